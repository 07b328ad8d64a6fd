// Explicit instantiations of the VALU decode kernel (templates in
// kvq_attn_impl.h) for pre-RoPE keys (with and without side tables), 2, 4 and 8 bits.
#include "kvq_attn_impl.h"

namespace kvq {

#define KVQ_VALU_INST(DT, D, BITS, MODE)                                                       \
  template hipError_t launch_attn_valu<DT, D, BITS, MODE>(const AttnArgs&, int, hipStream_t);  \
  template int attn_valu_blocks_per_cu<DT, D, BITS, MODE>();
#define KVQ_VALU_INST_W(BITS, MODE)                                                              \
  KVQ_VALU_INST(DT_F32, 64, BITS, MODE) KVQ_VALU_INST(DT_F32, 128, BITS, MODE)                 \
  KVQ_VALU_INST(DT_F16, 64, BITS, MODE) KVQ_VALU_INST(DT_F16, 128, BITS, MODE)                 \
  KVQ_VALU_INST(DT_BF16, 64, BITS, MODE) KVQ_VALU_INST(DT_BF16, 128, BITS, MODE)
KVQ_VALU_INST_W(2, 2) KVQ_VALU_INST_W(2, 3)
KVQ_VALU_INST_W(4, 2) KVQ_VALU_INST_W(4, 3)
KVQ_VALU_INST_W(8, 2) KVQ_VALU_INST_W(8, 3)

}  // namespace kvq
