// Explicit instantiations of the VALU decode kernel (templates in
// kvq_attn_impl.h) for pre-RoPE keys (with and without side tables), 1, 3, 5, 6 and 7 bits.
#include "kvq_attn_impl.h"

namespace kvq {

#define KVQ_VALU_INST(DT, D, BITS, MODE)                                                       \
  template hipError_t launch_attn_valu<DT, D, BITS, MODE>(const AttnArgs&, int, hipStream_t);  \
  template int attn_valu_blocks_per_cu<DT, D, BITS, MODE>();
#define KVQ_VALU_INST_W(BITS, MODE)                                                              \
  KVQ_VALU_INST(DT_F32, 64, BITS, MODE) KVQ_VALU_INST(DT_F32, 128, BITS, MODE)                 \
  KVQ_VALU_INST(DT_F16, 64, BITS, MODE) KVQ_VALU_INST(DT_F16, 128, BITS, MODE)                 \
  KVQ_VALU_INST(DT_BF16, 64, BITS, MODE) KVQ_VALU_INST(DT_BF16, 128, BITS, MODE)
KVQ_VALU_INST_W(1, 2) KVQ_VALU_INST_W(1, 3)
KVQ_VALU_INST_W(3, 2) KVQ_VALU_INST_W(3, 3)
KVQ_VALU_INST_W(5, 2) KVQ_VALU_INST_W(5, 3)
KVQ_VALU_INST_W(6, 2) KVQ_VALU_INST_W(6, 3)
KVQ_VALU_INST_W(7, 2) KVQ_VALU_INST_W(7, 3)

}  // namespace kvq
