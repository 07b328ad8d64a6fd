// Explicit instantiations of the VALU decode kernel (templates in
// kvq_attn_impl.h) for 1, 3, 5, 6 and 7 bits (codes read as a bit stream), plain caches and caches with side tables.
#include "kvq_attn_impl.h"

namespace kvq {

#define KVQ_VALU_INST(DT, D, BITS, MODE)                                                       \
  template hipError_t launch_attn_valu<DT, D, BITS, MODE>(const AttnArgs&, int, hipStream_t);  \
  template int attn_valu_blocks_per_cu<DT, D, BITS, MODE>();
#define KVQ_VALU_INST_W(BITS, MODE)                                                              \
  KVQ_VALU_INST(DT_F32, 64, BITS, MODE) KVQ_VALU_INST(DT_F32, 128, BITS, MODE)                 \
  KVQ_VALU_INST(DT_F16, 64, BITS, MODE) KVQ_VALU_INST(DT_F16, 128, BITS, MODE)                 \
  KVQ_VALU_INST(DT_BF16, 64, BITS, MODE) KVQ_VALU_INST(DT_BF16, 128, BITS, MODE)
#define KVQ_DIRECT_INST(BITS)                                                                    \
  template bool attn_valu_direct_ok<DT_F32, 64, BITS>();                                         \
  template bool attn_valu_direct_ok<DT_F32, 128, BITS>();                                        \
  template bool attn_valu_direct_ok<DT_F16, 64, BITS>();                                         \
  template bool attn_valu_direct_ok<DT_F16, 128, BITS>();                                        \
  template bool attn_valu_direct_ok<DT_BF16, 64, BITS>();                                        \
  template bool attn_valu_direct_ok<DT_BF16, 128, BITS>();

KVQ_VALU_INST_W(1, 0) KVQ_VALU_INST_W(1, 1) KVQ_DIRECT_INST(1)
KVQ_VALU_INST_W(3, 0) KVQ_VALU_INST_W(3, 1) KVQ_DIRECT_INST(3)
KVQ_VALU_INST_W(5, 0) KVQ_VALU_INST_W(5, 1) KVQ_DIRECT_INST(5)
KVQ_VALU_INST_W(6, 0) KVQ_VALU_INST_W(6, 1) KVQ_DIRECT_INST(6)
KVQ_VALU_INST_W(7, 0) KVQ_VALU_INST_W(7, 1) KVQ_DIRECT_INST(7)

}  // namespace kvq
