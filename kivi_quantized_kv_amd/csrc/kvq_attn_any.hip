// Explicit instantiations of the VALU decode kernel and the split merge
// (templates in kvq_attn_impl.h) for 1, 3, 5, 6 and 7 bits (codes read as a bit stream).
#include "kvq_attn_impl.h"

namespace kvq {

#define KVQ_VALU_INST(DT, D, BITS)                                                      \
  template hipError_t launch_attn_valu<DT, D, BITS>(const AttnArgs&, int, hipStream_t); \
  template int attn_valu_blocks_per_cu<DT, D, BITS>();                                 \
  template bool attn_valu_direct_ok<DT, D, BITS>();
#define KVQ_VALU_INST_W(BITS)                                                            \
  KVQ_VALU_INST(DT_F32, 64, BITS) KVQ_VALU_INST(DT_F32, 128, BITS)                     \
  KVQ_VALU_INST(DT_F16, 64, BITS) KVQ_VALU_INST(DT_F16, 128, BITS)                     \
  KVQ_VALU_INST(DT_BF16, 64, BITS) KVQ_VALU_INST(DT_BF16, 128, BITS)

KVQ_VALU_INST_W(1)
KVQ_VALU_INST_W(3)
KVQ_VALU_INST_W(5)
KVQ_VALU_INST_W(6)
KVQ_VALU_INST_W(7)

}  // namespace kvq
