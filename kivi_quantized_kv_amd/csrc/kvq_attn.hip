// Explicit instantiations of the VALU decode kernel and the split merge (templates in
// kvq_attn_impl.h) for 2, 4 and 8 bits, plain caches and caches with side tables.
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

KVQ_VALU_INST_W(2, 0) KVQ_VALU_INST_W(2, 1) KVQ_DIRECT_INST(2)
KVQ_VALU_INST_W(4, 0) KVQ_VALU_INST_W(4, 1) KVQ_DIRECT_INST(4)
KVQ_VALU_INST_W(8, 0) KVQ_VALU_INST_W(8, 1) KVQ_DIRECT_INST(8)

#define KVQ_INST_MERGE(DT)                                                     \
  template hipError_t launch_merge<DT, 64>(const AttnArgs&, int, hipStream_t); \
  template hipError_t launch_merge<DT, 128>(const AttnArgs&, int, hipStream_t);
KVQ_INST_MERGE(DT_F32)
KVQ_INST_MERGE(DT_F16)
KVQ_INST_MERGE(DT_BF16)

}  // namespace kvq
