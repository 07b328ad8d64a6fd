// Explicit instantiations of the GQA-grouped VALU decode kernel (templates
// in kvq_gqa_impl.h): pre-RoPE keys with side tables, every width.
#include "kvq_gqa_impl.h"

namespace kvq {

#define KVQ_GQA_INST(DT, D, BITS, MODE)                                                       \
  template hipError_t launch_attn_gqa<DT, D, BITS, MODE>(const AttnArgs&, int, hipStream_t);  \
  template int attn_gqa_blocks_per_cu<DT, D, BITS, MODE>();
#define KVQ_GQA_INST_W(BITS, MODE)                                                              \
  KVQ_GQA_INST(DT_F32, 64, BITS, MODE) KVQ_GQA_INST(DT_F32, 128, BITS, MODE)                  \
  KVQ_GQA_INST(DT_F16, 64, BITS, MODE) KVQ_GQA_INST(DT_F16, 128, BITS, MODE)                  \
  KVQ_GQA_INST(DT_BF16, 64, BITS, MODE) KVQ_GQA_INST(DT_BF16, 128, BITS, MODE)

KVQ_GQA_INST_W(1, 3)
KVQ_GQA_INST_W(2, 3)
KVQ_GQA_INST_W(3, 3)
KVQ_GQA_INST_W(4, 3)
KVQ_GQA_INST_W(5, 3)
KVQ_GQA_INST_W(6, 3)
KVQ_GQA_INST_W(7, 3)
KVQ_GQA_INST_W(8, 3)

}  // namespace kvq
