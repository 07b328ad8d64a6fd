// Explicit instantiations of the quantize kernels (templates in
// kvq_quant_impl.h) for the widths whose codes fill whole bytes (2, 4 and 8
// bits).
#include "kvq_quant_impl.h"

namespace kvq {

#define KVQ_QUANT_INST(DT, D, BITS)                                                        \
  template hipError_t launch_quant_keys<DT, D, BITS>(const QuantArgs&, int64_t, int, int, hipStream_t); \
  template hipError_t launch_quant_values<DT, D, BITS>(const QuantArgs&, int64_t, int, int, hipStream_t); \
  template hipError_t launch_append<DT, D, BITS>(const AppendArgs&, int, int, hipStream_t);
#define KVQ_QUANT_INST_W(BITS)                                                             \
  KVQ_QUANT_INST(DT_F32, 64, BITS) KVQ_QUANT_INST(DT_F32, 128, BITS)                     \
  KVQ_QUANT_INST(DT_F16, 64, BITS) KVQ_QUANT_INST(DT_F16, 128, BITS)                     \
  KVQ_QUANT_INST(DT_BF16, 64, BITS) KVQ_QUANT_INST(DT_BF16, 128, BITS)

KVQ_QUANT_INST_W(2)
KVQ_QUANT_INST_W(4)
KVQ_QUANT_INST_W(8)

}  // namespace kvq
