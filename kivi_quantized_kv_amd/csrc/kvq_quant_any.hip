// Explicit instantiations of the quantize kernels (templates in
// kvq_quant_impl.h) for 1 bit and the widths whose codes straddle bytes (3, 5, 6 and 7 bits).
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

KVQ_QUANT_INST_W(1)
KVQ_QUANT_INST_W(3)
KVQ_QUANT_INST_W(5)
KVQ_QUANT_INST_W(6)
KVQ_QUANT_INST_W(7)

}  // namespace kvq
