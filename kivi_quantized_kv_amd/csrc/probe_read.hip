// Streaming-read probe: a plain kernel that reads every 16-byte vector of up
// to 16 device buffers once (non-temporal loads; all threads sweep one buffer
// after the other, grid-stride, U loads in flight per thread) and writes one
// word per thread, so that the loads stay live.  The benchmark times it on a
// cache's own buffers: a measured read ceiling for those bytes and that
// layout, beside the decode-attention call.  A measurement aid, built as its
// own library (libkvq_probe.so); it is not part of the kvq C ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kMaxBufs = 16;
struct ReadSet {
  const uint8_t* p[kMaxBufs];
  int64_t nv[kMaxBufs];   // 16-byte vectors per buffer
  int n;
};
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(512) void k_stream_read(ReadSet s, uint32_t* out) {
  const int64_t stride = int64_t(gridDim.x) * 512;
  const int64_t t0 = int64_t(blockIdx.x) * 512 + threadIdx.x;
  uint32_t acc = 0;
  for (int b = 0; b < s.n; ++b) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(s.p[b]);
    const int64_t nv = s.nv[b];
    int64_t i = t0;
    for (; i + (U - 1) * stride < nv; i += U * stride) {
      u32x4_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < nv; i += stride) {
      const u32x4_t v = __builtin_nontemporal_load(p + i);
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  out[t0] = acc;
}

}  // namespace

// Reads n <= 16 buffers (ptrs[i], bytes[i]: device pointers 16-byte aligned,
// sizes multiples of 16) with grid workgroups of 512 threads and u (4 or 8)
// loads in flight per thread; out: device memory of grid * 512 words,
// overwritten.  Returns 0, or a hipError_t value (hipErrorInvalidValue for
// bad arguments, nothing enqueued).
extern "C" int kvqprobe_stream_read(const void* const* ptrs, const int64_t* bytes, int n, void* out,
                                    int grid, int u, void* stream) {
  if (n < 1 || n > kMaxBufs || grid < 1 || out == nullptr || ptrs == nullptr || bytes == nullptr ||
      (u != 4 && u != 8))
    return int(hipErrorInvalidValue);
  ReadSet s{};
  s.n = n;
  for (int i = 0; i < n; ++i) {
    if (ptrs[i] == nullptr || bytes[i] < 0 || bytes[i] % 16 != 0 ||
        reinterpret_cast<uintptr_t>(ptrs[i]) % 16 != 0)
      return int(hipErrorInvalidValue);
    s.p[i] = static_cast<const uint8_t*>(ptrs[i]);
    s.nv[i] = bytes[i] / 16;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (u == 4)
    hipLaunchKernelGGL(k_stream_read<4>, dim3(grid), dim3(512), 0, st, s, static_cast<uint32_t*>(out));
  else
    hipLaunchKernelGGL(k_stream_read<8>, dim3(grid), dim3(512), 0, st, s, static_cast<uint32_t*>(out));
  return int(hipGetLastError());
}
