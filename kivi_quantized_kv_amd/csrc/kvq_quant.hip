// Quantize-and-pack kernels: prefill of keys (per channel over G-token
// groups) and values (per token), and the streaming append with its group
// freeze.  Method: pigeon guide "KV-cache quantization", How it works steps
// 1-4; tract PR "quantized KV-cache storage op (int8/int4)" (frozen
// fixed-size key blocks, values per token, sinks kept exact).
#include "kvq_kernels.h"

namespace kvq {

// ----------------------------------------------------------------------------
// Key group: per-channel min/max over the G rows of an fp32 LDS tile, then
// delta / zero point and the packed rows.  256 threads.
// ----------------------------------------------------------------------------
template <int D, int BITS>
__device__ void key_group_from_tile(const float* tile, int G, float* s_red, float* s_delta,
                                    float* s_zp, float* k_scale, float* k_zero,
                                    uint8_t* code_rows) {
  constexpr float kLevels = float((1 << BITS) - 1);
  constexpr int kSeg = 256 / D;  // threads per channel
  const int t = threadIdx.x;
  const int c = t % D, seg = t / D;
  float mn = __builtin_inff(), mx = -__builtin_inff();
  for (int r = seg; r < G; r += kSeg) {
    float x = tile[r * D + c];
    mn = __builtin_fminf(mn, x);
    mx = __builtin_fmaxf(mx, x);
  }
  s_red[seg * D + c] = mn;
  s_red[(kSeg + seg) * D + c] = mx;
  __syncthreads();
  if (t < D) {
#pragma unroll
    for (int k = 1; k < kSeg; ++k) {
      mn = __builtin_fminf(mn, s_red[k * D + t]);
      mx = __builtin_fmaxf(mx, s_red[(kSeg + k) * D + t]);
    }
    float delta, zp;
    affine_params(mn, mx, kLevels, delta, zp);
    s_delta[t] = delta;
    s_zp[t] = zp;
    k_scale[t] = delta;
    k_zero[t] = zp;
  }
  __syncthreads();
  constexpr int kPerWord = 32 / BITS;
  constexpr int kWordsPerRow = D * BITS / 32;
  uint32_t* rows = reinterpret_cast<uint32_t*>(code_rows);
  for (int w = t; w < G * kWordsPerRow; w += 256) {
    const int r = w / kWordsPerRow, wi = w % kWordsPerRow;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < kPerWord; ++i) {
      const int ch = wi * kPerWord + i;
      word |= affine_code(tile[r * D + ch], s_delta[ch], s_zp[ch], kLevels) << (BITS * i);
    }
    rows[w] = word;
  }
}

// ----------------------------------------------------------------------------
// Value tokens [u0, u0 + n) (u0 and n multiples of 32) from an fp32 LDS
// tile: per-token min/max by wave reductions, delta / zero point, and the
// bytes of the value-code units that hold these tokens.  256 threads.
// ----------------------------------------------------------------------------
template <int D, int BITS>
__device__ void value_tokens_from_tile(const float* tile, int64_t u0, int n, float* s_delta,
                                       float* s_zp, float* v_scale, float* v_zero,
                                       uint8_t* v_codes_head) {
  constexpr float kLevels = float((1 << BITS) - 1);
  using VL = VLayout<BITS>;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int i = wave; i < n; i += 4) {
    float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
    for (int c = lane; c < D; c += 64) {
      float x = tile[i * D + c];
      mn = __builtin_fminf(mn, x);
      mx = __builtin_fmaxf(mx, x);
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
      float delta, zp;
      affine_params(mn, mx, kLevels, delta, zp);
      s_delta[i] = delta;
      s_zp[i] = zp;
      v_scale[u0 + i] = delta;
      v_zero[u0 + i] = zp;
    }
  }
  __syncthreads();
  const int64_t blk0 = u0 / VL::L;
  const int64_t blk1 = (u0 + n + VL::L - 1) / VL::L;
  const int units = int(blk1 - blk0) * 4 * D;
  for (int x = t; x < units; x += 256) {
    const int64_t blk = blk0 + x / (4 * D);
    const int uin = x % (4 * D);
    const int g = uin / (16 * (D / 16));
    const int rem = uin % (16 * (D / 16));
    const int j = rem / (D / 16), nn = rem % (D / 16);
    const int d = nn * 16 + j;
    uint64_t bits = 0;
    uint32_t step_in = 0;  // bit s set when 32-token step s of the block is in range
#pragma unroll
    for (int i = 0; i < VL::U; ++i) {
      const int o = vslot_token<BITS>(g, i);
      const int64_t u = blk * VL::L + o;
      if (u >= u0 && u < u0 + n) {
        const int li = int(u - u0);
        bits |= uint64_t(affine_code(tile[li * D + d], s_delta[li], s_zp[li], kLevels))
                << (BITS * i);
        step_in |= 1u << (o / 32);
      }
    }
    uint8_t* dst = v_codes_head + (blk * 4 * D + uin) * VL::UB;
    const uint32_t all_steps = (1u << (VL::L / 32)) - 1;
    if (step_in == all_steps) {
      if constexpr (VL::UB == 8) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(uint32_t(bits), uint32_t(bits >> 32));
      } else {
        *reinterpret_cast<uint32_t*>(dst) = uint32_t(bits);
      }
    } else {
      // partial block (2-bit codes): byte k holds slots 4k..4k+3, step k % 2
#pragma unroll
      for (int k = 0; k < VL::UB; ++k) {
        const int s = (4 * k >> 2) % (VL::U / 8);
        if (step_in & (1u << s)) dst[k] = uint8_t(bits >> (8 * k));
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Prefill kernels
// ----------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(64) void k_copy_fp_rows(FpCopyArgs a) {
  // grid: x = fp row (sinks first, then residual tokens), y = head, z = batch
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t row = blockIdx.x;
  const int64_t tok = row < a.n_sink ? row : a.first_resid + (row - a.n_sink);
  constexpr int EB = Elem<DT>::bytes;
  const uint8_t* src = reinterpret_cast<const uint8_t*>(a.src) +
                       (b * a.sb + h * a.sh + tok * a.st) * EB;
  uint8_t* dst;
  if (tok < a.S) {
    dst = reinterpret_cast<uint8_t*>(a.sink) + ((int64_t(b) * a.H + h) * a.S + tok) * D * EB;
  } else {
    const int64_t slot = (tok - a.S) % a.ring;
    dst = reinterpret_cast<uint8_t*>(a.resid) + ((int64_t(b) * a.H + h) * a.ring + slot) * D * EB;
  }
  constexpr int kVec = D * EB / 16;  // 16-byte vectors per row
  for (int v = threadIdx.x; v < kVec; v += 64)
    reinterpret_cast<uint4*>(dst)[v] = reinterpret_cast<const uint4*>(src)[v];
}

template <int DT, int D>
__device__ void load_rows_to_tile(const void* base, int64_t row0_elem, int64_t stride_t, int rows,
                                  int rows_valid, float* tile) {
  constexpr int kV = D / 4;
  for (int x = threadIdx.x; x < rows * kV; x += blockDim.x) {
    const int r = x / kV, c4 = x % kV;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (r < rows_valid) load4<DT>(base, row0_elem + r * stride_t + c4 * 4, v);
#pragma unroll
    for (int k = 0; k < 4; ++k) tile[r * D + c4 * 4 + k] = v[k];
  }
}

template <int DT, int D, int BITS>
__global__ __launch_bounds__(256) void k_quant_keys(QuantArgs a) {
  // grid: x = key group k, y = head, z = batch
  extern __shared__ float smem[];
  const int G = a.G;
  float* tile = smem;                       // G * D
  float* s_red = tile + G * D;              // 2 * (256/D) * D
  float* s_delta = s_red + 2 * 256;         // D
  float* s_zp = s_delta + D;                // D
  const int64_t k = blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t row0 = b * a.sb + h * a.sh + (a.S + k * G) * a.st;
  load_rows_to_tile<DT, D>(a.src, row0, a.st, G, G, tile);
  __syncthreads();
  const int64_t bh = int64_t(b) * a.H + h;
  float* ks = a.scale + (bh * (a.qcap / G) + k) * D;
  float* kz = a.zero + (bh * (a.qcap / G) + k) * D;
  uint8_t* rows = a.codes + (bh * a.qcap + k * G) * (D * BITS / 8);
  key_group_from_tile<D, BITS>(tile, G, s_red, s_delta, s_zp, ks, kz, rows);
}

template <int DT, int D, int BITS>
__global__ __launch_bounds__(256) void k_quant_values(QuantArgs a) {
  // grid: x = 32-token step of the quantized range, y = head, z = batch
  __shared__ float tile[32 * D];
  __shared__ float s_delta[32], s_zp[32];
  const int64_t u0 = int64_t(blockIdx.x) * 32;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t row0 = b * a.sb + h * a.sh + (a.S + u0) * a.st;
  load_rows_to_tile<DT, D>(a.src, row0, a.st, 32, 32, tile);
  __syncthreads();
  const int64_t bh = int64_t(b) * a.H + h;
  value_tokens_from_tile<D, BITS>(tile, u0, 32, s_delta, s_zp, a.scale + bh * a.qcap,
                                  a.zero + bh * a.qcap,
                                  a.codes + bh * (a.qcap * D * BITS / 8));
}

// ----------------------------------------------------------------------------
// Streaming append: write token t = n_before to its sink or ring slot; when
// the full-precision count reaches R + G, quantize and freeze the oldest G
// ring tokens as the next key group and G value tokens.
// ----------------------------------------------------------------------------
template <int DT, int D, int BITS>
__global__ __launch_bounds__(256) void k_append(AppendArgs a) {
  // grid: y = head, z = batch
  extern __shared__ float smem[];
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = int64_t(b) * a.H + h;
  constexpr int EB = Elem<DT>::bytes;
  const int64_t t = a.n_before;
  const int64_t ring = a.R + a.G;
  // 1) the new token, K and V
  {
    const uint8_t* ks = reinterpret_cast<const uint8_t*>(a.k_new) + (b * a.k_sb + h * a.k_sh) * EB;
    const uint8_t* vs = reinterpret_cast<const uint8_t*>(a.v_new) + (b * a.v_sb + h * a.v_sh) * EB;
    uint8_t *kd, *vd;
    if (t < a.S) {
      kd = reinterpret_cast<uint8_t*>(a.k_sink) + (bh * a.S + t) * D * EB;
      vd = reinterpret_cast<uint8_t*>(a.v_sink) + (bh * a.S + t) * D * EB;
    } else {
      const int64_t slot = (t - a.S) % ring;
      kd = reinterpret_cast<uint8_t*>(a.k_resid) + (bh * ring + slot) * D * EB;
      vd = reinterpret_cast<uint8_t*>(a.v_resid) + (bh * ring + slot) * D * EB;
    }
    constexpr int kVec = D * EB / 16;
    for (int v = threadIdx.x; v < 2 * kVec; v += blockDim.x) {
      if (v < kVec)
        reinterpret_cast<uint4*>(kd)[v] = reinterpret_cast<const uint4*>(ks)[v];
      else
        reinterpret_cast<uint4*>(vd)[v - kVec] = reinterpret_cast<const uint4*>(vs)[v - kVec];
    }
  }
  if (!a.flush) return;
  // 2) flush: tokens S + q_old .. S + q_old + G - 1, read from their ring
  // slots except the new token itself, which is read from the input (it may
  // be part of the group when R == 0).
  const int G = a.G;
  float* ktile = smem;                  // G * D
  float* vtile = ktile + G * D;         // G * D
  float* s_red = vtile + G * D;         // 512
  float* s_delta = s_red + 512;         // max(D, G)
  float* s_zp = s_delta + 128;          // max(D, G)
  constexpr int kV = D / 4;
  for (int x = threadIdx.x; x < G * kV; x += blockDim.x) {
    const int r = x / kV, c4 = x % kV;
    const int64_t tok = a.S + a.q_old + r;
    float kv4[4], vv4[4];
    if (tok == t) {
      load4<DT>(a.k_new, b * a.k_sb + h * a.k_sh + c4 * 4, kv4);
      load4<DT>(a.v_new, b * a.v_sb + h * a.v_sh + c4 * 4, vv4);
    } else {
      const int64_t slot = (tok - a.S) % ring;
      load4<DT>(a.k_resid, (bh * ring + slot) * D + c4 * 4, kv4);
      load4<DT>(a.v_resid, (bh * ring + slot) * D + c4 * 4, vv4);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ktile[r * D + c4 * 4 + k] = kv4[k];
      vtile[r * D + c4 * 4 + k] = vv4[k];
    }
  }
  __syncthreads();
  const int64_t kgrp = a.q_old / G;
  float* ks = a.k_scale + (bh * (a.qcap / G) + kgrp) * D;
  float* kz = a.k_zero + (bh * (a.qcap / G) + kgrp) * D;
  uint8_t* rows = a.k_codes + (bh * a.qcap + a.q_old) * (D * BITS / 8);
  key_group_from_tile<D, BITS>(ktile, G, s_red, s_delta, s_zp, ks, kz, rows);
  __syncthreads();
  value_tokens_from_tile<D, BITS>(vtile, a.q_old, G, s_delta, s_zp, a.v_scale + bh * a.qcap,
                                  a.v_zero + bh * a.qcap,
                                  a.v_codes + bh * (a.qcap * D * BITS / 8));
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------
template <int DT, int D, int BITS>
hipError_t launch_quant_keys(const QuantArgs& a, int64_t n_groups, int B, int H, hipStream_t s) {
  size_t lds = (size_t(a.G) * D + 2 * 256 + 2 * D) * sizeof(float);
  hipLaunchKernelGGL((k_quant_keys<DT, D, BITS>), dim3(unsigned(n_groups), H, B), dim3(256), lds,
                     s, a);
  return hipGetLastError();
}
template <int DT, int D, int BITS>
hipError_t launch_quant_values(const QuantArgs& a, int64_t n_steps, int B, int H, hipStream_t s) {
  hipLaunchKernelGGL((k_quant_values<DT, D, BITS>), dim3(unsigned(n_steps), H, B), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}
template <int DT, int D>
hipError_t launch_copy_fp(const FpCopyArgs& a, int64_t n_rows, int B, int H, hipStream_t s) {
  hipLaunchKernelGGL((k_copy_fp_rows<DT, D>), dim3(unsigned(n_rows), H, B), dim3(64), 0, s, a);
  return hipGetLastError();
}
template <int DT, int D, int BITS>
hipError_t launch_append(const AppendArgs& a, int B, int H, hipStream_t s) {
  size_t lds = a.flush ? (size_t(2) * a.G * D + 512 + 256) * sizeof(float) : 0;
  hipLaunchKernelGGL((k_append<DT, D, BITS>), dim3(1, H, B), dim3(256), lds, s, a);
  return hipGetLastError();
}

#define KVQ_DISPATCH_DT_D_BITS(FN, ...)                                              \
  template hipError_t FN<DT_F32, 64, 2>(__VA_ARGS__);                                \
  template hipError_t FN<DT_F32, 64, 4>(__VA_ARGS__);                                \
  template hipError_t FN<DT_F32, 64, 8>(__VA_ARGS__);                                \
  template hipError_t FN<DT_F32, 128, 2>(__VA_ARGS__);                               \
  template hipError_t FN<DT_F32, 128, 4>(__VA_ARGS__);                               \
  template hipError_t FN<DT_F32, 128, 8>(__VA_ARGS__);                               \
  template hipError_t FN<DT_F16, 64, 2>(__VA_ARGS__);                                \
  template hipError_t FN<DT_F16, 64, 4>(__VA_ARGS__);                                \
  template hipError_t FN<DT_F16, 64, 8>(__VA_ARGS__);                                \
  template hipError_t FN<DT_F16, 128, 2>(__VA_ARGS__);                               \
  template hipError_t FN<DT_F16, 128, 4>(__VA_ARGS__);                               \
  template hipError_t FN<DT_F16, 128, 8>(__VA_ARGS__);                               \
  template hipError_t FN<DT_BF16, 64, 2>(__VA_ARGS__);                               \
  template hipError_t FN<DT_BF16, 64, 4>(__VA_ARGS__);                               \
  template hipError_t FN<DT_BF16, 64, 8>(__VA_ARGS__);                               \
  template hipError_t FN<DT_BF16, 128, 2>(__VA_ARGS__);                              \
  template hipError_t FN<DT_BF16, 128, 4>(__VA_ARGS__);                              \
  template hipError_t FN<DT_BF16, 128, 8>(__VA_ARGS__);

KVQ_DISPATCH_DT_D_BITS(launch_quant_keys, const QuantArgs&, int64_t, int, int, hipStream_t)
KVQ_DISPATCH_DT_D_BITS(launch_quant_values, const QuantArgs&, int64_t, int, int, hipStream_t)
KVQ_DISPATCH_DT_D_BITS(launch_append, const AppendArgs&, int, int, hipStream_t)

template hipError_t launch_copy_fp<DT_F32, 64>(const FpCopyArgs&, int64_t, int, int, hipStream_t);
template hipError_t launch_copy_fp<DT_F32, 128>(const FpCopyArgs&, int64_t, int, int, hipStream_t);
template hipError_t launch_copy_fp<DT_F16, 64>(const FpCopyArgs&, int64_t, int, int, hipStream_t);
template hipError_t launch_copy_fp<DT_F16, 128>(const FpCopyArgs&, int64_t, int, int, hipStream_t);
template hipError_t launch_copy_fp<DT_BF16, 64>(const FpCopyArgs&, int64_t, int, int, hipStream_t);
template hipError_t launch_copy_fp<DT_BF16, 128>(const FpCopyArgs&, int64_t, int, int, hipStream_t);

}  // namespace kvq
