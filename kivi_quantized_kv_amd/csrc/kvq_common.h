// Device-side helpers shared by the libkvq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

constexpr int kWave = 64;

// ---------------------------------------------------------------- dtypes
template <int DT> struct Elem;
template <> struct Elem<DT_F32> { using T = float; static constexpr int bytes = 4; };
template <> struct Elem<DT_F16> { using T = uint16_t; static constexpr int bytes = 2; };
template <> struct Elem<DT_BF16> { using T = uint16_t; static constexpr int bytes = 2; };

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
// Through the bf16 type rather than a bit cast: the same shift, but the
// compiler then knows the value is canonical and adds no canonicalization
// before min / max (the inputs are finite, so the two agree bit for bit).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(__bf16, (uint16_t)h);
}

// Four consecutive elements at element index `i` (16-byte aligned for f32,
// 8-byte aligned for 16-bit types), widened exactly to fp32.
template <int DT>
__device__ __forceinline__ void load4(const void* base, int64_t i, float out[4]) {
  if constexpr (DT == DT_F32) {
    float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + i);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  } else {
    uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + i);
    uint32_t w[4] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      out[k] = (DT == DT_F16) ? f16_bits_to_f32(w[k]) : bf16_bits_to_f32(w[k]);
  }
}

template <int DT>
__device__ __forceinline__ float load1(const void* base, int64_t i) {
  if constexpr (DT == DT_F32) {
    return reinterpret_cast<const float*>(base)[i];
  } else {
    uint32_t w = reinterpret_cast<const uint16_t*>(base)[i];
    return (DT == DT_F16) ? f16_bits_to_f32(w) : bf16_bits_to_f32(w);
  }
}

// ---------------------------------------------------------------- quantizer
// delta = fl32(fl32(max - min) / (2^b - 1)), zero point = min + 0.0f, and
// code = clamp(rint(fl32(fl32(x - zp) / delta)), 0, 2^b - 1) with a
// correctly rounded IEEE division (pigeon guide "KV-cache quantization",
// How it works step 3; round half to even as numpy's round in its Source
// code section).
__device__ __forceinline__ void affine_params(float mn, float mx, float levels, float& delta,
                                              float& zp) {
  delta = __fdiv_rn((mx - mn) + 0.0f, levels);   // a range of zeros of either signs: +0
  zp = mn + 0.0f;
}

__device__ __forceinline__ uint32_t affine_code(float x, float delta, float zp, float levels) {
  if (delta == 0.0f) return 0u;
  float q = __fdiv_rn(x - zp, delta);
  float r = __builtin_rintf(q);
  r = __builtin_fminf(__builtin_fmaxf(r, 0.0f), levels);
  return (uint32_t)r;
}

// ---------------------------------------------------------------- wave ops
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Row rotation with bound_ctrl set: every lane has a source in a rotation,
// and the form lets the compiler fold the move into the consuming add.
template <int CTRL>
__device__ __forceinline__ float dpp_rot(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

__device__ __forceinline__ float swz_xor16(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}
__device__ __forceinline__ float xor32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                       (int)((threadIdx.x ^ 32u) & 63u) << 2, __builtin_bit_cast(int, v)));
}

// v combined with its partner lane l ^ 16 / l ^ 32 by a symmetric op, on
// the VALU: the gfx950 permlane swaps with both operands holding v leave
// {own, partner} in the two results, in lane-dependent order.  The second
// operand and both results pass through empty asm statements: the compiler
// otherwise takes the two results of such a swap to be equal.
__device__ __forceinline__ float opaque_f(unsigned u) {
  asm volatile("" : "+v"(u));
  return __builtin_bit_cast(float, u);
}
template <bool X32>
__device__ __forceinline__ void partner_pair(float v, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  unsigned w = u;
  asm volatile("" : "+v"(w));
  if constexpr (X32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, w, false, false);
    a = opaque_f(r[0]);
    b = opaque_f(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(u, w, false, false);
    a = opaque_f(r[0]);
    b = opaque_f(r[1]);
  }
}
__device__ __forceinline__ float max_xor16(float v) {
  float a, b;
  partner_pair<false>(v, a, b);
  return __builtin_fmaxf(a, b);
}
__device__ __forceinline__ float max_xor32(float v) {
  float a, b;
  partner_pair<true>(v, a, b);
  return __builtin_fmaxf(a, b);
}
__device__ __forceinline__ float sum_xor16(float v) {
  float a, b;
  partner_pair<false>(v, a, b);
  return a + b;
}
__device__ __forceinline__ float sum_xor32(float v) {
  float a, b;
  partner_pair<true>(v, a, b);
  return a + b;
}

// All-reduce over the 4 lanes of a quad.
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp_mov<kQuadXor1>(v);
  v += dpp_mov<kQuadXor2>(v);
  return v;
}
// All-reduce over the 16 lanes of a row.
__device__ __forceinline__ float row_max(float v) {
  v = __builtin_fmaxf(v, dpp_mov<kQuadXor1>(v));
  v = __builtin_fmaxf(v, dpp_mov<kQuadXor2>(v));
  v = __builtin_fmaxf(v, dpp_mov<kRowRor4>(v));
  v = __builtin_fmaxf(v, dpp_mov<kRowRor8>(v));
  return v;
}
__device__ __forceinline__ float row_min(float v) {
  v = __builtin_fminf(v, dpp_mov<kQuadXor1>(v));
  v = __builtin_fminf(v, dpp_mov<kQuadXor2>(v));
  v = __builtin_fminf(v, dpp_mov<kRowRor4>(v));
  v = __builtin_fminf(v, dpp_mov<kRowRor8>(v));
  return v;
}
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_mov<kQuadXor1>(v);
  v += dpp_mov<kQuadXor2>(v);
  v += dpp_mov<kRowRor4>(v);
  v += dpp_mov<kRowRor8>(v);
  return v;
}
// All-reduce over the whole wave (rows of 16 joined by swizzle / permute).
__device__ __forceinline__ float wave_max(float v) {
  v = row_max(v);
  v = __builtin_fmaxf(v, swz_xor16(v));
  return __builtin_fmaxf(v, xor32(v));
}
__device__ __forceinline__ float wave_min(float v) {
  v = row_min(v);
  v = __builtin_fminf(v, swz_xor16(v));
  return __builtin_fminf(v, xor32(v));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum(v);
  v += swz_xor16(v);
  return v + xor32(v);
}

// Order this lane's earlier LDS writes before its later LDS reads, for
// exchanges between lanes of one wave (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- partition
// With n = max(0, T - S): Q = G * floor((n - R) / G) if n >= R, else 0.
__host__ __device__ __forceinline__ int64_t quantized_count(int64_t T, int64_t S, int64_t R,
                                                            int64_t G) {
  int64_t n = T - S;
  if (n < 0) n = 0;
  return n >= R ? G * ((n - R) / G) : 0;
}

// ---------------------------------------------------------------- value layout
// Tokens per value-code block, codes per unit, bytes per unit.
template <int BITS> struct VLayout {
  static constexpr int L = (BITS == 2) ? 64 : 32;
  static constexpr int U = (BITS == 2) ? 16 : 8;
  static constexpr int UB = U * BITS / 8;  // 4, 4, 8
};
// Token offset inside a block held by code slot i of a lane-group-g unit:
// slot i = r + 4*s + (U/2)*h  <->  o = 32*s + 16*h + 4*g + r.
template <int BITS>
__host__ __device__ constexpr int vslot_token(int g, int i) {
  constexpr int U = VLayout<BITS>::U;
  int r = i & 3;
  int h = i / (U / 2);
  int s = (i >> 2) % (U / 8);
  return 32 * s + 16 * h + 4 * g + r;
}

}  // namespace kvq
