// Quantize-and-pack kernels: prefill of keys (per channel over G-token
// groups) and values (per token), and the streaming append with its group
// freeze.  Method: pigeon guide "KV-cache quantization", How it works steps
// 1-4; tract PR "quantized KV-cache storage op (int8/int4)" (frozen
// fixed-size key blocks, values per token, sinks kept exact).
//
// Both halves work from registers: every thread loads 16-byte pieces of its
// rows up front, the min / max reductions run across lanes (DPP and the
// permlane swaps) with one small LDS step across waves, and codes go
// straight from registers to the packed rows.  The affine code of an
// element is rint(fl(fl(x - zp) / delta)) with a correctly rounded division;
// it is computed as rint(y), y = fl(fl(x - zp) * r) with r the hardware
// reciprocal of delta (within 2 ulp), which equals it unless y lies within
// |y| 2^-21 of a half integer (r, the product and the division's own
// rounding move the quotient by less than |y| 1.5 2^-22).  Since 0 <= y <=
// (2^b - 1)(1 + 2^-21), one band (2^b) 2^-21 wide around the half integers
// covers every element.  Inputs of few significant bits (bf16) put many
// quotients exactly on a half integer h; such an exact tie is recognised
// by the residual fma(-h, delta, x - zp), which is zero exactly when x - zp
// = h delta (delta >= 2^-125 keeps every nonzero residual representable),
// and takes rint(h).  Any other element in the band, or an element whose
// delta is below 2^-125 (kept off the reciprocal), takes the exact
// division; it runs once per element index of a wave that holds one.  The
// prefill and the freeze run the same group and step routines; only the
// row source differs (input tensor or residual ring).
#pragma once

#include "kvq_kernels.h"

namespace kvq {

// Minimum and maximum in the IEEE 754-2019 sense (-0 below +0; the inputs
// are finite): one gfx950 instruction each, with no canonicalization of
// operands that come from loads, LDS or cross-lane moves.
__device__ __forceinline__ float fmin2(float a, float b) { return __builtin_elementwise_minimum(a, b); }
__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// ----------------------------------------------------------------------------
// Row sources: the byte address of row r of the group / step being quantized.
// ----------------------------------------------------------------------------
struct InputRows {            // rows of the caller's [.., T, D] tensor
  const uint8_t* base;        // row 0
  int64_t stride;             // bytes between rows
  __device__ const uint8_t* row(int r) const { return base + r * stride; }
};
struct RingRows {             // tokens first .. first + n of the residual ring
  const uint8_t* ring;        // slot 0 of this (batch, head)
  const uint8_t* fresh;       // the token being appended (read from its input)
  int64_t slot0, ring_len;    // ring slot of row 0; slots in the ring
  int fresh_row;              // row index of the appended token, or -1
  int row_bytes;
  __device__ const uint8_t* row(int r) const {
    if (r == fresh_row) return fresh;
    int64_t s = slot0 + r;
    if (s >= ring_len) s -= ring_len;
    return ring + s * row_bytes;
  }
};

// 16 bytes of a row widened exactly to fp32 (4 or 8 elements).
template <int DT>
__device__ __forceinline__ void widen16(uint4 v, float* out) {
  if constexpr (DT == DT_F32) {
    out[0] = __builtin_bit_cast(float, v.x); out[1] = __builtin_bit_cast(float, v.y);
    out[2] = __builtin_bit_cast(float, v.z); out[3] = __builtin_bit_cast(float, v.w);
  } else {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      out[2 * k] = DT == DT_F16 ? f16_bits_to_f32(w[k] & 0xFFFFu) : bf16_bits_to_f32(w[k] & 0xFFFFu);
      out[2 * k + 1] = DT == DT_F16 ? f16_bits_to_f32(w[k] >> 16) : bf16_bits_to_f32(w[k] >> 16);
    }
  }
}

// Reciprocal used by affine_codes: 1 / delta within 2 ulp (v_rcp_f32), 0
// for delta == 0 (every code 0).  `exact` is set for a delta in (0, 2^-125).
__device__ __forceinline__ float code_rcp(float delta, bool& exact) {
  exact |= delta != 0.0f && !(delta >= 0x1p-125f);
  return delta == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(delta);
}

// Codes of n elements x[i] against per-element (delta, zero, 1/delta):
// guarded reciprocal first.  An element index for which some lane is in the
// band (or flagged `exact`) checks those lanes for exact ties, and the
// lanes holding any other such element run the exact division (the other
// lanes keep their codes; with none, the division is skipped).
template <int N, int BITS>
__device__ __forceinline__ void affine_codes(const float* x, const float* delta, const float* zp,
                                             const float* rcp, bool exact, uint32_t* code) {
  constexpr float levels = float((1 << BITS) - 1);
  constexpr float kBand = 0.5f - float(1 << BITS) * 0x1p-21f;
  const uint64_t ex = __builtin_amdgcn_ballot_w64(exact);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float a = x[i] - zp[i];
    const float y = a * rcp[i];
    const float r = __builtin_rintf(y);
    const float d = y - r;   // NaN for an infinite quotient: never in the band
    // clamped (one median): an entry kept exact in a side table lies
    // outside the dense range; y is never NaN (x - zp is finite for inputs
    // below 2^127, and the reciprocal is finite), an infinite y clamps too
    float ci = __builtin_amdgcn_fmed3f(r, 0.0f, levels);
    if ((__builtin_amdgcn_ballot_w64(__builtin_fabsf(d) >= kBand) | ex) != 0) {
      const bool near = exact || __builtin_fabsf(d) >= kBand;
      const float h = r + __builtin_copysignf(0.5f, d);   // the half integer next to y
      const bool tie = !exact && __builtin_fmaf(-h, delta[i], a) == 0.0f;
      if (near) {
        if (tie) {
          ci = __builtin_amdgcn_fmed3f(__builtin_rintf(h), 0.0f, levels);
        } else if (delta[i] != 0.0f) {
          ci = __builtin_amdgcn_fmed3f(__builtin_rintf(__fdiv_rn(a, delta[i])), 0.0f, levels);
        } else {
          ci = 0.0f;
        }
      }
    }
    code[i] = uint32_t(ci);
  }
}

// min / max of v and the v of the lane a DPP pattern selects, in one
// instruction (the move fused into the operation; inline assembly, as the
// compiler's min / max carry an operand canonicalization that blocks the
// fusion; the s_nop gives the two wait states a DPP read needs after the
// VALU write of its source, which the compiler does not see in the asm).  For finite inputs the result equals the IEEE minimum / maximum
// except that a +0 / -0 pair may give either zero: the reductions' callers
// take zp = mn + 0 and delta from (mx - mn) + 0, which are then the same.
#define KVQ_DPP_MINMAX(NAME, OP, CTRL)                                                             \
  __device__ __forceinline__ float NAME(float v) {                                                \
    float d;                                                                                       \
    asm volatile("s_nop 1\n\t" OP " %0, %1, %1 " CTRL " row_mask:0xf bank_mask:0xf" : "=v"(d) : "v"(v)); \
    return d;                                                                                      \
  }
KVQ_DPP_MINMAX(min_qx1, "v_min_f32_dpp", "quad_perm:[1,0,3,2]")
KVQ_DPP_MINMAX(max_qx1, "v_max_f32_dpp", "quad_perm:[1,0,3,2]")
KVQ_DPP_MINMAX(min_qx2, "v_min_f32_dpp", "quad_perm:[2,3,0,1]")
KVQ_DPP_MINMAX(max_qx2, "v_max_f32_dpp", "quad_perm:[2,3,0,1]")
KVQ_DPP_MINMAX(min_hmir, "v_min_f32_dpp", "row_half_mirror")
KVQ_DPP_MINMAX(max_hmir, "v_max_f32_dpp", "row_half_mirror")
KVQ_DPP_MINMAX(min_mir, "v_min_f32_dpp", "row_mirror")
KVQ_DPP_MINMAX(max_mir, "v_max_f32_dpp", "row_mirror")
#undef KVQ_DPP_MINMAX

// All-reduce of min and max over aligned runs of N consecutive lanes (N =
// 4, 8, 16 or 32).
template <int N>
__device__ __forceinline__ void minmax_run(float& mn, float& mx) {
  mn = min_qx1(mn);
  mx = max_qx1(mx);
  mn = min_qx2(mn);
  mx = max_qx2(mx);
  if constexpr (N >= 8) {
    mn = min_hmir(mn);   // quads of a half row meet
    mx = max_hmir(mx);
  }
  if constexpr (N >= 16) {
    mn = min_mir(mn);    // halves of a row meet
    mx = max_mir(mx);
  }
  if constexpr (N >= 32) {
    float a, b;
    partner_pair<false>(mn, a, b); mn = fmin2(a, b);
    partner_pair<false>(mx, a, b); mx = fmax2(a, b);
  }
}

// ----------------------------------------------------------------------------
// Dense-and-sparse split (pigeon guide "KV-cache quantization", KVQuant
// adds: outliers kept in a sparse side table).  A vector keeps at most one
// entry exact: the maximum or the minimum, whichever leaves the smaller
// range.  The reductions carry the two largest and two smallest entries,
// with multiplicity.
// ----------------------------------------------------------------------------
struct Ext2 {
  float lo1, lo2, hi1, hi2;   // lo1 <= lo2, hi1 >= hi2
};
__device__ __forceinline__ Ext2 ext2_of(float x) { return {x, __builtin_inff(), x, -__builtin_inff()}; }
__device__ __forceinline__ void ext2_add(Ext2& e, float x) {
  e.hi2 = fmax2(e.hi2, fmin2(e.hi1, x));
  e.hi1 = fmax2(e.hi1, x);
  e.lo2 = fmin2(e.lo2, fmax2(e.lo1, x));
  e.lo1 = fmin2(e.lo1, x);
}
__device__ __forceinline__ void ext2_merge(Ext2& e, const Ext2& o) {
  e.hi2 = fmax2(fmin2(e.hi1, o.hi1), fmax2(e.hi2, o.hi2));
  e.hi1 = fmax2(e.hi1, o.hi1);
  e.lo2 = fmin2(fmax2(e.lo1, o.lo1), fmin2(e.lo2, o.lo2));
  e.lo1 = fmin2(e.lo1, o.lo1);
}
template <int CTRL>
__device__ __forceinline__ void ext2_dpp_merge(Ext2& e) {
  const Ext2 o{dpp_mov<CTRL>(e.lo1), dpp_mov<CTRL>(e.lo2), dpp_mov<CTRL>(e.hi1), dpp_mov<CTRL>(e.hi2)};
  ext2_merge(e, o);
}
// ext2 all-reduce over aligned runs of N = 4, 8 or 16 lanes (as minmax_run)
template <int N>
__device__ __forceinline__ void ext2_run(Ext2& e) {
  ext2_dpp_merge<kQuadXor1>(e);
  ext2_dpp_merge<kQuadXor2>(e);
  if constexpr (N >= 8) ext2_dpp_merge<0x141>(e);   // half-row mirror
  if constexpr (N >= 16) ext2_dpp_merge<0x140>(e);   // row mirror
}
// The dense range [lo, hi] and the kept entry's value kv; returns 1 (the
// maximum kept), -1 (the minimum) or 0 (none: neither removal shrinks the
// range).  Gaps in fp32; a tie keeps the maximum.
__device__ __forceinline__ int dense_split(const Ext2& e, float& lo, float& hi, float& kv) {
  const float gh = e.hi1 - e.hi2, gl = e.lo2 - e.lo1;
  const bool th = gh >= gl && gh > 0.0f;
  const bool tl = !th && gl > 0.0f;
  lo = tl ? e.lo2 : e.lo1;
  hi = th ? e.hi2 : e.hi1;
  kv = th ? e.hi1 : e.lo1;
  return th ? 1 : (tl ? -1 : 0);
}
// Side-table slot i: position and the value, exactly, in the input dtype
// (the value came from that dtype, so narrowing is exact).
template <int DT>
__device__ __forceinline__ void store_side(uint8_t* idx, uint8_t* val, int64_t i, int pos, float v) {
  idx[i] = uint8_t(pos);
  if constexpr (DT == DT_F32) reinterpret_cast<float*>(val)[i] = v;
  else if constexpr (DT == DT_F16) reinterpret_cast<_Float16*>(val)[i] = _Float16(v);
  else reinterpret_cast<uint16_t*>(val)[i] = uint16_t(__builtin_bit_cast(uint32_t, v) >> 16);
}
// Side tables of one unit (a key group: D entries; a value step: rows of
// the head), or none.
struct Side {
  uint8_t* idx;
  uint8_t* val;   // input dtype
  bool on;
};

// Store the n = 8 b bits of eight b-bit codes at p (aligned to b bytes):
// one store at 1, 2, 4 and 8 bits, byte stores at the widths whose codes
// straddle bytes.
template <int BITS>
__device__ __forceinline__ void store_codes8(uint8_t* p, uint64_t v) {
  if constexpr (BITS == 1) *p = uint8_t(v);
  else if constexpr (BITS == 2) *reinterpret_cast<uint16_t*>(p) = uint16_t(v);
  else if constexpr (BITS == 4) *reinterpret_cast<uint32_t*>(p) = uint32_t(v);
  else if constexpr (BITS == 8) *reinterpret_cast<uint2*>(p) = make_uint2(uint32_t(v), uint32_t(v >> 32));
  else {
#pragma unroll
    for (int k = 0; k < BITS; ++k) p[k] = uint8_t(v >> (8 * k));
  }
}

// Rows are split into pieces of 8 channels (16 bytes of 16-bit inputs, 32
// bytes of fp32), so that a thread's codes fill whole bytes at any width.
template <int DT, int D>
struct RowSplit {
  static constexpr int kVE = 8;                       // channels per piece
  static constexpr int kTPR = D / kVE;                // threads per row: 8 or 16
  static constexpr int kRPP = 256 / kTPR;             // rows per pass of 256 threads
};

// A piece of a row: its 16-byte loads.
template <int DT>
struct Piece {
  uint4 v[Elem<DT>::bytes / 2];
};
template <int DT>
__device__ __forceinline__ void load_piece(const uint8_t* p, Piece<DT>& pc) {
#pragma unroll
  for (int i = 0; i < Elem<DT>::bytes / 2; ++i) pc.v[i] = reinterpret_cast<const uint4*>(p)[i];
}
template <int DT>
__device__ __forceinline__ void widen_piece(const Piece<DT>& pc, float* out) {
#pragma unroll
  for (int i = 0; i < Elem<DT>::bytes / 2; ++i) widen16<DT>(pc.v[i], out + i * (16 / Elem<DT>::bytes));
}

// ----------------------------------------------------------------------------
// One key group of G rows, 256 threads: per-channel min / max over the rows,
// delta and zero point, the packed code rows.  The kRW = 64 / kTPR rows a
// wave holds per pass sit in consecutive lanes, so the reduction over them
// runs within DPP rows: lane l of wave w holds piece l / kRW (channels kVE *
// (l / kRW) ..) of rows kRW w + l % kRW + kRPP * i.
// ----------------------------------------------------------------------------
template <int DT, int D, int G>
struct KeyRows {
  static constexpr int kRPT = G / RowSplit<DT, D>::kRPP;   // rows per thread
  static_assert(kRPT >= 1 && G % RowSplit<DT, D>::kRPP == 0, "group rows per thread");
  Piece<DT> raw[kRPT];
};
template <int DT, int D>
struct KeyLane {
  static constexpr int kRW = 64 / RowSplit<DT, D>::kTPR;   // rows per wave and pass
  int cs, r0;
  __device__ KeyLane() {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    cs = lane / kRW;
    r0 = wave * kRW + lane % kRW;
  }
};

// This thread's pieces of a key group's rows.
template <int DT, int D, int G, class Rows>
__device__ __forceinline__ void load_key_rows(const Rows& rows, KeyRows<DT, D, G>& kr) {
  using RS = RowSplit<DT, D>;
  const KeyLane<DT, D> kl;
  const int cs = kl.cs, r0 = kl.r0;
#pragma unroll
  for (int i = 0; i < KeyRows<DT, D, G>::kRPT; ++i)
    load_piece<DT>(rows.row(r0 + i * RS::kRPP) + cs * RS::kVE * Elem<DT>::bytes, kr.raw[i]);
}

template <int DT, int D, int BITS, int G>
__device__ __forceinline__ void key_group(const KeyRows<DT, D, G>& kr, float* k_scale, float* k_zero,
                                          uint8_t* code_rows, Side side, float (*s_red)[D],
                                          float (*s_par)[D]) {
  using RS = RowSplit<DT, D>;
  constexpr int kVE = RS::kVE, kTPR = RS::kTPR, kRPP = RS::kRPP;
  constexpr int kRPT = KeyRows<DT, D, G>::kRPT;
  constexpr float kLevels = float((1 << BITS) - 1);
  constexpr int kRW = KeyLane<DT, D>::kRW;
  const KeyLane<DT, D> kl;
  const int t = threadIdx.x, cs = kl.cs, r0 = kl.r0;
  const int lane = t & 63, wave = t >> 6;
  const Piece<DT>* raw = kr.raw;
  float x[kRPT][kVE];
#pragma unroll
  for (int i = 0; i < kRPT; ++i) widen_piece<DT>(raw[i], x[i]);
  // the waves meet in LDS: rows 0..3 of s_red hold minima, 4..7 maxima
  // (with a side table, 8..11 the second smallest, 12..15 the second
  // largest)
  if (side.on) {
#pragma unroll
    for (int e = 0; e < kVE; ++e) {
      Ext2 ex2 = ext2_of(x[0][e]);
#pragma unroll
      for (int i = 1; i < kRPT; ++i) ext2_add(ex2, x[i][e]);
      ext2_run<kRW>(ex2);
      if (lane % kRW == 0) {
        s_red[wave][cs * kVE + e] = ex2.lo1;
        s_red[4 + wave][cs * kVE + e] = ex2.hi1;
        s_red[8 + wave][cs * kVE + e] = ex2.lo2;
        s_red[12 + wave][cs * kVE + e] = ex2.hi2;
      }
    }
  } else {
    float mn[kVE], mx[kVE];
#pragma unroll
    for (int e = 0; e < kVE; ++e) {
      mn[e] = x[0][e];
      mx[e] = x[0][e];
#pragma unroll
      for (int i = 1; i < kRPT; ++i) {
        mn[e] = fmin2(mn[e], x[i][e]);
        mx[e] = fmax2(mx[e], x[i][e]);
      }
      minmax_run<kRW>(mn[e], mx[e]);
    }
    if (lane % kRW == 0) {
#pragma unroll
      for (int e = 0; e < kVE; ++e) {
        s_red[wave][cs * kVE + e] = mn[e];
        s_red[4 + wave][cs * kVE + e] = mx[e];
      }
    }
  }
  __syncthreads();
  // one thread per channel: delta, zero point and reciprocal, written out
  // and shared through LDS (row 3 of s_par flags a delta that needs the
  // exact division; rows 4 and 5 the kept entry: flag and value)
  if (t < D) {
    float lo, hi;
    if (side.on) {
      Ext2 ex2{s_red[0][t], s_red[8][t], s_red[4][t], s_red[12][t]};
#pragma unroll
      for (int w = 1; w < 4; ++w) ext2_merge(ex2, Ext2{s_red[w][t], s_red[8 + w][t], s_red[4 + w][t], s_red[12 + w][t]});
      float kv;
      const int keep = dense_split(ex2, lo, hi, kv);
      s_par[4][t] = keep != 0 ? 1.0f : 0.0f;
      s_par[5][t] = kv;
      if (keep == 0) store_side<DT>(side.idx, side.val, t, 255, 0.0f);
    } else {
      lo = fmin2(fmin2(s_red[0][t], s_red[1][t]), fmin2(s_red[2][t], s_red[3][t]));
      hi = fmax2(fmax2(s_red[4][t], s_red[5][t]), fmax2(s_red[6][t], s_red[7][t]));
    }
    float dl, z;
    bool ex = false;
    affine_params(lo, hi, kLevels, dl, z);
    const float rc = code_rcp(dl, ex);
    s_par[0][t] = dl;
    s_par[1][t] = z;
    s_par[2][t] = rc;
    s_par[3][t] = ex ? 1.0f : 0.0f;
    k_scale[t] = dl;
    k_zero[t] = z;
  }
  __syncthreads();
  float delta[kVE], zp[kVE], rcp[kVE];
  bool exact = false;
#pragma unroll
  for (int e = 0; e < kVE; e += 4) {
    const int c = cs * kVE + e;
    const float4 d4 = *reinterpret_cast<const float4*>(&s_par[0][c]);
    const float4 z4 = *reinterpret_cast<const float4*>(&s_par[1][c]);
    const float4 r4 = *reinterpret_cast<const float4*>(&s_par[2][c]);
    const float4 x4 = *reinterpret_cast<const float4*>(&s_par[3][c]);
    delta[e] = d4.x; delta[e + 1] = d4.y; delta[e + 2] = d4.z; delta[e + 3] = d4.w;
    zp[e] = z4.x; zp[e + 1] = z4.y; zp[e + 2] = z4.z; zp[e + 3] = z4.w;
    rcp[e] = r4.x; rcp[e + 1] = r4.y; rcp[e + 2] = r4.z; rcp[e + 3] = r4.w;
    exact |= (x4.x + x4.y + x4.z + x4.w) != 0.0f;
  }
  if (side.on) {   // the thread holding a kept entry writes its side-table slot
#pragma unroll
    for (int e = 0; e < kVE; ++e) {
      const int c = cs * kVE + e;
      if (s_par[4][c] != 0.0f) {
        const float kv = s_par[5][c];
#pragma unroll
        for (int i = 0; i < kRPT; ++i)
          if (x[i][e] == kv) store_side<DT>(side.idx, side.val, c, r0 + i * kRPP, x[i][e]);
      }
    }
  }
  constexpr int kRB = D * BITS / 8;
#pragma unroll
  for (int i = 0; i < kRPT; ++i) {
    uint32_t code[kVE];
    affine_codes<kVE, BITS>(x[i], delta, zp, rcp, exact, code);
    uint64_t packed = 0;
#pragma unroll
    for (int e = 0; e < kVE; ++e) packed |= uint64_t(code[e]) << (BITS * e);
    store_codes8<BITS>(code_rows + (r0 + i * kRPP) * kRB + cs * BITS, packed);
  }
}

// ----------------------------------------------------------------------------
// One 32-token step of values (storage rows u0 .. u0 + 31, u0 a multiple
// of 32), 256 threads: per-token min / max across the lanes of the token,
// delta and zero point, codes through LDS (channel-major) into the value-code
// units of the layout in kvq.h.  At 2 bits a block holds two steps; a step
// writes its own bytes of each unit (bytes s and s + 2).
// ----------------------------------------------------------------------------
constexpr int kStepPitch = 36;   // bytes per channel row of the LDS code tile

// Value rows of a step: thread t holds kVE channels of token t / 8 (8
// threads per row, one token each), as kNV 16-byte vectors kSeg channels
// apart, so that each load instruction reads whole 128-byte spans of rows.
template <int DT, int D>
struct VSplit {
  static constexpr int kVE = D == 128 ? 16 : 8;    // channels per thread
  static constexpr int kTPR = D / kVE;             // threads per row: 8
  static constexpr int kEPV = 16 / Elem<DT>::bytes;  // channels per vector
  static constexpr int kNV = kVE / kEPV;           // vectors per thread
  static constexpr int kSeg = D / kNV;             // channels between a thread's vectors
  static_assert(kTPR * 32 == 256, "one token per thread");
  // channel of element e of thread column cs
  static __device__ __forceinline__ int chan(int cs, int e) { return (e / kEPV) * kSeg + cs * kEPV + e % kEPV; }
};

template <int DT, int D>
struct StepRows {
  uint4 raw[VSplit<DT, D>::kNV];
};

// This thread's vectors of its value row of a step.
template <int DT, int D, class Rows>
__device__ __forceinline__ void load_step_rows(const Rows& rows, StepRows<DT, D>& sr) {
  using VS = VSplit<DT, D>;
  const int t = threadIdx.x, cs = t % VS::kTPR;
  const uint8_t* row = rows.row(t / VS::kTPR);
#pragma unroll
  for (int i = 0; i < VS::kNV; ++i)
    sr.raw[i] = *reinterpret_cast<const uint4*>(row + (i * VS::kSeg + cs * VS::kEPV) * Elem<DT>::bytes);
}

template <int DT, int D, int BITS>
__device__ __forceinline__ void value_step(const StepRows<DT, D>& sr, int64_t u0, float* v_scale,
                                           float* v_zero, uint8_t* v_codes_head, Side side,
                                           uint8_t* s_codes) {
  using VS = VSplit<DT, D>;
  using VL = VLayout<BITS>;
  constexpr int kVE = VS::kVE, kTPR = VS::kTPR;
  constexpr float kLevels = float((1 << BITS) - 1);
  const int t = threadIdx.x, cs = t % kTPR, tok = t / kTPR;
  {
    float x[kVE];
#pragma unroll
    for (int i = 0; i < VS::kNV; ++i) widen16<DT>(sr.raw[i], x + i * VS::kEPV);
    float mn, mx;
    if (side.on) {
      Ext2 ex2 = ext2_of(x[0]);
#pragma unroll
      for (int e = 1; e < kVE; ++e) ext2_add(ex2, x[e]);
      ext2_run<kTPR>(ex2);
      float kv;
      const int keep = dense_split(ex2, mn, mx, kv);
      // the lane holding the kept entry writes the token's slot; lane 0 of
      // the token writes "none"
      if (keep == 0) {
        if (cs == 0) store_side<DT>(side.idx, side.val, u0 + tok, 255, 0.0f);
      } else {
#pragma unroll
        for (int e = 0; e < kVE; ++e)
          if (x[e] == kv) store_side<DT>(side.idx, side.val, u0 + tok, VS::chan(cs, e), x[e]);
      }
    } else {
      mn = x[0];
      mx = x[0];
#pragma unroll
      for (int e = 1; e < kVE; ++e) {
        mn = fmin2(mn, x[e]);
        mx = fmax2(mx, x[e]);
      }
      minmax_run<kTPR>(mn, mx);
    }
    float delta[kVE], zp[kVE], rcp[kVE];
    bool exact = false;
    affine_params(mn, mx, kLevels, delta[0], zp[0]);
    rcp[0] = code_rcp(delta[0], exact);
#pragma unroll
    for (int e = 1; e < kVE; ++e) {
      delta[e] = delta[0];
      zp[e] = zp[0];
      rcp[e] = rcp[0];
    }
    if (cs == 0) {
      v_scale[u0 + tok] = delta[0];
      v_zero[u0 + tok] = zp[0];
    }
    uint32_t code[kVE];
    affine_codes<kVE, BITS>(x, delta, zp, rcp, exact, code);
#pragma unroll
    for (int e = 0; e < kVE; ++e) s_codes[VS::chan(cs, e) * kStepPitch + tok] = uint8_t(code[e]);
  }
  __syncthreads();
  // units of this step: unit x of the block holds channel d = 16 n + jj for
  // lane group g; its tokens (h, r) of this step are offsets 16 h + 4 g + r
  constexpr int kUnits = 4 * D;
  const int64_t blk = u0 / VL::L;
  const int s = int((u0 % VL::L) / 32);
  for (int x = t; x < kUnits; x += 256) {
    const int g = x / D, rem = x % D, jj = rem / (D / 16), n = rem % (D / 16);
    const int d = 16 * n + jj;
    const uint32_t w0 = *reinterpret_cast<const uint32_t*>(s_codes + d * kStepPitch + 4 * g);
    const uint32_t w1 = *reinterpret_cast<const uint32_t*>(s_codes + d * kStepPitch + 16 + 4 * g);
    uint8_t* dst = v_codes_head + (blk * kUnits + x) * VL::UB;
    if constexpr (BITS == 8) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);         // slots r (h 0), 4 + r (h 1)
    } else if constexpr (BITS == 4) {
      const uint32_t a = w0 | (w0 >> 4), b = w1 | (w1 >> 4);        // nibble pairs in bytes 0, 2
      *reinterpret_cast<uint32_t*>(dst) = (a & 0xFFu) | ((a >> 8) & 0xFF00u) | ((b & 0xFFu) << 16) |
                                          ((b << 8) & 0xFF000000u);
    } else if constexpr (BITS == 2) {
      // slot r + 4 s + 8 h sits in byte s + 2 h
      uint32_t a = w0 | (w0 >> 6), b = w1 | (w1 >> 6);
      a = (a | (a >> 12)) & 0xFFu;
      b = (b | (b >> 12)) & 0xFFu;
      dst[s] = uint8_t(a);
      dst[s + 2] = uint8_t(b);
    } else {
      // any other width: slots r (h 0) and 4 + r (h 1) of an 8-code unit of
      // BITS bytes, slot i at bit i * BITS
      uint64_t v = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v |= uint64_t((w0 >> (8 * r)) & 0xFFu) << (BITS * r);
        v |= uint64_t((w1 >> (8 * r)) & 0xFFu) << (BITS * (4 + r));
      }
      store_codes8<BITS>(dst, v);
    }
  }
}

// ----------------------------------------------------------------------------
// Prefill kernels
// ----------------------------------------------------------------------------
// One workgroup's share of the full-precision rows of head (b, h): 16-byte
// vectors blk * 256 .. blk * 256 + 255 of the n_rows rows (sinks first,
// then the residual tokens, each to its sink or ring slot).
template <int DT, int D>
__device__ __forceinline__ void copy_fp_block(const FpCopyArgs& a, int64_t n_rows, int64_t blk, int h, int b) {
  constexpr int EB = Elem<DT>::bytes;
  constexpr int kVec = D * EB / 16;  // 16-byte vectors per row
  const int64_t v = blk * 256 + threadIdx.x;
  const int64_t row = v / kVec;
  if (row >= n_rows) return;
  const int64_t tok = row < a.n_sink ? row : a.first_resid + (row - a.n_sink);
  const uint8_t* src = reinterpret_cast<const uint8_t*>(a.src) + (b * a.sb + h * a.sh + tok * a.st) * EB;
  uint8_t* dst;
  if (tok < a.S) {
    dst = reinterpret_cast<uint8_t*>(a.sink) + ((int64_t(b) * a.H + h) * a.S + tok) * D * EB;
  } else {
    const int64_t slot = (tok - a.S) % a.ring;
    dst = reinterpret_cast<uint8_t*>(a.resid) + ((int64_t(b) * a.H + h) * a.ring + slot) * D * EB;
  }
  reinterpret_cast<uint4*>(dst)[v % kVec] = reinterpret_cast<const uint4*>(src)[v % kVec];
}

// grid: x = unit (key group, or 32-token value step) of the quantized range
// from unit a.k0 on, y = head, z = batch; unit k is stored at storage row
// (k * unit tokens) mod qcap.  One unit per workgroup: many small resident
// workgroups at different phases overlap loads with arithmetic better than
// fewer workgroups streaming several units each (measured).  Workgroups
// x >= n_units copy the full-precision rows, so a prefill half is one
// launch.
template <int DT, int D, int BITS, int G>
__global__ __launch_bounds__(256) void k_quant_keys(QuantArgs a) {
  __shared__ __attribute__((aligned(16))) float s_red[16][D];
  __shared__ __attribute__((aligned(16))) float s_par[6][D];
  if (blockIdx.x >= a.n_units) {
    copy_fp_block<DT, D>(a.fp, a.n_fp_rows, blockIdx.x - a.n_units, blockIdx.y, blockIdx.z);
    return;
  }
  const int64_t k = a.k0 + blockIdx.x;
  const int64_t ks = k % (a.qcap / G);              // storage slot of group k
  const int h = blockIdx.y, b = blockIdx.z;
  constexpr int EB = Elem<DT>::bytes;
  const int64_t bh = int64_t(b) * a.H + h;
  KeyRows<DT, D, G> kr;
  load_key_rows<DT, D, G>(
      InputRows{reinterpret_cast<const uint8_t*>(a.src) + (b * a.sb + h * a.sh + (a.S + k * G) * a.st) * EB,
                a.st * EB},
      kr);
  const int64_t gi = (bh * (a.qcap / G) + ks) * D;   // first parameter of the group
  key_group<DT, D, BITS, G>(kr, a.scale + gi, a.zero + gi, a.codes + (bh * a.qcap + ks * G) * (D * BITS / 8),
                            Side{a.oidx + gi, a.oval + gi * EB, a.outliers != 0}, s_red, s_par);
}

template <int DT, int D, int BITS>
__global__ __launch_bounds__(256) void k_quant_values(QuantArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[D * kStepPitch];
  if (blockIdx.x >= a.n_units) {
    copy_fp_block<DT, D>(a.fp, a.n_fp_rows, blockIdx.x - a.n_units, blockIdx.y, blockIdx.z);
    return;
  }
  const int64_t st = a.k0 + blockIdx.x;
  const int64_t r0 = (32 * st) % a.qcap;            // storage row of the step's first token
  const int h = blockIdx.y, b = blockIdx.z;
  constexpr int EB = Elem<DT>::bytes;
  const int64_t bh = int64_t(b) * a.H + h;
  StepRows<DT, D> sr;
  load_step_rows<DT, D>(
      InputRows{reinterpret_cast<const uint8_t*>(a.src) + (b * a.sb + h * a.sh + (a.S + 32 * st) * a.st) * EB,
                a.st * EB},
      sr);
  value_step<DT, D, BITS>(sr, r0, a.scale + bh * a.qcap, a.zero + bh * a.qcap,
                          a.codes + bh * (a.qcap * D * BITS / 8),
                          Side{a.oidx + bh * a.qcap, a.oval + bh * a.qcap * EB, a.outliers != 0}, s_codes);
}

// ----------------------------------------------------------------------------
// Streaming append: block 0 writes token t = n_before to its sink or ring
// slot.  When the full-precision count reaches R + G, block 1 quantizes the
// oldest G ring tokens as the next key group and blocks 2 .. 1 + G/32 their
// values, one 32-token step each.  The appended token itself is read from
// its input (it belongs to the group when R == 0), so the blocks need no
// ordering among themselves.
// ----------------------------------------------------------------------------
template <int DT, int D, int BITS, int G>
__global__ __launch_bounds__(256) void k_append(AppendArgs a) {
  // grid: x = role, y = head, z = batch
  const int role = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = int64_t(b) * a.H + h;
  constexpr int EB = Elem<DT>::bytes;
  const int64_t t = a.n_before;
  const int64_t ring = a.R + G;
  const uint8_t* kin = reinterpret_cast<const uint8_t*>(a.k_new) + (b * a.k_sb + h * a.k_sh) * EB;
  const uint8_t* vin = reinterpret_cast<const uint8_t*>(a.v_new) + (b * a.v_sb + h * a.v_sh) * EB;
  if (role == 0) {
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
        reinterpret_cast<uint4*>(kd)[v] = reinterpret_cast<const uint4*>(kin)[v];
      else
        reinterpret_cast<uint4*>(vd)[v - kVec] = reinterpret_cast<const uint4*>(vin)[v - kVec];
    }
    return;
  }
  // freeze of tokens S + q_old .. S + q_old + G - 1
  const int64_t first = a.S + a.q_old;
  const int fresh_row = int(t - first);          // in [0, G) when t is in the group
  if (role == 1) {
    __shared__ __attribute__((aligned(16))) float s_red[16][D];
    __shared__ __attribute__((aligned(16))) float s_par[6][D];
    const RingRows rows{reinterpret_cast<const uint8_t*>(a.k_resid) + bh * ring * D * EB, kin,
                        (first - a.S) % ring, ring, fresh_row, D * EB};
    const int64_t kgrp = a.r_old / G;                 // storage slot of the group
    const int64_t gi = (bh * (a.qcap / G) + kgrp) * D;
    KeyRows<DT, D, G> kr;
    load_key_rows<DT, D, G>(rows, kr);
    key_group<DT, D, BITS, G>(kr, a.k_scale + gi, a.k_zero + gi,
                              a.k_codes + (bh * a.qcap + a.r_old) * (D * BITS / 8),
                              Side{a.k_oidx + gi, a.k_oval + gi * EB, a.outliers != 0}, s_red, s_par);
  } else {
    __shared__ __attribute__((aligned(16))) uint8_t s_codes[D * kStepPitch];
    const int step = role - 2;
    const RingRows rows{reinterpret_cast<const uint8_t*>(a.v_resid) + bh * ring * D * EB, vin,
                        (first + 32 * step - a.S) % ring, ring, fresh_row - 32 * step, D * EB};
    StepRows<DT, D> sr;
    load_step_rows<DT, D>(rows, sr);
    value_step<DT, D, BITS>(sr, a.r_old + 32 * step, a.v_scale + bh * a.qcap, a.v_zero + bh * a.qcap,
                            a.v_codes + bh * (a.qcap * D * BITS / 8),
                            Side{a.v_oidx + bh * a.qcap, a.v_oval + bh * a.qcap * EB, a.outliers != 0},
                            s_codes);
  }
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------
template <int DT, int D, int BITS>
hipError_t launch_quant_keys(const QuantArgs& a, int64_t n_blocks, int B, int H, hipStream_t s) {
  const dim3 grid(unsigned(n_blocks), H, B);
  if (a.G == 32) hipLaunchKernelGGL((k_quant_keys<DT, D, BITS, 32>), grid, dim3(256), 0, s, a);
  else if (a.G == 64) hipLaunchKernelGGL((k_quant_keys<DT, D, BITS, 64>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_quant_keys<DT, D, BITS, 128>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}
template <int DT, int D, int BITS>
hipError_t launch_quant_values(const QuantArgs& a, int64_t n_blocks, int B, int H, hipStream_t s) {
  hipLaunchKernelGGL((k_quant_values<DT, D, BITS>), dim3(unsigned(n_blocks), H, B), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}
template <int DT, int D, int BITS>
hipError_t launch_append(const AppendArgs& a, int B, int H, hipStream_t s) {
  const dim3 grid(a.flush ? 2 + a.G / 32 : 1, H, B);
  if (a.G == 32) hipLaunchKernelGGL((k_append<DT, D, BITS, 32>), grid, dim3(256), 0, s, a);
  else if (a.G == 64) hipLaunchKernelGGL((k_append<DT, D, BITS, 64>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_append<DT, D, BITS, 128>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
