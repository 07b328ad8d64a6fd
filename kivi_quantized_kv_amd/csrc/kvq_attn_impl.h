// Split-K decode attention over the quantized cache, VALU form, and the
// log-sum-exp merge of the split partials.
//
// out = softmax(scale * q K^T) V with K and V dequantized on the fly
// (pigeon guide "KV-cache quantization", How it works step 5: dequantized
// group by group inside the kernel, never materialized).  GQA: q head hq
// reads KV head hq / (Hq / Hkv) (tract PR "KIVI-style KV-cache
// quantization", What's in the PR: GQA handled).
//
// Dequantization is folded so the inner loops only turn codes into
// numbers.  With key group delta_d, zero z_d and value token delta_t, zero
// z_t:
//   q . k_hat       = sum_d (q_d delta_d) c_d + sum_d q_d z_d
//   sum_t p_t v_hat = sum_t (p_t delta_t) c_t + sum_t p_t z_t
// where the codes c enter as exact fp16 subnormal bit fields (below).
// Scores are kept in the log2 domain (scale * log2 e folded into q).
#pragma once

#include "kvq_kernels.h"

namespace kvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Codes as fp16 subnormals.  A masked bit field of one 16-bit half of a code
// word, read as fp16, is exactly n * 2^-24 for the field's integer n < 1024;
// the fp32 FMA that consumes it (v_fma_mix) then multiplies by an fp32
// coefficient that carries 2^24.  Field sets of one word, each giving a
// (low half, high half) pair:
//   8-bit : byte 0|2, byte 1|3                               (code j  -> x_j)
//   4-bit : byte 0|2, nibble 0|4, byte 1|3, nibble 2|6
//   2-bit : masks 0xFF, 0x3F, 0x0F, 0x03 of bytes 0|2 (part 0) or 1|3 (part 1)
// A run of codes sharing a byte is recovered by nested masks, so its field
// coefficients are differences of the per-code values x_j, where x_j already
// carries 2^-(bits * (j mod codes per byte)) (run_coefs).
// ---------------------------------------------------------------------------
template <int BITS, int PART>
__device__ __forceinline__ void word_fields(uint32_t w, uint32_t f[4]) {
  if constexpr (BITS == 8) {
    f[0] = w & 0x00FF00FFu;
    f[1] = __builtin_amdgcn_perm(w, w, 0x0C030C01u);   // bytes 1 and 3, zero-extended
  } else if constexpr (BITS == 4) {
    const uint32_t t = __builtin_amdgcn_perm(w, w, 0x0C030C01u);
    f[0] = w & 0x00FF00FFu;
    f[1] = w & 0x000F000Fu;
    f[2] = t;
    f[3] = t & 0x000F000Fu;
  } else if constexpr (PART == 0) {
    f[0] = w & 0x00FF00FFu;
    f[1] = w & 0x003F003Fu;
    f[2] = w & 0x000F000Fu;
    f[3] = w & 0x00030003u;
  } else {
    const uint32_t t = __builtin_amdgcn_perm(w, w, 0x0C030C01u);
    f[0] = t;
    f[1] = t & 0x003F003Fu;
    f[2] = t & 0x000F000Fu;
    f[3] = t & 0x00030003u;
  }
}

// Codes of a word grouped as (part, half, run position): word code index
// i = pt * kRun + hf * (32 / BITS / 2) + j sits at coefficient slot
// (pt * 2 + hf) * kRun + j.
template <int BITS> struct WordShape {
  static constexpr int kCPW = 32 / BITS;            // codes per word
  static constexpr int kParts = BITS == 2 ? 2 : 1;  // field sets per half
  static constexpr int kRun = BITS == 8 ? 2 : 4;    // codes per half of a field set
};

// Field coefficients of one run from its per-code values x (scaled).
template <int BITS>
__device__ __forceinline__ void run_coefs(const float* x, float* c) {
  if constexpr (BITS == 8) {
    c[0] = x[0];
    c[1] = x[1];
  } else if constexpr (BITS == 4) {
    c[0] = x[1];
    c[1] = x[0] - x[1];
    c[2] = x[3];
    c[3] = x[2] - x[3];
  } else {
    c[0] = x[3];
    c[1] = x[2] - x[3];
    c[2] = x[1] - x[2];
    c[3] = x[0] - x[1];
  }
}

// Coefficients of NW words from per-code values x[NW * kCPW] in code order.
template <int BITS, int NW>
__device__ __forceinline__ void word_coefs(const float* x, float* c) {
  using WS = WordShape<BITS>;
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int pt = 0; pt < WS::kParts; ++pt)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        run_coefs<BITS>(x + i * WS::kCPW + pt * WS::kRun + hf * (WS::kCPW / 2),
                        c + i * WS::kCPW + (pt * 2 + hf) * WS::kRun);
}

// acc += sum over the codes of word w of code * x (through the coefficients
// c of that word).
template <int BITS>
__device__ __forceinline__ void word_dot(uint32_t w, const float* c, float& acc) {
  using WS = WordShape<BITS>;
  constexpr int kNF = BITS == 8 ? 2 : 4;
#pragma unroll
  for (int pt = 0; pt < WS::kParts; ++pt) {
    uint32_t f[4];
    if (pt == 0) word_fields<BITS, 0>(w, f);
    else word_fields<BITS, 1>(w, f);
    const float* clo = c + pt * 2 * WS::kRun;
    const float* chi = clo + WS::kRun;
#pragma unroll
    for (int k = 0; k < kNF; ++k) {
      const half2_t h = __builtin_bit_cast(half2_t, f[k]);
      acc = __builtin_fmaf((float)h[0], clo[k], acc);
      acc = __builtin_fmaf((float)h[1], chi[k], acc);
    }
  }
}

// Widths read as fp16-subnormal fields (2, 4, 8 bits); every other width is
// read as a bit stream, one code at a time.
template <int BITS>
constexpr bool field_codes() { return BITS == 2 || BITS == 4 || BITS == 8; }

// 2^-(bits * (j mod codes per byte)): weight of code j's field position (1
// for codes read one at a time).
template <int BITS>
__device__ __forceinline__ float code_field_scale(int j) {
  if constexpr (!field_codes<BITS>() || BITS == 8) return 1.0f;
  else return __builtin_amdgcn_ldexpf(1.0f, -BITS * (j % (8 / BITS)));
}

// Code at bit offset pos of a little-endian bit stream held in words w
// (pos known at compile time after unrolling: one bit-field extract, or a
// funnel shift and a mask for a code that crosses a word boundary), as a
// float.
template <int BITS>
__device__ __forceinline__ float stream_code(const uint32_t* w, int pos) {
  const int wi = pos >> 5, sh = pos & 31;
  uint32_t v = w[wi] >> sh;
  if (sh + BITS > 32) v = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh);
  return float(v & ((1u << BITS) - 1));
}

// Lane N of each row of 16, broadcast to the row.
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + N, 0xF, 0xF, false));
}
// Sum over the wave on the VALU (row DPP, then the two permlane swaps).
__device__ __forceinline__ float wave_sum_valu(float v) {
  return sum_xor32(sum_xor16(row_sum(v)));
}

// N consecutive elements at element index i (16-byte aligned) widened to
// fp32; N is a multiple of 8 (16-bit types) or 4 (fp32).
template <int DT, int N>
__device__ __forceinline__ void load_row_run(const void* base, int64_t i, float* out) {
  if constexpr (DT == DT_F32) {
    const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + i);
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
      const float4 v = src[k];
      out[4 * k] = v.x; out[4 * k + 1] = v.y; out[4 * k + 2] = v.z; out[4 * k + 3] = v.w;
    }
  } else {
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + i);
#pragma unroll
    for (int k = 0; k < N / 8; ++k) {
      const uint4 v = src[k];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        out[8 * k + 2 * j] = DT == DT_F16 ? f16_bits_to_f32(w[j] & 0xFFFFu) : bf16_bits_to_f32(w[j] & 0xFFFFu);
        out[8 * k + 2 * j + 1] = DT == DT_F16 ? f16_bits_to_f32(w[j] >> 16) : bf16_bits_to_f32(w[j] >> 16);
      }
    }
  }
}
// N = 1 or 2 consecutive elements at element index i (aligned to N elements).
template <int DT, int N>
__device__ __forceinline__ void load_small(const void* base, int64_t i, float* out) {
  if constexpr (N == 1) {
    out[0] = load1<DT>(base, i);
  } else if constexpr (DT == DT_F32) {
    const float2 v = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(base) + i);
    out[0] = v.x; out[1] = v.y;
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(base) + i);
    out[0] = DT == DT_F16 ? f16_bits_to_f32(w & 0xFFFFu) : bf16_bits_to_f32(w & 0xFFFFu);
    out[1] = DT == DT_F16 ? f16_bits_to_f32(w >> 16) : bf16_bits_to_f32(w >> 16);
  }
}

// ---------------------------------------------------------------------------
// VALU kernel: one workgroup of NW waves per (split, q head, batch).  A
// split owns a run of value-code blocks of L tokens (32 at 4/8 bits, 64 at 2
// bits) and a run of the full-precision tokens; its waves share both evenly
// and fold them into one softmax state each.  With NW = 4 the workgroup
// writes its split's partial for the log-sum-exp merge; with NW = 16 it is
// the only split of its row (the rows alone fill the GPU), merges its waves
// in LDS and writes the output row itself.
//
// Full-precision tokens go first, in tiles of 16: lane (qt, tl) scores
// token tl over channel quarter qt, and lane l then adds channels
// l * D/64 .. of each value row.
//
// Quantized blocks: each wave keeps two register sets, so the next block's
// code words, value parameters and key-group parameters are in flight while
// a block is processed.
// q . K: lane (qt, tl) takes channel quarter qt of token tl of a 16-token
//   sub-tile; the quarter sums meet by quad DPP.  The coefficients of a key
//   group, x_d = q_d delta_d 2^-(b (d mod codes per byte)), are formed
//   once per 32 tokens: each lane scales D/64 channels, the wave trades them
//   through LDS, and kappa = sum_d q_d z_d is a wave sum.  The factor 2^24
//   of the code fields is applied to the finished dot product, so neither
//   a wide key range nor a subnormal one leaves fp32's range on the way.
// P . V: lane (vg, vj) holds code units of channels vj + 16n for the tokens
//   of lane group vg; the probabilities of those tokens come from their
//   score lanes by row broadcasts.  Their coefficients p_t delta_t carry
//   2^(24 + vexp) (2^24 cancels the code fields' 2^-24, so the accumulators
//   hold sums times 2^vexp), where the wave's exponent vexp puts the
//   largest value delta seen so far in [2^6, 2^7); it only decreases, with
//   an exact power-of-two rescale of the accumulators.
// ---------------------------------------------------------------------------
// Waves per SIMD the register budget is held to: four (128 VGPRs) where the
// kernel fits without spilling, else three.
template <int DT, int D, int BITS>
constexpr int valu_waves_per_simd() {
  return (field_codes<BITS>() && (D == 64 || (BITS == 4 && DT == DT_F16))) ? 4 : 3;
}

// MODE: bit 0 caches with side tables, bit 1 pre-RoPE keys (three waves
// per SIMD; two for fp32 rows of 128 channels, and for pre-RoPE keys of 128
// channels, whose unrolled pair loop needs the registers).
constexpr int kModeOutliers = 1, kModeRope = 2;
template <int DT, int D, int BITS, int MODE>
constexpr int valu_waves() {
  if constexpr (MODE != 0) return ((DT == DT_F32 || (MODE & kModeRope)) && D == 128) ? 2 : 3;
  else return valu_waves_per_simd<DT, D, BITS>();
}

// Revolutions x in [0, 1) -> sin(2 pi x), cos(2 pi x) (the hardware
// transcendental units take revolutions).
__device__ __forceinline__ void sincos_rev(float x, float& sn, float& cs) {
  sn = __builtin_amdgcn_sinf(x);
  cs = __builtin_amdgcn_cosf(x);
}

template <int DT, int D, int BITS, int NW, int MODE>
__global__ __launch_bounds__(64 * NW, (NW == 16 ? 4 : valu_waves<DT, D, BITS, MODE>())) void k_attn_valu(
    AttnArgs a) {
  constexpr bool OUTL = (MODE & kModeOutliers) != 0;
  constexpr bool ROPE = (MODE & kModeRope) != 0;
  using VL = VLayout<BITS>;
  using WS = WordShape<BITS>;
  constexpr bool kFields = field_codes<BITS>();
  // 2^24: unit of a subnormal field (codes read one at a time are whole numbers)
  constexpr float kS = kFields ? 16777216.0f : 1.0f;
  constexpr int kCodeExp = kFields ? 24 : 0;
  constexpr int kRowBytes = D * BITS / 8;
  constexpr int kQuarterCh = D / 4;              // channels per lane in q.K
  constexpr int kQBytes = kQuarterCh * BITS / 8; // bytes of a lane's quarter row
  // key words per lane per sub-tile (a bit stream's last word may be half full)
  constexpr int kQW = kFields ? kQuarterCh / WS::kCPW : (kQBytes + 3) / 4;
  constexpr int kNST = VL::L / 16;               // 16-token sub-tiles per block
  constexpr int kHalves = VL::L / 32;            // 32-token key-group steps per block
  constexpr int kUnits = D / 16;                 // value units per lane per block
  constexpr int kVW = kUnits * VL::UB / 4;       // value-code words per lane per block
  constexpr int kUW = kFields ? VL::UB / 4 : 1;  // words per value unit (field widths)
  constexpr int kWC = D / 64;                    // channels per lane when scaling a group / adding a row

  const int split = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int h = hq / a.gqa;
  const int64_t bh = int64_t(b) * a.H + h;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qt = lane & 3;          // q.K: channel quarter
  const int tl = lane >> 2;         // q.K: token within a 16-token tile
  const int vg = lane >> 4;         // P.V: lane group
  const int vj = lane & 15;         // P.V: channel within 16

  __shared__ __attribute__((aligned(16))) float s_q[D];
  constexpr int kThreads = 64 * NW;
  __shared__ __attribute__((aligned(16))) float s_x[NW][kHalves][D];
  __shared__ float s_out[NW][D + 2];
  // side-table corrections: per key-group half, to the scores of its 32
  // tokens; per block, to the value sums of each channel
  __shared__ float s_kc[NW][kHalves * 32];
  __shared__ float s_vc[NW][D];
  constexpr bool outl = OUTL;
  // pre-RoPE keys: per frequency i < D/2 the rate C_i = theta_i / (2 pi) in
  // revolutions per token (fp64, and rounded to fp32), and per wave the
  // fraction of a revolution at its current block's first token; per wave
  // and key-group half the delta and zero point of every channel
  __shared__ double s_cd[ROPE ? D / 2 : 1];
  __shared__ float s_c[ROPE ? D / 2 : 1];
  __shared__ float s_fb[ROPE ? NW : 1][ROPE ? D / 2 : 1];
  __shared__ float s_dz[ROPE ? NW : 1][ROPE ? kHalves : 1][2][ROPE ? D : 1];

  for (int d = threadIdx.x; d < D; d += kThreads)
    s_q[d] = load1<DT>(a.q, b * a.q_sb + hq * a.q_sh + d) * a.sm_scale_log2;
  if constexpr (ROPE) {
    for (int i = threadIdx.x; i < D / 2; i += kThreads) {
      // theta_i = base^(-2i/D) (P1)
      const double c = exp2(-2.0 * double(i) / double(D) * a.rope_log2_base) *
                       0.15915494309189535;
      s_cd[i] = c;
      s_c[i] = float(c);
    }
  }
  if constexpr (outl) {
    for (int i = threadIdx.x; i < NW * kHalves * 32; i += kThreads) (&s_kc[0][0])[i] = 0.f;
    for (int i = threadIdx.x; i < NW * D; i += kThreads) (&s_vc[0][0])[i] = 0.f;
  }
  __syncthreads();

  float m = -__builtin_inff(), l = 0.f, z = 0.f;
  float acc[kUnits], accf[kWC];
#pragma unroll
  for (int n = 0; n < kUnits; ++n) acc[n] = 0.f;
#pragma unroll
  for (int c = 0; c < kWC; ++c) accf[c] = 0.f;
  // l and z gain each token once per lane of its quad (four times); the
  // quad-first wave sums at the end divide that out exactly.
  auto raise_max = [&](float bm) {
    const float new_m = __builtin_fmaxf(m, bm);
    if (new_m > m) {   // wave-uniform
      const float alpha = __builtin_amdgcn_exp2f(m - new_m);
      l *= alpha;
      z *= alpha;
#pragma unroll
      for (int n = 0; n < kUnits; ++n) acc[n] *= alpha;
#pragma unroll
      for (int c = 0; c < kWC; ++c) accf[c] *= alpha;
      m = new_m;
    }
  };
  auto tile_max = [&](float v) {   // over the 16 tokens of the tile(s)
    v = __builtin_fmaxf(v, dpp_mov<kRowRor4>(v));
    v = __builtin_fmaxf(v, dpp_mov<kRowRor8>(v));
    return max_xor32(max_xor16(v));
  };

  // Blocks are numbered from the first one the query attends to (block c0,
  // the first of the sliding window; 0 without one).
  const int64_t nblk = (a.Q + VL::L - 1) / VL::L - a.c0;
  const int64_t blk0 = int64_t(split) * a.blocks_per_split;
  const int64_t blk1 = blk0 + a.blocks_per_split < nblk ? blk0 + a.blocks_per_split : nblk;
  const int64_t per_wave = blk1 > blk0 ? (blk1 - blk0 + NW - 1) / NW : 0;
  const int64_t wb0 = blk0 + wave * per_wave;
  const int64_t wb1 = wb0 + per_wave < blk1 ? wb0 + per_wave : blk1;

  // group scaling: this lane's channels lane*kWC + c
  float sq_w[kWC], xs_w[kWC];
#pragma unroll
  for (int c = 0; c < kWC; ++c) {
    const int ch = lane * kWC + c;
    sq_w[c] = s_q[ch];
    xs_w[c] = s_q[ch] * code_field_scale<BITS>(ch);
  }
  // Pre-RoPE keys: lane quarter qt pairs with quarter qt ^ 2 (channel i with
  // i + D/2).  At step m2 a lane holds its channels 2 m2 and 2 m2 + 1;
  // lanes of the low half take the pair of channel 2 m2, lanes of the high
  // half that of their channel 2 m2 + 1, each receiving the partner's key
  // by a quad swap.  rope_pair returns A = q_i k_i + q_i' k_i' and sets B =
  // q_i' k_i - q_i k_i', so that the pair adds cos A + sin B to the score.
  const bool rp_hi = qt >= 2;
  const int rp_own = qt * kQuarterCh;                            // first own channel
  const int rp_par = rp_hi ? rp_own - D / 2 : rp_own + D / 2;    // its partner
  auto fr_index = [&](int m2) { return (rp_hi ? rp_own - D / 2 : rp_own) + 2 * m2 + (rp_hi ? 1 : 0); };
  auto rope_pair = [&](float k0, float k1, int m2, float& bb) {
    const float par = dpp_mov<kQuadXor2>(rp_hi ? k0 : k1);
    const float own = rp_hi ? k1 : k0;
    const int j = 2 * m2 + (rp_hi ? 1 : 0);
    const float qo = s_q[rp_own + j], qp = s_q[rp_par + j];
    const float cross = __builtin_fmaf(qp, own, -qo * par);
    bb = rp_hi ? -cross : cross;
    return __builtin_fmaf(qo, own, qp * par);
  };
  // exponent of this lane's score token's value code field
  const int fsh = (!kFields || BITS == 8) ? 0 : -BITS * (tl % (8 / (kFields ? BITS : 8)));
  // value exponent; before any delta is seen the threshold 2^(7 - vexp) is
  // the smallest fp32 subnormal, so the first nonzero delta sets it
  int vexp = 156;
  float vthr = __builtin_amdgcn_ldexpf(1.0f, 7 - vexp);
  // Uniform bases and 32-bit lane offsets (loads take the scalar-base form).
  const uint8_t* kc_head = a.k_codes + bh * a.qcap * kRowBytes;
  const uint8_t* vc_head = a.v_codes + bh * a.qcap * kRowBytes;
  const float* vs_head = a.v_scale + bh * a.qcap;
  const float* vz_head = a.v_zero + bh * a.qcap;
  const float* ks_head = a.k_scale + bh * a.kgroups * D;
  const float* kz_head = a.k_zero + bh * a.kgroups * D;
  const uint32_t k_off = uint32_t(tl * kRowBytes + qt * kQBytes);
  const uint32_t v_off = uint32_t((vg * 16 + vj) * kUnits * VL::UB);
  const uint32_t c_off = uint32_t(lane * kWC);

  struct Blk {
    uint32_t kw[kNST][kQW];
    uint32_t vw[kVW];
    float dv[kNST], zv[kNST];
    float ks[kHalves][kWC], kz[kHalves][kWC];
  };
  // Every address lies inside the allocation: qcap is a multiple of
  // max(64, G) tokens, so whole blocks and their key groups are in range;
  // tokens past the quantized count are masked after the loads.  Code words
  // are read once per call: non-temporal loads keep them out of the way of
  // the parameters in the caches.
  // first storage row of block blk: the ring's block slot (c0 + blk) mod
  // (qcap / L), by one conditional subtraction (the live blocks span at most
  // qcap / L + 1 slots)
  auto blk_base = [&](int64_t blk) -> int64_t {
    int64_t s = a.c0 + blk - a.cw;
    if (s >= a.ncap) s -= a.ncap;
    return s * VL::L;
  };
  auto load_blk = [&](int64_t blk, Blk& r) {
    const int64_t base = blk_base(blk);
    const uint8_t* kb = kc_head + base * kRowBytes;
#pragma unroll
    for (int st = 0; st < kNST; ++st) {
      if constexpr (kQBytes % 4 == 0) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(kb + k_off + st * 16 * kRowBytes);
#pragma unroll
        for (int i = 0; i < kQW; ++i) r.kw[st][i] = __builtin_nontemporal_load(src + i);
      } else {
        // a quarter row of 2 * BITS bytes (D 64, odd width) starts on a
        // 2-byte boundary: 16-bit loads, paired into words
        const uint16_t* src = reinterpret_cast<const uint16_t*>(kb + k_off + st * 16 * kRowBytes);
#pragma unroll
        for (int i = 0; i < kQW; ++i) {
          const uint32_t lo = src[2 * i];
          const uint32_t hi = 2 * i + 1 < kQBytes / 2 ? uint32_t(src[2 * i + 1]) : 0u;
          r.kw[st][i] = lo | (hi << 16);
        }
      }
    }
    const uint32_t* vsrc = reinterpret_cast<const uint32_t*>(vc_head + base * kRowBytes + v_off);
#pragma unroll
    for (int i = 0; i < kVW; ++i) r.vw[i] = __builtin_nontemporal_load(vsrc + i);
    const float* vs = vs_head + base;
    const float* vz = vz_head + base;
#pragma unroll
    for (int st = 0; st < kNST; ++st) {
      r.dv[st] = vs[uint32_t(tl + st * 16)];
      r.zv[st] = vz[uint32_t(tl + st * 16)];
    }
#pragma unroll
    for (int k = 0; k < kHalves; ++k) {
      const int64_t grp = (base + 32 * k) >> a.g_shift;
      const float* ks = ks_head + grp * D;
      const float* kz = kz_head + grp * D;
#pragma unroll
      for (int c = 0; c < kWC; ++c) {
        r.ks[k][c] = ks[c_off + c];
        r.kz[k][c] = kz[c_off + c];
      }
    }
  };

  Blk ra, rb;
  if (wb0 < wb1) load_blk(wb0, ra);

  // ---- full-precision tokens of this split (sinks, then the residual ring)
  {
    const int64_t f0 = int64_t(split) * a.fp_per_split;
    const int64_t f1 = f0 + a.fp_per_split < a.n_fp ? f0 + a.fp_per_split : a.n_fp;
    const int64_t fpw = f1 > f0 ? (f1 - f0 + NW - 1) / NW : 0;
    const int64_t fw0 = f0 + wave * fpw;
    const int64_t fw1 = fw0 + fpw < f1 ? fw0 + fpw : f1;
    // element offset of exact token i's row and the store holding it
    auto fp_row = [&](int64_t i, bool& sink) {
      sink = i < a.n_sink;
      int64_t slot = a.resid_slot0 + (i - a.n_sink);   // < 2 * ring
      slot -= slot >= a.ring ? a.ring : 0;
      return (sink ? bh * a.S + i : bh * a.ring + slot) * D;
    };
    if (fw0 < fw1) {
      for (int64_t t0 = fw0; t0 < fw1; t0 += 16) {
        // scores: token t0 + tl (addresses clamped into the run)
        bool sk;
        const int64_t ik = t0 + tl < fw1 ? t0 + tl : fw1 - 1;
        const int64_t ko = fp_row(ik, sk);
        float kr[kQuarterCh];
        load_row_run<DT, kQuarterCh>(sk ? a.k_sink : a.k_resid, ko + qt * kQuarterCh, kr);
        float dot = 0.f;
        if constexpr (ROPE) {
          // the token's position (its index) and the key rotated to it
          const int64_t pos = ik < a.n_sink ? ik : a.first_resid + (ik - a.n_sink);
#pragma unroll
          for (int m2 = 0; m2 < kQuarterCh / 2; ++m2) {
            float fr;
            const float pr = rope_pair(kr[2 * m2], kr[2 * m2 + 1], m2, fr);
            const double x = double(pos) * s_cd[fr_index(m2)];
            const float rev = float(x - __builtin_floor(x));
            float sn, cs;
            sincos_rev(rev, sn, cs);
            dot = __builtin_fmaf(cs, pr, __builtin_fmaf(sn, fr, dot));
          }
        } else {
#pragma unroll
          for (int j = 0; j < kQuarterCh; ++j) dot = __builtin_fmaf(kr[j], s_q[qt * kQuarterCh + j], dot);
        }
        // value rows of the tile's tokens, channels lane*kWC ..
        float vr[16][kWC];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          bool sv;
          const int64_t iv = t0 + t < fw1 ? t0 + t : fw1 - 1;
          const int64_t vo = fp_row(iv, sv);
          load_small<DT, kWC>(sv ? a.v_sink : a.v_resid, vo + lane * kWC, vr[t]);
        }
        const float sc = quad_sum(dot) + (t0 + tl < fw1 ? 0.f : -__builtin_inff());
        raise_max(tile_max(sc));
        const float p = __builtin_amdgcn_exp2f(sc - m);   // 0 past the run
        l += p;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const float pt = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), 4 * t));
#pragma unroll
          for (int c = 0; c < kWC; ++c) accf[c] = __builtin_fmaf(pt, vr[t][c], accf[c]);
        }
      }
    }
  }

  // ---- quantized blocks
  auto process = [&](int64_t blk, const Blk& r) {
    const int64_t base = (a.c0 + blk) * VL::L;   // quantized index of the block's first token
    const int nvalid = int(a.Q - base < VL::L ? a.Q - base : VL::L);
    const int lo = blk == 0 ? a.lo_off : 0;      // tokens before the window
    // key-group coefficients of each 32-token half (pre-RoPE keys: the
    // deltas and zero points themselves, and the block's angle base)
    float kap[kHalves];
#pragma unroll
    for (int k = 0; k < kHalves; ++k) {
      float kp = 0.f;
#pragma unroll
      for (int c = 0; c < kWC; ++c) {
        if constexpr (ROPE) {
          s_dz[wave][k][0][lane * kWC + c] = r.ks[k][c];
          s_dz[wave][k][1][lane * kWC + c] = r.kz[k][c];
        } else {
          s_x[wave][k][lane * kWC + c] = xs_w[c] * r.ks[k][c];
          kp = __builtin_fmaf(sq_w[c], r.kz[k][c], kp);
        }
      }
      kap[k] = ROPE ? 0.f : wave_sum_valu(kp);
    }
    if constexpr (ROPE) {
      if (lane < D / 2) {   // revolutions at the block's first token, position S + base
        const double x = double(a.S + base) * s_cd[lane];
        s_fb[wave][lane] = float(x - __builtin_floor(x));
      }
    }
    wave_lds_sync();
    if constexpr (outl) {
      // keys kept exact: a channel's entry at group offset j adds
      // s_q (x - dense) to the score of token j of its half, dense = zp +
      // delta (2^b - 1) for an entry above the zero point, else zp (its
      // code clamps to 2^b - 1 or 0)
      constexpr float kLev = float((1 << BITS) - 1);
#pragma unroll
      for (int k = 0; k < kHalves; ++k) {
        const int64_t row = blk_base(blk) + 32 * k;          // storage row of the half
        const int64_t gi = ((row >> a.g_shift) + bh * a.kgroups) * D;
        const int off = int(row & (a.G - 1));                 // the half's offset in its group
#pragma unroll
        for (int c = 0; c < kWC; ++c) {
          const int ch = lane * kWC + c;
          const int j = int(a.k_oidx[gi + ch]) - off;
          if (j >= 0 && j < 32) {
            const float xv = load1<DT>(a.k_oval, gi + ch);
            const float dense = xv < r.kz[k][c] ? r.kz[k][c] : __builtin_fmaf(kLev, r.ks[k][c], r.kz[k][c]);
            float qe = sq_w[c];
            if constexpr (ROPE) {
              // the query rotated back by the token's angle, channel ch
              const int fi = ch & (D / 2 - 1);
              float rev = __builtin_fmaf(float(k * 32 + j), s_c[fi], s_fb[wave][fi]);
              rev -= __builtin_floorf(rev);
              float sn, cs;
              sincos_rev(rev, sn, cs);
              const float qp = s_q[ch ^ (D / 2)];
              qe = __builtin_fmaf(sq_w[c], cs, (ch < D / 2 ? qp : -qp) * sn);
            }
            atomicAdd(&s_kc[wave][k * 32 + j], qe * (xv - dense));
          }
        }
      }
      wave_lds_sync();
    }
    // scores (log2 domain); lane (qt, tl) ends with token st*16 + tl
    float sc[kNST];
#pragma unroll
    for (int k = 0; k < kHalves; ++k) {
      float dot[2] = {0.f, 0.f};
      if constexpr (ROPE) {
        // dequantized pairs rotated to their positions: token st*16 + tl
        // of the block turns its pair by its offset times C_i past the
        // block's base
#pragma unroll
        for (int m2 = 0; m2 < kQuarterCh / 2; ++m2) {
          const int c0 = rp_own + 2 * m2;
          const float d0 = s_dz[wave][k][0][c0], z0 = s_dz[wave][k][1][c0];
          const float d1 = s_dz[wave][k][0][c0 + 1], z1 = s_dz[wave][k][1][c0 + 1];
          const int fi = fr_index(m2);
          const float ci = s_c[fi], fb = s_fb[wave][fi];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int st = 2 * k + u;
            const float k0 = __builtin_fmaf(stream_code<BITS>(r.kw[st], (2 * m2) * BITS), d0, z0);
            const float k1 = __builtin_fmaf(stream_code<BITS>(r.kw[st], (2 * m2 + 1) * BITS), d1, z1);
            float bb;
            const float aa = rope_pair(k0, k1, m2, bb);
            float rev = __builtin_fmaf(float(st * 16 + tl), ci, fb);
            rev -= __builtin_floorf(rev);
            float sn, cs;
            sincos_rev(rev, sn, cs);
            dot[u] = __builtin_fmaf(cs, aa, __builtin_fmaf(sn, bb, dot[u]));
          }
        }
      } else if constexpr (kFields) {
#pragma unroll
        for (int i = 0; i < kQW; ++i) {   // one word's coefficients at a time
          float x[WS::kCPW], qc[WS::kCPW];
#pragma unroll
          for (int j = 0; j < WS::kCPW; ++j) x[j] = s_x[wave][k][qt * kQuarterCh + i * WS::kCPW + j];
          word_coefs<BITS, 1>(x, qc);
#pragma unroll
          for (int u = 0; u < 2; ++u) word_dot<BITS>(r.kw[2 * k + u][i], qc, dot[u]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kQuarterCh; ++j) {   // one code at a time
          const float xj = s_x[wave][k][qt * kQuarterCh + j];
#pragma unroll
          for (int u = 0; u < 2; ++u) dot[u] = __builtin_fmaf(stream_code<BITS>(r.kw[2 * k + u], j * BITS), xj, dot[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        // -inf past the quantized count (selected: the key parameters of a
        // group past the count are never written and may hold anything)
        const int st = 2 * k + u;
        float v = ROPE ? quad_sum(dot[u]) : __builtin_fmaf(quad_sum(dot[u]), kS, kap[k]);
        if constexpr (outl) v += s_kc[wave][st * 16 + tl];
        sc[st] = st * 16 + tl < nvalid && st * 16 + tl >= lo ? v : -__builtin_inff();
      }
    }
    wave_lds_sync();
    if constexpr (outl) if (qt == 0) {   // cleared for the next block (each wave reads in order)
#pragma unroll
      for (int st = 0; st < kNST; ++st) s_kc[wave][st * 16 + tl] = 0.f;
    }
    float lmax = sc[0];
#pragma unroll
    for (int st = 1; st < kNST; ++st) lmax = __builtin_fmaxf(lmax, sc[st]);
    raise_max(tile_max(lmax));
    float pp[kNST], dvs[kNST];
    float vmax = 0.f;
#pragma unroll
    for (int st = 0; st < kNST; ++st) {
      dvs[st] = st * 16 + tl < nvalid && st * 16 + tl >= lo ? r.dv[st] : 0.f;
      vmax = __builtin_fmaxf(vmax, dvs[st]);
    }
    if (__builtin_amdgcn_ballot_w64(vmax >= vthr) != 0) {   // rare: a larger value delta
      const int knew = __builtin_amdgcn_readfirstlane(7 - __builtin_amdgcn_frexp_expf(wave_max(vmax)));
#pragma unroll
      for (int n = 0; n < kUnits; ++n) acc[n] = __builtin_amdgcn_ldexpf(acc[n], knew - vexp);
      vexp = knew;
      vthr = __builtin_amdgcn_ldexpf(1.0f, 7 - vexp);
    }
    const int vke = vexp + kCodeExp + fsh;
#pragma unroll
    for (int st = 0; st < kNST; ++st) {
      const bool ok = st * 16 + tl < nvalid && st * 16 + tl >= lo;
      const float p = __builtin_amdgcn_exp2f(sc[st] - m);   // 0 past the range
      const float zv = ok ? r.zv[st] : 0.f;
      l += p;
      z = __builtin_fmaf(p, zv, z);
      pp[st] = p * __builtin_amdgcn_ldexpf(dvs[st], vke);
      if constexpr (outl) if (qt == 0 && ok) {
        // a value kept exact: p (x - dense) on its channel
        const int64_t row = blk_base(blk) + st * 16 + tl;
        const int vi = a.v_oidx[bh * a.qcap + row];
        if (vi != 255) {
          constexpr float kLev = float((1 << BITS) - 1);
          const float xv = load1<DT>(a.v_oval, bh * a.qcap + row);
          const float dense = xv < r.zv[st] ? r.zv[st] : __builtin_fmaf(kLev, r.dv[st], r.zv[st]);
          atomicAdd(&s_vc[wave][vi], p * (xv - dense));
        }
      }
    }
    if constexpr (outl) {   // folded into the exact-token sums, which share p's scale
      wave_lds_sync();
#pragma unroll
      for (int c = 0; c < kWC; ++c) {
        accf[c] += s_vc[wave][lane * kWC + c];
        s_vc[wave][lane * kWC + c] = 0.f;
      }
    }
    // P . V: code slot i of lane group vg is token vslot_token(vg, i), whose
    // p sits in lane 4 * (i & 3) of this row, sub-tile o / 16
    float pv[VL::U], vc[VL::U];
#pragma unroll
    for (int i = 0; i < VL::U; ++i) {
      const int st = vslot_token<BITS>(0, i) / 16;
      switch (i & 3) {
        case 0: pv[i] = row_bcast<0>(pp[st]); break;
        case 1: pv[i] = row_bcast<4>(pp[st]); break;
        case 2: pv[i] = row_bcast<8>(pp[st]); break;
        default: pv[i] = row_bcast<12>(pp[st]); break;
      }
    }
    if constexpr (kFields) {
      word_coefs<BITS, kUW>(pv, vc);
#pragma unroll
      for (int n = 0; n < kUnits; ++n)
#pragma unroll
        for (int wi = 0; wi < kUW; ++wi) word_dot<BITS>(r.vw[n * kUW + wi], vc + wi * WS::kCPW, acc[n]);
    } else {
      // unit n: slot i at bit (8 n + i) * BITS of the lane's value words
#pragma unroll
      for (int n = 0; n < kUnits; ++n)
#pragma unroll
        for (int i = 0; i < VL::U; ++i) acc[n] = __builtin_fmaf(stream_code<BITS>(r.vw, (8 * n + i) * BITS), pv[i], acc[n]);
    }
  };

  if (wb0 < wb1) {
    for (int64_t blk = wb0;; blk += 2) {
      load_blk(blk + 1 < wb1 ? blk + 1 : blk, rb);
      process(blk, ra);
      if (blk + 1 >= wb1) break;
      load_blk(blk + 2 < wb1 ? blk + 2 : blk + 1, ra);
      process(blk + 1, rb);
      if (blk + 2 >= wb1) break;
    }
  }

  // ---- wave result: the four lane groups of the quantized part each hold
  // a quarter of the tokens; exact-token sums are per channel already
#pragma unroll
  for (int n = 0; n < kUnits; ++n) acc[n] = sum_xor32(sum_xor16(acc[n]));
  l = 0.25f * wave_sum_valu(l);
  z = 0.25f * wave_sum_valu(z);
  if (lane < 16) {
#pragma unroll
    for (int n = 0; n < kUnits; ++n) s_out[wave][n * 16 + lane] = __builtin_amdgcn_ldexpf(acc[n], -vexp) + z;
  }
  wave_lds_sync();
#pragma unroll
  for (int c = 0; c < kWC; ++c) s_out[wave][lane * kWC + c] += accf[c];
  if (lane == 0) {
    s_out[wave][D] = m;
    s_out[wave][D + 1] = l;
  }
  __syncthreads();
  // merge the waves; a wave with no tokens left m = -inf, l = 0 and a zero
  // row.  NW = 4: this split's partial; NW = 16: the output row.
  float M = s_out[0][D];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = __builtin_fmaxf(M, s_out[w][D]);
  const float Mref = M == -__builtin_inff() ? 0.f : M;
  float f[NW];
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    f[w] = __builtin_amdgcn_exp2f(s_out[w][D] - Mref);
    L = __builtin_fmaf(f[w], s_out[w][D + 1], L);
  }
  if constexpr (NW == 16) {
    float* dst = a.out + (int64_t(b) * a.Hq + hq) * D;
    for (int d = threadIdx.x; d < D; d += kThreads) {
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) o = __builtin_fmaf(f[w], s_out[w][d], o);
      dst[d] = o / L;
    }
  } else {
    const int64_t row = int64_t(b) * a.Hq + hq;
    float* dst = partial_o(a, row, split, D);
    for (int d = threadIdx.x; d < D; d += kThreads) {
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) o = __builtin_fmaf(f[w], s_out[w][d], o);
      dst[d] = o;
    }
    if (threadIdx.x == 0) *reinterpret_cast<float2*>(partial_ml(a, row, split)) = float2{M, L};
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the split partials: M = max_j m_j,
// L = sum_j 2^(m_j - M) l_j, out = sum_j 2^(m_j - M) o_j / L.
// Above 64 splits: one workgroup per (32-channel block, q head, batch), one
// round of loads up to 64 splits: thread (slot, c4) folds channels [4 c4, 4 c4 + 4) of the
// block for splits slot, slot + 32, ... (float4 loads) into a running
// state of its own (local max, sums); the 32 slot states then meet through
// LDS by the same rule, with each slot's weight 2^(M_slot - M) computed once.
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(256) void k_merge(AttnArgs a) {
  constexpr int kCW = 32;                   // channels per workgroup
  constexpr int kQ = kCW / 4;               // float4 columns per split row
  constexpr int kSlots = 256 / kQ;          // 32 split slots
  constexpr int kPer = 2;                   // splits per slot per load round
  __shared__ float s_m[kSlots], s_l[kSlots], s_w[kSlots];
  __shared__ float4 s_acc[kSlots][kQ];
  const int cb = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, c4 = t % kQ, slot = t / kQ;
  const int ns = a.n_split;
  const int64_t row = int64_t(b) * a.Hq + hq;
  const float2* ml = reinterpret_cast<const float2*>(partial_ml(a, row, 0));
  const float* ob = partial_o(a, row, 0, D) + cb * kCW + 4 * c4;
  float M = -__builtin_inff(), L = 0.f;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = slot; j0 < ns; j0 += kSlots * kPer) {
    float2 p[kPer];
    float4 o[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int j = j0 + kSlots * i;
      const int jj = j < ns ? j : ns - 1;   // in bounds; weight 0 below
      p[i] = ml[jj];
      o[i] = *reinterpret_cast<const float4*>(ob + int64_t(jj) * D);
      if (j >= ns) p[i].x = -__builtin_inff();
    }
    float cm = p[0].x;
#pragma unroll
    for (int i = 1; i < kPer; ++i) cm = __builtin_fmaxf(cm, p[i].x);
    if (cm > M) {
      const float f = __builtin_amdgcn_exp2f(M - cm);   // 0 while M = -inf
      acc.x *= f; acc.y *= f; acc.z *= f; acc.w *= f;
      L *= f;
      M = cm;
    }
    const float Mref = M == -__builtin_inff() ? 0.f : M;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const float w = __builtin_amdgcn_exp2f(p[i].x - Mref);   // 0 for empty splits
      acc.x = __builtin_fmaf(w, o[i].x, acc.x);
      acc.y = __builtin_fmaf(w, o[i].y, acc.y);
      acc.z = __builtin_fmaf(w, o[i].z, acc.z);
      acc.w = __builtin_fmaf(w, o[i].w, acc.w);
      L = __builtin_fmaf(w, p[i].y, L);
    }
  }
  s_acc[slot][c4] = acc;
  if (c4 == 0) {
    s_m[slot] = M;
    s_l[slot] = L;
  }
  __syncthreads();
  // the slot weights 2^(M_k - M), once per slot
  if (t < kSlots) {
    float Mt = s_m[t];
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) Mt = __builtin_fmaxf(Mt, __shfl_xor(Mt, o, 32));
    const float Mref = Mt == -__builtin_inff() ? 0.f : Mt;
    s_w[t] = __builtin_amdgcn_exp2f(s_m[t] - Mref);
  }
  __syncthreads();
  if (t < kCW) {
    float sum = 0.f, Lt = 0.f;
    const int q = t / 4, e = t % 4;
#pragma unroll 8
    for (int k = 0; k < kSlots; ++k) {
      const float f = s_w[k];
      sum = __builtin_fmaf(f, reinterpret_cast<const float*>(&s_acc[k][q])[e], sum);
      Lt = __builtin_fmaf(f, s_l[k], Lt);
    }
    a.out[row * D + cb * kCW + t] = sum / Lt;
  }
}

// Workgroups of the VALU kernel resident per CU (its register use decides),
// asked of the runtime once per instantiation.
template <int DT, int D, int BITS, int MODE>
int attn_valu_blocks_per_cu() {
  static const int n = [] {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, k_attn_valu<DT, D, BITS, 4, MODE>, 256, 0) != hipSuccess ||
        v < 1)
      v = 1;
    return v;
  }();
  return n;
}
// Whether the one-split form (16 waves, output written directly) exists for
// this instantiation: it needs the kernel to fit four waves per SIMD (plain
// caches only).
template <int DT, int D, int BITS>
bool attn_valu_direct_ok() {
  return valu_waves_per_simd<DT, D, BITS>() == 4;
}

template <int DT, int D, int BITS, int MODE>
hipError_t launch_attn_valu(const AttnArgs& a, int B, hipStream_t s) {
  if (a.n_split == 1 && a.direct) {
    if constexpr (MODE == 0 && valu_waves_per_simd<DT, D, BITS>() == 4) {
      hipLaunchKernelGGL((k_attn_valu<DT, D, BITS, 16, 0>), dim3(1, a.Hq, B), dim3(1024), 0, s, a);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  hipLaunchKernelGGL((k_attn_valu<DT, D, BITS, 4, MODE>), dim3(a.n_split, a.Hq, B), dim3(256), 0, s, a);
  return hipGetLastError();
}
// Merge for up to 64 splits: one wave per (batch, q head) row.  Lane l
// folds float4 column l % kQ (kQ = D / 4) over splits l / kQ, l / kQ + kS,
// ... (kS = 64 / kQ slices), 16 per slice per round of loads, in
// registers; the slices then meet across lanes.
template <int DT, int D>
__global__ __launch_bounds__(64) void k_merge_row(AttnArgs a) {
  constexpr int kQ = D / 4;
  constexpr int kS = 64 / kQ;
  constexpr int kU = 16;
  const int lane = threadIdx.x, c4 = lane % kQ, ss = lane / kQ;
  const int64_t row = blockIdx.x;
  const int ns = a.n_split;
  const float2* ml = reinterpret_cast<const float2*>(partial_ml(a, row, 0));
  const float* ob = partial_o(a, row, 0, D) + 4 * c4;
  float M = -__builtin_inff(), L = 0.f;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = ss; j0 < ns; j0 += kS * kU) {
    float2 p[kU];
    float4 o[kU];
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const int j = j0 + kS * i;
      const int jj = j < ns ? j : ns - 1;   // in bounds; weight 0 below
      p[i] = ml[jj];
      o[i] = *reinterpret_cast<const float4*>(ob + int64_t(jj) * D);
      if (j >= ns) p[i].x = -__builtin_inff();
    }
    float cm = p[0].x;
#pragma unroll
    for (int i = 1; i < kU; ++i) cm = __builtin_fmaxf(cm, p[i].x);
    if (cm > M) {
      const float f = __builtin_amdgcn_exp2f(M - cm);   // 0 while M = -inf
      acc.x *= f; acc.y *= f; acc.z *= f; acc.w *= f;
      L *= f;
      M = cm;
    }
    const float Mref = M == -__builtin_inff() ? 0.f : M;
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const float w = __builtin_amdgcn_exp2f(p[i].x - Mref);   // 0 for empty splits
      acc.x = __builtin_fmaf(w, o[i].x, acc.x);
      acc.y = __builtin_fmaf(w, o[i].y, acc.y);
      acc.z = __builtin_fmaf(w, o[i].z, acc.z);
      acc.w = __builtin_fmaf(w, o[i].w, acc.w);
      L = __builtin_fmaf(w, p[i].y, L);
    }
  }
  // the slices meet: lanes kQ, 2 kQ apart hold the same column
#pragma unroll
  for (int x = kQ; x < 64; x <<= 1) {
    const float M2 = __shfl_xor(M, x, 64), L2 = __shfl_xor(L, x, 64);
    const float4 a2 = {__shfl_xor(acc.x, x, 64), __shfl_xor(acc.y, x, 64), __shfl_xor(acc.z, x, 64),
                       __shfl_xor(acc.w, x, 64)};
    const float Mn = __builtin_fmaxf(M, M2);
    const float Mr = Mn == -__builtin_inff() ? 0.f : Mn;
    const float f1 = __builtin_amdgcn_exp2f(M - Mr), f2 = __builtin_amdgcn_exp2f(M2 - Mr);
    acc.x = __builtin_fmaf(acc.x, f1, a2.x * f2);
    acc.y = __builtin_fmaf(acc.y, f1, a2.y * f2);
    acc.z = __builtin_fmaf(acc.z, f1, a2.z * f2);
    acc.w = __builtin_fmaf(acc.w, f1, a2.w * f2);
    L = __builtin_fmaf(L, f1, L2 * f2);
    M = Mn;
  }
  if (ss == 0) {
    float4 r = {acc.x / L, acc.y / L, acc.z / L, acc.w / L};
    *reinterpret_cast<float4*>(a.out + row * D + 4 * c4) = r;
  }
}

template <int DT, int D>
hipError_t launch_merge(const AttnArgs& a, int B, hipStream_t s) {
  if (a.n_split <= 64)
    hipLaunchKernelGGL((k_merge_row<DT, D>), dim3(unsigned(int64_t(B) * a.Hq)), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((k_merge<DT, D>), dim3(D / 32, a.Hq, B), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
