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
// numbers.  A code c becomes the fp16 value u = 1 + c / 2^b by placing its
// bits at the top of a 1.0 mantissa (exact).  With F = 2^b:
//   keys   (group delta_d, zero z_d):  q . k_hat = sum_d (F q_d delta_d) u_d
//                                               + sum_d q_d (z_d - F delta_d)
//   values (token delta_t, zero z_t):  sum_t p_t v_hat_t
//                                     = sum_t (F p_t delta_t) u_t
//                                       + (sum_t p_t (z_t - F delta_t)) * 1
// Scores are kept in the log2 domain (scale * log2 e folded into q).
#include "kvq_kernels.h"

namespace kvq {

// fp16 pair (code r, code r + 16/BITS) of a 32-bit code word, as 1 + c/2^b.
template <int BITS, int R>
__device__ __forceinline__ uint32_t code_pair_f16(uint32_t w) {
  constexpr int kNet = (10 - BITS) - BITS * R;  // shift bringing code R to bit 10-b
  constexpr uint32_t kMask = (((1u << BITS) - 1u) << (10 - BITS)) * 0x00010001u;
  uint32_t x;
  if constexpr (kNet > 0) x = w << kNet;
  else if constexpr (kNet < 0) x = w >> (-kNet);
  else x = w;
  return (x & kMask) | 0x3C003C00u;
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float lo_f16(uint32_t p) {
  return (float)__builtin_bit_cast(half2_t, p)[0];
}
__device__ __forceinline__ float hi_f16(uint32_t p) {
  return (float)__builtin_bit_cast(half2_t, p)[1];
}

// dot += sum over the codes of one 32-bit word of u(code) * coef[code index]
template <int BITS, int R = 0>
__device__ __forceinline__ void word_dot(uint32_t w, const float* coef, float& dot) {
  if constexpr (R < 16 / BITS) {
    const uint32_t p = code_pair_f16<BITS, R>(w);
    dot = __builtin_fmaf(lo_f16(p), coef[R], dot);
    dot = __builtin_fmaf(hi_f16(p), coef[R + 16 / BITS], dot);
    word_dot<BITS, R + 1>(w, coef, dot);
  }
}

// ---------------------------------------------------------------------------
// VALU kernel: one workgroup of 4 waves per (split, q head, batch).
// ---------------------------------------------------------------------------
template <int DT, int D, int BITS>
__global__ __launch_bounds__(256) void k_attn_valu(AttnArgs a) {
  using VL = VLayout<BITS>;
  constexpr float F = float(1 << BITS);
  constexpr int kRowBytes = D * BITS / 8;
  constexpr int kQuarterCh = D / 4;              // channels per lane in QK
  constexpr int kQuarterWords = kQuarterCh * BITS / 32;
  constexpr int kNST = VL::L / 16;               // 16-token sub-tiles per block
  constexpr int kUnits = D / 16;                 // value units per lane per block
  constexpr int kUnitWords = VL::UB / 4;

  const int split = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int h = hq / a.gqa;
  const int64_t bh = int64_t(b) * a.H + h;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  __shared__ float s_q[D];
  __shared__ float s_p[4][64];
  __shared__ float s_out[4][D + 2];

  for (int d = threadIdx.x; d < D; d += 256)
    s_q[d] = load1<DT>(a.q, b * a.q_sb + hq * a.q_sh + d) * a.sm_scale_log2;
  __syncthreads();

  float m = -__builtin_inff(), l = 0.f, z = 0.f;

  if (split < a.n_split_q) {
    float acc[kUnits];
#pragma unroll
    for (int n = 0; n < kUnits; ++n) acc[n] = 0.f;
    const int64_t nblk = (a.Q + VL::L - 1) / VL::L;
    const int64_t blk0 = int64_t(split) * a.blocks_per_split;
    const int64_t blk1 = blk0 + a.blocks_per_split < nblk ? blk0 + a.blocks_per_split : nblk;
    const int64_t per_wave = (blk1 - blk0 + 3) / 4;
    const int64_t wb0 = blk0 + wave * per_wave;
    const int64_t wb1 = wb0 + per_wave < blk1 ? wb0 + per_wave : blk1;

    const int qt = lane & 3;          // QK: channel quarter
    const int tl = lane >> 2;         // QK: token within the 16-token sub-tile
    const int vg = lane >> 4;         // PV: lane group g
    const int vj = lane & 15;         // PV: channel within 16
    float qpp[kQuarterCh];
    float kappa = 0.f;
    int64_t cur_grp = -1;
    const uint8_t* kc_head = a.k_codes + bh * a.qcap * kRowBytes;
    const uint8_t* vc_head = a.v_codes + bh * a.qcap * kRowBytes;

    for (int64_t blk = wb0; blk < wb1; ++blk) {
      const int64_t base_u = blk * VL::L;
      const int nvalid = int(a.Q - base_u < VL::L ? a.Q - base_u : VL::L);
      float sc[kNST];
#pragma unroll
      for (int st = 0; st < kNST; ++st) {
        if (st * 16 >= nvalid) { sc[st] = -__builtin_inff(); continue; }
        const int64_t u = base_u + st * 16 + tl;
        const int64_t grp = (base_u + st * 16) >> a.g_shift;
        if (grp != cur_grp) {
          cur_grp = grp;
          const float* ks = a.k_scale + (bh * a.kgroups + grp) * D + qt * kQuarterCh;
          const float* kz = a.k_zero + (bh * a.kgroups + grp) * D + qt * kQuarterCh;
          float kp = 0.f;
#pragma unroll
          for (int c = 0; c < kQuarterCh; ++c) {
            const float sq = s_q[qt * kQuarterCh + c];
            const float dl = ks[c];
            qpp[c] = F * sq * dl;
            kp = __builtin_fmaf(sq, kz[c] - F * dl, kp);
          }
          kappa = quad_sum(kp);
        }
        const uint32_t* src =
            reinterpret_cast<const uint32_t*>(kc_head + u * kRowBytes) + qt * kQuarterWords;
        uint32_t w[kQuarterWords];
#pragma unroll
        for (int i = 0; i < kQuarterWords; ++i) w[i] = src[i];
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < kQuarterWords; ++i) word_dot<BITS>(w[i], qpp + i * (32 / BITS), dot);
        sc[st] = quad_sum(dot) + kappa;
      }
      // online softmax (log2 domain)
      float lmax = sc[0];
#pragma unroll
      for (int st = 1; st < kNST; ++st) lmax = __builtin_fmaxf(lmax, sc[st]);
      const float bm = wave_max(lmax);
      const float new_m = __builtin_fmaxf(m, bm);
      const float alpha = __builtin_amdgcn_exp2f(m - new_m);
      m = new_m;
      l *= alpha;
      z *= alpha;
#pragma unroll
      for (int n = 0; n < kUnits; ++n) acc[n] *= alpha;
#pragma unroll
      for (int st = 0; st < kNST; ++st) {
        const int o = st * 16 + tl;
        if (qt == 0) {
          float pp = 0.f;
          if (o < nvalid) {
            const float p = __builtin_amdgcn_exp2f(sc[st] - m);
            const int64_t u = base_u + o;
            const float dv = a.v_scale[bh * a.qcap + u];
            const float zv = a.v_zero[bh * a.qcap + u];
            l += p;
            z = __builtin_fmaf(p, zv - F * dv, z);
            pp = F * p * dv;
          }
          s_p[wave][o] = pp;
        }
      }
      wave_lds_sync();
      // P . V over the block's value units
      float pv[VL::U];
#pragma unroll
      for (int i = 0; i < VL::U; ++i) pv[i] = s_p[wave][vslot_token<BITS>(vg, i)];
      const uint32_t* vsrc = reinterpret_cast<const uint32_t*>(
          vc_head + blk * (VL::L * kRowBytes) + (vg * 16 + vj) * kUnits * VL::UB);
#pragma unroll
      for (int n = 0; n < kUnits; ++n) {
#pragma unroll
        for (int wi = 0; wi < kUnitWords; ++wi) {
          const uint32_t w = vsrc[n * kUnitWords + wi];
          word_dot<BITS>(w, pv + wi * (32 / BITS), acc[n]);
        }
      }
      wave_lds_sync();
    }
    // combine the four lane groups (each summed a quarter of the tokens)
#pragma unroll
    for (int n = 0; n < kUnits; ++n) {
      acc[n] += swz_xor16(acc[n]);
      acc[n] += xor32(acc[n]);
    }
    l = wave_sum(l);
    z = wave_sum(z);
    if (lane < 16) {
#pragma unroll
      for (int n = 0; n < kUnits; ++n) s_out[wave][n * 16 + lane] = acc[n] + z;
    }
  } else {
    // full-precision tokens: sinks, then the residual ring
    constexpr int kC = D / 64;
    float acc[kC];
#pragma unroll
    for (int k = 0; k < kC; ++k) acc[k] = 0.f;
    const int64_t f0 = int64_t(split - a.n_split_q) * a.fp_per_split;
    const int64_t f1 = f0 + a.fp_per_split < a.n_fp ? f0 + a.fp_per_split : a.n_fp;
    for (int64_t i = f0 + wave; i < f1; i += 4) {
      const void* kb;
      const void* vb;
      int64_t off;
      if (i < a.n_sink) {
        kb = a.k_sink; vb = a.v_sink; off = (bh * a.S + i) * D;
      } else {
        int64_t slot = a.resid_slot0 + (i - a.n_sink);   // < 2 * ring
        if (slot >= a.ring) slot -= a.ring;
        kb = a.k_resid; vb = a.v_resid; off = (bh * a.ring + slot) * D;
      }
      float dot = 0.f;
#pragma unroll
      for (int k = 0; k < kC; ++k) dot = __builtin_fmaf(load1<DT>(kb, off + lane + 64 * k), s_q[lane + 64 * k], dot);
      const float s = wave_sum(dot);
      const float new_m = __builtin_fmaxf(m, s);
      const float alpha = __builtin_amdgcn_exp2f(m - new_m);
      const float p = __builtin_amdgcn_exp2f(s - new_m);
      m = new_m;
      l = l * alpha + p;
#pragma unroll
      for (int k = 0; k < kC; ++k) acc[k] = __builtin_fmaf(p, load1<DT>(vb, off + lane + 64 * k), acc[k] * alpha);
    }
#pragma unroll
    for (int k = 0; k < kC; ++k) s_out[wave][lane + 64 * k] = acc[k];
  }
  if (lane == 0) {
    s_out[wave][D] = m;
    s_out[wave][D + 1] = l;
  }
  __syncthreads();
  // merge the four waves and write this split's partial
  float* dst = a.ws + ((int64_t(b) * a.Hq + hq) * a.n_split + split) * (D + 2);
  float M = s_out[0][D];
#pragma unroll
  for (int w = 1; w < 4; ++w) M = __builtin_fmaxf(M, s_out[w][D]);
  float f[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) f[w] = __builtin_amdgcn_exp2f(s_out[w][D] - M);
  for (int d = threadIdx.x; d < D; d += 256) {
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) o = __builtin_fmaf(f[w], s_out[w][d], o);
    dst[d] = o;
  }
  if (threadIdx.x == 0) {
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) L = __builtin_fmaf(f[w], s_out[w][D + 1], L);
    dst[D] = M;
    dst[D + 1] = L;
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the split partials: one workgroup per (q head, batch).
// M = max_j m_j, L = sum_j 2^(m_j - M) l_j, out = sum_j 2^(m_j - M) o_j / L.
// All partial loads are independent: splits spread over the threads for M
// and the weights, then (channel, split-subset) pairs for the outputs.
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(256) void k_merge(AttnArgs a) {
  constexpr int kSub = 256 / D;             // token / split subsets per channel
  __shared__ float s_w[KVQ_MAX_SPLITS_DEV];
  __shared__ float s_red[8];
  __shared__ float s_part[kSub][D];
  const int hq = blockIdx.x, b = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int d = t % D, sub = t / D;

  // ---- split partials
  const int ns = a.n_split;
  const float* src = a.ws + (int64_t(b) * a.Hq + hq) * ns * (D + 2);
  float mx = -__builtin_inff();
  for (int j = t; j < ns; j += 256) mx = __builtin_fmaxf(mx, src[j * (D + 2) + D]);
  mx = wave_max(mx);
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  const float M = __builtin_fmaxf(__builtin_fmaxf(s_red[0], s_red[1]),
                                  __builtin_fmaxf(s_red[2], s_red[3]));
  float lsum = 0.f;
  for (int j = t; j < ns; j += 256) {
    const float e = __builtin_amdgcn_exp2f(src[j * (D + 2) + D] - M);
    s_w[j] = e;
    lsum = __builtin_fmaf(e, src[j * (D + 2) + D + 1], lsum);
  }
  lsum = wave_sum(lsum);
  __syncthreads();
  if (lane == 0) s_red[4 + wave] = lsum;
  float o = 0.f;
#pragma unroll 8
  for (int j = sub; j < ns; j += kSub) o = __builtin_fmaf(s_w[j], src[j * (D + 2) + d], o);
  s_part[sub][d] = o;
  __syncthreads();
  if (t < D) {
    const float L = s_red[4] + s_red[5] + s_red[6] + s_red[7];
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < kSub; ++k) acc += s_part[k][t];
    a.out[(int64_t(b) * a.Hq + hq) * D + t] = acc / L;
  }
}

template <int DT, int D, int BITS>
hipError_t launch_attn_valu(const AttnArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL((k_attn_valu<DT, D, BITS>), dim3(a.n_split, a.Hq, B), dim3(256), 0, s, a);
  return hipGetLastError();
}
template <int DT, int D>
hipError_t launch_merge(const AttnArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL((k_merge<DT, D>), dim3(a.Hq, B), dim3(256), 0, s, a);
  return hipGetLastError();
}

#define KVQ_INST_VALU(DT, D)                                                        \
  template hipError_t launch_attn_valu<DT, D, 2>(const AttnArgs&, int, hipStream_t); \
  template hipError_t launch_attn_valu<DT, D, 4>(const AttnArgs&, int, hipStream_t); \
  template hipError_t launch_attn_valu<DT, D, 8>(const AttnArgs&, int, hipStream_t);
KVQ_INST_VALU(DT_F32, 64)
KVQ_INST_VALU(DT_F32, 128)
KVQ_INST_VALU(DT_F16, 64)
KVQ_INST_VALU(DT_F16, 128)
KVQ_INST_VALU(DT_BF16, 64)
KVQ_INST_VALU(DT_BF16, 128)
#define KVQ_INST_MERGE(DT)                                                     \
  template hipError_t launch_merge<DT, 64>(const AttnArgs&, int, hipStream_t); \
  template hipError_t launch_merge<DT, 128>(const AttnArgs&, int, hipStream_t);
KVQ_INST_MERGE(DT_F32)
KVQ_INST_MERGE(DT_F16)
KVQ_INST_MERGE(DT_BF16)

}  // namespace kvq
