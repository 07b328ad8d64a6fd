// Split-K decode attention, VALU form, with up to four query heads of one
// KV head in one workgroup (GQA; tract PR "KIVI-style KV-cache
// quantization", What's in the PR: GQA handled).  It serves the cases the matrix-core
// kernel has no form for at GQA 2..8: code widths other than 2 and 4 bits
// (read as a bit stream), caches with outlier side tables (pigeon guide
// "KV-cache quantization", KVQuant adds: a sparse side table of outliers)
// and keys cached before the rotary position embedding (same section:
// quantize keys before RoPE).
//
// Every code is extracted once and feeds one FMA per head; with pre-RoPE
// keys every key is dequantized and rotated once and then feeds one FMA per
// head.  The dequantization folds as in the per-head kernel:
//   q_h . k_hat     = sum_d (q_hd delta_d) c_d + sum_d q_hd z_d
//   sum_t p_ht v_hat = sum_t (p_ht delta_t) c_t + sum_t p_ht z_t
// Scores are in the log2 domain (scale * log2 e folded into q).
//
// Lanes: q.K lane (qt, tl) takes channel quarter qt of token tl of each
// 16-token tile; P.V lane (vg, vj) holds value units of channels vj + 16n
// for the tokens of lane group vg (the value layout of kvq.h).  Per head a
// lane keeps its running max, sum, zero-point sum, scores and P.V
// accumulators; a GQA group of g heads takes ceil(g / 4) workgroups, and
// heads past the group's count are skipped by uniform branches.
#pragma once

#include "kvq_attn_impl.h"

namespace kvq {

constexpr int kGqaMax = 8;   // query heads per KV head this kernel takes
constexpr int kGqaHeads = 4; // query heads per workgroup

template <int DT, int D, int BITS, int MODE>
__global__ __launch_bounds__(256, 2) void k_attn_gqa(AttnArgs a) {
  constexpr bool OUTL = (MODE & kModeOutliers) != 0;
  constexpr bool ROPE = (MODE & kModeRope) != 0;
  constexpr int NW = 4, H8 = kGqaHeads;
  using VL = VLayout<BITS>;
  constexpr int kRowBytes = D * BITS / 8;
  constexpr int kQuarterCh = D / 4;               // channels per lane in q.K
  constexpr int kQBytes = kQuarterCh * BITS / 8;  // bytes of a lane's quarter row
  constexpr int kQW = (kQBytes + 3) / 4;          // its words (the last may be part full)
  constexpr int kNST = VL::L / 16;                // 16-token sub-tiles per block
  constexpr int kHalves = VL::L / 32;             // 32-token key-group steps per block
  constexpr int kUnits = D / 16;                  // value units per lane per block
  constexpr int kVW = kUnits * VL::UB / 4;        // value-code words per lane per block
  constexpr int kWC = D / 64;                     // channels per lane in row-wise work
  constexpr float kLev = float((1 << BITS) - 1);

  const int ngrp = (a.gqa + H8 - 1) / H8;       // workgroups per KV head
  const int split = blockIdx.x, h = blockIdx.y / ngrp, b = blockIdx.z;
  const int hg = blockIdx.y % ngrp;
  const int g = a.gqa - hg * H8 < H8 ? a.gqa - hg * H8 : H8;   // heads of this workgroup
  const int64_t bh = int64_t(b) * a.H + h;
  const int hq0 = h * a.gqa + hg * H8;           // its first query head
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qt = lane & 3, tl = lane >> 2;
  const int vg = lane >> 4, vj = lane & 15;

  // s_q[d][h]: scale * log2e * q of head h; s_x: per wave and key-group
  // half, q_hd * delta_d (or, with pre-RoPE keys, delta_d and z_d)
  __shared__ __attribute__((aligned(16))) float s_q[D][H8];
  __shared__ __attribute__((aligned(16))) float s_x[NW][kHalves][D][ROPE ? 2 : H8];
  __shared__ float s_out[NW][H8][D + 2];
  __shared__ float s_kc[OUTL ? NW : 1][OUTL ? H8 : 1][OUTL ? kHalves * 32 : 1];
  __shared__ float s_vc[OUTL ? NW : 1][OUTL ? H8 : 1][OUTL ? D : 1];
  __shared__ double s_cd[ROPE ? D / 2 : 1];
  __shared__ float s_c[ROPE ? D / 2 : 1];
  __shared__ float s_fb[ROPE ? NW : 1][ROPE ? D / 2 : 1];

  for (int i = threadIdx.x; i < D * H8; i += 256) {
    const int d = i / H8, hh = i % H8;
    s_q[d][hh] = hh < g ? load1<DT>(a.q, b * a.q_sb + (hq0 + hh) * a.q_sh + d) * a.sm_scale_log2 : 0.f;
  }
  if constexpr (OUTL) {
    for (int i = threadIdx.x; i < NW * H8 * kHalves * 32; i += 256) (&s_kc[0][0][0])[i] = 0.f;
    for (int i = threadIdx.x; i < NW * H8 * D; i += 256) (&s_vc[0][0][0])[i] = 0.f;
  }
  if constexpr (ROPE) {
    for (int i = threadIdx.x; i < D / 2; i += 256) {
      const double c = exp2(-2.0 * double(i) / double(D) * a.rope_log2_base) * 0.15915494309189535;
      s_cd[i] = c;
      s_c[i] = float(c);
    }
  }
  __syncthreads();

  float m[H8], l[H8], z[H8];
  float acc[H8][kUnits], accf[H8][kWC];
#pragma unroll
  for (int hh = 0; hh < H8; ++hh) {
    m[hh] = -__builtin_inff();
    l[hh] = 0.f;
    z[hh] = 0.f;
#pragma unroll
    for (int n = 0; n < kUnits; ++n) acc[hh][n] = 0.f;
#pragma unroll
    for (int c = 0; c < kWC; ++c) accf[hh][c] = 0.f;
  }
  auto raise_max = [&](int hh, float bm) {
    const float new_m = __builtin_fmaxf(m[hh], bm);
    if (new_m > m[hh]) {   // wave-uniform
      const float alpha = __builtin_amdgcn_exp2f(m[hh] - new_m);
      l[hh] *= alpha;
      z[hh] *= alpha;
#pragma unroll
      for (int n = 0; n < kUnits; ++n) acc[hh][n] *= alpha;
#pragma unroll
      for (int c = 0; c < kWC; ++c) accf[hh][c] *= alpha;
      m[hh] = new_m;
    }
  };
  auto tile_max = [&](float v) {   // over the 16 tokens of the tile(s)
    v = __builtin_fmaxf(v, dpp_mov<kRowRor4>(v));
    v = __builtin_fmaxf(v, dpp_mov<kRowRor8>(v));
    return max_xor32(max_xor16(v));
  };
  // Heads' query values of channel d, four at a time from LDS.
  auto heads4 = [&](const float* row, int hh0, float* out4) {
    const float4 v = *reinterpret_cast<const float4*>(row + hh0);
    out4[0] = v.x; out4[1] = v.y; out4[2] = v.z; out4[3] = v.w;
  };
  // Pre-RoPE keys: quarter qt pairs with qt ^ 2 (channel i with i + D/2);
  // the frequency of a lane's channel j and the sign of its partner term.
  const bool rp_hi = qt >= 2;
  const int rp_f0 = (rp_hi ? qt - 2 : qt) * kQuarterCh;
  const float rp_sgn = rp_hi ? 1.f : -1.f;   // k' = k cos + sgn * partner * sin

  // Blocks are numbered from the first one the query attends to (block c0).
  const int64_t nblk = (a.Q + VL::L - 1) / VL::L - a.c0;
  const int64_t blk0 = int64_t(split) * a.blocks_per_split;
  const int64_t blk1 = blk0 + a.blocks_per_split < nblk ? blk0 + a.blocks_per_split : nblk;
  const int64_t per_wave = blk1 > blk0 ? (blk1 - blk0 + NW - 1) / NW : 0;
  const int64_t wb0 = blk0 + wave * per_wave;
  const int64_t wb1 = wb0 + per_wave < blk1 ? wb0 + per_wave : blk1;

  int vexp = 156;
  float vthr = __builtin_amdgcn_ldexpf(1.0f, 7 - vexp);
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
  // Every address lies inside the allocation (qcap is a multiple of max(64,
  // G) tokens); tokens past the quantized count are masked after the loads.
  auto blk_base = [&](int64_t blk) -> int64_t {   // first storage row of block blk
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
#pragma unroll
    for (int st = 0; st < kNST; ++st) {
      r.dv[st] = vs_head[base + uint32_t(tl + st * 16)];
      r.zv[st] = vz_head[base + uint32_t(tl + st * 16)];
    }
#pragma unroll
    for (int k = 0; k < kHalves; ++k) {
      const int64_t grp = (base + 32 * k) >> a.g_shift;
#pragma unroll
      for (int c = 0; c < kWC; ++c) {
        r.ks[k][c] = ks_head[grp * D + c_off + c];
        r.kz[k][c] = kz_head[grp * D + c_off + c];
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
    auto fp_row = [&](int64_t i, bool& sink) {
      sink = i < a.n_sink;
      int64_t slot = a.resid_slot0 + (i - a.n_sink);   // < 2 * ring
      slot -= slot >= a.ring ? a.ring : 0;
      return (sink ? bh * a.S + i : bh * a.ring + slot) * D;
    };
    for (int64_t t0 = fw0; t0 < fw1; t0 += 16) {
      bool sk;
      const int64_t ik = t0 + tl < fw1 ? t0 + tl : fw1 - 1;
      const int64_t ko = fp_row(ik, sk);
      float kr[kQuarterCh];
      load_row_run<DT, kQuarterCh>(sk ? a.k_sink : a.k_resid, ko + qt * kQuarterCh, kr);
      if constexpr (ROPE) {
        // rotate the key to its position (its token index)
        const int64_t pos = ik < a.n_sink ? ik : a.first_resid + (ik - a.n_sink);
#pragma unroll
        for (int j = 0; j < kQuarterCh; ++j) {
          const float par = dpp_mov<kQuadXor2>(kr[j]);
          const double x = double(pos) * s_cd[rp_f0 + j];
          float sn, cs;
          sincos_rev(float(x - __builtin_floor(x)), sn, cs);
          kr[j] = __builtin_fmaf(kr[j], cs, rp_sgn * par * sn);
        }
      }
      float dot[H8];
#pragma unroll
      for (int hh = 0; hh < H8; ++hh) dot[hh] = 0.f;
#pragma unroll
      for (int j = 0; j < kQuarterCh; ++j) {
        const float* qrow = s_q[qt * kQuarterCh + j];
#pragma unroll
        for (int h4 = 0; h4 < H8; h4 += 4) {
          if (h4 < g) {
            float q4[4];
            heads4(qrow, h4, q4);
#pragma unroll
            for (int e = 0; e < 4; ++e) dot[h4 + e] = __builtin_fmaf(kr[j], q4[e], dot[h4 + e]);
          }
        }
      }
      float vr[16][kWC];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        bool sv;
        const int64_t iv = t0 + t < fw1 ? t0 + t : fw1 - 1;
        const int64_t vo = fp_row(iv, sv);
        load_small<DT, kWC>(sv ? a.v_sink : a.v_resid, vo + lane * kWC, vr[t]);
      }
      const float mask = t0 + tl < fw1 ? 0.f : -__builtin_inff();
#pragma unroll
      for (int hh = 0; hh < H8; ++hh) {
        if (hh < g) {
          const float sc = quad_sum(dot[hh]) + mask;
          raise_max(hh, tile_max(sc));
          const float p = __builtin_amdgcn_exp2f(sc - m[hh]);   // 0 past the run
          l[hh] += p;
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const float pt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), 4 * t));
#pragma unroll
            for (int c = 0; c < kWC; ++c) accf[hh][c] = __builtin_fmaf(pt, vr[t][c], accf[hh][c]);
          }
        }
      }
    }
  }

  // ---- quantized blocks
  auto process = [&](int64_t blk, const Blk& r) {
    const int64_t base = (a.c0 + blk) * VL::L;   // quantized index of the block's first token
    const int nvalid = int(a.Q - base < VL::L ? a.Q - base : VL::L);
    const int lo = blk == 0 ? a.lo_off : 0;      // tokens before the window
    // per key-group half: the weights q_hd delta_d (or delta, zero) and kappa_h
    float kap[kHalves][H8];
#pragma unroll
    for (int k = 0; k < kHalves; ++k) {
#pragma unroll
      for (int hh = 0; hh < H8; ++hh) kap[k][hh] = 0.f;
#pragma unroll
      for (int c = 0; c < kWC; ++c) {
        const int ch = lane * kWC + c;
        if constexpr (ROPE) {
          s_x[wave][k][ch][0] = r.ks[k][c];
          s_x[wave][k][ch][1] = r.kz[k][c];
        } else {
#pragma unroll
          for (int hh = 0; hh < H8; ++hh) {
            const float qv = s_q[ch][hh];
            s_x[wave][k][ch][hh] = qv * r.ks[k][c];
            kap[k][hh] = __builtin_fmaf(qv, r.kz[k][c], kap[k][hh]);
          }
        }
      }
      if constexpr (!ROPE) {
#pragma unroll
        for (int hh = 0; hh < H8; ++hh)
          if (hh < g) kap[k][hh] = wave_sum_valu(kap[k][hh]);
      }
    }
    if constexpr (ROPE) {
      if (lane < D / 2) {   // revolutions at the block's first token, position S + base
        const double x = double(a.S + base) * s_cd[lane];
        s_fb[wave][lane] = float(x - __builtin_floor(x));
      }
    }
    wave_lds_sync();
    if constexpr (OUTL) {
      // keys kept exact: channel ch's entry at group offset j adds
      // q'_h,ch (x - dense) to token j of its half for every head, dense =
      // zp + delta (2^b - 1) above the zero point, else zp; q' is q rotated
      // back by the token's angle with pre-RoPE keys
#pragma unroll
      for (int k = 0; k < kHalves; ++k) {
        const int64_t row = blk_base(blk) + 32 * k;
        const int64_t gi = ((row >> a.g_shift) + bh * a.kgroups) * D;
        const int off = int(row & (a.G - 1));
#pragma unroll
        for (int c = 0; c < kWC; ++c) {
          const int ch = lane * kWC + c;
          const int j = int(a.k_oidx[gi + ch]) - off;
          if (j >= 0 && j < 32) {
            const float xv = load1<DT>(a.k_oval, gi + ch);
            const float dense = xv < r.kz[k][c] ? r.kz[k][c] : __builtin_fmaf(kLev, r.ks[k][c], r.kz[k][c]);
            float cs = 1.f, sn = 0.f, sg = 0.f;
            if constexpr (ROPE) {
              const int fi = ch & (D / 2 - 1);
              float rev = __builtin_fmaf(float(k * 32 + j), s_c[fi], s_fb[wave][fi]);
              rev -= __builtin_floorf(rev);
              sincos_rev(rev, sn, cs);
              sg = ch < D / 2 ? 1.f : -1.f;
            }
#pragma unroll
            for (int hh = 0; hh < H8; ++hh) {
              if (hh < g) {
                float qe = s_q[ch][hh];
                if constexpr (ROPE) qe = __builtin_fmaf(qe, cs, sg * s_q[ch ^ (D / 2)][hh] * sn);
                atomicAdd(&s_kc[wave][hh][k * 32 + j], qe * (xv - dense));
              }
            }
          }
        }
      }
      wave_lds_sync();
    }
    // scores (log2 domain); lane (qt, tl) ends with token st*16 + tl
    float sc[kNST][H8];
#pragma unroll
    for (int k = 0; k < kHalves; ++k) {
      float dot[2][H8];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int hh = 0; hh < H8; ++hh) dot[u][hh] = 0.f;
#pragma unroll
      for (int j = 0; j < kQuarterCh; ++j) {
        const int ch = qt * kQuarterCh + j;
        float kv[2];
        if constexpr (ROPE) {
          const float dl = s_x[wave][k][ch][0], zp = s_x[wave][k][ch][1];
          const int fi = rp_f0 + j;
          const float ci = s_c[fi], fb = s_fb[wave][fi];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int st = 2 * k + u;
            const float own = __builtin_fmaf(stream_code<BITS>(r.kw[st], j * BITS), dl, zp);
            const float par = dpp_mov<kQuadXor2>(own);
            float rev = __builtin_fmaf(float(st * 16 + tl), ci, fb);
            rev -= __builtin_floorf(rev);
            float sn, cs;
            sincos_rev(rev, sn, cs);
            kv[u] = __builtin_fmaf(own, cs, rp_sgn * par * sn);
          }
        } else {
#pragma unroll
          for (int u = 0; u < 2; ++u) kv[u] = stream_code<BITS>(r.kw[2 * k + u], j * BITS);
        }
        const float* wrow = ROPE ? s_q[ch] : s_x[wave][k][ch];
#pragma unroll
        for (int h4 = 0; h4 < H8; h4 += 4) {
          if (h4 < g) {
            float w4[4];
            heads4(wrow, h4, w4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
              for (int u = 0; u < 2; ++u) dot[u][h4 + e] = __builtin_fmaf(kv[u], w4[e], dot[u][h4 + e]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int st = 2 * k + u;
        const bool ok = st * 16 + tl < nvalid && st * 16 + tl >= lo;
#pragma unroll
        for (int hh = 0; hh < H8; ++hh) {
          if (hh < g) {
            float v = quad_sum(dot[u][hh]) + kap[k][hh];
            if constexpr (OUTL) v += s_kc[wave][hh][st * 16 + tl];
            // -inf past the quantized count (selected: parameters of a group
            // past the count are never written and may hold anything)
            sc[st][hh] = ok ? v : -__builtin_inff();
          }
        }
      }
    }
    wave_lds_sync();
    if constexpr (OUTL) if (qt == 0) {   // cleared for the next block (each wave reads in order)
#pragma unroll
      for (int hh = 0; hh < H8; ++hh)
        if (hh < g)
#pragma unroll
          for (int st = 0; st < kNST; ++st) s_kc[wave][hh][st * 16 + tl] = 0.f;
    }
    // value exponent (shared by the heads: it follows the value deltas)
    float dvs[kNST];
    float vmax = 0.f;
#pragma unroll
    for (int st = 0; st < kNST; ++st) {
      dvs[st] = st * 16 + tl < nvalid && st * 16 + tl >= lo ? r.dv[st] : 0.f;
      vmax = __builtin_fmaxf(vmax, dvs[st]);
    }
    if (__builtin_amdgcn_ballot_w64(vmax >= vthr) != 0) {   // rare: a larger value delta
      const int knew = __builtin_amdgcn_readfirstlane(7 - __builtin_amdgcn_frexp_expf(wave_max(vmax)));
#pragma unroll
      for (int hh = 0; hh < H8; ++hh)
#pragma unroll
        for (int n = 0; n < kUnits; ++n) acc[hh][n] = __builtin_amdgcn_ldexpf(acc[hh][n], knew - vexp);
      vexp = knew;
      vthr = __builtin_amdgcn_ldexpf(1.0f, 7 - vexp);
    }
    // softmax weights of the block's tokens, per head, scaled for P . V
    float pp[H8][kNST];
#pragma unroll
    for (int hh = 0; hh < H8; ++hh) {
      if (hh < g) {
        float lmax = sc[0][hh];
#pragma unroll
        for (int st = 1; st < kNST; ++st) lmax = __builtin_fmaxf(lmax, sc[st][hh]);
        raise_max(hh, tile_max(lmax));
#pragma unroll
        for (int st = 0; st < kNST; ++st) {
          const bool ok = st * 16 + tl < nvalid && st * 16 + tl >= lo;
          const float p = __builtin_amdgcn_exp2f(sc[st][hh] - m[hh]);   // 0 past the range
          l[hh] += p;
          z[hh] = __builtin_fmaf(p, ok ? r.zv[st] : 0.f, z[hh]);
          pp[hh][st] = p * __builtin_amdgcn_ldexpf(dvs[st], vexp);
          if constexpr (OUTL) if (qt == 0 && ok) {
            // a value kept exact: p (x - dense) on its channel
            const int64_t row = blk_base(blk) + st * 16 + tl;
            const int vi = a.v_oidx[bh * a.qcap + row];
            if (vi != 255) {
              const float xv = load1<DT>(a.v_oval, bh * a.qcap + row);
              const float dense = xv < r.zv[st] ? r.zv[st] : __builtin_fmaf(kLev, r.dv[st], r.zv[st]);
              atomicAdd(&s_vc[wave][hh][vi], p * (xv - dense));
            }
          }
        }
      }
    }
    if constexpr (OUTL) {   // folded into the exact-token sums, which share p's scale
      wave_lds_sync();
#pragma unroll
      for (int hh = 0; hh < H8; ++hh) {
        if (hh < g) {
#pragma unroll
          for (int c = 0; c < kWC; ++c) {
            accf[hh][c] += s_vc[wave][hh][lane * kWC + c];
            s_vc[wave][hh][lane * kWC + c] = 0.f;
          }
        }
      }
    }
    // P . V, four code slots at a time: slot i of lane group vg is token
    // vslot_token(vg, i), whose weight sits in lane 4 (i & 3) of this row,
    // sub-tile vslot_token / 16; unit n holds slot i at bit (U n + i) b, and
    // each code is extracted once for all heads
#pragma unroll
    for (int i0 = 0; i0 < VL::U; i0 += 4) {
      float pv[H8][4];
#pragma unroll
      for (int hh = 0; hh < H8; ++hh) {
        if (hh < g) {
          pv[hh][0] = row_bcast<0>(pp[hh][vslot_token<BITS>(0, i0) / 16]);
          pv[hh][1] = row_bcast<4>(pp[hh][vslot_token<BITS>(0, i0 + 1) / 16]);
          pv[hh][2] = row_bcast<8>(pp[hh][vslot_token<BITS>(0, i0 + 2) / 16]);
          pv[hh][3] = row_bcast<12>(pp[hh][vslot_token<BITS>(0, i0 + 3) / 16]);
        }
      }
#pragma unroll
      for (int n = 0; n < kUnits; ++n) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c = stream_code<BITS>(r.vw, (VL::U * n + i0 + e) * BITS);
#pragma unroll
          for (int hh = 0; hh < H8; ++hh)
            if (hh < g) acc[hh][n] = __builtin_fmaf(c, pv[hh][e], acc[hh][n]);
        }
      }
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

  // ---- wave results: the four lane groups each hold a quarter of the
  // tokens; l and z were gathered four times per token (once per quad lane)
#pragma unroll
  for (int hh = 0; hh < H8; ++hh) {
    if (hh < g) {
#pragma unroll
      for (int n = 0; n < kUnits; ++n) acc[hh][n] = sum_xor32(sum_xor16(acc[hh][n]));
      const float lh = 0.25f * wave_sum_valu(l[hh]);
      const float zh = 0.25f * wave_sum_valu(z[hh]);
      if (lane < 16) {
#pragma unroll
        for (int n = 0; n < kUnits; ++n)
          s_out[wave][hh][n * 16 + lane] = __builtin_amdgcn_ldexpf(acc[hh][n], -vexp) + zh;
      }
      wave_lds_sync();
#pragma unroll
      for (int c = 0; c < kWC; ++c) s_out[wave][hh][lane * kWC + c] += accf[hh][c];
      if (lane == 0) {
        s_out[wave][hh][D] = m[hh];
        s_out[wave][hh][D + 1] = lh;
      }
    }
  }
  __syncthreads();
  // merge the waves into this split's partial of each head
  for (int i = threadIdx.x; i < g * D; i += 256) {
    const int hh = i / D, d = i % D;
    float M = s_out[0][hh][D];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = __builtin_fmaxf(M, s_out[w][hh][D]);
    const float Mref = M == -__builtin_inff() ? 0.f : M;
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = __builtin_amdgcn_exp2f(s_out[w][hh][D] - Mref);
      o = __builtin_fmaf(f, s_out[w][hh][d], o);
      L = __builtin_fmaf(f, s_out[w][hh][D + 1], L);
    }
    const int64_t row = int64_t(b) * a.Hq + hq0 + hh;
    partial_o(a, row, split, D)[d] = o;
    if (d == 0) *reinterpret_cast<float2*>(partial_ml(a, row, split)) = float2{M, L};
  }
}

template <int DT, int D, int BITS, int MODE>
int attn_gqa_blocks_per_cu() {
  static const int n = [] {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, k_attn_gqa<DT, D, BITS, MODE>, 256, 0) != hipSuccess ||
        v < 1)
      v = 1;
    return v;
  }();
  return n;
}

template <int DT, int D, int BITS, int MODE>
hipError_t launch_attn_gqa(const AttnArgs& a, int B, hipStream_t s) {
  if (a.gqa < 2 || a.gqa > kGqaMax) return hipErrorInvalidValue;
  const int ngrp = (a.gqa + kGqaHeads - 1) / kGqaHeads;
  hipLaunchKernelGGL((k_attn_gqa<DT, D, BITS, MODE>), dim3(a.n_split, a.H * ngrp, B), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
