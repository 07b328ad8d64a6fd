// Kernel argument blocks and launcher declarations shared by the libkvq
// host API and its kernels.
#pragma once

#include "kvq_common.h"

namespace kvq {

// Copy full-precision rows (sinks [0, n_sink), then residual tokens
// [first_resid, first_resid + n_rows - n_sink)) from an input tensor into
// the sink array / residual ring.
struct FpCopyArgs {
  const void* src;
  int64_t sb, sh, st;       // input strides (elements)
  void* sink;               // [B][H][S][D]
  void* resid;              // [B][H][ring][D]
  int64_t n_sink, first_resid, S, ring;
  int H;
};

// Prefill quantization of one half (keys or values).
struct QuantArgs {
  const void* src;
  int64_t sb, sh, st;
  uint8_t* codes;
  float* scale;
  float* zero;
  int64_t S, qcap;
  int64_t k0;               // first unit quantized (groups or 32-token steps); unit k goes to
                            // storage (k * unit tokens) mod qcap
  uint8_t* oidx;            // side table (outliers != 0): positions, laid out as scale
  uint8_t* oval;            // and the kept values in the input dtype
  int H, G, outliers;
  // Workgroups x >= n_units copy the full-precision rows instead (sinks,
  // then the residual tokens: n_fp_rows per head, 256 16-byte vectors per
  // workgroup).
  FpCopyArgs fp;
  int64_t n_units, n_fp_rows;
};

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  int64_t k_sb, k_sh, v_sb, v_sh;
  uint8_t* k_codes;
  uint8_t* v_codes;
  float *k_scale, *k_zero, *v_scale, *v_zero;
  void *k_sink, *v_sink, *k_resid, *v_resid;
  int64_t n_before, q_old, S, R, qcap;
  int64_t r_old;            // storage row of quantized token q_old: q_old mod qcap
  uint8_t *k_oidx, *k_oval, *v_oidx, *v_oval;   // side tables (outliers != 0)
  int H, G, flush, outliers;
};

// Decode attention.  Split partials of row r = b*Hq + hq: o (D floats,
// unnormalized) at ws[(r*n_split + split)*D], and the pair (m, l) (m in the
// log2 domain) at ws[ml_offset + 2*(r*n_split + split)], with ml_offset =
// B*Hq*n_split*D: the o rows stay 16-byte aligned for vector loads.
struct AttnArgs {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float *k_scale, *k_zero, *v_scale, *v_zero;
  const void *k_sink, *v_sink, *k_resid, *v_resid;
  const void* q;
  int64_t q_sb, q_sh;
  float* ws;
  float* out;
  float sm_scale_log2;      // softmax scale * log2(e)
  int64_t T, S, Q, qcap, ring, first_resid, n_sink, n_fp;
  int64_t kgroups;          // qcap / G
  int64_t resid_slot0;      // ring slot of the first residual token, Q mod ring
  int H, Hq, gqa, G, g_shift;
  int n_split;              // splits per (batch, q head)
  int direct;               // VALU kernel, one split per row: write out, no merge
  int blocks_per_split;     // value-code blocks per split (VALU kernel; the matrix-core
                            // kernel's waves take chunks from a counter instead)
  int fp_per_split;         // full-precision tokens per split
  int64_t ml_offset;        // floats before the (m, l) pairs in ws
  // Sliding window: quantized tokens before u_lo are outside it.  The
  // kernel's units (64-token chunks, or value blocks for the VALU kernel)
  // start at unit c0; unit c sits at storage unit c - cw, less ncap when
  // that reaches ncap (live units span at most ncap + 1, so one subtraction
  // suffices); lo_off = u_lo - c0 * unit tokens of unit c0 are masked.
  int64_t u_lo, c0, cw, ncap;
  int lo_off;
  // Dense-and-sparse outliers (outliers != 0, VALU kernel): side tables of
  // one kept entry per key group channel and per value token.
  const uint8_t *k_oidx, *v_oidx;
  const void *k_oval, *v_oval;
  int outliers;
  // Pre-RoPE keys (rope != 0): log2 of the rotation base.
  double rope_log2_base;
  int rope;
};

__device__ __forceinline__ float* partial_o(const AttnArgs& a, int64_t row, int split, int D) {
  return a.ws + (row * a.n_split + split) * D;
}
__device__ __forceinline__ float* partial_ml(const AttnArgs& a, int64_t row, int split) {
  return a.ws + a.ml_offset + (row * a.n_split + split) * 2;
}

template <int DT, int D, int BITS>
hipError_t launch_quant_keys(const QuantArgs& a, int64_t n_blocks, int B, int H, hipStream_t s);
template <int DT, int D, int BITS>
hipError_t launch_quant_values(const QuantArgs& a, int64_t n_blocks, int B, int H, hipStream_t s);
template <int DT, int D, int BITS>
hipError_t launch_append(const AppendArgs& a, int B, int H, hipStream_t s);
// MODE bit 0: side tables; bit 1: pre-RoPE keys.
template <int DT, int D, int BITS, int MODE>
hipError_t launch_attn_valu(const AttnArgs& a, int B, hipStream_t s);
template <int DT, int D, int BITS, int MODE>
int attn_valu_blocks_per_cu();
template <int DT, int D, int BITS>
bool attn_valu_direct_ok();
// GQA groups of 2..8 query heads, up to four per workgroup (MODE as above).
template <int DT, int D, int BITS, int MODE>
hipError_t launch_attn_gqa(const AttnArgs& a, int B, hipStream_t s);
template <int DT, int D, int BITS, int MODE>
int attn_gqa_blocks_per_cu();
// The matrix-core kernel: one workgroup of kMfmaWaves waves per CU.  Each
// wave stages the rows of its exact (sink and residual) tokens in 4 KB of
// LDS, so a split takes at most mfma_exact_cap(element bytes, D) of them.
constexpr int kMfmaWaves = 8;
constexpr int mfma_exact_cap(int esz, int D) {
  return kMfmaWaves * (4096 / (2 * D * esz)) < 64 ? kMfmaWaves * (4096 / (2 * D * esz)) : 64;
}
template <int DT, int D, int BITS, int GQA>
hipError_t launch_attn_mfma(const AttnArgs& a, int B, hipStream_t s);
template <int DT, int D>
hipError_t launch_merge(const AttnArgs& a, int B, hipStream_t s);

}  // namespace kvq
