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
  int H, G;
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
  int H, G, flush;
};

// Decode attention.  Partials: ws[((b*Hq + hq)*n_split + split)*(D+2) + ...]
// holds o (D floats, unnormalized), then m (log2 domain), then l.  With the
// merge fused into the attention kernel, splits are merged in groups of
// merge_group as they arrive: group g's merged partial goes to
// ws2[((b*Hq + hq)*n_groups + g)*(D+2) + ...], and the last group to
// arrive writes the output.  Arrival counters (zero between calls):
// counters[row*n_groups + g] per group, counters[n_rows*n_groups + row] per
// row, with row = b * gridDim.y + blockIdx.y and n_rows = gridDim.y * gridDim.z.
struct AttnArgs {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float *k_scale, *k_zero, *v_scale, *v_zero;
  const void *k_sink, *v_sink, *k_resid, *v_resid;
  const void* q;
  int64_t q_sb, q_sh;
  float* ws;
  float* ws2;               // merged partials of split groups (fused merge)
  uint32_t* counters;       // arrival counters (fused merge)
  float* out;
  float sm_scale_log2;      // softmax scale * log2(e)
  int64_t T, S, Q, qcap, ring, first_resid, n_sink, n_fp;
  int64_t kgroups;          // qcap / G
  int64_t resid_slot0;      // ring slot of the first residual token, Q mod ring
  int H, Hq, gqa, G, g_shift;
  int n_split;              // splits per (batch, q head)
  int direct;               // VALU kernel, one split per row: write out, no merge
  int fused;                // splits merge inside the attention kernel (no k_merge)
  int merge_group;          // splits per first-level merge group
  int n_groups;             // ceil(n_split / merge_group)
  int blocks_per_split;     // value-code blocks per quantized split
  int fp_per_split;         // full-precision tokens per split that takes them
};

// Fused split merge, run by every workgroup of an attention grid after it
// has stored its partial for heads hq0 .. hq0 + H - 1 with st_dev: the last
// split of each group to arrive merges the group, and the last group of the
// row to arrive writes the output rows.
template <int H, int D>
__device__ __forceinline__ void merge_split(const AttnArgs& a, int b, int hq0, int split) {
  __shared__ int s_flag;
  const int64_t row = int64_t(blockIdx.z) * gridDim.y + blockIdx.y;
  const int64_t n_rows = int64_t(gridDim.y) * gridDim.z;
  const int g = split / a.merge_group;
  const int gsize = a.n_split - g * a.merge_group < a.merge_group ? a.n_split - g * a.merge_group : a.merge_group;
  if (!arrive_last(a.counters + row * a.n_groups + g, uint32_t(gsize), &s_flag)) return;
  const int64_t head0 = int64_t(b) * a.Hq + hq0;
  const float* src = a.ws + (head0 * a.n_split + int64_t(g) * a.merge_group) * (D + 2);
  float* out = a.out + head0 * D;
  if (a.n_groups == 1) {
    merge_partials<H, D>(src, a.n_split, gsize, true, out, D);
    return;
  }
  float* dst2 = a.ws2 + (head0 * a.n_groups + g) * (D + 2);
  merge_partials<H, D>(src, a.n_split, gsize, false, dst2, int64_t(a.n_groups) * (D + 2));
  if (!arrive_last(a.counters + n_rows * a.n_groups + row, uint32_t(a.n_groups), &s_flag)) return;
  merge_partials<H, D>(a.ws2 + head0 * a.n_groups * (D + 2), a.n_groups, a.n_groups, true, out, D);
}

template <int DT, int D, int BITS>
hipError_t launch_quant_keys(const QuantArgs& a, int64_t n_groups, int B, int H, hipStream_t s);
template <int DT, int D, int BITS>
hipError_t launch_quant_values(const QuantArgs& a, int64_t n_steps, int B, int H, hipStream_t s);
template <int DT, int D>
hipError_t launch_copy_fp(const FpCopyArgs& a, int64_t n_rows, int B, int H, hipStream_t s);
template <int DT, int D, int BITS>
hipError_t launch_append(const AppendArgs& a, int B, int H, hipStream_t s);
template <int DT, int D, int BITS>
hipError_t launch_attn_valu(const AttnArgs& a, int B, hipStream_t s);
template <int DT, int D, int BITS>
int attn_valu_blocks_per_cu();
template <int DT, int D, int BITS>
bool attn_valu_direct_ok();
template <int DT, int D, int BITS, int GQA>
hipError_t launch_attn_mfma(const AttnArgs& a, int B, hipStream_t s);
template <int DT, int D>
hipError_t launch_merge(const AttnArgs& a, int B, hipStream_t s);

}  // namespace kvq
