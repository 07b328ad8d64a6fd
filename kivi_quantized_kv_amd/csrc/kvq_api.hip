// Host side of libkvq: the four C-ABI entry points.  Each validates its
// arguments on the host, derives the token partition and launch geometry,
// and enqueues kernels on the caller's stream.  Nothing here allocates,
// frees or synchronizes.
#include <atomic>
#include <cmath>
#include <cstdint>

#include "../../include/kvq.h"
#include "kvq_kernels.h"

using namespace kvq;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int device_cu_count();

// One workgroup per (batch, q head) row fills the GPU when the rows come in
// whole rounds of CUs (or so many rounds that a partial last one is cheap).
bool direct_rows(int64_t rows) {
  const int64_t cu = device_cu_count();
  return rows >= cu && (rows % cu == 0 || rows >= 4 * cu);
}

// Compute units of the current device (cached per device id; a host query,
// no allocation).  Falls back to 256 if the query fails.
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

kvq_status check_config(const kvq_config* c) {
  if (!c) return KVQ_EINVAL;
  if (c->batch < 1 || c->n_kv_heads < 1 || c->sink < 0 || c->residual < 0 || c->capacity < 1)
    return KVQ_EINVAL;
  if (c->head_dim != 64 && c->head_dim != 128) return KVQ_EUNSUPPORTED;
  if (c->bits < 1 || c->bits > 8) return KVQ_EUNSUPPORTED;
  if (c->group != 32 && c->group != 64 && c->group != 128) return KVQ_EUNSUPPORTED;
  if (c->dtype != KVQ_F32 && c->dtype != KVQ_F16 && c->dtype != KVQ_BF16) return KVQ_EUNSUPPORTED;
  if (c->capacity > (int64_t(1) << 40)) return KVQ_EINVAL;
  // a window holds at least the full-precision tokens
  if (c->window < 0 || (c->window > 0 && c->window < int64_t(c->residual) + c->group)) return KVQ_EINVAL;
  if (c->outliers != 0 && c->outliers != 1) return KVQ_EINVAL;
  if (!(c->rope_base >= 0.0f) || std::isinf(c->rope_base)) return KVQ_EINVAL;
  return KVQ_OK;
}

// Rows of 16-bit tensors are read 8 or 16 bytes at a time: every row must
// start on a 16-byte boundary.
kvq_status check_tensor(const kvq_tensor& t, int32_t dtype, bool needs_t) {
  if (!t.ptr || !aligned16(t.ptr)) return KVQ_EINVAL;
  const int64_t eb = kvq_dtype_bytes(dtype);
  if (t.stride_b < 0 || t.stride_h < 0 || (needs_t && t.stride_t < 0)) return KVQ_EINVAL;
  if ((t.stride_b * eb) % 16 || (t.stride_h * eb) % 16 || (needs_t && (t.stride_t * eb) % 16))
    return KVQ_EINVAL;
  return KVQ_OK;
}

kvq_status check_cache(const kvq_config* c, const kvq_cache* k) {
  if (!k) return KVQ_EINVAL;
  const bool q = kvq_qcap(c) > 0;
  if (q && (!k->k_codes || !k->v_codes || !k->k_scale || !k->k_zero || !k->v_scale || !k->v_zero))
    return KVQ_EINVAL;
  if (c->sink > 0 && (!k->k_sink || !k->v_sink)) return KVQ_EINVAL;
  if (!k->k_resid || !k->v_resid) return KVQ_EINVAL;
  if (q && c->outliers && (!k->k_oidx || !k->k_oval || !k->v_oidx || !k->v_oval)) return KVQ_EINVAL;
  const void* ptrs[] = {k->k_codes, k->v_codes, k->k_scale, k->k_zero, k->v_scale, k->v_zero,
                        k->k_sink,  k->v_sink,  k->k_resid, k->v_resid, k->k_oidx,  k->k_oval,
                        k->v_oidx,  k->v_oval};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KVQ_EINVAL;
  return KVQ_OK;
}

// dispatch over (dtype, head_dim, bits)
template <template <int, int, int> class Fn, typename... Args>
auto dispatch3(const kvq_config* c, Args&&... args) -> decltype(Fn<DT_F32, 64, 2>::run(args...)) {
#define KVQ_CASE_B(DT, D)                                                \
  switch (c->bits) {                                                     \
    case 1: return Fn<DT, D, 1>::run(args...);                           \
    case 2: return Fn<DT, D, 2>::run(args...);                           \
    case 3: return Fn<DT, D, 3>::run(args...);                           \
    case 4: return Fn<DT, D, 4>::run(args...);                           \
    case 5: return Fn<DT, D, 5>::run(args...);                           \
    case 6: return Fn<DT, D, 6>::run(args...);                           \
    case 7: return Fn<DT, D, 7>::run(args...);                           \
    default: return Fn<DT, D, 8>::run(args...);                          \
  }
#define KVQ_CASE_D(DT)                                                   \
  if (c->head_dim == 64) { KVQ_CASE_B(DT, 64) } else { KVQ_CASE_B(DT, 128) }
  switch (c->dtype) {
    case KVQ_F32: KVQ_CASE_D(DT_F32)
    case KVQ_F16: KVQ_CASE_D(DT_F16)
    default: KVQ_CASE_D(DT_BF16)
  }
#undef KVQ_CASE_D
#undef KVQ_CASE_B
}

template <int DT, int D, int BITS> struct QuantKeysFn {
  static hipError_t run(const QuantArgs& a, int64_t n, int B, int H, hipStream_t s) {
    return launch_quant_keys<DT, D, BITS>(a, n, B, H, s);
  }
};
template <int DT, int D, int BITS> struct QuantValuesFn {
  static hipError_t run(const QuantArgs& a, int64_t n, int B, int H, hipStream_t s) {
    return launch_quant_values<DT, D, BITS>(a, n, B, H, s);
  }
};
template <int DT, int D, int BITS> struct AppendFn {
  static hipError_t run(const AppendArgs& a, int B, int H, hipStream_t s) {
    return launch_append<DT, D, BITS>(a, B, H, s);
  }
};
template <int DT, int D, int BITS> struct AttnMfma4Fn {
  static hipError_t run(const AttnArgs& a, int B, hipStream_t s) {
    if constexpr (BITS != 2 && BITS != 4) return hipErrorInvalidValue;
    else return launch_attn_mfma<DT, D, BITS, 4>(a, B, s);
  }
};
template <int DT, int D, int BITS> struct AttnMfma8Fn {
  static hipError_t run(const AttnArgs& a, int B, hipStream_t s) {
    if constexpr (BITS != 2 && BITS != 4) return hipErrorInvalidValue;
    else return launch_attn_mfma<DT, D, BITS, 8>(a, B, s);
  }
};
// VALU kernel modes: bit 0 side tables, bit 1 pre-RoPE keys
template <int DT, int D, int BITS> struct AttnValuFn {
  static hipError_t run(const AttnArgs& a, int B, hipStream_t s) {
    switch ((a.outliers ? 1 : 0) | (a.rope ? 2 : 0)) {
      case 0: return launch_attn_valu<DT, D, BITS, 0>(a, B, s);
      case 1: return launch_attn_valu<DT, D, BITS, 1>(a, B, s);
      case 2: return launch_attn_valu<DT, D, BITS, 2>(a, B, s);
      default: return launch_attn_valu<DT, D, BITS, 3>(a, B, s);
    }
  }
};
template <int DT, int D, int BITS> struct AttnValuOccFn {
  static int run(int mode) {
    switch (mode) {
      case 0: return attn_valu_blocks_per_cu<DT, D, BITS, 0>();
      case 1: return attn_valu_blocks_per_cu<DT, D, BITS, 1>();
      case 2: return attn_valu_blocks_per_cu<DT, D, BITS, 2>();
      default: return attn_valu_blocks_per_cu<DT, D, BITS, 3>();
    }
  }
};
template <int DT, int D, int BITS> struct AttnGqaFn {
  static hipError_t run(const AttnArgs& a, int B, hipStream_t s) {
    switch ((a.outliers ? 1 : 0) | (a.rope ? 2 : 0)) {
      case 0: return launch_attn_gqa<DT, D, BITS, 0>(a, B, s);
      case 1: return launch_attn_gqa<DT, D, BITS, 1>(a, B, s);
      case 2: return launch_attn_gqa<DT, D, BITS, 2>(a, B, s);
      default: return launch_attn_gqa<DT, D, BITS, 3>(a, B, s);
    }
  }
};
template <int DT, int D, int BITS> struct AttnGqaOccFn {
  static int run(int mode) {
    switch (mode) {
      case 0: return attn_gqa_blocks_per_cu<DT, D, BITS, 0>();
      case 1: return attn_gqa_blocks_per_cu<DT, D, BITS, 1>();
      case 2: return attn_gqa_blocks_per_cu<DT, D, BITS, 2>();
      default: return attn_gqa_blocks_per_cu<DT, D, BITS, 3>();
    }
  }
};
template <int DT, int D, int BITS> struct AttnValuDirectOkFn {
  static bool run() { return attn_valu_direct_ok<DT, D, BITS>(); }
};

// Prefill of one half in one launch: the quantized range (keys per group or
// values per 32-token step) and, in the workgroups past it, the fp copies
// of the sinks and residual tokens.
kvq_status prefill_half(const kvq_config* c, const kvq_cache* k, const kvq_tensor& x,
                        int64_t n_tokens, void* stream, bool keys) {
  kvq_status st = check_config(c);
  if (st != KVQ_OK) return st;
  if ((st = check_cache(c, k)) != KVQ_OK) return st;
  if ((st = check_tensor(x, c->dtype, true)) != KVQ_OK) return st;
  if (n_tokens < 0) return KVQ_EINVAL;
  if (n_tokens > c->capacity) return KVQ_ECAPACITY;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t S = c->sink, R = c->residual, G = c->group, D = c->head_dim;
  const int64_t Q = quantized_count(n_tokens, S, R, G);
  const int64_t n_sink = n_tokens < S ? n_tokens : S;
  const int64_t n_res = n_tokens > S ? n_tokens - S - Q : 0;
  const int B = c->batch, H = c->n_kv_heads;
  QuantArgs q{};
  q.src = x.ptr; q.sb = x.stride_b; q.sh = x.stride_h; q.st = x.stride_t;
  q.codes = keys ? k->k_codes : k->v_codes;
  q.scale = keys ? k->k_scale : k->v_scale;
  q.zero = keys ? k->k_zero : k->v_zero;
  q.S = S; q.qcap = kvq_qcap(c); q.H = H; q.G = int(G);
  q.outliers = c->outliers;
  q.oidx = keys ? k->k_oidx : k->v_oidx;
  q.oval = static_cast<uint8_t*>(keys ? k->k_oval : k->v_oval);
  // with a window only the groups of the last qcap quantized tokens are
  // kept (older ones would be evicted by them), each storage slot once
  const int64_t k_first = Q > q.qcap ? (Q - q.qcap) / G : 0;
  q.k0 = keys ? k_first : k_first * G / 32;
  q.n_units = Q > 0 ? (keys ? Q / G - k_first : (Q - k_first * G) / 32) : 0;
  FpCopyArgs& f = q.fp;
  f.src = x.ptr; f.sb = x.stride_b; f.sh = x.stride_h; f.st = x.stride_t;
  f.sink = keys ? k->k_sink : k->v_sink;
  f.resid = keys ? k->k_resid : k->v_resid;
  f.n_sink = n_sink; f.first_resid = S + Q; f.S = S; f.ring = R + G; f.H = H;
  q.n_fp_rows = n_sink + n_res;
  const int64_t vec_per_row = D * int64_t(kvq_dtype_bytes(c->dtype)) / 16;
  const int64_t n_copy = (q.n_fp_rows * vec_per_row + 255) / 256;
  const int64_t n_blocks = q.n_units + n_copy;
  if (n_blocks > 0) {
    hipError_t e = keys ? dispatch3<QuantKeysFn>(c, q, n_blocks, B, H, s)
                        : dispatch3<QuantValuesFn>(c, q, n_blocks, B, H, s);
    if (e != hipSuccess) return KVQ_EHIP;
  }
  return KVQ_OK;
}

}  // namespace

extern "C" kvq_status kvq_quantize_keys(const kvq_config* cfg, const kvq_cache* cache,
                                        kvq_tensor k, int64_t n_tokens, void* stream) {
  try {
    return prefill_half(cfg, cache, k, n_tokens, stream, true);
  } catch (...) {
    return KVQ_EINVAL;
  }
}

extern "C" kvq_status kvq_quantize_values(const kvq_config* cfg, const kvq_cache* cache,
                                          kvq_tensor v, int64_t n_tokens, void* stream) {
  try {
    return prefill_half(cfg, cache, v, n_tokens, stream, false);
  } catch (...) {
    return KVQ_EINVAL;
  }
}

extern "C" kvq_status kvq_append_token(const kvq_config* cfg, const kvq_cache* cache,
                                       int64_t n_before, kvq_tensor k_new, kvq_tensor v_new,
                                       void* stream) {
  try {
    kvq_status st = check_config(cfg);
    if (st != KVQ_OK) return st;
    if ((st = check_cache(cfg, cache)) != KVQ_OK) return st;
    if ((st = check_tensor(k_new, cfg->dtype, false)) != KVQ_OK) return st;
    if ((st = check_tensor(v_new, cfg->dtype, false)) != KVQ_OK) return st;
    if (n_before < 0) return KVQ_EINVAL;
    if (n_before + 1 > cfg->capacity) return KVQ_ECAPACITY;
    const int64_t S = cfg->sink, R = cfg->residual, G = cfg->group;
    const int64_t q_old = quantized_count(n_before, S, R, G);
    const int64_t q_new = quantized_count(n_before + 1, S, R, G);
    AppendArgs a{};
    a.k_new = k_new.ptr; a.v_new = v_new.ptr;
    a.k_sb = k_new.stride_b; a.k_sh = k_new.stride_h;
    a.v_sb = v_new.stride_b; a.v_sh = v_new.stride_h;
    a.k_codes = cache->k_codes; a.v_codes = cache->v_codes;
    a.k_scale = cache->k_scale; a.k_zero = cache->k_zero;
    a.v_scale = cache->v_scale; a.v_zero = cache->v_zero;
    a.k_sink = cache->k_sink; a.v_sink = cache->v_sink;
    a.k_resid = cache->k_resid; a.v_resid = cache->v_resid;
    a.n_before = n_before; a.q_old = q_old; a.S = S; a.R = R; a.qcap = kvq_qcap(cfg);
    a.r_old = a.qcap > 0 ? q_old % a.qcap : 0;
    a.H = cfg->n_kv_heads; a.G = int(G); a.flush = q_new > q_old ? 1 : 0;
    a.outliers = cfg->outliers;
    a.k_oidx = cache->k_oidx; a.k_oval = static_cast<uint8_t*>(cache->k_oval);
    a.v_oidx = cache->v_oidx; a.v_oval = static_cast<uint8_t*>(cache->v_oval);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (dispatch3<AppendFn>(cfg, a, cfg->batch, cfg->n_kv_heads, s) != hipSuccess) return KVQ_EHIP;
    return KVQ_OK;
  } catch (...) {
    return KVQ_EINVAL;
  }
}

namespace {

// Argument checks of decode attention that need no workspace.
kvq_status check_decode_args(const kvq_config* cfg, const kvq_cache* cache, int64_t n_tokens,
                             int32_t n_q_heads, const kvq_tensor& q, float softmax_scale,
                             const float* out) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if ((st = check_cache(cfg, cache)) != KVQ_OK) return st;
  if ((st = check_tensor(q, cfg->dtype, false)) != KVQ_OK) return st;
  if (!out || !aligned16(out)) return KVQ_EINVAL;
  if (n_q_heads < 1 || n_q_heads % cfg->n_kv_heads) return KVQ_EINVAL;
  if (n_tokens < 1) return KVQ_EINVAL;
  if (n_tokens > cfg->capacity) return KVQ_ECAPACITY;
  if (!(softmax_scale == softmax_scale) || std::isinf(softmax_scale)) return KVQ_EINVAL;
  return KVQ_OK;
}

// Decode attention after the argument checks, with the split partials in
// `workspace` (workspace_bytes bytes, 16-byte aligned).
kvq_status decode_attention(const kvq_config* cfg, const kvq_cache* cache, int64_t n_tokens,
                            int32_t n_q_heads, const kvq_tensor& q, float softmax_scale, float* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  const int B = cfg->batch, H = cfg->n_kv_heads, D = cfg->head_dim;
  const int64_t S = cfg->sink, R = cfg->residual, G = cfg->group;
  const int64_t T = n_tokens;
  const int64_t Q = quantized_count(T, S, R, G);
  const int64_t n_sink = T < S ? T : S;
  const int64_t n_res = T > S ? T - S - Q : 0;
  const int64_t n_fp = n_sink + n_res;
  const int64_t per_split_bytes = int64_t(B) * n_q_heads * (D + 2) * 4;
  int64_t cap_splits = int64_t(workspace_bytes) / per_split_bytes;
  if (cap_splits > KVQ_MAX_SPLITS) cap_splits = KVQ_MAX_SPLITS;
  if (int64_t(workspace_bytes) < kvq_workspace_bytes_min(cfg, n_q_heads) || cap_splits < 1)
    return KVQ_EWORKSPACE;

  // The matrix-core kernel covers GQA groups of 4 and 8 with 2- and 4-bit
  // codes, once at least one token is quantized (its chunk loads assume a
  // chunk 0), for caches without side tables or pre-RoPE keys.  It works
  // per KV head on 64-token chunks, with the grid sized to one round of
  // one workgroup per CU, and spreads the full-precision tokens evenly over
  // its splits.  Everything else runs a VALU kernel on
  // value-code blocks, again with the full-precision tokens spread evenly
  // over the splits: GQA groups of 2..8 heads the grouped one, MHA and
  // larger groups the per-head one.
  const int gqa = n_q_heads / H;
  const bool rope = cfg->rope_base > 0.0f;
  const int valu_mode = (cfg->outliers ? 1 : 0) | (rope ? 2 : 0);
  const bool mfma = (gqa == 4 || gqa == 8) && (cfg->bits == 2 || cfg->bits == 4) && Q > 0 &&
                    valu_mode == 0;
  // other GQA groups of 2..8 heads: the grouped VALU kernel, up to four
  // heads per workgroup sharing each code's extraction
  const bool grouped = !mfma && gqa >= 2 && gqa <= 8;
  const int64_t L = mfma ? 64 : (cfg->bits == 2 ? 64 : 32);
  const int64_t qcap = kvq_qcap(cfg);
  // sliding window: quantized tokens before u_lo are not attended; the
  // kernels' units (chunks or value blocks) start at c0
  const int64_t u_lo = cfg->window > 0 && T - cfg->window - S > 0 ? T - cfg->window - S : 0;
  const int64_t c0 = u_lo / L;
  const int64_t nblk = (Q + L - 1) / L - c0;   // live units
  int64_t fp_per_split = 32;
  int64_t bps = 1;
  int64_t n_split = 0;
  bool direct = false;
  if (mfma) {
    // one round of workgroups, one per CU
    const int64_t slots = int64_t(device_cu_count());
    const int64_t rows = int64_t(B) * H;
    int64_t want = slots / rows > 0 ? slots / rows : 1;
    if (want > nblk) want = nblk;
    if (want > cap_splits) want = cap_splits;
    bps = want > 0 ? (nblk + want - 1) / want : 1;
    n_split = nblk > 0 ? (nblk + bps - 1) / bps : 0;
    // at most mfma_exact_cap exact tokens per split (their rows are staged
    // in LDS): splits past the chunks, if any, take exact tokens only
    const int64_t xcap = kvq::mfma_exact_cap(int(kvq_dtype_bytes(cfg->dtype)), int(D));
    int64_t want_fp = (n_fp + xcap - 1) / xcap;
    if (want_fp > cap_splits) want_fp = cap_splits;
    if (n_split < want_fp) n_split = want_fp;
    if (n_split < 1) n_split = 1;
    fp_per_split = (n_fp + n_split - 1) / n_split;
  } else if (grouped) {
    // one round of resident workgroups over (b, KV head, head group) rows,
    // at least one block per wave
    const int64_t slots = int64_t(dispatch3<AttnGqaOccFn>(cfg, valu_mode)) * device_cu_count();
    const int64_t rows = int64_t(B) * H * ((gqa + 3) / 4);
    int64_t want = slots / rows > 0 ? slots / rows : 1;
    if (want > (nblk + 3) / 4) want = (nblk + 3) / 4;
    if (want > cap_splits) want = cap_splits;
    bps = want > 0 ? (nblk + want - 1) / want : 1;
    n_split = nblk > 0 ? (nblk + bps - 1) / bps : 0;
    int64_t want_fp = (n_fp + 63) / 64;
    if (want_fp > cap_splits) want_fp = cap_splits;
    if (n_split < want_fp) n_split = want_fp;
    if (n_split < 1) n_split = 1;
    fp_per_split = (n_fp + n_split - 1) / n_split;
  } else if ((direct_rows(int64_t(B) * n_q_heads) || (nblk <= 16 && n_fp <= 256)) && valu_mode == 0 &&
             dispatch3<AttnValuDirectOkFn>(cfg)) {
    // the rows alone fill the GPU, or each row is short (at most one value
    // block per wave; longer rows gain more from spreading over the CUs
    // than the merge launch costs, measured at 30 blocks per row): one
    // 16-wave workgroup per row takes all of its tokens, merges in LDS and
    // writes the output, with no merge launch
    direct = true;
    n_split = 1;
    bps = nblk > 0 ? nblk : 1;
    fp_per_split = n_fp > 0 ? n_fp : 1;
  } else {
    // one round of resident workgroups, at least one block per wave
    const int64_t slots = int64_t(dispatch3<AttnValuOccFn>(cfg, valu_mode)) * device_cu_count();
    const int64_t rows = int64_t(B) * n_q_heads;
    int64_t want = slots / rows > 0 ? slots / rows : 1;
    if (want > (nblk + 3) / 4) want = (nblk + 3) / 4;
    if (want > cap_splits) want = cap_splits;
    bps = want > 0 ? (nblk + want - 1) / want : 1;
    n_split = nblk > 0 ? (nblk + bps - 1) / bps : 0;
    int64_t want_fp = (n_fp + 63) / 64;
    if (want_fp > cap_splits) want_fp = cap_splits;
    if (n_split < want_fp) n_split = want_fp;
    if (n_split < 1) n_split = 1;
    fp_per_split = (n_fp + n_split - 1) / n_split;
  }
  AttnArgs a{};
  a.k_codes = cache->k_codes; a.v_codes = cache->v_codes;
  a.k_scale = cache->k_scale; a.k_zero = cache->k_zero;
  a.v_scale = cache->v_scale; a.v_zero = cache->v_zero;
  a.k_sink = cache->k_sink; a.v_sink = cache->v_sink;
  a.k_resid = cache->k_resid; a.v_resid = cache->v_resid;
  a.q = q.ptr; a.q_sb = q.stride_b; a.q_sh = q.stride_h;
  a.ws = reinterpret_cast<float*>(workspace);
  a.out = out;
  const double scale = softmax_scale > 0 ? double(softmax_scale) : 1.0 / std::sqrt(double(D));
  a.sm_scale_log2 = float(scale * 1.4426950408889634);
  a.T = T; a.S = S; a.Q = Q; a.qcap = kvq_qcap(cfg); a.ring = R + G;
  a.first_resid = S + Q; a.n_sink = n_sink; a.n_fp = n_fp;
  a.kgroups = kvq_qcap(cfg) / G;
  a.resid_slot0 = Q % (R + G);
  a.H = H; a.Hq = n_q_heads; a.gqa = n_q_heads / H; a.G = int(G);
  a.g_shift = G == 32 ? 5 : (G == 64 ? 6 : 7);
  a.n_split = int(n_split);
  a.direct = direct ? 1 : 0;
  a.blocks_per_split = int(bps);
  a.fp_per_split = int(fp_per_split);
  a.ml_offset = int64_t(B) * n_q_heads * n_split * D;
  a.u_lo = u_lo;
  a.c0 = c0;
  a.ncap = qcap / L;
  a.cw = a.ncap > 0 ? c0 / a.ncap * a.ncap : 0;
  a.lo_off = int(u_lo - c0 * L);
  a.outliers = cfg->outliers;
  a.rope = rope ? 1 : 0;
  a.rope_log2_base = rope ? std::log2(double(cfg->rope_base)) : 0.0;
  a.k_oidx = cache->k_oidx; a.k_oval = cache->k_oval;
  a.v_oidx = cache->v_oidx; a.v_oval = cache->v_oval;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t ea = hipSuccess;
  if (a.n_split > 0) {
    if (mfma && gqa == 8) ea = dispatch3<AttnMfma8Fn>(cfg, a, B, s);
    else if (mfma) ea = dispatch3<AttnMfma4Fn>(cfg, a, B, s);
    else if (grouped) ea = dispatch3<AttnGqaFn>(cfg, a, B, s);
    else ea = dispatch3<AttnValuFn>(cfg, a, B, s);
  }
  if (ea != hipSuccess) return KVQ_EHIP;
  if (direct) return KVQ_OK;
  hipError_t e;
  if (cfg->dtype == KVQ_F32) e = D == 64 ? launch_merge<DT_F32, 64>(a, B, s) : launch_merge<DT_F32, 128>(a, B, s);
  else if (cfg->dtype == KVQ_F16) e = D == 64 ? launch_merge<DT_F16, 64>(a, B, s) : launch_merge<DT_F16, 128>(a, B, s);
  else e = D == 64 ? launch_merge<DT_BF16, 64>(a, B, s) : launch_merge<DT_BF16, 128>(a, B, s);
  if (e != hipSuccess) return KVQ_EHIP;
  return KVQ_OK;
}

}  // namespace

extern "C" kvq_status kvq_decode_attention(const kvq_config* cfg, const kvq_cache* cache,
                                           int64_t n_tokens, int32_t n_q_heads, kvq_tensor q,
                                           float softmax_scale, float* out, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  try {
    kvq_status st = check_decode_args(cfg, cache, n_tokens, n_q_heads, q, softmax_scale, out);
    if (st != KVQ_OK) return st;
    if (!workspace || !aligned16(workspace)) return KVQ_EINVAL;
    return decode_attention(cfg, cache, n_tokens, n_q_heads, q, softmax_scale, out, workspace,
                            workspace_bytes, stream);
  } catch (...) {
    return KVQ_EINVAL;
  }
}

// ---------------------------------------------------------------------------
// Decode attention without a caller workspace: the split partials live in a
// file-scope device array of KVQ_NOALLOC_SCRATCH_BYTES, one per GPU the
// library runs on, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device
// address): its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and cached.  The partials
// need no clearing (every split writes its own before the merge reads it).
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of this device's copy of `scratch`, or null on failure.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  g_scratch_ptr[dev].store(ptr, std::memory_order_release);   // same value from any racing thread
  return ptr;
}

}  // namespace

extern "C" kvq_status kvq_decode_attention_noalloc(const kvq_config* cfg, const kvq_cache* cache,
                                                   int64_t n_tokens, int32_t n_q_heads,
                                                   kvq_tensor q, float softmax_scale, float* out,
                                                   void* stream) {
  try {
    kvq_status st = check_decode_args(cfg, cache, n_tokens, n_q_heads, q, softmax_scale, out);
    if (st != KVQ_OK) return st;
    // one split per (batch, q head) must fit the array
    if (kvq_workspace_bytes_min(cfg, n_q_heads) > int64_t(KVQ_NOALLOC_SCRATCH_BYTES))
      return KVQ_EWORKSPACE;
    void* ws = scratch_address();
    if (!ws) return KVQ_EHIP;
    return decode_attention(cfg, cache, n_tokens, n_q_heads, q, softmax_scale, out, ws,
                            KVQ_NOALLOC_SCRATCH_BYTES, stream);
  } catch (...) {
    return KVQ_EINVAL;
  }
}
