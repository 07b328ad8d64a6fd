/*
 * kvq.h -- C ABI of libkvq: a KIVI-style quantized KV cache for AMD
 * Instinct MI355X (gfx950).
 *
 * The method (web pages the library follows; cited by title and section):
 *  - sonos/tract PR "KIVI-style KV-cache quantization - packed u8 storage":
 *    "The idea" (Keys quantized per channel, Values per token), "What's in
 *    the PR" (u8 stores: per-token values = D bytes + 2 f32 params; per-
 *    channel keys; fused op taking [Q, K_new, V_new], output of Q's shape,
 *    GQA handled), commit messages (bits are a parameter; optional scale).
 *  - sonos/tract PR "quantized KV-cache storage op (int8/int4)": keys per
 *    channel in frozen fixed-size blocks for streaming consistency, values
 *    per token; the first SINK_TOKENS kept exact in both stores.
 *  - pigeon guide "KV-cache quantization", "How it works" steps 1-5: keys
 *    per channel over G-token groups, values per token, asymmetric
 *    q = round((x - min)/delta) with delta = (max - min)/(2^b - 1), a
 *    full-precision window of the R most recent tokens quantized once a
 *    group fills, and softmax(q K^T / sqrt(d)) V over the cache dequantized
 *    on the fly without materializing a full-precision copy.
 *
 * Readings of points the pages leave open:
 *  - Partition of T cached tokens: with n = max(0, T - S), the quantized
 *    count is Q = G * floor((n - R) / G) if n >= R, else 0.  Tokens [0, S)
 *    are sinks, [S, S+Q) are quantized, [S+Q, T) stay in full precision
 *    (R..R+G-1 of them once n >= R): the R most recent are always exact and
 *    a group of G freezes when the full-precision count reaches R + G.
 *  - Arithmetic: delta = fl32(fl32(max - min) / (2^b - 1)); zero point =
 *    min + 0.0f (fp32); code = clamp(rint_half_even(fl32(fl32(x - zp) /
 *    delta)), 0, 2^b - 1), a true IEEE division; delta == 0 gives code 0.
 *    Subnormals are kept.  Inputs must be finite with magnitude below
 *    2^127, so that max - min is finite in fp32.
 *  - Decode attention accumulates in fp32: every score scale * q . k_hat
 *    and every partial sum of its terms must be finite in fp32.  Within
 *    that, any key or value range is handled (the kernels track power-of-
 *    two exponents for both); outputs inside fp32's subnormal range carry
 *    its absolute rounding.
 *  - Sink and residual tokens are stored bit-exactly in the input dtype.
 *  - GQA: query head hq reads KV head hq / (Hq / Hkv).
 *  - The decode query attends to all n_tokens cached tokens (no mask);
 *    softmax_scale <= 0 selects 1/sqrt(D).
 *  - Sliding window (tract PR "KIVI-style KV-cache quantization", The idea
 *    and Relationship to other PRs: the quantized store composes with a
 *    bounded sliding-window cache): with window W > 0 the query attends to
 *    the sinks and to the last W tokens [max(S, n_tokens - W), n_tokens),
 *    exactly to the token; W >= R + G is required.  The quantized store is
 *    then a ring: quantized token u (token S + u) lives at storage row
 *    u mod qcap, so each group that freezes evicts the oldest one, and the
 *    cache's size no longer grows with n_tokens.
 *  - Dense-and-sparse outliers (pigeon guide "KV-cache quantization",
 *    KVQuant adds, third bullet: about 1% of outlier values kept in a
 *    sparse side table), with outliers = 1: each quantization vector (a
 *    key group's channel over G tokens; a value token over D channels)
 *    keeps at most one entry exact.  With the two largest entries max1 >=
 *    max2 and the two smallest min1 <= min2, gap_hi = fl32(max1 - max2),
 *    gap_lo = fl32(min2 - min1): the maximum is kept if gap_hi >= gap_lo
 *    and gap_hi > 0, else the minimum if gap_lo > 0, else none.  delta and
 *    the zero point come from the other entries; every entry, the kept
 *    one too, is coded with them (the kept one's code clamps to 2^b - 1
 *    or 0, so its dense value is zp + delta (2^b - 1) if it is >= zp,
 *    else zp).  Attention reads the kept entry at its exact value.
 *  - Pre-RoPE keys (pigeon guide "KV-cache quantization", KVQuant adds,
 *    first bullet: keys quantized before the rotary position embedding,
 *    which would otherwise mix channel pairs and smear the per-channel
 *    structure), with rope_base > 0: the cache holds keys as given, before
 *    the rotation; decode rotates each dequantized (or exact) key to its
 *    position, the token index t: channel i pairs with channel i + D/2 at
 *    frequency theta_i = rope_base^(-2i/D), k_i' = k_i cos(t theta_i) -
 *    k_{i+D/2} sin(t theta_i), k_{i+D/2}' = k_{i+D/2} cos(t theta_i) + k_i
 *    sin(t theta_i).  The query is passed already rotated to its own
 *    position; values are not rotated.
 *
 * Conventions for every entry point:
 *  - All pointers except `cfg`, `cache` (the structs themselves) are
 *    DEVICE pointers.  The caller owns every buffer; the library never
 *    allocates, frees or synchronizes.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL =
 *    the default stream) and is asynchronous.  Calls on one cache must be
 *    ordered on one stream by the caller.  Inputs must not alias the cache.
 *  - Validation happens on the host before any launch; a bad argument
 *    returns an error code and enqueues nothing.  A launch failure returns
 *    KVQ_EHIP; faults during execution surface at the caller's next sync.
 *  - No entry point throws across the ABI; there is no global mutable
 *    state.
 *
 * Supported: bits 1 to 8 (2 and 4 are the method's settings; the other
 * widths use the same affine codes, packed as a bit stream); head_dim in
 * {64, 128}; group in {32, 64, 128}; sink >= 0; residual >= 0; dtype f32,
 * f16 or bf16.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KVQ_F32 = 0, KVQ_F16 = 1, KVQ_BF16 = 2 } kvq_dtype;

typedef enum {
  KVQ_OK = 0,
  KVQ_EINVAL = 1,       /* null pointer, bad shape, n_tokens out of range */
  KVQ_EUNSUPPORTED = 2, /* bits / head_dim / group / dtype not supported  */
  KVQ_ECAPACITY = 3,    /* n_tokens exceeds the cache capacity            */
  KVQ_EWORKSPACE = 4,   /* workspace too small                            */
  KVQ_EHIP = 5          /* a HIP launch failed                            */
} kvq_status;

/* Shape of one cache (one attention layer). */
typedef struct {
  int32_t batch;      /* B                                              */
  int32_t n_kv_heads; /* Hkv                                            */
  int32_t head_dim;   /* D: 64 or 128                                   */
  int32_t bits;       /* b: code width, 1 .. 8                          */
  int32_t group;      /* G: key group length in tokens, 32/64/128       */
  int32_t sink;       /* S: first tokens kept exact                     */
  int32_t residual;   /* R: most recent tokens kept exact               */
  int32_t dtype;      /* kvq_dtype of K, V, q and the exact stores      */
  int64_t capacity;   /* maximum number of cached tokens                */
  int64_t window;     /* W: sliding window in tokens, 0 = none (below)  */
  int32_t outliers;   /* 1: keep one exact entry per quantization       */
                      /*    vector in side tables (above); 0: none       */
  float rope_base;    /* > 0: keys are stored before RoPE of this base  */
                      /*    and rotated in decode (above); 0: none       */
} kvq_config;

/*
 * Cache buffers (device memory, caller-allocated; sizes below).
 *
 * qcap = max(0, capacity - S), at most W + G with a window, rounded up to
 * a multiple of max(64, G).  Storage row r holds quantized token u with
 * r = u mod qcap (r = u without a window, as u < qcap).
 *
 * k_codes  u8 [B][Hkv][qcap][D*b/8]: token-major key codes.  Row r holds
 *          quantized token t = S + u; channel d sits at bit offset d*b of
 *          the row (byte d*b/8, bits (d*b)%8 .. +b), low bits first.
 * k_scale, k_zero  f32 [B][Hkv][qcap/G][D]: delta and zero point of key
 *          group k (tokens S+kG .. S+kG+G-1) in slot (kG mod qcap)/G, per
 *          channel.  Frozen once written.
 * v_codes  u8 [B][Hkv][vbytes]: value codes in blocks of L storage rows
 *          (L = 64 at 2 bits, 32 at every other width), vbytes =
 *          qcap/L * L*D*b/8.  A
 *          token offset o inside its block is split as
 *          o = 32*s + 16*h + 4*g + r (s < L/32, h < 2, g < 4, r < 4).  A
 *          block holds 4*D units; unit (g*16 + d%16)*(D/16) + d/16 holds
 *          the U codes of channel d for the tokens sharing g (U = 16 at 2
 *          bits in 4 bytes, U = 8 in b bytes at every other width b);
 *          token (s, h, r) is code slot i = r + 4*s + (U/2)*h at
 *          bit offset i*b of the unit, low bits first.  This places, for
 *          each 32-token step, the 8 tokens one wave lane needs for one
 *          channel in one contiguous run.
 * v_scale, v_zero  f32 [B][Hkv][qcap]: delta and zero point of each
 *          quantized value token, at its storage row.
 * k_sink, v_sink   dtype [B][Hkv][S][D]: tokens 0..S-1, exact.
 * k_resid, v_resid dtype [B][Hkv][R+G][D]: full-precision ring; token
 *          t >= S lives in slot (t - S) mod (R + G).
 * Side tables (outliers = 1 only; NULL otherwise):
 * k_oidx   u8 [B][Hkv][qcap/G][D]: token offset (0..G-1) inside key group
 *          slot k of channel d's kept entry, 255 = none.
 * k_oval   dtype [B][Hkv][qcap/G][D]: its value (+0 when none).
 * v_oidx   u8 [B][Hkv][qcap]: channel of the kept entry of the value token
 *          at that storage row, 255 = none.
 * v_oval   dtype [B][Hkv][qcap]: its value (+0 when none).
 *
 * Bytes of codes that belong to no quantized token yet are never written.
 */
typedef struct {
  uint8_t *k_codes;
  uint8_t *v_codes;
  float *k_scale;
  float *k_zero;
  float *v_scale;
  float *v_zero;
  void *k_sink;
  void *v_sink;
  void *k_resid;
  void *v_resid;
  uint8_t *k_oidx;
  void *k_oval;
  uint8_t *v_oidx;
  void *v_oval;
} kvq_cache;

/* A strided device tensor whose last axis (D) is contiguous.  Strides are
 * in elements.  K/V inputs are [B][Hkv][T][D]; q is [B][Hq][D] (stride_t
 * unused); appended tokens are [B][Hkv][D] (stride_t unused). */
typedef struct {
  const void *ptr;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_t;
} kvq_tensor;

/* ---- buffer sizes (closed forms) ---------------------------------- */
static inline int64_t kvq_qcap(const kvq_config *c) {
  int64_t step = c->group > 64 ? c->group : 64;
  int64_t n = c->capacity - c->sink;
  if (n < 0) n = 0;
  if (c->window > 0 && n > c->window + c->group) n = c->window + c->group;
  return (n + step - 1) / step * step;
}
static inline int64_t kvq_dtype_bytes(int32_t dt) { return dt == KVQ_F32 ? 4 : 2; }
static inline int64_t kvq_k_codes_bytes(const kvq_config *c) {
  return (int64_t)c->batch * c->n_kv_heads * kvq_qcap(c) * c->head_dim * c->bits / 8;
}
static inline int64_t kvq_v_codes_bytes(const kvq_config *c) { return kvq_k_codes_bytes(c); }
static inline int64_t kvq_k_params_count(const kvq_config *c) { /* floats per array */
  return (int64_t)c->batch * c->n_kv_heads * (kvq_qcap(c) / c->group) * c->head_dim;
}
static inline int64_t kvq_v_params_count(const kvq_config *c) {
  return (int64_t)c->batch * c->n_kv_heads * kvq_qcap(c);
}
static inline int64_t kvq_sink_bytes(const kvq_config *c) {
  return (int64_t)c->batch * c->n_kv_heads * c->sink * c->head_dim * kvq_dtype_bytes(c->dtype);
}
static inline int64_t kvq_k_side_count(const kvq_config *c) { /* entries per k_oidx / k_oval */
  return c->outliers ? kvq_k_params_count(c) : 0;
}
static inline int64_t kvq_v_side_count(const kvq_config *c) { /* entries per v_oidx / v_oval */
  return c->outliers ? kvq_v_params_count(c) : 0;
}
static inline int64_t kvq_resid_bytes(const kvq_config *c) {
  return (int64_t)c->batch * c->n_kv_heads * (c->residual + c->group) * c->head_dim *
         kvq_dtype_bytes(c->dtype);
}

/* Decode-attention workspace: per (batch, query head) up to
 * KVQ_MAX_SPLITS partial results of D + 2 floats.  Any size of at least
 * kvq_workspace_bytes_min (room for one split) works; the kernels use
 * fewer splits when given less room, down to one.  Results agree across
 * split counts to fp32 rounding. */
#define KVQ_MAX_SPLITS 1024
static inline int64_t kvq_workspace_bytes(const kvq_config *c, int32_t n_q_heads) {
  return (int64_t)c->batch * n_q_heads * KVQ_MAX_SPLITS * (c->head_dim + 2) * 4;
}
static inline int64_t kvq_workspace_bytes_min(const kvq_config *c, int32_t n_q_heads) {
  return (int64_t)c->batch * n_q_heads * (c->head_dim + 2) * 4;
}

/* ---- entry points -------------------------------------------------- */

/*
 * kvq_quantize_keys: load the first n_tokens keys of every sequence into
 * an empty cache (prefill).  Keys of the sink tokens go to k_sink; the
 * Q = partition(n_tokens) quantized tokens are quantized per channel over
 * G-token groups into k_codes / k_scale / k_zero (pigeon guide "KV-cache
 * quantization", How it works steps 1 and 3; tract "quantized KV-cache
 * storage op": frozen fixed-size blocks); the rest go to their k_resid
 * ring slots.  The result is byte-identical to n_tokens calls of
 * kvq_append_token on the key half.
 *   k: [B][Hkv][>= n_tokens][D] in cfg->dtype.
 * Errors: KVQ_EINVAL (null pointers, n_tokens < 0), KVQ_ECAPACITY
 * (n_tokens > capacity), KVQ_EUNSUPPORTED, KVQ_EHIP.
 */
kvq_status kvq_quantize_keys(const kvq_config *cfg, const kvq_cache *cache, kvq_tensor k,
                             int64_t n_tokens, void *stream);

/*
 * kvq_quantize_values: the value half of the prefill.  Quantized value
 * tokens are quantized per token (pigeon guide "KV-cache quantization",
 * How it works step 2; tract "KIVI-style KV-cache quantization", What's in
 * the PR: per-token store with 2 f32 params) into v_codes / v_scale /
 * v_zero; sinks and residual tokens go to v_sink / v_resid.
 *   v: [B][Hkv][>= n_tokens][D] in cfg->dtype.
 * Errors as kvq_quantize_keys.
 */
kvq_status kvq_quantize_values(const kvq_config *cfg, const kvq_cache *cache, kvq_tensor v,
                               int64_t n_tokens, void *stream);

/*
 * kvq_append_token: streaming append of token t = n_before (K and V) to a
 * cache holding n_before tokens.  The token is written to its sink slot
 * (t < S) or ring slot; if the full-precision count then reaches R + G,
 * the oldest G ring tokens are quantized as key group Q/G (per channel)
 * and as G value tokens (per token) and frozen: they are never
 * recomputed (tract "quantized KV-cache storage op": frozen blocks for
 * streaming consistency; pigeon guide, How it works step 4).
 *   k_new, v_new: [B][Hkv][D] in cfg->dtype.
 * Errors: KVQ_EINVAL, KVQ_ECAPACITY (n_before + 1 > capacity),
 * KVQ_EUNSUPPORTED, KVQ_EHIP.
 */
kvq_status kvq_append_token(const kvq_config *cfg, const kvq_cache *cache, int64_t n_before,
                            kvq_tensor k_new, kvq_tensor v_new, void *stream);

/*
 * kvq_decode_attention: out[b][hq] = softmax(scale * q[b][hq] . K^T) V over
 * the n_tokens cached tokens of KV head hq / (Hq/Hkv), with quantized keys
 * and values dequantized on the fly inside the kernel (pigeon guide, How
 * it works step 5; tract "KIVI-style KV-cache quantization", What's in the
 * PR: GQA handled, output of Q's shape).  Split-K over the token axis with
 * a log-sum-exp merge; fp32 accumulation.
 *   q:   [B][n_q_heads][D] in cfg->dtype; n_q_heads a multiple of Hkv.
 *   out: f32 [B][n_q_heads][D], written densely.
 *   softmax_scale: <= 0 selects 1/sqrt(D).
 *   workspace: device scratch of workspace_bytes bytes (see above); its
 *   contents need no initialization and are garbage afterwards.
 * Errors: KVQ_EINVAL (null pointers, n_tokens < 1, bad n_q_heads),
 * KVQ_ECAPACITY, KVQ_EWORKSPACE, KVQ_EUNSUPPORTED, KVQ_EHIP.
 */
kvq_status kvq_decode_attention(const kvq_config *cfg, const kvq_cache *cache, int64_t n_tokens,
                                int32_t n_q_heads, kvq_tensor q, float softmax_scale, float *out,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * kvq_decode_attention_noalloc: kvq_decode_attention without a workspace
 * argument, for callers that cannot allocate device memory (code under
 * stream / graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It allocates nothing and frees nothing.  The split partials
 * go to a device array inside the library of KVQ_NOALLOC_SCRATCH_BYTES
 * bytes, one per GPU the library runs on, held until the process ends;
 * the result equals kvq_decode_attention's with a workspace of that size.
 *   Limit: one split per (batch, query head) must fit, i.e.
 *   kvq_workspace_bytes_min(cfg, n_q_heads) <= KVQ_NOALLOC_SCRATCH_BYTES
 *   (B * n_q_heads * (D + 2) * 4 bytes); larger calls return
 *   KVQ_EWORKSPACE before any work is enqueued.
 *   Sharing: every call on one GPU uses that GPU's array and leaves its
 *   partials there (they need no clearing).  Calls that can overlap in time
 *   on one GPU (on different streams) race on it and must be ordered by
 *   the caller.
 * Arguments and other errors as kvq_decode_attention; KVQ_EHIP also when
 * the array's device address cannot be obtained.
 */
#define KVQ_NOALLOC_SCRATCH_BYTES (16u << 20)
kvq_status kvq_decode_attention_noalloc(const kvq_config *cfg, const kvq_cache *cache,
                                        int64_t n_tokens, int32_t n_q_heads, kvq_tensor q,
                                        float softmax_scale, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
