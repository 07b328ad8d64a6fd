// Split-K decode attention on the matrix cores, for GQA groups of 4 or 8
// query heads per KV head (the group makes q.K^T and P.V dense tiles),
// with 2- or 4-bit codes.
//
// Method: softmax(scale * q K^T) V over the cache dequantized inside the
// kernel (pigeon guide "KV-cache quantization", How it works step 5), GQA
// as in tract PR "KIVI-style KV-cache quantization", What's in the PR.
//
// Codes enter the matrix cores as fp16 subnormals: a 32-bit code word
// masked to a few bits per 16-bit half is, bit for bit, a pair of fp16
// numbers n * 2^-24 with n the masked field, and the matrix instructions
// take subnormal inputs exactly.  A field can hold several codes at once:
// with 4-bit codes a byte field is c0 + 16 c1, and the pair (byte, low
// nibble) carries (c0, c1) with weights (w1/16, w0 - w1/16); with 2-bit
// codes the fields are nested masks 0xFF, 0x3F, 0x0F, 0x03 of a byte, with
// weights (w3/64, w2/16 - w3/64, w1/4 - w2/16, w0 - w1/4).  So four
// and/perm instructions turn a word into one 8-element operand, and the
// per-code scale factors 2^-(bits * position) ride on the other operand.
//
// Per wave and 64-token chunk:
//   q.K^T : S^T[16 tokens x 16 cols] = C[16 x D] . W[D x 16] per 16-token
//           tile, v_mfma_f32_16x16x32_f16.  W holds the field weights of
//           w_d = scale*log2e * q_d * delta_d split into an fp16 high part
//           (cols 0..GQA-1) and low part (cols GQA..2GQA-1), ~22 bits in
//           all; the accumulator starts at kappa * 2^-24 with kappa =
//           sum_d scale*log2e * q_d * zero_d, and the high and low columns
//           are joined with one DPP rotate-add.  Scores are acc * 2^24.
//   P.V   : O[16 rows x 16 ch] += P'[16 x 32 tokens] . Vc[32 x 16 ch],
//           v_mfma_f32_16x16x32_f16, rows = heads (fp16 high and low parts
//           of the field weights of P''_t = p_t delta_t 2^k), Vc = code
//           fields.  sum_t p_t zero_t is kept per head on the side.  The
//           exponent k puts the largest value scale seen so far at
//           [2^14, 2^15) so P'' stays in fp16's normal range; it only ever
//           decreases, with an exact power-of-two rescale of O.
// The value-code layout puts, for each 32-token step, the 8 tokens a lane
// holds in the S^T accumulator for one channel in one 32-bit unit, so the
// P' operand comes straight from the q.K^T output registers.
//
// Work split: one workgroup of kMfmaWaves waves per CU and split of a
// (batch, KV head); split s owns chunks s, s + n_split, ..., so at any
// moment the splits stream one contiguous stretch of the cache.  Its waves
// take those chunks in order from a counter in LDS (the first two each
// fixed), so a wave whose loads come back early takes more of them and the
// waves of a CU finish together.  While a wave computes one chunk the codes
// of its next one are already in flight into registers (non-temporal
// loads: read once, not kept in the caches), and so are its key/value
// parameters, which are staged through wave-private LDS (broadcast reads).
// The sink and residual tokens of a split are spread over its waves: each
// wave copies its tokens' rows into LDS before the chunk batches and folds
// them in after its last chunk.  The workgroup merge joins the waves'
// states.
//
// MFMA operand layout (16x16x32, 64 lanes): lane l holds A[row l%16][k in
// group l/16] and B[k in group l/16][col l%16] (8 values each, the same
// k order for A and B), and D[rows 4*(l/16) .. +3][col l%16].
#include <type_traits>

#include "kvq_kernels.h"

namespace kvq {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef float f2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_t mfma_f16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
// Round-to-nearest-even packing of two floats (v_cvt_pk_f16_f32 /
// v_cvt_pk_bf16_f32).  Nearest rounding keeps the high/low splits
// unbiased, so their errors do not accumulate over long token ranges.
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, h2_t));
}

// (a, b) as an fp16 pair for the high columns/rows, (a - high(a), b -
// high(b)) for the low ones (neg_lo = 0 / -1).
__device__ __forceinline__ uint32_t split_pack(float a, float b, float neg_lo) {
  const h2_t hv = __builtin_bit_cast(h2_t, pack_f16(a, b));
  const float r0 = __builtin_fmaf((float)hv[0], neg_lo, a);
  const float r1 = __builtin_fmaf((float)hv[1], neg_lo, b);
  return pack_f16(r0, r1);
}

// The four fp16-subnormal fields of a code word that make one operand.
// 4-bit: bytes 0|2, nibbles 0|4, bytes 1|3, nibbles 2|6 (low|high half).
// 2-bit, PART 0 / 1: nested masks of bytes 0|2 / bytes 1|3.
template <int BITS, int PART>
__device__ __forceinline__ u32x4_t code_fields(uint32_t w) {
  u32x4_t r;
  if constexpr (BITS == 4) {
    const uint32_t t = __builtin_amdgcn_perm(w, w, 0x0C030C01u);   // bytes 1, 3 down
    r[0] = w & 0x00FF00FFu;
    r[1] = w & 0x000F000Fu;
    r[2] = t;
    r[3] = t & 0x000F000Fu;
  } else if constexpr (PART == 0) {
    r[0] = w & 0x00FF00FFu;
    r[1] = w & 0x003F003Fu;
    r[2] = w & 0x000F000Fu;
    r[3] = w & 0x00030003u;
  } else {
    const uint32_t t = __builtin_amdgcn_perm(w, w, 0x0C030C01u);
    r[0] = t;
    r[1] = t & 0x003F003Fu;
    r[2] = t & 0x000F000Fu;
    r[3] = t & 0x00030003u;
  }
  return r;
}

// Field weights of four codes at byte positions 0..3 of their run, from
// per-code factors x_j * f_j, where f_j already carries 2^-(bits * (j mod
// codes-per-byte)); the order matches code_fields.
template <int BITS>
__device__ __forceinline__ void field_weights(const float x[4], const float f[4], float w[4]) {
  if constexpr (BITS == 4) {
    w[0] = x[1] * f[1];                          // c0 + 16 c1 : w1 / 16
    w[1] = __builtin_fmaf(x[0], f[0], -w[0]);    // c0         : w0 - w1 / 16
    w[2] = x[3] * f[3];
    w[3] = __builtin_fmaf(x[2], f[2], -w[2]);
  } else {
    const float y3 = x[3] * f[3], y2 = x[2] * f[2], y1 = x[1] * f[1];
    w[0] = y3;                                   // c0 + 4c1 + 16c2 + 64c3
    w[1] = y2 - y3;                              // c0 + 4c1 + 16c2
    w[2] = y1 - y2;                              // c0 + 4c1
    w[3] = __builtin_fmaf(x[0], f[0], -y1);      // c0
  }
}

// 2^-(bits * (j mod codes-per-byte)): the field scale of code index j.
template <int BITS>
__device__ __forceinline__ float field_scale(int j) {
  return __builtin_amdgcn_ldexpf(1.0f, -BITS * (j % (8 / BITS)));
}

// N consecutive 32-bit words from a 4*N-byte aligned address, as wide
// loads (non-temporal for the 16-byte ones).
template <int N>
__device__ __forceinline__ void load_words(const uint8_t* p, uint32_t* out) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + i / 4);
      out[i] = v[0]; out[i + 1] = v[1]; out[i + 2] = v[2]; out[i + 3] = v[3];
    }
  } else if constexpr (N == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    out[0] = v.x; out[1] = v.y;
  } else {
    out[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

// Code registers of one 64-token chunk in flight.
template <int D, int BITS>
struct ChunkRegs {
  static constexpr int kQW = (D / 4) * BITS / 32;    // key words per lane per tile
  static constexpr int kNB = D / 16;                 // value words per lane per block
  static constexpr int kVB = 64 / VLayout<BITS>::L;  // value blocks per chunk
  uint32_t kw[4][kQW];
  uint32_t vw[kVB][kNB];
};

// Asynchronous copy of 4 or 16 bytes per lane from global memory into LDS
// (lane l's bytes land at lds + l * bytes, lds wave-uniform), counted by
// vmcnt like a load.  Written as assembly so that the compiler, which
// would otherwise hold every later LDS read behind the newest copy in
// flight, leaves the ordering to the explicit waits of the caller; the
// memory clobber keeps the copy in place relative to the wave's other
// memory instructions.  M0 carries the LDS address, as the instruction
// requires.
template <int BYTES>
__device__ __forceinline__ void copy_to_lds(const void* src, const void* lds) {
  static_assert(BYTES == 4 || BYTES == 16, "copy size");
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(l) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(l) : "memory", "m0");
}

// s_waitcnt for the vector-memory counter only (expcnt and lgkmcnt left
// at their maxima), N < 64 (the count's low four bits sit in bits 3:0 of
// the immediate, its high two in bits 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

template <int DT, int D, int BITS, int GQA, bool G32>
__global__ __launch_bounds__(64 * kMfmaWaves, 1) void k_attn_mfma(AttnArgs a) {
  constexpr int kW = kMfmaWaves;
  constexpr int kT = 64 * kW;
  using VLy = VLayout<BITS>;
  using CR = ChunkRegs<D, BITS>;
  constexpr int kRB = D * BITS / 8;        // bytes per key row
  constexpr int kQCH = D / 4;              // channels of a lane's quarter row
  constexpr int kCPW = 32 / BITS;          // codes per 32-bit word
  constexpr int kQW = CR::kQW;
  constexpr int kKS = D / 32;              // K-steps of q.K^T
  constexpr int kNB = CR::kNB;
  constexpr int kVB = CR::kVB;
  constexpr int kNG = G32 ? 2 : 1;         // key groups per chunk
  constexpr int kStepsPerWord = kCPW / 8;  // K-steps covered by one code word
  // GQA 4 with 32-token key groups: the 8 matrix columns a GQA-4 group
  // leaves free take the chunk's second key group (columns 0-3 / 8-11:
  // group 0 high / low parts, 4-7 / 12-15: group 1), so one weight pass
  // serves both groups; the high and low columns of a head are then 8
  // apart, as with GQA 8.
  constexpr bool DUAL = GQA == 4 && G32;
  constexpr int kJoin = (GQA == 8 || DUAL) ? kRowRor8 : kRowRor4;   // high <-> low column
  constexpr float kS = 16777216.0f;        // 2^24: unit of a subnormal code field
  constexpr float kSlack = 8.0f;           // running max kept within 2^8 of the true one
  // value exponent before any scale is seen: the threshold 2^(7 - kNoScale)
  // is the smallest fp32 subnormal, so the first nonzero delta sets it
  constexpr int kNoScale = 156;
  // vector-memory instructions per chunk batch: code loads, then the
  // parameter copies (key groups: one 16-byte copy per group at D = 128,
  // two 4-byte copies at D = 64; values: delta and zero, 4 bytes each)
  constexpr int kCodeLoads = 4 * ((kQW * 4 + 15) / 16) + kVB * ((kNB * 4 + 15) / 16);
  constexpr int kBatch = kCodeLoads + kNG * (D == 128 ? 1 : 2) + 2;
  static_assert(kBatch < 16, "batch must fit the vmcnt field");
  static_assert(D == 64 || D == 128, "head_dim");

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = int64_t(b) * a.H + h;
  // the wave index is uniform: kept in a scalar register, it makes the LDS
  // copy destinations scalar as the copy instructions require
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, lg = lane >> 4;
  const int hh = col % GQA;                          // head of this column
  const bool is_lo = DUAL ? col >= 8 : ((col / GQA) & 1) != 0;   // low part column
  const bool owner = col < GQA;                      // counts l and z once
  const int grp = DUAL ? (col >> 2) & 1 : 0;         // key group of this column (dual form)
  // v from lane l ^ 4: the other key group's column of the same head
  auto other_group = [&](float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 4) << 2, __builtin_bit_cast(int, v)));
  };

  __shared__ float s_q[GQA][D + 4];    // scale*log2e * q; rows padded against bank conflicts
  __shared__ float s_qf[GQA][D + 4];   // the same times each channel's field scale
  __shared__ float s_o[kW][D][16];     // each wave's accumulator rows, channel-major
  __shared__ float s_m[kW][GQA], s_l[kW][GQA], s_z[kW][GQA];
  // wave-private parameter buffers of the chunks in register sets a / b,
  // filled by LDS copies.  Two separate arrays, so that the compiler, which
  // orders reads of an array after the copies in flight into it, does not
  // hold the reads of one buffer behind the other's copies.
  __shared__ float4 s_kp0[kW][2][2 * D / 4], s_kp1[kW][2][2 * D / 4];   // [wave][group][delta | zero]
  __shared__ float s_vp0[kW][2][64], s_vp1[kW][2][64];                  // [wave][delta | zero][token]
  // wave-private rows of the wave's exact tokens (key row, value row each)
  __shared__ uint32_t s_x[kW][1024];
  __shared__ int s_next;                                               // the chunk counter

  // Chunks are numbered from the first one the query attends to (chunk c0,
  // the first of the sliding window; 0 without one).  This workgroup's
  // chunks: j = 0, 1, ... is chunk split + j * n_split (none for splits past
  // the chunk count, which only take exact tokens).  Only the last chunk of
  // the quantized range can be a half chunk (32 tokens).
  const int64_t nch = ((a.Q + 63) >> 6) - a.c0;
  const int64_t nsp = a.n_split;
  const int nj = split < nch ? int((nch - split + nsp - 1) / nsp) : 0;
  const bool wg_half = (a.Q & 63) != 0 && nj > 0 && split + int64_t(nj - 1) * nsp == nch - 1;
  const int nfull = nj - (wg_half ? 1 : 0);
  // 1: a full chunk, 2: the half chunk, 0: past the workgroup's chunks
  auto state_of = [&](int j) { return j < nfull ? 1 : (j == nfull && wg_half ? 2 : 0); };
  auto chunk_of = [&](int j) { return int64_t(split) + int64_t(j) * nsp; };
  // first storage row of chunk ch: the ring's chunk slot (c0 + ch) mod
  // (qcap / 64), by one conditional subtraction (the live chunks span at
  // most qcap / 64 + 1 slots)
  auto chunk_base = [&](int64_t ch) -> int64_t {
    int64_t s = a.c0 + ch - a.cw;
    if (s >= a.ncap) s -= a.ncap;
    return s << 6;
  };
  const uint8_t* kc_head = a.k_codes + bh * a.qcap * kRB;
  const uint8_t* vc_head = a.v_codes + bh * a.qcap * kRB;
  const float* vs_head = a.v_scale + bh * a.qcap;
  const float* vz_head = a.v_zero + bh * a.qcap;
  const float* ks_head = a.k_scale + bh * a.kgroups * D;
  const float* kz_head = a.k_zero + bh * a.kgroups * D;
  const int gsh = a.g_shift;

  // Issue the batch of chunk ch: its code words into r, then its key and
  // value parameters into parameter buffer ch & 1.  Every address lies
  // inside the allocation (qcap >= 64 * ceil(Q / 64) tokens, qcap / G key
  // groups); whatever lies past the quantized range is skipped or masked
  // later.  The instruction count is fixed (kBatch), so waiting for
  // vmcnt <= kBatch completes every batch but the last one issued.
  // A batch that is not live (past the wave's last chunk) keeps the same
  // instructions, with every lane of each on the same 16 bytes of chunk 0:
  // one cache line per instruction.
  auto issue_batch = [&](int64_t ch, bool live, CR& r, auto buf_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    auto& kpb = BUF == 0 ? s_kp0 : s_kp1;
    auto& vpb = BUF == 0 ? s_vp0 : s_vp1;
    const int64_t base = live ? chunk_base(ch) : 0;
    const int cl = live ? col : 0, lgl = live ? lg : 0, ll = live ? lane : 0;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      load_words<kQW>(kc_head + (base + 16 * t + cl) * kRB + lgl * (kQW * 4), r.kw[t]);
#pragma unroll
    for (int vb = 0; vb < kVB; ++vb)
      load_words<kNB>(vc_head + (base / VLy::L + vb) * (VLy::L * kRB) + (lgl * 16 + cl) * kNB * 4,
                      r.vw[vb]);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t g0 = base >> gsh;
#pragma unroll
    for (int gi = 0; gi < kNG; ++gi) {
      float* dst = reinterpret_cast<float*>(&kpb[wave][gi][0]);
      if constexpr (D == 128) {
        // lanes 0..31: delta[4l..4l+3], lanes 32..63: zero[4(l-32)..]
        const float* src = (lane < 32 ? ks_head : kz_head) + (g0 + gi) * D + (ll & 31) * 4;
        copy_to_lds<16>(src, dst);
      } else {
        copy_to_lds<4>(ks_head + (g0 + gi) * D + ll, dst);
        copy_to_lds<4>(kz_head + (g0 + gi) * D + ll, dst + D);
      }
    }
    copy_to_lds<4>(vs_head + base + ll, &vpb[wave][0][0]);
    copy_to_lds<4>(vz_head + base + ll, &vpb[wave][1][0]);
    __builtin_amdgcn_sched_barrier(0);
  };

  // q (raw elements) is copied into LDS by the waves ahead of any chunk
  // batch (requests issued after the first batches of all CUs would queue
  // behind them, and every wave needs q for its first chunk), then each
  // wave issues its first batch and waits for its q copies alone.  Its
  // second batch and the copies of its exact-token rows (four, always;
  // those past its rows copy 16 bytes of chunk 0) go out during its first
  // chunk: a CU's memory pipeline takes requests in issue order and holds
  // a wave's issue while it is full, so a wave that issued two batches up
  // front could not start its first chunk, landed, before the second one
  // had gone out.
  using QE = typename Elem<DT>::T;
  constexpr int kEsz = Elem<DT>::bytes;
  constexpr int kQRowB = D * kEsz;                 // bytes per q row
  constexpr int kQI = GQA * kQRowB / 256;          // 256-byte copies of q
  __shared__ uint32_t s_qraw[GQA * kQRowB / 4];
#pragma unroll
  for (int i0 = 0; i0 < (kQI + kW - 1) / kW; ++i0) {
    const int i = i0 * kW + wave;
    if (i < kQI) {
      const int o = i * 256 + lane * 4, qh = o / kQRowB;
      const char* src = reinterpret_cast<const char*>(a.q) +
                        (b * a.q_sb + (h * GQA + qh) * a.q_sh) * kEsz + o % kQRowB;
      copy_to_lds<4>(src, reinterpret_cast<const char*>(&s_qraw[0]) + i * 256);
    }
  }
  // This wave's first batch (a wave without chunks issues a batch that is
  // not live, on chunk 0, which exists: the kernel runs only with Q > 0),
  // behind q; then q alone is waited for.
  CR ra, rb;
  const int jA0 = wave, jB0 = wave + kW;
  issue_batch(chunk_of(jA0), state_of(jA0) != 0, ra, std::integral_constant<int, 0>{});
  wait_vmcnt<kBatch>();
  __syncthreads();
  // The split's exact tokens (sinks and the residual window) are [f0, f1);
  // this wave's are f0 + wave, f0 + wave + kW, ...  The rows of the first
  // kXPer of them (4 KB; the planner keeps a split's count within
  // mfma_exact_cap, unless the workspace is too small for more splits) are
  // copied into s_x[wave] (token i: key row, then value row); all are
  // folded in after the wave's last chunk.
  const int64_t f0 = int64_t(split) * a.fp_per_split;
  const int64_t f1 = f0 + a.fp_per_split < a.n_fp ? f0 + a.fp_per_split : a.n_fp;
  auto fp_row = [&](int64_t i, const void*& kb, const void*& vb, int64_t& off) {
    if (i < a.n_sink) {
      kb = a.k_sink; vb = a.v_sink; off = (bh * a.S + i) * D;
    } else {
      int64_t slot = a.resid_slot0 + (i - a.n_sink);   // < 2 * ring
      if (slot >= a.ring) slot -= a.ring;
      kb = a.k_resid; vb = a.v_resid; off = (bh * a.ring + slot) * D;
    }
  };
  constexpr int kRowB = D * kEsz;                  // bytes per row
  constexpr int kXPer = 4096 / (2 * kRowB);         // tokens staged per wave
  const int nxw = f0 + wave < f1 ? int((f1 - f0 - wave + kW - 1) / kW) : 0;
  __shared__ float s_qmx[kW];
  float qmx = 0.f;                                 // max |scale*log2e * q| of the workgroup
  constexpr int kQPer = (GQA * D + kT - 1) / kT;
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    const int x = threadIdx.x + kT * j, qh = x / D, d = x % D;
    if (x < GQA * D) {
      float qf;
      if constexpr (DT == DT_F32) qf = reinterpret_cast<const float*>(&s_qraw[0])[x];
      else if constexpr (DT == DT_F16) qf = f16_bits_to_f32(reinterpret_cast<const QE*>(&s_qraw[0])[x]);
      else qf = bf16_bits_to_f32(reinterpret_cast<const QE*>(&s_qraw[0])[x]);
      const float v = qf * a.sm_scale_log2;
      s_q[qh][d] = v;
      s_qf[qh][d] = v * field_scale<BITS>(d);
      qmx = __builtin_fmaxf(qmx, __builtin_fabsf(v));
    }
  }
  qmx = wave_max(qmx);
  if (lane == 0) s_qmx[wave] = qmx;
  if (threadIdx.x == 0) s_next = 2 * kW;
  __syncthreads();
  float qmax = s_qmx[0];
#pragma unroll
  for (int w = 1; w < kW; ++w) qmax = __builtin_fmaxf(qmax, s_qmx[w]);
  // issue_second starts this wave's second batch and its exact-token
  // copies.
  auto issue_second = [&]() {
    {
      const int bytes = (nxw < kXPer ? nxw : kXPer) * 2 * kRowB;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int o = k * 1024 + lane * 16;
        const int r = o / kRowB, i = r >> 1;
        const char* src = reinterpret_cast<const char*>(kc_head);
        if (k * 1024 < bytes) {
          const void* kb;
          const void* vb;
          int64_t off;
          fp_row(f0 + wave + int64_t(i < nxw ? i : 0) * kW, kb, vb, off);
          const char* row = reinterpret_cast<const char*>((r & 1) ? vb : kb) + off * kEsz;
          // lanes past the wave's rows copy the start of its first row (in bounds)
          src = i < nxw ? row + o % kRowB : row;
        }
        copy_to_lds<16>(src, reinterpret_cast<const char*>(&s_x[wave][0]) + k * 1024);
      }
    }
    issue_batch(chunk_of(jB0), state_of(jB0) != 0, rb, std::integral_constant<int, 1>{});
  };
  // Key weights w = x * delta with |x| <= qmax: every field weight is at
  // most 1.25 qmax delta_max, so the fp16 high parts stay finite while the
  // chunk's largest key delta is below 2^15 / qmax.  A chunk at or above
  // 2^12 / qmax takes the rare branch, which scales the weights by 2^-e and
  // forms its scores in one rounding: below it, kappa - m and the products
  // stay under ~2^26, so the split sum kappa - m + products keeps the
  // running-max slack.
  const float kthr = 4096.0f / qmax;                // +inf when q is zero

  f32x4_t acc[kNB];
#pragma unroll
  for (int n = 0; n < kNB; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff(), l = 0.f, z = 0.f;
  int kexp = kNoScale;                               // P'' = p * delta * 2^kexp
  const float neg_lo = is_lo ? -1.0f : 0.0f;
  // byte selector of v_perm: identity on high lanes, 16-bit halves swapped
  // on low lanes
  const uint32_t swap_sel = is_lo ? 0x01000302u : 0x03020100u;

  // Running-max update shared by both token kinds: the max moves only when
  // a score exceeds it by more than the slack, so p <= 2^8 in between.
  auto raise_max = [&](float cm) {
    if (__builtin_amdgcn_ballot_w64(cm > m + kSlack) != 0) {
      const float new_m = __builtin_fmaxf(m, cm);
      const float alpha = __builtin_amdgcn_exp2f(m - new_m);
      l *= alpha;
      z *= alpha;
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ar[i] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                              ((4 * lg + i) % GQA) << 2, __builtin_bit_cast(int, alpha)));
#pragma unroll
      for (int n = 0; n < kNB; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[n][i] *= ar[i];
      m = new_m;
    }
  };

  // Wave state into LDS: l and z reduced over the owner columns' lane
  // groups; the accumulator (in real units by then) written whole, rows
  // channel-major, its high and low rows joined in the workgroup merge.
  auto stash = [&]() {
    float lr = l + dpp_rot<kJoin>(l);     // owner (even tiles or exact tokens) + partner (odd tiles)
    float zr = z + dpp_rot<kJoin>(z);
    if constexpr (DUAL) {
      lr += other_group(lr);
      zr += other_group(zr);
    }
    if (!owner) {
      lr = 0.f;
      zr = 0.f;
    }
    lr = sum_xor32(sum_xor16(lr));
    zr = sum_xor32(sum_xor16(zr));
    if (lane < GQA) {
      s_m[wave][lane] = m;
      s_l[wave][lane] = lr;
      s_z[wave][lane] = zr;
    }
#pragma unroll
    for (int n = 0; n < kNB; ++n) *reinterpret_cast<f32x4_t*>(&s_o[wave][n * 16 + col][4 * lg]) = acc[n];
  };

  // An exact token folded into the state, from its partial score over the
  // lane's quarter row (an fp32 dot product) and its values vv, which are
  // added to the high rows in the accumulator's units.
  auto fold_score = [&](float part, const float* vv) {
    part = sum_xor16(part);
    const float sc = sum_xor32(part);             // score of head hh
    raise_max(sc);
    const float p = __builtin_amdgcn_exp2f(sc - m);
    if (lg == 0 && owner) l += p;                 // one lane group of the owner columns
    float pr[4];
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      const float v = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                                    ((4 * lg + i2) % GQA) << 2, __builtin_bit_cast(int, p)));
      pr[i2] = (4 * lg + i2) < GQA ? v : 0.f;     // high rows only
    }
#pragma unroll
    for (int n = 0; n < kNB; ++n)
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) acc[n][i2] = __builtin_fmaf(pr[i2], vv[n], acc[n][i2]);
  };

  // The wave's exact token i: its partial score over the lane's quarter
  // row and its values, from its rows in s_x (i < kXPer; the key row is
  // read four channels at a time, so few registers stay live), or past
  // the staged ones from the cache.
  auto exact_part = [&](int i) -> float {
    float part = 0.f;
    if (i >= kXPer) {
      const void* kb;
      const void* vb;
      int64_t off;
      fp_row(f0 + wave + int64_t(i) * kW, kb, vb, off);
#pragma unroll
      for (int c = 0; c < kQCH; c += 4) {
        float k4[4];
        load4<DT>(kb, off + lg * kQCH + c, k4);
        const float4 q4 = *reinterpret_cast<const float4*>(&s_q[hh][lg * kQCH + c]);
        part = __builtin_fmaf(k4[0], q4.x, part);
        part = __builtin_fmaf(k4[1], q4.y, part);
        part = __builtin_fmaf(k4[2], q4.z, part);
        part = __builtin_fmaf(k4[3], q4.w, part);
      }
      return part;
    }
    const char* xk = reinterpret_cast<const char*>(&s_x[wave][0]) + i * 2 * kRowB;
#pragma unroll
    for (int c = 0; c < kQCH; c += 4) {
      float k4[4];
      if constexpr (DT == DT_F32) {
        const float4 v = *reinterpret_cast<const float4*>(xk + (lg * kQCH + c) * 4);
        k4[0] = v.x; k4[1] = v.y; k4[2] = v.z; k4[3] = v.w;
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(xk + (lg * kQCH + c) * 2);
        const uint32_t e[4] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16};
#pragma unroll
        for (int t = 0; t < 4; ++t) k4[t] = DT == DT_F16 ? f16_bits_to_f32(e[t]) : bf16_bits_to_f32(e[t]);
      }
      const float4 q4 = *reinterpret_cast<const float4*>(&s_q[hh][lg * kQCH + c]);
      part = __builtin_fmaf(k4[0], q4.x, part);
      part = __builtin_fmaf(k4[1], q4.y, part);
      part = __builtin_fmaf(k4[2], q4.z, part);
      part = __builtin_fmaf(k4[3], q4.w, part);
    }
    return part;
  };
  auto exact_values = [&](int i, float* vv) {
    if (i >= kXPer) {
      const void* kb;
      const void* vb;
      int64_t off;
      fp_row(f0 + wave + int64_t(i) * kW, kb, vb, off);
#pragma unroll
      for (int n = 0; n < kNB; ++n) vv[n] = load1<DT>(vb, off + 16 * n + col);
      return;
    }
    const char* xv = reinterpret_cast<const char*>(&s_x[wave][0]) + i * 2 * kRowB + kRowB;
#pragma unroll
    for (int n = 0; n < kNB; ++n) {
      if constexpr (DT == DT_F32) {
        vv[n] = reinterpret_cast<const float*>(xv)[16 * n + col];
      } else {
        const uint32_t e = reinterpret_cast<const uint16_t*>(xv)[16 * n + col];
        vv[n] = DT == DT_F16 ? f16_bits_to_f32(e) : bf16_bits_to_f32(e);
      }
    }
  };
  int x_done = 0;                                  // exact tokens folded in so far

  {
    // ------------------------------------------------------------ quantized
    // exponents of the value field scales of rows i (token 4g + i of a
    // tile) plus kexp: P''_t = p_t * ldexp(delta_t, vke[i]).  ldexp keeps
    // exponents outside fp32's range of powers of two (kexp up to 156 for
    // subnormal deltas) exact.
    int vke[4];
    auto set_vke = [&]() {
#pragma unroll
      for (int i = 0; i < 4; ++i) vke[i] = kexp - BITS * (i % (8 / BITS));
    };
    set_vke();
    const int vtok = (lane & 31) * 2;                // value deltas this lane checks

    u32x4_t qB[kKS];

    // Field weights of one key group into qB (high or low parts): x_d
    // (field-scaled q) times delta_d.  A high column and its low partner
    // (kJoin apart in the row) split the K-steps: each computes both fp16
    // parts of its own half (high lanes K-steps [0, kKS/2), low lanes the
    // rest), keeps the part of its own kind and takes the other half's part
    // of its kind from the partner by a DPP move masked to its banks.
    constexpr int kHalfKS = kKS / 2;
    constexpr int kHiBanks = (GQA == 8 || DUAL) ? 0x3 : 0x5;   // banks of high columns
    constexpr int kLoBanks = 0xF ^ kHiBanks;
    const int kk_own = is_lo ? kHalfKS : 0;
    auto group_weights = [&](const float* kpd) {
#pragma unroll
      for (int j = 0; j < kHalfKS; ++j) {
        const int kk = j + kk_own;
        const int wk = kk / kStepsPerWord, sp = kk % kStepsPerWord;
        // the 8 channels of this K-step: runs [cA, cA+4) (low halves of
        // the fields) and [cB, cB+4) (high halves) of word wk
        const int cA = lg * kQCH + wk * kCPW + 4 * sp;
        const int cB = cA + kCPW / 2;
        const float4 qa = *reinterpret_cast<const float4*>(&s_qf[hh][cA]);
        const float4 qb = *reinterpret_cast<const float4*>(&s_qf[hh][cB]);
        const float4 da = *reinterpret_cast<const float4*>(kpd + cA);
        const float4 db = *reinterpret_cast<const float4*>(kpd + cB);
        const float xa[4] = {qa.x, qa.y, qa.z, qa.w}, xb[4] = {qb.x, qb.y, qb.z, qb.w};
        const float fa[4] = {da.x, da.y, da.z, da.w}, fb[4] = {db.x, db.y, db.z, db.w};
        float wa[4], wb[4];
        field_weights<BITS>(xa, fa, wa);
        field_weights<BITS>(xb, fb, wb);
#pragma unroll
        for (int r2 = 0; r2 < 4; ++r2) {
          const uint32_t hi = pack_f16(wa[r2], wb[r2]);
          const h2_t hv = __builtin_bit_cast(h2_t, hi);
          const uint32_t lo = pack_f16(wa[r2] - (float)hv[0], wb[r2] - (float)hv[1]);
          // K-step j: high lanes keep theirs, low lanes take the high
          // partner's low part; K-step j + kHalfKS: the other way round
          qB[j][r2] = uint32_t(__builtin_amdgcn_update_dpp(int(hi), int(lo), kJoin, 0xF, kLoBanks, false));
          qB[j + kHalfKS][r2] = uint32_t(__builtin_amdgcn_update_dpp(int(lo), int(hi), kJoin, 0xF, kHiBanks, false));
        }
      }
    };
    // S^T tiles [t_begin, t_end) of chunk r from the weights in qB.
    auto tile_products = [&](const CR& r, f32x4_t* sc, int t_begin, int t_end) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t >= t_begin && t < t_end) sc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kKS; ++kk) {
        const int wk = kk / kStepsPerWord;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (t < t_begin || t >= t_end) continue;
          u32x4_t av;
          if (kk % kStepsPerWord == 0) av = code_fields<BITS, 0>(r.kw[t][wk]);
          else av = code_fields<BITS, 1>(r.kw[t][wk]);
          sc[t] = mfma_f16(av, qB[kk], sc[t]);
        }
      }
    };

    // A half chunk (only ever the last of the quantized range) holds 32
    // tokens: tiles 0 and 1, the first 32-token step of P.V.
    // The wave's staged exact tokens, folded into the state in the units of
    // the accumulator (values times 2^(kexp - 24)); kexp is lowered first
    // where the largest value needs it, so that p * v stays below 2^108.
    auto fold_exact_scaled = [&]() {
      const int nst = nxw < kXPer ? nxw : kXPer;   // the staged ones
      for (int i = 0; i < nst; ++i) {
        const float part = exact_part(i);
        float vv[kNB];
        exact_values(i, vv);
        float vm = 0.f;
#pragma unroll
        for (int n = 0; n < kNB; ++n) vm = __builtin_fmaxf(vm, __builtin_fabsf(vv[n]));
        const int ev = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(wave_max(vm)));
        if (kexp - 24 + ev > 100) {
          const int knew = 124 - ev;
#pragma unroll
          for (int n = 0; n < kNB; ++n)
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2) acc[n][i2] = __builtin_amdgcn_ldexpf(acc[n][i2], knew - kexp);
          kexp = knew;
          set_vke();
        }
#pragma unroll
        for (int n = 0; n < kNB; ++n) vv[n] = __builtin_amdgcn_ldexpf(vv[n], kexp - 24);
        fold_score(part, vv);
      }
      x_done = nst;
    };
    // ORD 1: the wave's first chunk, whose batch is the only one issued: it
    // waits for all of it and starts the second batch after its q.K^T.
    auto process_chunk = [&](const CR& r, int64_t ch, auto half_tag, auto buf_tag, auto ord_tag) {
      constexpr bool HALF = decltype(half_tag)::value;
      constexpr bool FIRST = decltype(ord_tag)::value == 1;
      constexpr int kTiles = HALF ? 2 : 4;
      constexpr int BUF = decltype(buf_tag)::value;
      const auto& kpb = BUF == 0 ? s_kp0 : s_kp1;
      const auto& vpb = BUF == 0 ? s_vp0 : s_vp1;
      constexpr int nv = HALF ? 32 : 64;
      constexpr int kSegTiles = G32 ? 2 : 4;
      constexpr int kPasses = (G32 && !DUAL) ? 2 : 1;
      // key groups of this chunk that hold quantized tokens (a half chunk
      // with 32-token groups has one)
      constexpr int kLiveGroups = (G32 && !HALF) ? 2 : 1;
      // this chunk's batch is complete once at most the next one is in flight
      if constexpr (FIRST) wait_vmcnt<0>();
      else wait_vmcnt<kBatch>();
      // ---- value scale: a delta at or above 2^(7-kexp) lowers kexp so
      // that the largest delta seen sits in [2^6, 2^7); with p <= 2^8 the
      // value weights stay below 2^15.  Checked here, acted on (rarely)
      // together with the running max before P.V, so that one branch per
      // chunk splits its instruction stream.
      const float2 dv = *reinterpret_cast<const float2*>(&vpb[wave][0][vtok]);
      const float vmax = vtok < nv ? __builtin_fmaxf(dv.x, dv.y) : 0.0f;
      const bool v_over = vmax >= __builtin_amdgcn_ldexpf(1.0f, 7 - kexp);
      // ---- key range: the lanes share the chunk's key deltas, a disjoint
      // few each; any at or above kthr sends the chunk to the rare branch
      float kdm;
      {
        // lanes [64/kLiveGroups * g, ...) cover group g, kPer deltas each
        constexpr int kPer = kLiveGroups * D / 64;
        constexpr int kLanesPerGroup = 64 / kLiveGroups;
        const float* kp = reinterpret_cast<const float*>(&kpb[wave][lane / kLanesPerGroup][0]) +
                          (lane % kLanesPerGroup) * kPer;
        if constexpr (kPer == 4) {
          const float4 x = *reinterpret_cast<const float4*>(kp);
          kdm = __builtin_fmaxf(__builtin_fmaxf(x.x, x.y), __builtin_fmaxf(x.z, x.w));
        } else if constexpr (kPer == 2) {
          const float2 x = *reinterpret_cast<const float2*>(kp);
          kdm = __builtin_fmaxf(x.x, x.y);
        } else {
          kdm = kp[0];
        }
      }
      const bool k_over = kdm >= kthr;
      auto seg_range = [&](int seg, int& t_begin, int& t_end) {
        t_begin = DUAL ? 0 : seg * kSegTiles;
        t_end = DUAL ? kTiles : (t_begin + kSegTiles < kTiles ? t_begin + kSegTiles : kTiles);
      };
      auto seg_params = [&](int seg) {
        return reinterpret_cast<const float*>(&kpb[wave][DUAL ? grp : (G32 ? seg : 0)][0]);
      };
      // ---- q.K^T: per key-group segment, K-steps outer, tiles inner
      f32x4_t sc[4];
      float kap[2] = {0.f, 0.f};               // kappa of each segment's group
#pragma unroll
      for (int seg = 0; seg < kPasses; ++seg) {
        int t_begin, t_end;
        seg_range(seg, t_begin, t_end);
        if (t_begin >= kTiles) break;
        {
          const float* kpd = seg_params(seg);
          group_weights(kpd);
          // kappa = sum_d q_d zero_d: high columns take the first half of
          // the K-steps, low columns the second, joined by the rotate-add;
          // it is added to the scores after the matrix products
          float kpart = 0.f;
#pragma unroll
          for (int j = 0; j < kKS / 2; ++j) {
            const int kk = j + (is_lo ? kKS / 2 : 0);
            const int wk = kk / kStepsPerWord, sp = kk % kStepsPerWord;
            const int cA = lg * kQCH + wk * kCPW + 4 * sp;
            const int cB = cA + kCPW / 2;
            const float4 qa = *reinterpret_cast<const float4*>(&s_q[hh][cA]);
            const float4 qb = *reinterpret_cast<const float4*>(&s_q[hh][cB]);
            const float4 za = *reinterpret_cast<const float4*>(kpd + D + cA);
            const float4 zb = *reinterpret_cast<const float4*>(kpd + D + cB);
            kpart = __builtin_fmaf(qa.x, za.x, kpart);
            kpart = __builtin_fmaf(qa.y, za.y, kpart);
            kpart = __builtin_fmaf(qa.z, za.z, kpart);
            kpart = __builtin_fmaf(qa.w, za.w, kpart);
            kpart = __builtin_fmaf(qb.x, zb.x, kpart);
            kpart = __builtin_fmaf(qb.y, zb.y, kpart);
            kpart = __builtin_fmaf(qb.z, zb.z, kpart);
            kpart = __builtin_fmaf(qb.w, zb.w, kpart);
          }
          kpart += dpp_rot<kJoin>(kpart);
          kpart = sum_xor16(kpart);
          kap[seg] = sum_xor32(kpart);
        }
        tile_products(r, sc, t_begin, t_end);
      }
      if constexpr (FIRST) issue_second();
      // join the high and low columns of each head (scores - kappa, times
      // 2^-24)
      auto join_tiles = [&]() {
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[t][i] += dpp_rot<kJoin>(sc[t][i]);
        }
      };
      join_tiles();
      // ---- online softmax (log2 domain); m is per head, uniform over lanes
      auto chunk_max = [&]() {
        float cm_seg[2] = {-__builtin_inff(), -__builtin_inff()};
#pragma unroll
        for (int t = 0; t < kTiles; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) cm_seg[t / kSegTiles] = __builtin_fmaxf(cm_seg[t / kSegTiles], sc[t][i]);
        float c;
        if constexpr (DUAL) {
          c = __builtin_fmaf(grp ? cm_seg[1] : cm_seg[0], kS, kap[0]);   // this column's group's tiles
        } else {
          c = __builtin_fmaf(cm_seg[0], kS, kap[0]);
          if constexpr (G32 && !HALF) c = __builtin_fmaxf(c, __builtin_fmaf(cm_seg[1], kS, kap[1]));
        }
        return c;
      };
      // the sliding window's first chunk: scores of the tokens before the
      // window are -inf (p = 0)
      auto mask_front = [&]() {
        if (ch == 0 && a.lo_off > 0) {
#pragma unroll
          for (int t = 0; t < kTiles; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (16 * t + 4 * lg + i < a.lo_off) sc[t][i] = -__builtin_inff();
        }
      };
      mask_front();
      float cm = chunk_max();
      // the head's max over lanes is only needed when the running max
      // moves: any lane over m + slack means its head's max is
      // wave priority: 1 from the chunk's start, 2 from here to the issue
      // of the next batch, 0 after it; a wave that has reached P.V goes
      // ahead of its SIMD partner, so its chunk ends and its next loads go
      // out sooner (same-box A/B: -0.5 to -0.9 us per call)
      __builtin_amdgcn_s_setprio(2);
      const uint64_t need_k = __builtin_amdgcn_ballot_w64(k_over);
      const uint64_t need_v = __builtin_amdgcn_ballot_w64(v_over);
      uint64_t need_m = __builtin_amdgcn_ballot_w64(cm > m + kSlack);
      if ((need_k | need_v | need_m) != 0) {
        if (need_k != 0) {
          // a wide key range: the weights of this chunk again with x scaled
          // by 2^-e, e = exponent of qmax * (largest delta) less 14, so
          // every field weight is below 1.25 * 2^14; the products are
          // scaled back by 2^e (exact) before the scores are formed
          const float big = qmax * wave_max(kdm);
          const int e = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(big) - 14);
          const float xs = __builtin_amdgcn_ldexpf(1.0f, -e);
          // One K-step at a time, with the chunk's key codes loaded again
          // (ordinary loads), so that the branch needs few registers beyond
          // those live across it.
#pragma unroll
          for (int seg = 0; seg < kPasses; ++seg) {
            int t_begin, t_end;
            seg_range(seg, t_begin, t_end);
            if (t_begin >= kTiles) break;
            const float* kpd = seg_params(seg);
#pragma unroll
            for (int t = 0; t < 4; ++t)
              if (t >= t_begin && t < t_end) sc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < kKS; ++kk) {
              __builtin_amdgcn_sched_barrier(0);
              const int wk = kk / kStepsPerWord, sp = kk % kStepsPerWord;
              const int cA = lg * kQCH + wk * kCPW + 4 * sp;
              const int cB = cA + kCPW / 2;
              const float4 qa = *reinterpret_cast<const float4*>(&s_qf[hh][cA]);
              const float4 qb = *reinterpret_cast<const float4*>(&s_qf[hh][cB]);
              const float4 da = *reinterpret_cast<const float4*>(kpd + cA);
              const float4 db = *reinterpret_cast<const float4*>(kpd + cB);
              const float xa[4] = {qa.x * xs, qa.y * xs, qa.z * xs, qa.w * xs};
              const float xb[4] = {qb.x * xs, qb.y * xs, qb.z * xs, qb.w * xs};
              const float fa[4] = {da.x, da.y, da.z, da.w}, fb[4] = {db.x, db.y, db.z, db.w};
              float wa[4], wb[4];
              field_weights<BITS>(xa, fa, wa);
              field_weights<BITS>(xb, fb, wb);
              u32x4_t wq;
#pragma unroll
              for (int r2 = 0; r2 < 4; ++r2) wq[r2] = split_pack(wa[r2], wb[r2], neg_lo);
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                if (t < t_begin || t >= t_end) continue;
                const uint32_t w = reinterpret_cast<const uint32_t*>(
                    kc_head + (chunk_base(ch) + 16 * t + col) * kRB + lg * (kQW * 4))[wk];
                u32x4_t av;
                if (kk % kStepsPerWord == 0) av = code_fields<BITS, 0>(w);
                else av = code_fields<BITS, 1>(w);
                sc[t] = mfma_f16(av, wq, sc[t]);
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          join_tiles();
          // whole scores, rounded once, back in units of 2^24 (kappa folded
          // in and then zero): with scores this large, kappa - m rounded on
          // its own would leave an error of ulp(kappa) in the largest score
#pragma unroll
          for (int t = 0; t < kTiles; ++t) {
            const float kp = DUAL ? kap[0] : kap[t / kSegTiles];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sc[t][i] = __builtin_amdgcn_ldexpf(
                  __builtin_fmaf(__builtin_amdgcn_ldexpf(sc[t][i], e), kS, kp), -24);
          }
          kap[0] = 0.f;
          kap[1] = 0.f;
          mask_front();
          cm = chunk_max();
          need_m = __builtin_amdgcn_ballot_w64(cm > m + kSlack);
        }
        if (need_v != 0) {
          const int knew = __builtin_amdgcn_readfirstlane(7 - __builtin_amdgcn_frexp_expf(wave_max(vmax)));
#pragma unroll
          for (int n = 0; n < kNB; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[n][i] = __builtin_amdgcn_ldexpf(acc[n][i], knew - kexp);
          kexp = knew;
          set_vke();
        }
        if (need_m != 0) {
          cm = max_xor16(cm);
          cm = max_xor32(cm);
          if constexpr (DUAL) cm = __builtin_fmaxf(cm, other_group(cm));
          raise_max(cm);
        }
      }
      const float km0 = kap[0] - m, km1 = kap[1] - m;
      // ---- P.V per 32-token step (tiles 2ps, 2ps+1).  A high column and
      // its low partner (GQA lanes apart in the row) hold the same scores:
      // the high one weighs tile 2ps, the low one tile 2ps+1, and each takes
      // the other tile's weights from its partner; both then pack the pair
      // in tile order (high or low parts).  l and z gather per tile parity
      // and meet at the end.
      if constexpr (DUAL) {
        // dual-group form: a column weighs only its own group's 32-token
        // step (tiles 2 grp and 2 grp + 1; none in a half chunk for group
        // 1), so its weights are computed once and placed in that step's
        // operand, with zeros in the other step's
        const int t_own = 2 * grp + (is_lo ? 1 : 0);
        const int tok = 16 * t_own + 4 * lg;
        const float4 dv = *reinterpret_cast<const float4*>(&vpb[wave][0][tok]);
        const float4 zv = *reinterpret_cast<const float4*>(&vpb[wave][1][tok]);
        const float ds[4] = {__builtin_amdgcn_ldexpf(dv.x, vke[0]), __builtin_amdgcn_ldexpf(dv.y, vke[1]),
                             __builtin_amdgcn_ldexpf(dv.z, vke[2]), __builtin_amdgcn_ldexpf(dv.w, vke[3])};
        // group 1 of a half chunk has no tokens: its zero points are never
        // written, so they are not read into z
        const float zs[4] = {(HALF && grp) ? 0.f : zv.x, (HALF && grp) ? 0.f : zv.y,
                             (HALF && grp) ? 0.f : zv.z, (HALF && grp) ? 0.f : zv.w};
        float pm[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float s0 = is_lo ? sc[1][i] : sc[0][i];
          float sm = s0;
          if constexpr (!HALF) sm = grp ? (is_lo ? sc[3][i] : sc[2][i]) : s0;
          pm[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sm, kS, km0));
          if constexpr (HALF) pm[i] = grp ? 0.f : pm[i];
          l += pm[i];
          z = __builtin_fmaf(pm[i], zs[i], z);
        }
        float wm[4];
        field_weights<BITS>(pm, ds, wm);
        u32x4_t ap_own;
#pragma unroll
        for (int r2 = 0; r2 < 4; ++r2) {
          const float wo = dpp_rot<kJoin>(wm[r2]);
          ap_own[r2] = __builtin_amdgcn_perm(0u, split_pack(wm[r2], wo, neg_lo), swap_sel);
        }
#pragma unroll
        for (int ps = 0; ps < kTiles / 2; ++ps) {
          u32x4_t ap;
#pragma unroll
          for (int r2 = 0; r2 < 4; ++r2) ap[r2] = ps == grp ? ap_own[r2] : 0u;
#pragma unroll
          for (int n = 0; n < kNB; ++n) {
            u32x4_t bv;
            if constexpr (kVB == 2) {
              bv = code_fields<BITS, 0>(r.vw[ps][n]);
            } else {
              if (ps == 0) bv = code_fields<BITS, 0>(r.vw[0][n]);
              else bv = code_fields<BITS, 1>(r.vw[0][n]);
            }
            acc[n] = mfma_f16(ap, bv, acc[n]);
          }
        }
        return;
      }
#pragma unroll
      for (int ps = 0; ps < kTiles / 2; ++ps) {
        const int t0 = 2 * ps, t1 = 2 * ps + 1;
        const float kmp = (t0 / kSegTiles) == 0 ? km0 : km1;
        const int tok = 16 * (is_lo ? t1 : t0) + 4 * lg;
        const float4 dv = *reinterpret_cast<const float4*>(&vpb[wave][0][tok]);
        const float4 zv = *reinterpret_cast<const float4*>(&vpb[wave][1][tok]);
        const float ds[4] = {__builtin_amdgcn_ldexpf(dv.x, vke[0]), __builtin_amdgcn_ldexpf(dv.y, vke[1]),
                             __builtin_amdgcn_ldexpf(dv.z, vke[2]), __builtin_amdgcn_ldexpf(dv.w, vke[3])};
        const float zs[4] = {zv.x, zv.y, zv.z, zv.w};
        float pm[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sm = is_lo ? sc[t1][i] : sc[t0][i];
          pm[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sm, kS, kmp));
          l += pm[i];                         // every lane; owners and partners meet at the end
          z = __builtin_fmaf(pm[i], zs[i], z);
        }
        float wm[4];
        field_weights<BITS>(pm, ds, wm);
        u32x4_t ap;
#pragma unroll
        for (int r2 = 0; r2 < 4; ++r2) {
          const float wo = dpp_rot<kJoin>(wm[r2]);
          // (own, other) -> (tile 2ps, tile 2ps+1): halves swapped on low lanes
          ap[r2] = __builtin_amdgcn_perm(0u, split_pack(wm[r2], wo, neg_lo), swap_sel);
        }
#pragma unroll
        for (int n = 0; n < kNB; ++n) {
          u32x4_t bv;
          if constexpr (kVB == 2) {
            bv = code_fields<BITS, 0>(r.vw[ps][n]);
          } else {
            if (ps == 0) bv = code_fields<BITS, 0>(r.vw[0][n]);
            else bv = code_fields<BITS, 1>(r.vw[0][n]);
          }
          acc[n] = mfma_f16(ap, bv, acc[n]);
        }
      }
    };

    // The wave's first two chunks are fixed (j = wave and wave + kW); every
    // later index comes from the workgroup's counter, fetched one chunk
    // ahead so that its LDS round trip is hidden.  After a chunk, its
    // registers and parameter buffer are free: the batch of the next index
    // starts there.  Past the workgroup's chunks that batch is not live (one
    // cache line of chunk 0 per instruction), so that a batch always
    // follows each chunk, as the counter waits assume.  The copies into the
    // buffer are ordered after this wave's reads of it by the wait on the
    // LDS counter.
    int jA = jA0, jB = jB0;
    int stA = state_of(jA), stB = state_of(jB);
    auto fetch = [&]() {
      int v = 0;
      if (lane == 0) v = __hip_atomic_fetch_add(&s_next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return v;                                      // in lane 0
    };
    int jn = fetch();
    auto next_batch = [&](CR& r, int& j, int& st, auto buf_tag) {
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      j = __builtin_amdgcn_readfirstlane(jn);
      st = state_of(j);
      issue_batch(chunk_of(j), st != 0, r, buf_tag);
      jn = fetch();
    };
    auto run_chunk = [&](CR& r, int& j, int& st, auto buf_tag) {
      __builtin_amdgcn_s_setprio(1);
      process_chunk(r, chunk_of(j), std::false_type{}, buf_tag, std::integral_constant<int, 0>{});
      next_batch(r, j, st, buf_tag);
      __builtin_amdgcn_s_setprio(0);
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    // The first chunk (set a) issues set b's batch, and after it the
    // staged exact tokens are folded in (their copies went out ahead of set
    // b's batch, so waiting for them leaves both batches in flight); then
    // the sets alternate, b first, and the set checked is always the one
    // with the older (smaller) index, whose batch is not the newest, so the
    // compiler's own waits for its registers never reach far into the other
    // set's.  A set whose chunk is not a full one ends the loop; it may hold
    // the half chunk (the other set's index is larger, so it holds nothing).
    bool at_a = true;
    if (stA == 1) {
      __builtin_amdgcn_s_setprio(1);
      process_chunk(ra, chunk_of(jA), std::false_type{}, B0{}, std::integral_constant<int, 1>{});
      next_batch(ra, jA, stA, B0{});
      __builtin_amdgcn_s_setprio(0);
      if (nxw > 0) {
        wait_vmcnt<2 * kBatch>();
        fold_exact_scaled();
      }
      for (;;) {
        if (stB != 1) {
          at_a = false;
          break;
        }
        run_chunk(rb, jB, stB, B1{});
        if (stA != 1) break;
        run_chunk(ra, jA, stA, B0{});
      }
    } else {
      issue_second();
    }
    __builtin_amdgcn_s_setprio(1);
    if (at_a) {
      if (stA == 2) process_chunk(ra, chunk_of(jA), std::true_type{}, B0{}, std::integral_constant<int, 0>{});
    } else if (stB == 2) {
      process_chunk(rb, chunk_of(jB), std::true_type{}, B1{}, std::integral_constant<int, 0>{});
    }
    __builtin_amdgcn_s_setprio(0);
    // let every copy land before the buffers are left behind (and the
    // exact-token rows are read)
    wait_vmcnt<0>();
  }
  // ---- the accumulator in real units, then this wave's exact tokens
  {
    const int uexp = 24 - kexp;
#pragma unroll
    for (int n = 0; n < kNB; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[n][i] = __builtin_amdgcn_ldexpf(acc[n][i], uexp);
    for (int i = x_done; i < nxw; ++i) {
      const float part = exact_part(i);
      float vv[kNB];
      exact_values(i, vv);
      fold_score(part, vv);
    }
  }
  // ---- wave result
  stash();
  __syncthreads();
  // ---- merge the waves' states: the weights 2^(m_j - M) once per (head,
  // wave), then the rows (the high and low rows of each head joined);
  // write this split's partial for each head
  __shared__ float s_fac[GQA][kW], s_M[GQA];
  if (threadIdx.x < kW * GQA) {
    const int qh = threadIdx.x / kW, j = threadIdx.x % kW;
    float M = s_m[0][qh];
#pragma unroll
    for (int w = 1; w < kW; ++w) M = __builtin_fmaxf(M, s_m[w][qh]);
    // a split with no tokens at all leaves m = -inf, l = 0, o = 0
    const float Mref = M == -__builtin_inff() ? 0.f : M;
    s_fac[qh][j] = __builtin_amdgcn_exp2f(s_m[j][qh] - Mref);
    if (j == 0) s_M[qh] = M;
  }
  __syncthreads();
  constexpr int kHG = GQA / 4;                     // groups of four heads
  for (int x = threadIdx.x; x < kHG * D; x += kT) {
    const int hg = x / D, d = x % D;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      f32x4_t r = *reinterpret_cast<const f32x4_t*>(&s_o[w][d][4 * hg]);
      if constexpr (DUAL) {
        // rows r, r + 4, r + 8, r + 12: both key groups' high and low rows
        r += *reinterpret_cast<const f32x4_t*>(&s_o[w][d][4]);
        r += *reinterpret_cast<const f32x4_t*>(&s_o[w][d][8]);
        r += *reinterpret_cast<const f32x4_t*>(&s_o[w][d][12]);
      } else {
        r += *reinterpret_cast<const f32x4_t*>(&s_o[w][d][4 * hg + GQA]);   // the low rows
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qh = 4 * hg + i;
        o[i] = __builtin_fmaf(s_fac[qh][w], r[i] + s_z[w][qh], o[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qh = 4 * hg + i;
      const int64_t row = int64_t(b) * a.Hq + h * GQA + qh;
      partial_o(a, row, split, D)[d] = o[i];
      if (d == 0) {
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < kW; ++w) L = __builtin_fmaf(s_fac[qh][w], s_l[w][qh], L);
        *reinterpret_cast<float2*>(partial_ml(a, row, split)) = float2{s_M[qh], L};
      }
    }
  }
}

template <int DT, int D, int BITS, int GQA>
hipError_t launch_attn_mfma(const AttnArgs& a, int B, hipStream_t s) {
  if (a.G == 32)
    hipLaunchKernelGGL((k_attn_mfma<DT, D, BITS, GQA, true>), dim3(a.n_split, a.H, B), dim3(64 * kMfmaWaves), 0, s,
                       a);
  else
    hipLaunchKernelGGL((k_attn_mfma<DT, D, BITS, GQA, false>), dim3(a.n_split, a.H, B), dim3(64 * kMfmaWaves), 0,
                       s, a);
  return hipGetLastError();
}

#define KVQ_INST_MFMA(DT, D)                                                           \
  template hipError_t launch_attn_mfma<DT, D, 2, 4>(const AttnArgs&, int, hipStream_t); \
  template hipError_t launch_attn_mfma<DT, D, 2, 8>(const AttnArgs&, int, hipStream_t); \
  template hipError_t launch_attn_mfma<DT, D, 4, 4>(const AttnArgs&, int, hipStream_t); \
  template hipError_t launch_attn_mfma<DT, D, 4, 8>(const AttnArgs&, int, hipStream_t);
KVQ_INST_MFMA(DT_F32, 64)
KVQ_INST_MFMA(DT_F32, 128)
KVQ_INST_MFMA(DT_F16, 64)
KVQ_INST_MFMA(DT_F16, 128)
KVQ_INST_MFMA(DT_BF16, 64)
KVQ_INST_MFMA(DT_BF16, 128)

}  // namespace kvq
