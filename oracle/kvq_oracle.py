"""CPU oracle for KIVI-style KV-cache quantization and decode attention.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check of the package
entry point and the CPU-baseline leg of the benchmark may import or run this
module.  It shares no code with the HIP library and imports nothing from it:
it is written from the pages' definitions and from the cache layout as the
library's header states it in prose.

Sources (web pages, cited by title and section):
  [KIVI-PR]   sonos/tract PR "KIVI-style KV-cache quantization - packed u8
              storage": "The idea" (keys per channel, values per token),
              "What's in the PR" (per-token value store = D bytes + 2 f32
              params per token; per-channel key store = D bytes per token +
              D x 8 bytes of params; GQA handled; output has Q's shape),
              squashed commit messages (round-trip error <= scale/2, bits
              configurable, memory = bits/16 of an f16 cache).
  [STORE-PR]  sonos/tract PR "quantized KV-cache storage op (int8/int4)":
              PR description (keys per channel in frozen fixed-size blocks,
              values per token) and commit message (first SINK_TOKENS kept in
              f32 in both stores).
  [GUIDE]     pigeon guide page "KV-cache quantization": "How it works"
              steps 1-5 (per-channel keys over G-token groups, per-token
              values, q = round((x - min)/delta), delta = (max - min)/(2^b - 1),
              full-precision residual window of R tokens quantized once a
              group fills, softmax(q K^T / sqrt(d)) V over the dequantized
              cache) and "Source code" (numpy round = half to even, clip).

Readings where the pages are silent (each is listed in the design notes):
  R1 partition: with n = max(0, T - S) tokens past the sinks, the quantized
     count is Q = G * floor((n - R) / G) when n >= R, else 0; tokens
     [S, S+Q) are quantized, [S+Q, T) stay in full precision (between R and
     R+G-1 of them once n >= R), so the most recent R are always exact.
  R2 groups start right after the sinks.
  R3 K and V share the partition.
  R4 rounding is half to even (numpy.rint).
  R5 delta = fl32(fl32(max - min) / (2^b - 1)); code = rint(fl32(fl32(x - zp)
     / delta)), a true IEEE fp32 division.
  R6 max == min gives delta = +0 and every code 0.
  R7 the zero point is the fp32 minimum, stored as mn + 0.0f (so -0 -> +0).
  R8 sink and residual tokens are stored losslessly in the input dtype.
  R9 GQA: q head hq reads KV head hq // (Hq / Hkv).
  R10 default softmax scale 1/sqrt(D); the query attends to every cached token
      (every token of the window when a window is set, W1).
  R11 codes are clamped to [0, 2^b - 1].

Sliding window ([KIVI-PR] "The idea": the quantized store composes with the
sliding-window cache; "Relationship to other PRs": a bounded window cache
with int8 storage), readings:
  W1 with a window of W tokens the decode query attends to the sinks and to
     the last W tokens [max(S, T - W), T); with S = 0 this is plain sliding-
     window attention.  W >= R + G, so the full-precision tokens always lie
     inside the window.
  W2 the store is bounded: quantized token u (token S + u) is kept at
     storage row u mod qcap, with qcap = W + G rounded up to a multiple of
     max(64, G); a group that freezes overwrites the rows of the oldest
     one (eviction).  Tokens before the window inside a live chunk are
     masked, so the window is exact to the token.

Dense-and-sparse outliers ([GUIDE] "KVQuant adds", third bullet: about 1%
of outlier values kept in a sparse fp16 side table), readings:
  O1 the unit is the quantization vector: a key group's channel (G values)
     or a value token (D values).  Each keeps at most one entry exact, so
     1/G of the keys and 1/D of the values (about 1-2% at G 32..128, D 64
     or 128).
  O2 the kept entry is the largest or the smallest, whichever leaves the
     smaller range: with the two largest max1 >= max2 and the two smallest
     min1 <= min2, gap_hi = fl32(max1 - max2) and gap_lo = fl32(min2 -
     min1); the maximum if gap_hi >= gap_lo and gap_hi > 0, else the
     minimum if gap_lo > 0, else none (the range would not shrink).
  O3 delta and the zero point come from the other entries; every entry,
     the kept one too, is coded with them (the kept one clamps to 2^b - 1
     or 0).
  O4 the side table holds the kept entry's position (u8: token offset in
     the group for keys, channel for values; 255 = none) and its value,
     losslessly in the input dtype (fp16 for fp16 inputs, as the page has
     it); with none kept the value slot holds +0.
  O5 reconstruction: the kept entry takes its exact value, every other
     entry its dense dequantization.

Pre-RoPE keys ([GUIDE] "KVQuant adds", first bullet: quantize keys before
the rotary position embedding, which otherwise mixes channel pairs and
smears the per-channel structure), readings:
  P1 the rotation pairs channel i with channel i + D/2 (i < D/2) at
     frequency theta_i = base^(-2i/D): x_i' = x_i cos(p theta_i) -
     x_{i+D/2} sin(p theta_i), x_{i+D/2}' = x_{i+D/2} cos(p theta_i) + x_i
     sin(p theta_i).
  P2 cached token t sits at position p = t (its index in the sequence).
  P3 with a RoPE base set, the cache stores keys as given (before the
     rotation): sinks, residual and quantized alike; the query passed to
     decode is already rotated to its own position; attention rotates each
     (dequantized) key to its position before the dot product.  Values are
     not rotated.

Every function here is pinned by tests/test_oracle_pins.py against worked
examples, closed forms, brute force and library routines.
"""
from __future__ import annotations

import math
import numpy as np

SUPPORTED_BITS = (1, 2, 3, 4, 5, 6, 7, 8)   # [KIVI-PR] commit messages: bits configurable
_F32 = np.float32


# ----------------------------------------------------------------------------
# step 0: input dtype -> fp32 (exact for fp16 and bf16)
# ----------------------------------------------------------------------------
def to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored input values to fp32.  bf16 arrives as uint16 bit
    patterns and becomes the fp32 with those 16 bits on top."""
    if dtype == "f32":
        return np.asarray(x, dtype=_F32)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(_F32)
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(_F32)
    raise ValueError(dtype)


def from_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Narrow fp32 values that the input dtype represents exactly back to
    it (bf16 as uint16 bit patterns: the top 16 bits)."""
    x = np.asarray(x, dtype=_F32)
    if dtype == "f32":
        return x.copy()
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dtype)


def elem_bytes(dtype: str) -> int:
    return {"f32": 4, "f16": 2, "bf16": 2}[dtype]


def storage_np_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


# ----------------------------------------------------------------------------
# step 1: which tokens are sinks, quantized, or full-precision residual (R1)
# ----------------------------------------------------------------------------
def partition(T: int, S: int, R: int, G: int):
    """Returns (n_sink, Q, n_resid) for T cached tokens."""
    n_sink = min(T, S)
    n = max(0, T - S)
    Q = G * ((n - R) // G) if n >= R else 0
    return n_sink, Q, n - Q


def ring_slot(t: int, S: int, R: int, G: int) -> int:
    """Slot of token t (t >= S) in the (R+G)-slot full-precision ring."""
    return (t - S) % (R + G)


# ----------------------------------------------------------------------------
# steps 2-3: the asymmetric affine quantizer ([GUIDE] How it works, step 3)
# ----------------------------------------------------------------------------
def affine_params(mn: np.ndarray, mx: np.ndarray, bits: int):
    """delta = (max - min) / (2^b - 1) and zero point = min, in fp32 (R5, R7);
    delta = +0 when max = min (R6; which of -0 and +0 a min or max returns
    among equal zeros is not fixed, their difference's sign would be)."""
    mn = np.asarray(mn, dtype=_F32)
    mx = np.asarray(mx, dtype=_F32)
    delta = (mx - mn) / _F32(2 ** bits - 1)
    delta = np.where(mx == mn, _F32(0.0), delta)
    zp = mn + _F32(0.0)
    return delta.astype(_F32), zp.astype(_F32)


def affine_codes(x: np.ndarray, delta: np.ndarray, zp: np.ndarray, bits: int) -> np.ndarray:
    """code = clamp(round_half_even((x - zp) / delta), 0, 2^b - 1); delta == 0
    gives code 0 (R4, R5, R6, R11)."""
    x = np.asarray(x, dtype=_F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = (x - zp) / delta
    r = np.rint(quot)
    r = np.clip(r, _F32(0), _F32(2 ** bits - 1))
    r = np.where(delta == 0, _F32(0), r)
    return r.astype(np.uint8)


def split_outlier(v: np.ndarray):
    """Dense-and-sparse split of vectors along the last axis (O1, O2).
    v: [..., m] fp32, m >= 2.  Returns (pos, mn, mx): the position of the
    entry kept exact ([...] int64, -1 = none) and the minimum and maximum
    of the remaining (dense) entries."""
    v = np.asarray(v, dtype=_F32)
    s = np.sort(v, axis=-1)
    min1, min2, max2, max1 = s[..., 0], s[..., 1], s[..., -2], s[..., -1]
    gap_hi = (max1 - max2).astype(_F32)
    gap_lo = (min2 - min1).astype(_F32)
    take_hi = (gap_hi >= gap_lo) & (gap_hi > 0)
    take_lo = ~take_hi & (gap_lo > 0)
    # the kept extreme is unique (its gap is positive)
    pos = np.where(take_hi, np.argmax(v, axis=-1), np.where(take_lo, np.argmin(v, axis=-1), -1))
    mn = np.where(take_lo, min2, min1).astype(_F32)
    mx = np.where(take_hi, max2, max1).astype(_F32)
    return pos.astype(np.int64), mn, mx


def quantize_keys_per_channel(K: np.ndarray, G: int, bits: int, outliers: bool = False):
    """Keys per channel over G-token groups ([GUIDE] step 1; [STORE-PR] frozen
    fixed-size blocks).  K: [..., n, D] fp32 with n a multiple of G.
    Returns codes [..., n, D], delta and zp [..., n/G, D]; with outliers
    also the kept entry's token offset in its group [..., n/G, D] (-1 =
    none, O1-O3)."""
    *lead, n, D = K.shape
    assert n % G == 0
    Kg = K.reshape(*lead, n // G, G, D)
    if outliers:
        pos, mn, mx = split_outlier(np.swapaxes(Kg, -1, -2))
    else:
        mn = Kg.min(axis=-2)
        mx = Kg.max(axis=-2)
    delta, zp = affine_params(mn, mx, bits)
    codes = affine_codes(Kg, delta[..., None, :], zp[..., None, :], bits)
    if outliers:
        return codes.reshape(*lead, n, D), delta, zp, pos
    return codes.reshape(*lead, n, D), delta, zp


def quantize_values_per_token(V: np.ndarray, bits: int, outliers: bool = False):
    """Values per token ([GUIDE] step 2; [KIVI-PR] per-token value store).
    V: [..., n, D] fp32.  Returns codes [..., n, D], delta and zp [..., n];
    with outliers also the kept entry's channel [..., n] (-1 = none)."""
    if outliers:
        pos, mn, mx = split_outlier(V)
    else:
        mn = V.min(axis=-1)
        mx = V.max(axis=-1)
    delta, zp = affine_params(mn, mx, bits)
    codes = affine_codes(V, delta[..., None], zp[..., None], bits)
    if outliers:
        return codes, delta, zp, pos
    return codes, delta, zp


# ----------------------------------------------------------------------------
# step 4: packed byte layouts (the library header states them in prose)
# ----------------------------------------------------------------------------
def pack_bits(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack the last axis of `codes` (m codes, m * bits a multiple of 8) into
    m * bits / 8 bytes: code i at bit offset i * bits, low bits first.  At
    3, 5, 6 and 7 bits a code may straddle two bytes (its low bits end one
    byte, its high bits start the next)."""
    *lead, m = codes.shape
    assert (m * bits) % 8 == 0
    if 8 % bits == 0:                       # whole codes per byte
        per = 8 // bits
        c = codes.astype(np.uint8).reshape(*lead, m // per, per)
        out = np.zeros((*lead, m // per), dtype=np.uint8)
        for i in range(per):
            out |= (c[..., i] << np.uint8(bits * i)).astype(np.uint8)
        return out
    c = codes.astype(np.uint16)
    out = np.zeros((*lead, m * bits // 8), dtype=np.uint16)
    for i in range(m):
        byte, sh = divmod(i * bits, 8)
        v = c[..., i] << np.uint16(sh)
        out[..., byte] |= v & np.uint16(0xFF)
        if sh + bits > 8:
            out[..., byte + 1] |= v >> np.uint16(8)
    return out.astype(np.uint8)


def unpack_bits(packed: np.ndarray, bits: int, m: int) -> np.ndarray:
    """Inverse of pack_bits: [..., m * bits / 8] bytes -> [..., m] codes."""
    *lead, nb = packed.shape
    mask = 2 ** bits - 1
    if 8 % bits == 0:
        per = 8 // bits
        out = np.zeros((*lead, nb, per), dtype=np.uint8)
        for i in range(per):
            out[..., i] = (packed >> np.uint8(bits * i)) & np.uint8(mask)
        return out.reshape(*lead, m)
    p = packed.astype(np.uint16)
    out = np.zeros((*lead, m), dtype=np.uint8)
    for i in range(m):
        byte, sh = divmod(i * bits, 8)
        v = p[..., byte] >> np.uint16(sh)
        if sh + bits > 8:
            v = v | (p[..., byte + 1] << np.uint16(8 - sh))
        out[..., i] = (v & np.uint16(mask)).astype(np.uint8)
    return out


def pack_key_rows(codes: np.ndarray, bits: int) -> np.ndarray:
    """Key codes are token-major: row u holds D codes in D*b/8 bytes, channel
    d at bit offset d*b of the row, low bits first."""
    return pack_bits(codes, bits)


def unpack_key_rows(packed: np.ndarray, bits: int, D: int) -> np.ndarray:
    return unpack_bits(packed, bits, D)


def value_block_tokens(bits: int) -> int:
    """Tokens per value-code block: 64 at 2 bits, 32 at every other width."""
    return 64 if bits == 2 else 32


def value_unit_codes(bits: int) -> int:
    """Codes of one channel held in one unit: 16 at 2 bits (a 32-bit unit),
    8 at every other width (a unit of b bytes: 32 bits at 4, 64 at 8)."""
    return 16 if bits == 2 else 8


def value_code_location(u: int, d: int, bits: int, D: int):
    """(byte offset, bit shift) of value code (token u, channel d) inside one
    head's value-code array, straight from the layout's definition:

    * tokens are cut into blocks of L tokens (L = 64 at 2 bits, else 32);
    * inside a block, token offset o splits as o = 32*s + 16*h + 4*g + r with
      s in [0, L/32), h in {0, 1}, g in [0, 4), r in [0, 4);
    * one unit holds the codes of one channel for the tokens sharing (g);
      units are ordered in the block by g, then j = d % 16, then n = d // 16:
      unit index = (g*16 + j) * (D/16) + n, units of U*b/8 bytes;
    * inside the unit, the token (s, h, r) is code slot i = r + 4*s + (U/2)*h,
      slot i at bit offset i*b, low bits first.
    """
    L = value_block_tokens(bits)
    U = value_unit_codes(bits)
    unit_bytes = U * bits // 8
    blk, o = divmod(u, L)
    s, rem = divmod(o, 32)
    h, rem = divmod(rem, 16)
    g, r = divmod(rem, 4)
    j, n = d % 16, d // 16
    unit = blk * 4 * D + (g * 16 + j) * (D // 16) + n
    i = r + 4 * s + (U // 2) * h
    byte = unit * unit_bytes + (i * bits) // 8
    return byte, (i * bits) % 8


def value_codes_bytes(n_tokens_cap: int, bits: int, D: int) -> int:
    L = value_block_tokens(bits)
    nblk = -(-n_tokens_cap // L)
    return nblk * L * D * bits // 8


def pack_value_codes_loop(codes: np.ndarray, bits: int) -> np.ndarray:
    """Slow, literal form of the value layout for small cases.
    codes: [n, D] -> bytes [value_codes_bytes(n)]."""
    n, D = codes.shape
    out = np.zeros(value_codes_bytes(n, bits, D), dtype=np.uint8)
    for u in range(n):
        for d in range(D):
            byte, sh = value_code_location(u, d, bits, D)
            v = int(codes[u, d]) << sh
            out[byte] |= np.uint8(v & 0xFF)
            if sh + bits > 8:                 # a code straddling two bytes
                out[byte + 1] |= np.uint8(v >> 8)
    return out


def _value_perm_axes(bits: int):
    # codes[u, d] viewed as [blk, s, h, g, r, n, j] -> [blk, g, j, n, h, s, r]
    return (0, 3, 6, 5, 2, 1, 4)


def pack_value_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Vectorized value layout.  codes: [..., n, D] -> [..., bytes]; tokens
    past n (a partial last block) are packed as code 0 and are not part of
    the cache contents."""
    *lead, n, D = codes.shape
    L = value_block_tokens(bits)
    nblk = -(-n // L)
    c = np.zeros((*lead, nblk * L, D), dtype=np.uint8)
    c[..., :n, :] = codes
    S_ = L // 32
    c = c.reshape(*lead, nblk, S_, 2, 4, 4, D // 16, 16)
    nl = len(lead)
    axes = tuple(range(nl)) + tuple(nl + a for a in _value_perm_axes(bits))
    c = np.transpose(c, axes)  # [..., blk, g, j, n, h, s, r] -> slot i = r + 4s + (U/2)h
    U = value_unit_codes(bits)
    c = c.reshape(*lead, nblk * 4 * D, U)
    out = pack_bits(c, bits)                # units of U * b / 8 bytes
    return out.reshape(*lead, nblk * 4 * D * U * bits // 8)


def unpack_value_codes(packed: np.ndarray, bits: int, D: int, n: int) -> np.ndarray:
    """Inverse of pack_value_codes: [..., bytes] -> codes [..., n, D]."""
    *lead, nbytes = packed.shape
    L = value_block_tokens(bits)
    U = value_unit_codes(bits)
    nblk = nbytes // (L * D * bits // 8)
    p = packed.reshape(*lead, nblk * 4 * D, U * bits // 8)
    c = unpack_bits(p, bits, U)
    S_ = L // 32
    c = c.reshape(*lead, nblk, 4, 16, D // 16, 2, S_, 4)   # [blk, g, j, n, h, s, r]
    nl = len(lead)
    inv = np.argsort(_value_perm_axes(bits))
    axes = tuple(range(nl)) + tuple(nl + int(a) for a in inv)
    c = np.transpose(c, axes)  # back to [blk, s, h, g, r, n, j]
    return c.reshape(*lead, nblk * L, D)[..., :n, :]


def value_valid_byte_mask(n_valid: int, n_cap: int, bits: int, D: int) -> np.ndarray:
    """Bytes of a head's value-code array that hold codes of tokens < n_valid."""
    ones = np.zeros((n_cap, D), dtype=np.uint8)
    ones[:n_valid] = 2 ** bits - 1
    return pack_value_codes(ones, bits) != 0


# ----------------------------------------------------------------------------
# the cache state, in the library's buffer layout
# ----------------------------------------------------------------------------
class CacheGeometry:
    """Sizes of every cache buffer for a configuration.  The quantized-token
    capacity is cap - S (at most W + G with a window, W2) rounded up to a
    multiple of max(64, G)."""

    def __init__(self, B, Hkv, D, bits, G, S, R, capacity, dtype, window=0, outliers=0,
                 rope_base=0.0):
        assert bits in SUPPORTED_BITS
        assert window == 0 or window >= R + G
        assert outliers in (0, 1)
        self.B, self.Hkv, self.D, self.bits = B, Hkv, D, bits
        self.G, self.S, self.R, self.capacity, self.dtype = G, S, R, capacity, dtype
        self.window = window
        self.outliers = outliers
        assert rope_base >= 0
        self.rope_base = float(rope_base)
        step = max(64, G)
        qcap = max(0, capacity - S)
        if window:
            qcap = min(qcap, window + G)
        self.qcap = -(-qcap // step) * step
        self.ring = R + G
        self.k_row_bytes = D * bits // 8
        self.v_head_bytes = value_codes_bytes(self.qcap, bits, D)

    def empty_state(self):
        B, H, D = self.B, self.Hkv, self.D
        sd = storage_np_dtype(self.dtype)
        return {
            "k_codes": np.zeros((B, H, self.qcap, self.k_row_bytes), np.uint8),
            "v_codes": np.zeros((B, H, self.v_head_bytes), np.uint8),
            "k_scale": np.zeros((B, H, self.qcap // self.G, D), _F32),
            "k_zero": np.zeros((B, H, self.qcap // self.G, D), _F32),
            "v_scale": np.zeros((B, H, self.qcap), _F32),
            "v_zero": np.zeros((B, H, self.qcap), _F32),
            "k_sink": np.zeros((B, H, self.S, D), sd),
            "v_sink": np.zeros((B, H, self.S, D), sd),
            "k_resid": np.zeros((B, H, self.ring, D), sd),
            "v_resid": np.zeros((B, H, self.ring, D), sd),
            # side tables (O4), empty without outliers
            "k_oidx": np.zeros((B, H, self.qcap // self.G if self.outliers else 0, D), np.uint8),
            "k_oval": np.zeros((B, H, self.qcap // self.G if self.outliers else 0, D), sd),
            "v_oidx": np.zeros((B, H, self.qcap if self.outliers else 0), np.uint8),
            "v_oval": np.zeros((B, H, self.qcap if self.outliers else 0), sd),
        }


def _store_groups(geo: CacheGeometry, st: dict, u0: int, Kq: np.ndarray, Vq: np.ndarray):
    """Quantize tokens [S+u0, S+u0+n) (fp32 [B, H, n, D], n a multiple of G,
    u0 a multiple of G) into the state's code and parameter arrays, at
    storage rows u mod qcap (W2).  Groups are stored in token order, so a
    group that wraps the ring overwrites the oldest ones."""
    n = Kq.shape[2]
    if n == 0:
        return
    if u0 + n > geo.qcap or u0 >= geo.qcap:
        for k in range(n // geo.G):
            sl = slice(k * geo.G, (k + 1) * geo.G)
            _store_groups_at(geo, st, (u0 + k * geo.G) % geo.qcap, Kq[:, :, sl], Vq[:, :, sl])
        return
    _store_groups_at(geo, st, u0, Kq, Vq)


def _store_groups_at(geo: CacheGeometry, st: dict, r0: int, Kq: np.ndarray, Vq: np.ndarray):
    """Quantize n tokens (fp32 [B, H, n, D]) into storage rows r0 .. r0 + n
    (n and r0 multiples of G, no wrap)."""
    n = Kq.shape[2]
    b = geo.bits
    if geo.outliers:
        kc, kd, kz, kpos = quantize_keys_per_channel(Kq, geo.G, b, outliers=True)
        vc, vd, vz, vpos = quantize_values_per_token(Vq, b, outliers=True)
        # side tables (O4): position (255 = none) and the exact value
        g0, g1 = r0 // geo.G, (r0 + n) // geo.G
        Kg = Kq.reshape(geo.B, geo.Hkv, n // geo.G, geo.G, geo.D)
        kval = np.take_along_axis(Kg, np.maximum(kpos, 0)[..., None, :], axis=-2)[..., 0, :]
        st["k_oidx"][:, :, g0:g1] = np.where(kpos < 0, 255, kpos).astype(np.uint8)
        st["k_oval"][:, :, g0:g1] = from_f32(np.where(kpos < 0, _F32(0), kval), geo.dtype)
        vval = np.take_along_axis(Vq, np.maximum(vpos, 0)[..., None], axis=-1)[..., 0]
        st["v_oidx"][:, :, r0:r0 + n] = np.where(vpos < 0, 255, vpos).astype(np.uint8)
        st["v_oval"][:, :, r0:r0 + n] = from_f32(np.where(vpos < 0, _F32(0), vval), geo.dtype)
    else:
        kc, kd, kz = quantize_keys_per_channel(Kq, geo.G, b)
        vc, vd, vz = quantize_values_per_token(Vq, b)
    st["k_codes"][:, :, r0:r0 + n] = pack_key_rows(kc, b)
    st["k_scale"][:, :, r0 // geo.G:(r0 + n) // geo.G] = kd
    st["k_zero"][:, :, r0 // geo.G:(r0 + n) // geo.G] = kz
    st["v_scale"][:, :, r0:r0 + n] = vd
    st["v_zero"][:, :, r0:r0 + n] = vz
    # value codes: write only the bytes that belong to tokens [r0, r0+n).
    # Blocks are independent runs of bytes, so work on the covered blocks.
    L = value_block_tokens(b)
    blk0, blk1 = r0 // L, -(-(r0 + n) // L)
    span = (blk1 - blk0) * L
    part = np.zeros((geo.B, geo.Hkv, span, geo.D), np.uint8)
    part[:, :, r0 - blk0 * L:r0 - blk0 * L + n] = vc
    packed = pack_value_codes(part, b)
    touched = np.zeros((span, geo.D), np.uint8)
    touched[r0 - blk0 * L:r0 - blk0 * L + n] = 1
    tmask = pack_value_codes(touched, b) != 0      # bytes holding these tokens
    # a byte only ever holds tokens of one 32-token step, and a step lies in
    # one G-group (G is a multiple of 32), so whole bytes move.
    blk_bytes = L * geo.D * b // 8
    dst = st["v_codes"][:, :, blk0 * blk_bytes:blk1 * blk_bytes]
    dst[:, :, tmask] = packed[:, :, tmask]


def storage_row(geo: CacheGeometry, u):
    """Storage row of quantized token u (token S + u), W2."""
    return u % geo.qcap if geo.qcap else u


def prefill(geo: CacheGeometry, K: np.ndarray, V: np.ndarray, T: int) -> dict:
    """Cache state after loading T tokens at once (K, V in storage dtype,
    [B, H, >=T, D])."""
    st = geo.empty_state()
    ns, Q, nr = partition(T, geo.S, geo.R, geo.G)
    st["k_sink"][:, :, :ns] = K[:, :, :ns]
    st["v_sink"][:, :, :ns] = V[:, :, :ns]
    Kf = to_f32(K[:, :, geo.S:geo.S + Q], geo.dtype)
    Vf = to_f32(V[:, :, geo.S:geo.S + Q], geo.dtype)
    _store_groups(geo, st, 0, Kf, Vf)
    for t in range(geo.S + Q, T):
        sl = ring_slot(t, geo.S, geo.R, geo.G)
        st["k_resid"][:, :, sl] = K[:, :, t]
        st["v_resid"][:, :, sl] = V[:, :, t]
    return st


def append(geo: CacheGeometry, st: dict, n_before: int, k_new: np.ndarray,
           v_new: np.ndarray) -> dict:
    """Streaming append of token t = n_before ([B, H, D] in storage dtype).
    The token goes to its sink or ring slot; when the full-precision count
    reaches R + G the oldest G ring tokens are quantized as the next group
    and frozen ([STORE-PR] frozen blocks; [GUIDE] step 4)."""
    t = n_before
    if t < geo.S:
        st["k_sink"][:, :, t] = k_new
        st["v_sink"][:, :, t] = v_new
    else:
        sl = ring_slot(t, geo.S, geo.R, geo.G)
        st["k_resid"][:, :, sl] = k_new
        st["v_resid"][:, :, sl] = v_new
    _, q_old, _ = partition(t, geo.S, geo.R, geo.G)
    _, q_new, _ = partition(t + 1, geo.S, geo.R, geo.G)
    if q_new > q_old:
        assert q_new - q_old == geo.G
        toks = [geo.S + q_old + i for i in range(geo.G)]
        slots = [ring_slot(x, geo.S, geo.R, geo.G) for x in toks]
        Kf = to_f32(st["k_resid"][:, :, slots], geo.dtype)
        Vf = to_f32(st["v_resid"][:, :, slots], geo.dtype)
        _store_groups(geo, st, q_old, Kf, Vf)
    return st


def valid_masks(geo: CacheGeometry, T: int) -> dict:
    """Which parts of each buffer hold cache contents after T tokens: the
    sinks, the ring slots of the full-precision tokens, and the storage rows
    of the last min(Q, qcap) quantized tokens (all Q without a window)."""
    ns, Q, nr = partition(T, geo.S, geo.R, geo.G)
    ring = np.zeros(geo.ring, bool)
    for t in range(geo.S + Q, T):
        ring[ring_slot(t, geo.S, geo.R, geo.G)] = True
    rows = np.zeros(geo.qcap, bool)
    for u in range(max(0, Q - geo.qcap), Q):
        rows[storage_row(geo, u)] = True
    ones = np.zeros((geo.qcap, geo.D), np.uint8)
    ones[rows] = 2 ** geo.bits - 1
    groups = rows.reshape(-1, geo.G).all(axis=1) if geo.qcap else np.zeros(0, bool)
    return {
        "n_sink": ns, "Q": Q, "ring": ring, "rows": rows, "groups": groups,
        "v_bytes": pack_value_codes(ones, geo.bits) != 0,
    }


def window_start(geo: CacheGeometry, T: int) -> int:
    """First quantized token u the decode query attends to (W1): tokens
    before max(S, T - W) are outside the window."""
    if not geo.window:
        return 0
    return max(0, T - geo.window - geo.S)


# ----------------------------------------------------------------------------
# rotary position embedding of the keys (P1-P3)
# ----------------------------------------------------------------------------
def rope_angles(positions, D: int, base: float) -> np.ndarray:
    """Angles p * theta_i, theta_i = base^(-2i/D), fp64 [n, D/2] (P1)."""
    i = np.arange(D // 2, dtype=np.float64)
    theta = np.power(np.float64(base), -2.0 * i / D)
    return np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]


def apply_rope(x: np.ndarray, positions, base: float) -> np.ndarray:
    """Rotate x [..., n, D] (fp64) token by token to its position (P1)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = rope_angles(positions, D, base)
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :D // 2], x[..., D // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def attended_positions(geo: CacheGeometry, T: int) -> np.ndarray:
    """Positions (token indices, P2) of the tokens dequant_cache returns,
    in its order: the sinks, the attended quantized tokens, the residual
    tokens."""
    ns, Q, nr = partition(T, geo.S, geo.R, geo.G)
    u_lo = window_start(geo, T)
    return np.concatenate([np.arange(ns), geo.S + np.arange(u_lo, Q), np.arange(geo.S + Q, T)])


# ----------------------------------------------------------------------------
# step 5: dequantize in fp64 ([GUIDE] step 5: dequantized group by group)
# ----------------------------------------------------------------------------
def dequant_cache(geo: CacheGeometry, st: dict, T: int, heads=None):
    """K_hat, V_hat in fp64, [B, len(heads), n, D], of the n tokens the decode
    query attends to, in token order: all T without a window; the sinks and
    the last W tokens with one (W1)."""
    heads = range(geo.Hkv) if heads is None else heads
    heads = list(heads)
    ns, Q, nr = partition(T, geo.S, geo.R, geo.G)
    u_lo = window_start(geo, T)
    nq = max(0, Q - u_lo)
    n = ns + nq + nr
    B, D = geo.B, geo.D
    Kh = np.zeros((B, len(heads), n, D), np.float64)
    Vh = np.zeros((B, len(heads), n, D), np.float64)
    rows = storage_row(geo, np.arange(u_lo, Q))
    for i, h in enumerate(heads):
        Kh[:, i, :ns] = to_f32(st["k_sink"][:, h, :ns], geo.dtype)
        Vh[:, i, :ns] = to_f32(st["v_sink"][:, h, :ns], geo.dtype)
        if nq:
            kc = unpack_key_rows(st["k_codes"][:, h][:, rows], geo.bits, D).astype(np.float64)
            kd = st["k_scale"][:, h][:, rows // geo.G].astype(np.float64)
            kz = st["k_zero"][:, h][:, rows // geo.G].astype(np.float64)
            Kh[:, i, ns:ns + nq] = kc * kd + kz
            vc_all = unpack_value_codes(st["v_codes"][:, h], geo.bits, D, geo.qcap)
            vc = vc_all[:, rows].astype(np.float64)
            vd = st["v_scale"][:, h][:, rows].astype(np.float64)[..., None]
            vz = st["v_zero"][:, h][:, rows].astype(np.float64)[..., None]
            Vh[:, i, ns:ns + nq] = vc * vd + vz
            if geo.outliers:
                # kept entries take their exact values (O5)
                ki = st["k_oidx"][:, h][:, rows // geo.G]                      # [B, nq, D]
                kv = to_f32(st["k_oval"][:, h][:, rows // geo.G], geo.dtype)
                kmask = ki == (rows % geo.G)[None, :, None]
                Kh[:, i, ns:ns + nq] = np.where(kmask, kv, Kh[:, i, ns:ns + nq])
                vi = st["v_oidx"][:, h][:, rows]                               # [B, nq]
                vv = to_f32(st["v_oval"][:, h][:, rows], geo.dtype)
                vmask = np.arange(D)[None, None, :] == vi[..., None]
                Vh[:, i, ns:ns + nq] = np.where(vmask, vv[..., None], Vh[:, i, ns:ns + nq])
        for j, t in enumerate(range(geo.S + Q, T)):
            sl = ring_slot(t, geo.S, geo.R, geo.G)
            Kh[:, i, ns + nq + j] = to_f32(st["k_resid"][:, h, sl], geo.dtype)
            Vh[:, i, ns + nq + j] = to_f32(st["v_resid"][:, h, sl], geo.dtype)
    return Kh, Vh


# ----------------------------------------------------------------------------
# step 6: attention in fp64 ([GUIDE] step 5; [KIVI-PR] GQA handled)
# ----------------------------------------------------------------------------
def attention(q: np.ndarray, Kh: np.ndarray, Vh: np.ndarray, scale: float | None = None):
    """softmax(scale * q K^T) V per (batch, q head), fp64.
    q [B, Hq, D] (any float), Kh/Vh [B, Hkv, T, D] fp64.  Head hq reads
    KV head hq // (Hq / Hkv) (R9).  Returns [B, Hq, D] fp64."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = Kh.shape[1]
    g = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = np.zeros((B, Hq, D), np.float64)
    for b in range(B):
        for hq in range(Hq):
            kv = hq // g
            s = sc * (Kh[b, kv] @ q[b, hq])
            m = s.max()
            p = np.exp(s - m)
            out[b, hq] = (p @ Vh[b, kv]) / p.sum()
    return out


def decode(geo: CacheGeometry, st: dict, T: int, q_stored: np.ndarray,
           n_q_heads: int, scale: float | None = None, rows=None):
    """Decode attention of q (storage dtype [B, Hq, D]) over the T cached
    tokens, through the dequantized cache.  `rows` optionally restricts the
    computation to a list of (b, hq) pairs (others left as NaN)."""
    q = to_f32(q_stored, geo.dtype).astype(np.float64)
    B, Hq, D = q.shape
    g = Hq // geo.Hkv
    if rows is None:
        Kh, Vh = dequant_cache(geo, st, T)
        if geo.rope_base:
            Kh = apply_rope(Kh, attended_positions(geo, T), geo.rope_base)
        return attention(q, Kh, Vh, scale)
    out = np.full((B, Hq, D), np.nan)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    by_head = {}
    for (b, hq) in rows:
        by_head.setdefault(hq // g, []).append((b, hq))
    for kv, lst in by_head.items():
        Kh, Vh = dequant_cache(geo, st, T, heads=[kv])
        if geo.rope_base:
            Kh = apply_rope(Kh, attended_positions(geo, T), geo.rope_base)
        for (b, hq) in lst:
            s = sc * (Kh[b, 0] @ q[b, hq])
            p = np.exp(s - s.max())
            out[b, hq] = (p @ Vh[b, 0]) / p.sum()
    return out


def row_rel_error(o: np.ndarray, ref: np.ndarray) -> float:
    """Max over (b, hq) rows of max_d |o - ref| / max_d |ref| (R12)."""
    o = np.asarray(o, np.float64).reshape(-1, o.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    num = np.abs(o - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    return float((num / den).max())
