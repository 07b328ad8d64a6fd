"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bar: packed codes, scales, zero points and the exact sink / residual
copies bit-exact; decode attention within 2e-3 max-abs-relative error per
output row (max_d |o - ref| / max_d |ref|, against fp64 attention over the
oracle's dequantized cache).
"""
import numpy as np
import pytest
import torch

from oracle import kvq_oracle as O
from kivi_quantized_kv_amd import synth
from tests.gpu_util import compare_state, log, make, read_state, to_dev

pytestmark = pytest.mark.gpu

ATOL_ROW_REL = 2e-3


def _kvq():
    from kivi_quantized_kv_amd import kvq
    kvq.load_library()
    return kvq


def _run_prefill(kvq, cfg, data, T):
    cache = kvq.Cache(cfg)
    K = to_dev(data["K"], cfg.dtype)
    V = to_dev(data["V"], cfg.dtype)
    kvq.kvq_quantize_keys(cfg, cache, K, T)
    kvq.kvq_quantize_values(cfg, cache, V, T)
    torch.cuda.synchronize()
    return cache


def _cfg_kw(B, H, D, bits, G, S, R, cap, dtype, window=0, outliers=0):
    return dict(batch=B, n_kv_heads=H, head_dim=D, bits=bits, group=G, sink=S, residual=R,
                capacity=cap, dtype=dtype, window=window, outliers=outliers)


# ----------------------------------------------------------------- small cases
SMALL = [
    # B, Hq, Hkv, D, bits, G, S, R, T, dtype
    (1, 1, 1, 64, 4, 32, 4, 32, 256, "f32"),
    (2, 4, 2, 64, 2, 32, 0, 0, 333, "f16"),
    (1, 8, 1, 128, 8, 64, 3, 64, 517, "bf16"),
    (3, 6, 3, 128, 4, 128, 1, 0, 700, "f16"),
    (1, 4, 4, 64, 8, 32, 0, 32, 95, "bf16"),
    (2, 16, 2, 128, 2, 64, 4, 128, 1100, "bf16"),
    (1, 2, 1, 64, 4, 32, 7, 96, 96, "f32"),        # all full precision
    (1, 32, 8, 128, 4, 32, 4, 128, 2048, "bf16"),
    (1, 16, 4, 128, 2, 32, 4, 128, 2080, "bf16"),
    (2, 2, 2, 64, 2, 32, 2, 32, 98, "f32"),        # 2-bit with a half value block
    # matrix-core path: GQA 4 / 8, 2 / 4 bits, D 64 / 128, G 32 / 64 / 128,
    # chunks of 64 tokens with a half chunk at the end
    (1, 8, 1, 64, 4, 32, 4, 32, 1000, "f16"),
    (2, 16, 4, 64, 2, 64, 1, 64, 1377, "bf16"),
    (1, 8, 2, 128, 4, 128, 0, 0, 1000, "f32"),
    (1, 4, 1, 128, 2, 128, 3, 128, 2999, "f16"),
    (3, 24, 3, 128, 4, 64, 4, 128, 4100, "bf16"),
    (1, 32, 4, 128, 2, 32, 4, 32, 580, "bf16"),     # Q % 64 == 32: a half chunk
    (2, 16, 2, 64, 4, 32, 4, 32, 644, "f16"),       # half chunk, GQA 8
    (1, 8, 1, 128, 2, 32, 0, 64, 480, "bf16"),      # half chunk, GQA 8, 2-bit
    # 64 waves per KV head on a 256-CU part, 129 chunks: the wave with the
    # half chunk has three chunks (the half one on the first register set)
    (4, 32, 8, 128, 4, 32, 4, 32, 8260, "bf16"),
    # GQA 4 with 32-token key groups at D 64, 4-bit: the dual-group form
    # (both key groups of a chunk in one weight pass), several chunks per wave
    (4, 32, 8, 64, 4, 32, 4, 32, 10000, "f16"),
    (1, 64, 8, 128, 4, 64, 4, 128, 70000, "bf16"),
    # GQA 4 / 8 with nothing quantized yet (the VALU kernel takes these)
    (1, 8, 1, 128, 4, 64, 4, 128, 150, "bf16"),
    (2, 8, 2, 64, 2, 32, 2, 32, 50, "f16"),
    # VALU kernel, one 16-wave workgroup per (batch, q head) row when the
    # rows fill a 256-CU part: D 64 (every width), D 128 4-bit fp16, and a
    # cache with no quantized tokens yet
    (16, 16, 16, 64, 2, 32, 4, 32, 300, "f32"),
    (8, 32, 32, 128, 4, 32, 4, 128, 700, "f16"),
    (4, 64, 32, 64, 8, 64, 3, 64, 260, "bf16"),
    (16, 16, 16, 64, 4, 32, 4, 32, 40, "f16"),
    # widths whose codes straddle bytes, and 1 bit (VALU kernel, codes read
    # as a bit stream): D 64 quarter rows of 2b bytes, D 128 of 4b bytes;
    # GQA 4 / 8 at these widths stays on the VALU kernel
    (1, 4, 2, 64, 3, 32, 4, 32, 333, "f16"),
    (2, 8, 2, 128, 5, 64, 2, 64, 517, "bf16"),
    (1, 8, 1, 64, 6, 32, 0, 0, 700, "f32"),
    (1, 2, 1, 128, 7, 128, 3, 128, 1111, "f16"),
    (2, 2, 2, 64, 1, 32, 4, 32, 290, "bf16"),
    (1, 32, 8, 128, 3, 32, 4, 128, 2080, "bf16"),
    (1, 16, 2, 128, 1, 64, 4, 128, 1500, "f16"),
    (16, 16, 16, 64, 5, 32, 4, 32, 300, "f16"),     # one 16-wave workgroup per row
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_small_prefill_and_attention(case):
    kvq = _kvq()
    B, Hq, Hkv, D, bits, G, S, R, T, dt = case
    log("case", case)
    data = synth.random_case(sum(case[:9]), B, Hq, Hkv, D, T, dt)
    cfg, geo = make(_cfg_kw(B, Hkv, D, bits, G, S, R, T + 8, dt))
    cache = _run_prefill(kvq, cfg, data, T)
    ref = O.prefill(geo, data["K"], data["V"], T)
    compare_state(geo, read_state(cache), ref, T)
    q = to_dev(data["q"], dt)
    out = kvq.kvq_decode_attention(cfg, cache, T, q).cpu().numpy()
    exp = O.decode(geo, ref, T, data["q"], Hq)
    err = O.row_rel_error(out, exp)
    log("row rel err", err)
    assert err <= ATOL_ROW_REL


@pytest.mark.parametrize("T", [1, 2, 4, 5, 36, 67, 68, 69, 100, 131])
def test_short_caches(T):
    """Sinks only, all full precision, and the first group freezes."""
    kvq = _kvq()
    log("T", T)
    B, Hq, Hkv, D, G, S, R = 1, 4, 2, 64, 32, 4, 32
    data = synth.random_case(T, B, Hq, Hkv, D, T, "f16")
    cfg, geo = make(_cfg_kw(B, Hkv, D, 4, G, S, R, 200, "f16"))
    cache = _run_prefill(kvq, cfg, data, T)
    ref = O.prefill(geo, data["K"], data["V"], T)
    compare_state(geo, read_state(cache), ref, T)
    out = kvq.kvq_decode_attention(cfg, cache, T, to_dev(data["q"], "f16")).cpu().numpy()
    assert O.row_rel_error(out, O.decode(geo, ref, T, data["q"], Hq)) <= ATOL_ROW_REL
    if T == 1:   # one token: the output is that token's value
        v = data["V"][:, :, 0].astype(np.float32)
        assert np.abs(out - np.repeat(v, Hq // Hkv, axis=1)).max() < 1e-6


@pytest.mark.parametrize("bits", list(range(1, 9)))
def test_constructed_edge_values(bits):
    """Ties at half steps, all-equal groups and tokens, -0.0, groups of
    zeros of both signs, fp32 subnormal ranges, large magnitudes: every code
    and parameter bit-exact."""
    kvq = _kvq()
    log("bits", bits)
    rng = np.random.default_rng(bits)
    B, H, D, G, S, R = 1, 2, 64, 32, 2, 0
    T = S + 8 * G
    L = 2 ** bits - 1
    step = np.float32(2.0 ** -6)
    K = np.zeros((B, H, T, D), np.float32)
    V = np.zeros((B, H, T, D), np.float32)
    for h in range(H):
        for k in range(8):
            rows = slice(S + k * G, S + (k + 1) * G)
            if k == 0:    # ties: (c + 1/2) * step between a 0 and an L * step endpoint
                c = rng.integers(0, L, size=(G, D)).astype(np.float32) + np.float32(0.5)
                c[0] = 0
                c[1] = L
                K[0, h, rows] = c * step
                V[0, h, rows] = c * step
            elif k == 1:  # all equal
                K[0, h, rows] = np.float32(-3.25)
                V[0, h, rows] = np.float32(1.5)
            elif k == 2:  # negative zero minimum
                K[0, h, rows] = rng.uniform(0, 1, size=(G, D)).astype(np.float32)
                K[0, h, S + k * G] = np.float32(-0.0)
                V[0, h, rows] = rng.uniform(0, 1, size=(G, D)).astype(np.float32)
                V[0, h, rows, 0] = np.float32(-0.0)
            elif k == 3:  # subnormal ranges
                K[0, h, rows] = rng.integers(0, 40, size=(G, D)).astype(np.float32) * np.float32(2.0 ** -149)
                V[0, h, rows] = rng.integers(0, 40, size=(G, D)).astype(np.float32) * np.float32(2.0 ** -149)
            elif k == 4:  # large magnitudes
                K[0, h, rows] = rng.standard_normal((G, D)).astype(np.float32) * np.float32(1e30)
                V[0, h, rows] = rng.standard_normal((G, D)).astype(np.float32) * np.float32(1e30)
            elif k == 5:  # zeros of both signs: every key channel and value token all zero
                K[0, h, rows] = np.where(rng.random((G, D)) < 0.5, np.float32(-0.0), np.float32(0.0))
                V[0, h, rows] = np.where(rng.random((G, D)) < 0.5, np.float32(-0.0), np.float32(0.0))
            else:
                K[0, h, rows] = rng.standard_normal((G, D)).astype(np.float32) * np.float32(10.0 ** (k - 6))
                V[0, h, rows] = rng.standard_normal((G, D)).astype(np.float32)
    cfg, geo = make(_cfg_kw(B, H, D, bits, G, S, R, T, "f32"))
    cache = _run_prefill(kvq, cfg, {"K": K, "V": V}, T)
    ref = O.prefill(geo, K, V, T)
    compare_state(geo, read_state(cache), ref, T)



# Attention on caches built from edge values, on both kernels.  Each path is
# (Hq, Hkv, bits, G, D): the matrix-core kernel for GQA 8 (one and two key
# groups per chunk) and for the dual-group GQA-4 form, the VALU kernel for
# GQA 1 / 2, for 8-bit codes and for the bit-stream widths.  T = 524 with S = 2, R = 32 leaves a
# quantized count with Q % 64 == 32 at G = 32 (a half chunk / half value
# block at the end).
EDGE_PATHS = [
    (8, 1, 4, 64, 128),
    (8, 1, 2, 32, 64),
    (4, 1, 2, 32, 128),
    (4, 1, 4, 32, 64),
    (1, 1, 4, 32, 128),
    (2, 1, 2, 32, 64),
    (8, 1, 8, 32, 128),
    (1, 1, 3, 32, 128),
    (4, 1, 5, 32, 64),
    (8, 1, 1, 64, 128),
    (2, 1, 7, 32, 64),
]
EDGE_KINDS = ["ties", "constant", "negzero", "ksub", "vtiny", "kwide", "kwide30", "vwide30",
              "outlier300"]


def _edge_inputs(kind, B, Hq, Hkv, D, G, S, T, bits, seed):
    """fp32 K, V, q and the storage dtype of one edge-value case."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    K = rng.standard_normal((B, Hkv, T, D), dtype=f32)
    V = rng.standard_normal((B, Hkv, T, D), dtype=f32)
    q = rng.standard_normal((B, Hq, D), dtype=f32)
    L = 2 ** bits - 1
    dtype = "f32"
    if kind == "ties":
        # every quotient (x - min) / delta a half integer: delta = 1/16 with
        # both 0 and L/16 present in every key group channel and value token
        step = f32(2.0 ** -4)
        K = (rng.integers(0, L, size=K.shape).astype(f32) + f32(0.5)) * step
        V = (rng.integers(0, L, size=V.shape).astype(f32) + f32(0.5)) * step
        for g0 in range(S, T, G):
            K[:, :, g0] = 0
            if g0 + 1 < T:
                K[:, :, g0 + 1] = L * step
        V[..., 0] = 0
        V[..., 1] = L * step
        dtype = "f16"
    elif kind == "constant":
        # every key group constant per channel, every value token constant
        for g0 in range(S, T, G):
            K[:, :, g0:g0 + G] = rng.standard_normal((B, Hkv, 1, D), dtype=f32)
        V[:] = rng.standard_normal((B, Hkv, T, 1), dtype=f32)
    elif kind == "negzero":
        K = rng.uniform(0, 1, size=K.shape).astype(f32)
        V = rng.uniform(0, 1, size=V.shape).astype(f32)
        for g0 in range(S, T, G):
            K[:, :, g0, ::3] = f32(-0.0)
        V[..., 5] = f32(-0.0)
    elif kind == "ksub":     # subnormal key range: scores ~ 0, uniform weights
        K = rng.integers(0, 40, size=K.shape).astype(f32) * f32(2.0 ** -149)
    elif kind == "vtiny":    # value deltas near 2^-120 (normal fp32)
        V = V * f32(2.0 ** -118)
    elif kind == "kwide":    # one key channel wide enough that q * delta > 65504
        K[..., 7] *= f32(1e6)
        dtype = "bf16"
    elif kind == "kwide30":
        K *= f32(1e30)
    elif kind == "vwide30":
        V *= f32(1e30)
    elif kind == "outlier300":   # ten times the 70B-shaped workload's outliers
        for h in range(Hkv):
            K[:, h, :, rng.choice(D, 4, replace=False)] *= f32(300.0)
        dtype = "bf16"
    return {"K": synth.cast(K, dtype), "V": synth.cast(V, dtype), "q": synth.cast(q, dtype)}, dtype


def _fp32_score_floor(geo, st, T, q_stored, Hq, exp):
    """Row-rel error of attention whose exact log2-domain scores are each
    rounded once to fp32: what fp32 scores cost on this cache.  It is 0 to
    within rounding on every edge case but one: 1-bit codes with a key
    channel 1e6 wide, where half the tokens tie on that channel at scores
    near 3e5 and the softmax rests on their differences, far below fp32's
    resolution there (2^-6)."""
    import math
    Kh, Vh = O.dequant_cache(geo, st, T)
    q = O.to_f32(q_stored, geo.dtype).astype(np.float64)
    g = Hq // geo.Hkv
    out = np.zeros_like(exp)
    c = math.log2(math.e) / math.sqrt(geo.D)
    for b in range(geo.B):
        for hq in range(Hq):
            s = (c * (Kh[b, hq // g] @ q[b, hq])).astype(np.float32).astype(np.float64)
            p = np.exp2(s - s.max())
            out[b, hq] = (p @ Vh[b, hq // g]) / p.sum()
    return O.row_rel_error(out, exp)


@pytest.mark.parametrize("kind", EDGE_KINDS)
@pytest.mark.parametrize("path", EDGE_PATHS, ids=lambda c: "-".join(map(str, c)))
def test_attention_on_edge_value_caches(kind, path):
    """Ties, zero ranges, -0, subnormal key ranges, tiny value ranges, key
    ranges that push q * delta past fp16's range, 1e30 keys and values, and
    300x outlier channels: state bit-exact, attention within 2e-3 of the
    oracle on every row (plus twice the error fp32 scores alone cost, which
    is nonzero only where the result rests on score differences below
    fp32's resolution), on each kernel path."""
    kvq = _kvq()
    Hq, Hkv, bits, G, D = path
    B, S, R, T = 1, 2, 32, 524
    log("edge", kind, path)
    data, dt = _edge_inputs(kind, B, Hq, Hkv, D, G, S, T, bits, seed=11 + bits + D)
    cfg, geo = make(_cfg_kw(B, Hkv, D, bits, G, S, R, T, dt))
    cache = _run_prefill(kvq, cfg, data, T)
    ref = O.prefill(geo, data["K"], data["V"], T)
    compare_state(geo, read_state(cache), ref, T)
    out = kvq.kvq_decode_attention(cfg, cache, T, to_dev(data["q"], dt)).cpu().numpy()
    assert np.isfinite(out).all()
    exp = O.decode(geo, ref, T, data["q"], Hq)
    err = O.row_rel_error(out, exp)
    floor = _fp32_score_floor(geo, ref, T, data["q"], Hq, exp)
    log("row rel err", err, "fp32 score floor", floor)
    assert err <= ATOL_ROW_REL + 2 * floor


# Caches whose buffers start as 0xFF bytes (NaN as fp32): nothing the
# kernels read outside the cache contents may reach the result.
FILLED = [
    # B, Hq, Hkv, D, bits, G, S, R, T, dtype
    (1, 32, 8, 128, 2, 32, 4, 128, 1193, "bf16"),   # dual-group GQA 4, Q % 64 == 32
    (1, 8, 1, 128, 4, 32, 4, 32, 580, "bf16"),      # GQA 8, G 32, half chunk
    (1, 8, 1, 64, 2, 64, 4, 32, 600, "f16"),        # GQA 8, G 64
    (1, 2, 2, 64, 2, 32, 0, 32, 323, "f16"),        # VALU 2-bit, G 32, half value block
    (2, 16, 2, 64, 8, 64, 3, 64, 400, "f32"),       # VALU 8-bit
    (1, 4, 1, 128, 4, 32, 4, 128, 100, "bf16"),     # nothing quantized yet
    (1, 4, 2, 64, 3, 32, 4, 32, 330, "f16"),        # VALU 3-bit bit stream
    (1, 8, 1, 128, 7, 64, 2, 64, 450, "bf16"),      # VALU 7-bit bit stream
]


@pytest.mark.parametrize("case", FILLED, ids=lambda c: "-".join(map(str, c)))
def test_unwritten_cache_bytes_never_reach_the_result(case):
    kvq = _kvq()
    B, Hq, Hkv, D, bits, G, S, R, T, dt = case
    log("filled", case)
    data = synth.random_case(sum(case[:9]), B, Hq, Hkv, D, T, dt)
    cfg, geo = make(_cfg_kw(B, Hkv, D, bits, G, S, R, T + 70, dt))
    cache = kvq.Cache(cfg, fill=0xFF)
    kvq.prefill(cfg, cache, to_dev(data["K"], dt), to_dev(data["V"], dt), T)
    ref = O.prefill(geo, data["K"], data["V"], T)
    compare_state(geo, read_state(cache), ref, T)
    q = to_dev(data["q"], dt)
    out = kvq.kvq_decode_attention(cfg, cache, T, q).cpu().numpy()
    assert O.row_rel_error(out, O.decode(geo, ref, T, data["q"], Hq)) <= ATOL_ROW_REL
    # appends across the next freeze (the ring slots and the next group's
    # parameters start as 0xFF too)
    st = ref
    Kd, Vd = to_dev(data["K"], dt), to_dev(data["V"], dt)
    extra = synth.random_case(5 + T, B, Hq, Hkv, D, 70, dt)
    kn, vn = to_dev(extra["K"], dt), to_dev(extra["V"], dt)
    for i in range(70):
        kvq.kvq_append_token(cfg, cache, T + i, kn[:, :, i], vn[:, :, i])
        st = O.append(geo, st, T + i, extra["K"][:, :, i], extra["V"][:, :, i])
    del Kd, Vd
    T2 = T + 70
    compare_state(geo, read_state(cache), st, T2)
    out = kvq.kvq_decode_attention(cfg, cache, T2, q).cpu().numpy()
    assert O.row_rel_error(out, O.decode(geo, st, T2, data["q"], Hq)) <= ATOL_ROW_REL


STREAM = [
    # B, Hq, Hkv, D, bits, G, S, R, T0, steps, dtype
    (1, 2, 1, 64, 4, 32, 4, 32, 0, 140, "f32"),
    (2, 4, 2, 64, 2, 32, 0, 0, 10, 100, "bf16"),
    (1, 8, 2, 128, 8, 64, 3, 64, 100, 140, "f16"),
    (1, 8, 1, 128, 4, 64, 1, 128, 200, 150, "bf16"),
    (1, 4, 4, 128, 2, 32, 5, 32, 40, 130, "f16"),
    (1, 16, 4, 128, 2, 32, 4, 128, 100, 140, "bf16"),   # matrix-core path, GQA 4
    (2, 16, 2, 64, 4, 64, 2, 0, 30, 150, "f16"),        # matrix-core path, GQA 8, R 0
    (2, 8, 2, 64, 4, 32, 2, 32, 60, 130, "f16"),        # dual-group GQA 4, 4-bit, half chunks
    (1, 8, 1, 128, 4, 128, 4, 128, 250, 280, "bf16"),   # G 128 freezes at D 128 (largest LDS tile)
    (2, 4, 2, 64, 2, 128, 0, 0, 100, 300, "f16"),       # G 128 freezes at D 64
    # bit-stream widths: keys and value units straddle bytes
    (1, 2, 1, 64, 3, 32, 4, 32, 20, 120, "f32"),
    (1, 4, 2, 128, 5, 64, 2, 64, 90, 140, "bf16"),
    (2, 2, 2, 64, 1, 32, 0, 0, 10, 100, "f16"),
    (1, 8, 1, 128, 6, 128, 4, 128, 250, 280, "bf16"),
    (1, 4, 1, 64, 7, 32, 3, 32, 60, 110, "f16"),
]


@pytest.mark.parametrize("case", STREAM, ids=lambda c: "-".join(map(str, c)))
def test_streaming_appends_match_oracle_every_step(case):
    """[tract 'quantized KV-cache storage op'] frozen groups: the state after
    each append matches the oracle's streaming state and the GPU prefill of
    the same tokens, bit for bit; attention matches after every step."""
    kvq = _kvq()
    B, Hq, Hkv, D, bits, G, S, R, T0, steps, dt = case
    log("case", case)
    Tmax = T0 + steps
    data = synth.random_case(7 + sum(case[:9]), B, Hq, Hkv, D, Tmax, dt, steps=0)
    cfg, geo = make(_cfg_kw(B, Hkv, D, bits, G, S, R, Tmax, dt))
    cache = _run_prefill(kvq, cfg, data, T0)
    st = O.prefill(geo, data["K"], data["V"], T0)
    Kd = to_dev(data["K"], dt)
    Vd = to_dev(data["V"], dt)
    qd = to_dev(data["q"], dt)
    for n in range(T0, Tmax):
        kvq.kvq_append_token(cfg, cache, n, Kd[:, :, n], Vd[:, :, n])
        st = O.append(geo, st, n, data["K"][:, :, n], data["V"][:, :, n])
        T = n + 1
        compare_state(geo, read_state(cache), st, T)
        out = kvq.kvq_decode_attention(cfg, cache, T, qd).cpu().numpy()
        err = O.row_rel_error(out, O.decode(geo, st, T, data["q"], Hq))
        assert err <= ATOL_ROW_REL, (T, err)
    fresh = _run_prefill(kvq, cfg, data, Tmax)
    compare_state(geo, read_state(fresh), st, Tmax)


WINDOW = [
    # B, Hq, Hkv, D, bits, G, S, R, W, T0, steps, dtype
    (1, 16, 4, 128, 2, 32, 4, 32, 256, 900, 200, "bf16"),   # dual-group GQA 4, ring wraps
    (1, 8, 1, 128, 4, 64, 4, 128, 320, 1200, 150, "bf16"),  # GQA 8, G 64
    (2, 4, 4, 64, 4, 32, 0, 32, 100, 500, 130, "f16"),      # VALU, no sinks (plain window)
    (1, 8, 2, 64, 8, 32, 2, 32, 128, 400, 100, "f32"),      # VALU 8-bit, GQA 4
    (1, 8, 1, 64, 2, 32, 3, 0, 64, 300, 150, "f16"),        # R 0, small window, half chunks
    (1, 4, 2, 128, 2, 64, 4, 64, 192, 700, 140, "bf16"),    # VALU 2-bit (64-token blocks), G 64
    (1, 8, 2, 64, 3, 32, 4, 32, 160, 600, 120, "f16"),      # 3-bit bit stream
]


@pytest.mark.parametrize("case", WINDOW, ids=lambda c: "-".join(map(str, c)))
def test_sliding_window_prefill_and_streaming(case):
    """[KIVI-PR] the quantized store in a bounded sliding-window cache: the
    live ring rows bit-exact against the oracle after a prefill and after
    every append (groups evicted as they freeze), attention over the sinks
    and the last W tokens within 2e-3 after every step."""
    kvq = _kvq()
    B, Hq, Hkv, D, bits, G, S, R, W, T0, steps, dt = case
    log("window", case)
    Tmax = T0 + steps
    data = synth.random_case(31 + sum(case[:11]), B, Hq, Hkv, D, Tmax, dt)
    cfg, geo = make(_cfg_kw(B, Hkv, D, bits, G, S, R, Tmax, dt, window=W))
    assert cfg.qcap == geo.qcap < Tmax - S
    cache = _run_prefill(kvq, cfg, data, T0)
    st = O.prefill(geo, data["K"], data["V"], T0)
    compare_state(geo, read_state(cache), st, T0)
    Kd, Vd, qd = to_dev(data["K"], dt), to_dev(data["V"], dt), to_dev(data["q"], dt)
    out = kvq.kvq_decode_attention(cfg, cache, T0, qd).cpu().numpy()
    assert O.row_rel_error(out, O.decode(geo, st, T0, data["q"], Hq)) <= ATOL_ROW_REL
    for n in range(T0, Tmax):
        kvq.kvq_append_token(cfg, cache, n, Kd[:, :, n], Vd[:, :, n])
        st = O.append(geo, st, n, data["K"][:, :, n], data["V"][:, :, n])
        compare_state(geo, read_state(cache), st, n + 1)
        out = kvq.kvq_decode_attention(cfg, cache, n + 1, qd).cpu().numpy()
        err = O.row_rel_error(out, O.decode(geo, st, n + 1, data["q"], Hq))
        assert err <= ATOL_ROW_REL, (n + 1, err)


@pytest.mark.parametrize("Hq", [8, 4])
def test_split_count_invariance(Hq):
    """The log-sum-exp merge makes the result independent of the split count
    up to fp32 rounding.  Workspaces with room for 1, 3, 17, 64 and 1024
    splits per row: Q = 5856 quantized tokens (92 chunks of 64, the last a
    half chunk; 183 value blocks of 32) with 148 exact tokens.  On a 256-CU
    part the matrix-core path (Hq 8: GQA 4, dual-group form) then runs 1,
    3, 16, 46 and 92 splits, the VALU path (Hq 4: GQA 2) 1, 3, 17, 46 and
    46."""
    kvq = _kvq()
    B, Hkv, D, bits, G, S, R, T, dt = (1, 2, 128, 4, 32, 4, 128, 6000, "bf16")
    data = synth.random_case(99, B, Hq, Hkv, D, T, dt)
    cfg, geo = make(_cfg_kw(B, Hkv, D, bits, G, S, R, T, dt))
    cache = _run_prefill(kvq, cfg, data, T)
    q = to_dev(data["q"], dt)
    outs = []
    for splits in (1024, 1, 3, 17, 64):
        ws = torch.empty(cfg.workspace_bytes(Hq, splits), dtype=torch.uint8, device="cuda")
        outs.append(kvq.kvq_decode_attention(cfg, cache, T, q, workspace=ws).cpu().numpy())
    # Split counts change the summation order, the running-max rescales and
    # (one split) the length of each wave's accumulation chain; with the
    # matrix-core path's ~22-bit fp16 high/low weights the rows agree to
    # ~2e-5 (measured), well inside the parity bar checked below.
    for o in outs[1:]:
        assert O.row_rel_error(o, outs[0]) < 1e-4
    ref = O.decode(geo, O.prefill(geo, data["K"], data["V"], T), T, data["q"], Hq)
    for o in outs:
        assert O.row_rel_error(o, ref) <= ATOL_ROW_REL


@pytest.mark.parametrize("fill", [0x00, 0xFF, "random"])
def test_workspace_needs_no_initialization(fill):
    """Whatever the workspace holds, a call gives the same result, and so
    do repeated calls on it."""
    kvq = _kvq()
    B, Hq, Hkv, D, bits, G, S, R, T, dt = (2, 16, 2, 128, 4, 64, 4, 128, 3000, "bf16")
    data = synth.random_case(7, B, Hq, Hkv, D, T, dt)
    cfg, geo = make(_cfg_kw(B, Hkv, D, bits, G, S, R, T, dt))
    cache = _run_prefill(kvq, cfg, data, T)
    q = to_dev(data["q"], dt)
    n = cfg.workspace_bytes(Hq)
    if fill == "random":
        g = torch.Generator(device="cpu").manual_seed(5)
        ws = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).cuda()
    else:
        ws = torch.full((n,), fill, dtype=torch.uint8, device="cuda")
    ref = O.decode(geo, O.prefill(geo, data["K"], data["V"], T), T, data["q"], Hq)
    first = kvq.kvq_decode_attention(cfg, cache, T, q, workspace=ws).cpu().numpy()
    assert O.row_rel_error(first, ref) <= ATOL_ROW_REL
    for _ in range(3):
        again = kvq.kvq_decode_attention(cfg, cache, T, q, workspace=ws).cpu().numpy()
        assert np.array_equal(again, first)


# ----------------------------------------------------------------- workloads
def _workload(name):
    w = synth.WORKLOADS[name]
    cfg_kw = _cfg_kw(w.batch, w.n_kv_heads, w.head_dim, w.bits, w.group, w.sink, w.residual,
                     w.capacity, w.dtype, w.window, outliers=w.outliers)
    cfg_kw["rope_base"] = w.rope_base
    return w, cfg_kw


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_prefill_bit_exact_and_attention(name):
    kvq = _kvq()
    w, kw = _workload(name)
    log("workload", name)
    data = synth.generate(w, steps=0)
    cfg, geo = make(kw)
    T = w.n_tokens
    cache = _run_prefill(kvq, cfg, data, T)
    ref = O.prefill(geo, data["K"], data["V"], T)
    compare_state(geo, read_state(cache), ref, T)
    log("state bit-exact")
    q = to_dev(data["q"], w.dtype)
    out = kvq.kvq_decode_attention(cfg, cache, T, q).cpu().numpy()
    err = O.row_rel_error(out, O.decode(geo, ref, T, data["q"], w.n_q_heads))   # every row
    log("row rel err", err)
    assert err <= ATOL_ROW_REL


@pytest.mark.parametrize("name", ["gpt2", "llama70b", "mistral_swa"])
def test_workload_streaming(name):
    """The streaming workloads: append + attention per step, the state
    checked against the oracle's append path at the steps around both group
    freezes (every step for the GPT-2 shape), attention on every row at
    those steps."""
    kvq = _kvq()
    w, kw = _workload(name)
    log("workload", name)
    data = synth.generate(w)
    cfg, geo = make(kw)
    T0 = w.n_tokens
    cache = _run_prefill(kvq, cfg, data, T0)
    st = O.prefill(geo, data["K"], data["V"], T0)
    kn = to_dev(data["k_new"], w.dtype)
    vn = to_dev(data["v_new"], w.dtype)
    qn = to_dev(data["q_new"], w.dtype)
    flush_steps = [i + 1 for i in range(w.steps)
                   if O.partition(T0 + i + 1, w.sink, w.residual, w.group)[1]
                   > O.partition(T0 + i, w.sink, w.residual, w.group)[1]]
    assert len(flush_steps) >= 2
    check = set([1, w.steps] + flush_steps + [s + 1 for s in flush_steps if s < w.steps])
    if name == "gpt2":
        check = set(range(1, w.steps + 1))
    for i in range(w.steps):
        n = T0 + i
        kvq.kvq_append_token(cfg, cache, n, kn[i], vn[i])
        out = kvq.kvq_decode_attention(cfg, cache, n + 1, qn[i])
        st = O.append(geo, st, n, data["k_new"][i], data["v_new"][i])
        if i + 1 in check:
            log("step", i + 1)
            compare_state(geo, read_state(cache), st, n + 1)
            o = out.cpu().numpy()
            err = O.row_rel_error(o, O.decode(geo, st, n + 1, data["q_new"][i], w.n_q_heads))
            assert err <= ATOL_ROW_REL, (i + 1, err)


# Dense-and-sparse outliers: one exact entry per key group channel and per
# value token in side tables (both kept on the VALU kernel).
OUTLIER = [
    # B, Hq, Hkv, D, bits, G, S, R, T, dtype, window
    (1, 4, 2, 64, 4, 32, 4, 32, 333, "f16", 0),
    (2, 8, 2, 128, 2, 64, 2, 64, 700, "bf16", 0),      # GQA 4, 2-bit
    (1, 8, 1, 128, 4, 32, 4, 128, 1500, "bf16", 0),    # GQA 8, 4-bit
    (1, 2, 2, 64, 8, 128, 0, 0, 520, "f32", 0),
    (1, 4, 1, 128, 3, 32, 3, 32, 611, "f16", 0),       # bit-stream width
    (1, 2, 1, 128, 8, 32, 4, 32, 300, "f32", 0),       # fp32 rows of 128 channels
    (1, 8, 2, 64, 2, 32, 4, 32, 900, "bf16", 192),     # sliding window
]


@pytest.mark.parametrize("case", OUTLIER, ids=lambda c: "-".join(map(str, c)))
def test_outlier_side_tables_prefill_streaming_and_attention(case):
    """[pigeon guide 'KV-cache quantization', KVQuant adds] the side tables,
    codes and dense parameters bit-exact against the oracle after a prefill
    of spiky keys and values and after each of 70 appends (across freezes),
    and attention with the kept entries read exactly within 2e-3."""
    kvq = _kvq()
    B, Hq, Hkv, D, bits, G, S, R, T, dt, W = case
    log("outliers", case)
    steps = 70
    data = synth.spiky_case(41 + sum(case[:9]), B, Hq, Hkv, D, T + steps, dt)
    cfg, geo = make(_cfg_kw(B, Hkv, D, bits, G, S, R, T + steps, dt, window=W, outliers=1))
    cache = kvq.Cache(cfg, fill=0xFF)
    Kd, Vd, qd = to_dev(data["K"], dt), to_dev(data["V"], dt), to_dev(data["q"], dt)
    kvq.prefill(cfg, cache, Kd, Vd, T)
    torch.cuda.synchronize()
    st = O.prefill(geo, data["K"], data["V"], T)
    compare_state(geo, read_state(cache), st, T)
    assert (st["v_oidx"] != 255).any() and (st["k_oidx"] != 255).any()
    out = kvq.kvq_decode_attention(cfg, cache, T, qd).cpu().numpy()
    err = O.row_rel_error(out, O.decode(geo, st, T, data["q"], Hq))
    log("row rel err", err)
    assert err <= ATOL_ROW_REL
    for n in range(T, T + steps):
        kvq.kvq_append_token(cfg, cache, n, Kd[:, :, n], Vd[:, :, n])
        st = O.append(geo, st, n, data["K"][:, :, n], data["V"][:, :, n])
        if (n + 1) % 16 == 0 or n + 1 == T + steps:
            compare_state(geo, read_state(cache), st, n + 1)
            out = kvq.kvq_decode_attention(cfg, cache, n + 1, qd).cpu().numpy()
            err = O.row_rel_error(out, O.decode(geo, st, n + 1, data["q"], Hq))
            assert err <= ATOL_ROW_REL, (n + 1, err)
    fresh = kvq.Cache(cfg)
    kvq.prefill(cfg, fresh, Kd, Vd, T + steps)
    torch.cuda.synchronize()
    compare_state(geo, read_state(fresh), st, T + steps)


@pytest.mark.parametrize("kind", ["ties", "constant", "negzero", "vwide30", "outlier300"])
def test_outlier_side_tables_on_edge_values(kind):
    """Edge-value caches with side tables: tied extremes (nothing or the
    maximum kept), constant vectors (nothing kept), -0, 1e30 values and
    300x outlier channels, state bit-exact and attention within 2e-3."""
    kvq = _kvq()
    Hq, Hkv, bits, G, D = 4, 1, 4, 32, 128
    B, S, R, T = 1, 2, 32, 524
    log("outlier edge", kind)
    data, dt = _edge_inputs(kind, B, Hq, Hkv, D, G, S, T, bits, seed=77)
    cfg, geo = make(_cfg_kw(B, Hkv, D, bits, G, S, R, T, dt, outliers=1))
    cache = _run_prefill(kvq, cfg, data, T)
    ref = O.prefill(geo, data["K"], data["V"], T)
    compare_state(geo, read_state(cache), ref, T)
    out = kvq.kvq_decode_attention(cfg, cache, T, to_dev(data["q"], dt)).cpu().numpy()
    assert np.isfinite(out).all()
    exp = O.decode(geo, ref, T, data["q"], Hq)
    err = O.row_rel_error(out, exp)
    floor = _fp32_score_floor(geo, ref, T, data["q"], Hq, exp)
    log("row rel err", err, "floor", floor)
    assert err <= ATOL_ROW_REL + 2 * floor


# Pre-RoPE keys: the cache holds keys before the rotation, decode rotates
# each dequantized key to its token index (VALU kernel, every width).
ROPE = [
    # B, Hq, Hkv, D, bits, G, S, R, T, dtype, base, outliers, window
    (1, 4, 2, 64, 4, 32, 4, 32, 333, "f16", 10000.0, 0, 0),
    (2, 8, 2, 128, 2, 64, 2, 64, 700, "bf16", 500000.0, 0, 0),     # GQA 4, 2-bit (64-token blocks)
    (1, 8, 1, 128, 4, 32, 4, 128, 1500, "bf16", 500000.0, 0, 0),   # GQA 8
    (1, 2, 2, 64, 8, 128, 0, 0, 520, "f32", 10000.0, 0, 0),
    (1, 4, 1, 128, 3, 32, 3, 32, 611, "f16", 10000.0, 0, 0),       # bit-stream width
    (1, 2, 1, 128, 4, 32, 4, 32, 400, "f32", 10000.0, 1, 0),       # with side tables
    (1, 4, 2, 64, 2, 32, 4, 32, 900, "bf16", 10000.0, 1, 192),     # side tables and a window
    (1, 8, 2, 128, 5, 64, 4, 64, 800, "bf16", 1000000.0, 0, 256),  # window
]


@pytest.mark.parametrize("case", ROPE, ids=lambda c: "-".join(map(str, c)))
def test_pre_rope_keys_prefill_streaming_and_attention(case):
    """[pigeon guide 'KV-cache quantization', KVQuant adds] keys stored
    before RoPE: the stored state bit-exact (it is the plain state), and
    attention with every key rotated to its position within 2e-3 of the
    oracle after the prefill and across 70 appends."""
    kvq = _kvq()
    B, Hq, Hkv, D, bits, G, S, R, T, dt, base, outl, W = case
    log("rope", case)
    steps = 70
    data = synth.spiky_case(53 + sum(case[:9]), B, Hq, Hkv, D, T + steps, dt) if outl else \
        synth.random_case(53 + sum(case[:9]), B, Hq, Hkv, D, T + steps, dt)
    cfg, geo = make(dict(_cfg_kw(B, Hkv, D, bits, G, S, R, T + steps, dt, window=W, outliers=outl),
                         rope_base=base))
    cache = kvq.Cache(cfg, fill=0xFF)
    Kd, Vd, qd = to_dev(data["K"], dt), to_dev(data["V"], dt), to_dev(data["q"], dt)
    kvq.prefill(cfg, cache, Kd, Vd, T)
    torch.cuda.synchronize()
    st = O.prefill(geo, data["K"], data["V"], T)
    compare_state(geo, read_state(cache), st, T)
    out = kvq.kvq_decode_attention(cfg, cache, T, qd).cpu().numpy()
    err = O.row_rel_error(out, O.decode(geo, st, T, data["q"], Hq))
    log("row rel err", err)
    assert err <= ATOL_ROW_REL
    for n in range(T, T + steps):
        kvq.kvq_append_token(cfg, cache, n, Kd[:, :, n], Vd[:, :, n])
        st = O.append(geo, st, n, data["K"][:, :, n], data["V"][:, :, n])
        if (n + 1) % 17 == 0 or n + 1 == T + steps:
            out = kvq.kvq_decode_attention(cfg, cache, n + 1, qd).cpu().numpy()
            err = O.row_rel_error(out, O.decode(geo, st, n + 1, data["q"], Hq))
            assert err <= ATOL_ROW_REL, (n + 1, err)
    compare_state(geo, read_state(cache), st, T + steps)


def test_pre_rope_position_zero_is_the_plain_attention():
    """With only the first token cached, its position is 0 and the rotation
    is the identity: the output is that token's value, as without RoPE."""
    kvq = _kvq()
    data = synth.random_case(9, 1, 4, 2, 128, 1, "bf16")
    cfg, geo = make(dict(_cfg_kw(1, 2, 128, 4, 32, 4, 32, 64, "bf16"), rope_base=10000.0))
    cache = _run_prefill(kvq, cfg, data, 1)
    out = kvq.kvq_decode_attention(cfg, cache, 1, to_dev(data["q"], "bf16")).cpu().numpy()
    v = O.to_f32(data["V"][:, :, 0], "bf16")
    assert np.abs(out - np.repeat(v, 2, axis=1)).max() < 1e-6
