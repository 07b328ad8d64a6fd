"""Streaming through the C ABI beyond fixed scripts: a cache snapshotted to
host memory mid-stream and restored into fresh buffers continues bit for
bit like the original ([tract 'quantized KV-cache storage op'] frozen
blocks: the cache's state is its buffers and the token count, nothing
else), and randomized configurations and append sequences match the
oracle's streaming state."""
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


SNAP = [
    # B, Hq, Hkv, D, bits, G, S, R, T0, n_before_snapshot, n_after, dtype, window, outliers, rope
    (2, 8, 2, 128, 2, 32, 4, 64, 300, 50, 90, "bf16", 0, 0, 0.0),     # matrix-core path
    (1, 4, 4, 64, 3, 32, 2, 32, 200, 40, 80, "f16", 0, 1, 0.0),       # bit stream, side tables
    (1, 8, 2, 64, 4, 32, 4, 32, 500, 70, 100, "bf16", 160, 0, 10000.0),   # window, pre-RoPE keys
]


@pytest.mark.parametrize("case", SNAP, ids=lambda c: "-".join(map(str, c)))
def test_snapshot_restore_continues_bit_identically(case):
    kvq = _kvq()
    B, Hq, Hkv, D, bits, G, S, R, T0, n1, n2, dt, W, outl, rope = case
    log("snapshot", case)
    Tmax = T0 + n1 + n2
    data = synth.random_case(61 + sum(case[:8]), B, Hq, Hkv, D, Tmax, dt)
    kw = dict(batch=B, n_kv_heads=Hkv, head_dim=D, bits=bits, group=G, sink=S, residual=R,
              capacity=Tmax, dtype=dt, window=W, outliers=outl, rope_base=rope)
    cfg, geo = make(kw)
    Kd, Vd, qd = to_dev(data["K"], dt), to_dev(data["V"], dt), to_dev(data["q"], dt)
    a = kvq.Cache(cfg)
    kvq.prefill(cfg, a, Kd, Vd, T0)
    for n in range(T0, T0 + n1):
        kvq.kvq_append_token(cfg, a, n, Kd[:, :, n], Vd[:, :, n])
    torch.cuda.synchronize()
    # snapshot every buffer to host memory, restore into fresh buffers
    snap = {name: getattr(a, name).detach().cpu().clone() for name in a.BUFFERS}
    b = kvq.Cache(cfg, fill=0xA5)
    for name in b.BUFFERS:
        getattr(b, name).copy_(snap[name].to(getattr(b, name).device))
    torch.cuda.synchronize()
    for n in range(T0 + n1, Tmax):
        for c in (a, b):
            kvq.kvq_append_token(cfg, c, n, Kd[:, :, n], Vd[:, :, n])
        oa = kvq.kvq_decode_attention(cfg, a, n + 1, qd)
        ob = kvq.kvq_decode_attention(cfg, b, n + 1, qd)
        assert torch.equal(oa, ob), n
    torch.cuda.synchronize()
    for name in a.BUFFERS:
        assert torch.equal(getattr(a, name).view(torch.uint8), getattr(b, name).view(torch.uint8)), name
    # and both are the oracle's streaming state
    st = O.prefill(geo, data["K"], data["V"], T0)
    for n in range(T0, Tmax):
        st = O.append(geo, st, n, data["K"][:, :, n], data["V"][:, :, n])
    compare_state(geo, read_state(b), st, Tmax)
    out = kvq.kvq_decode_attention(cfg, b, Tmax, qd).cpu().numpy()
    assert O.row_rel_error(out, O.decode(geo, st, Tmax, data["q"], Hq)) <= ATOL_ROW_REL


@pytest.mark.parametrize("seed", range(8))
def test_random_configurations_and_append_sequences(seed):
    """A seeded random configuration (width, group, sinks, residual, GQA,
    head dim, dtype, window, side tables, RoPE base) and a random prefill
    length followed by a random run of appends: the state matches the
    oracle bit for bit and attention within 2e-3 at random checkpoints."""
    kvq = _kvq()
    rng = np.random.default_rng(1000 + seed)
    bits = int(rng.integers(1, 9))
    G = int(rng.choice([32, 64, 128]))
    S = int(rng.integers(0, 6))
    R = int(rng.choice([0, 32, 64, 128]))
    Hkv = int(rng.choice([1, 2, 4]))
    gqa = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    dt = str(rng.choice(["f32", "f16", "bf16"]))
    outl = int(rng.integers(0, 2))
    rope = float(rng.choice([0.0, 10000.0]))
    W = int(rng.choice([0, R + G + int(rng.integers(0, 200))]))
    T0 = int(rng.integers(0, 700))
    steps = int(rng.integers(20, 160))
    B = int(rng.integers(1, 3))
    Tmax = T0 + steps
    log("random", dict(seed=seed, bits=bits, G=G, S=S, R=R, Hkv=Hkv, gqa=gqa, D=D, dt=dt, outl=outl,
                       rope=rope, W=W, T0=T0, steps=steps, B=B))
    Hq = Hkv * gqa
    data = synth.spiky_case(seed, B, Hq, Hkv, D, Tmax, dt) if outl else \
        synth.random_case(seed, B, Hq, Hkv, D, Tmax, dt)
    kw = dict(batch=B, n_kv_heads=Hkv, head_dim=D, bits=bits, group=G, sink=S, residual=R,
              capacity=Tmax, dtype=dt, window=W, outliers=outl, rope_base=rope)
    cfg, geo = make(kw)
    Kd, Vd, qd = to_dev(data["K"], dt), to_dev(data["V"], dt), to_dev(data["q"], dt)
    cache = kvq.Cache(cfg, fill=0xFF)
    kvq.prefill(cfg, cache, Kd, Vd, T0)
    st = O.prefill(geo, data["K"], data["V"], T0)
    checks = set(rng.integers(T0 + 1, Tmax + 1, size=4).tolist()) | {Tmax}
    for n in range(T0, Tmax):
        kvq.kvq_append_token(cfg, cache, n, Kd[:, :, n], Vd[:, :, n])
        st = O.append(geo, st, n, data["K"][:, :, n], data["V"][:, :, n])
        if n + 1 in checks:
            torch.cuda.synchronize()
            compare_state(geo, read_state(cache), st, n + 1)
            out = kvq.kvq_decode_attention(cfg, cache, n + 1, qd).cpu().numpy()
            err = O.row_rel_error(out, O.decode(geo, st, n + 1, data["q"], Hq))
            assert err <= ATOL_ROW_REL, (n + 1, err)
