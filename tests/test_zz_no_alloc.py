"""kvq_decode_attention_noalloc, the decode entry point that allocates
nothing (its split partials live in a device array inside the library),
through the C ABI: two calls in a row, the second on a smaller input, each
bit-identical to kvq_decode_attention with a workspace of the same size
(same kernels, same split count) and within 2e-3 of the oracle."""
import numpy as np
import pytest
import torch

from oracle import kvq_oracle as O
from kivi_quantized_kv_amd import synth
from tests.gpu_util import log, make, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, D, bits, G, S, R, T, dtype
    (1, 64, 8, 128, 4, 64, 4, 128, 20000, "bf16"),   # matrix-core path
    (1, 8, 8, 64, 4, 32, 4, 32, 3000, "f16"),        # VALU path, smaller
]


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    from kivi_quantized_kv_amd import kvq
    kvq.load_library()
    for case in CASES:
        B, Hq, Hkv, D, bits, G, S, R, T, dt = case
        log("noalloc", case)
        data = synth.random_case(sum(case[:9]), B, Hq, Hkv, D, T, dt)
        cfg, geo = make(dict(batch=B, n_kv_heads=Hkv, head_dim=D, bits=bits, group=G, sink=S,
                             residual=R, capacity=T, dtype=dt))
        cache = kvq.Cache(cfg)
        kvq.prefill(cfg, cache, to_dev(data["K"], dt), to_dev(data["V"], dt), T)
        q = to_dev(data["q"], dt)
        out_na = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        kvq.kvq_decode_attention_noalloc(cfg, cache, T, q, out_na)
        ws = torch.empty(kvq.NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
        out_ws = kvq.kvq_decode_attention(cfg, cache, T, q, workspace=ws)
        torch.cuda.synchronize()
        a, b = out_na.cpu().numpy(), out_ws.cpu().numpy()
        assert np.array_equal(a, b)
        ref = O.decode(geo, O.prefill(geo, data["K"], data["V"], T), T, data["q"], Hq)
        err = O.row_rel_error(a, ref)
        log("row rel err", err)
        assert err <= 2e-3
