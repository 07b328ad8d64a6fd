"""Helpers for the GPU parity tests: move synthetic numpy inputs to the
device, run the library through its C ABI, read the cache back in the
oracle's layout and compare."""
import sys

import numpy as np
import torch

from oracle import kvq_oracle as O


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def make(cfg_kw):
    from kivi_quantized_kv_amd import kvq
    cfg = kvq.Config(**cfg_kw)
    geo = O.CacheGeometry(cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.bits, cfg.group,
                          cfg.sink, cfg.residual, cfg.capacity, cfg.dtype, cfg.window,
                          cfg.outliers, cfg.rope_base)
    return cfg, geo


def read_state(cache) -> dict:
    return {n: to_host(getattr(cache, n)) for n in cache.BUFFERS}


def _bits(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    return a


def compare_state(geo, got: dict, ref: dict, T: int, heads=None):
    """Bit-exact comparison of every buffer region that holds cache
    contents after T tokens.  Returns nothing; raises AssertionError."""
    vm = O.valid_masks(geo, T)
    rows, groups, ns = vm["rows"], vm["groups"], vm["n_sink"]
    sl = slice(None) if heads is None else heads

    def eq(name, a, b):
        a, b = _bits(a), _bits(b)
        if a.shape != b.shape or not np.array_equal(a, b):
            bad = np.argwhere(a != b) if a.shape == b.shape else None
            raise AssertionError(f"{name} differs (shape {a.shape} vs {b.shape}); "
                                 f"first mismatches {None if bad is None else bad[:5].tolist()}")

    eq("k_codes", got["k_codes"][:, sl][:, :, rows], ref["k_codes"][:, sl][:, :, rows])
    eq("k_scale", got["k_scale"][:, sl][:, :, groups], ref["k_scale"][:, sl][:, :, groups])
    eq("k_zero", got["k_zero"][:, sl][:, :, groups], ref["k_zero"][:, sl][:, :, groups])
    eq("v_scale", got["v_scale"][:, sl][:, :, rows], ref["v_scale"][:, sl][:, :, rows])
    eq("v_zero", got["v_zero"][:, sl][:, :, rows], ref["v_zero"][:, sl][:, :, rows])
    eq("v_codes", got["v_codes"][:, sl][:, :, vm["v_bytes"]], ref["v_codes"][:, sl][:, :, vm["v_bytes"]])
    eq("k_sink", got["k_sink"][:, sl, :ns], ref["k_sink"][:, sl, :ns])
    eq("v_sink", got["v_sink"][:, sl, :ns], ref["v_sink"][:, sl, :ns])
    eq("k_resid", got["k_resid"][:, sl][:, :, vm["ring"]], ref["k_resid"][:, sl][:, :, vm["ring"]])
    eq("v_resid", got["v_resid"][:, sl][:, :, vm["ring"]], ref["v_resid"][:, sl][:, :, vm["ring"]])
    if geo.outliers:
        for n in ("k_oidx", "k_oval"):
            eq(n, got[n][:, sl][:, :, groups], ref[n][:, sl][:, :, groups])
        for n in ("v_oidx", "v_oval"):
            eq(n, got[n][:, sl][:, :, rows], ref[n][:, sl][:, :, rows])
