"""Seeded synthetic inputs for the quantized KV-cache path.

This module only draws random numbers and casts them to the storage dtype.
It holds none of the quantization or attention arithmetic, so both the CPU
oracle (through the tests) and the HIP path (through the tests and the bench)
can be fed from it without sharing any of the method's code.

The workloads stand in for the real activations the pages validate on (GPT-2
K/V activations and OpenELM-270M on the tract pull requests), which are not
available: Keys are Gaussian with a few fixed large-magnitude outlier channels
(the outlier-channel structure the KIVI recipe on the pigeon "KV-cache
quantization" page, "How it works" step 1, motivates per-channel key scales
with), Values and queries are plain Gaussian.

Arrays are numpy.  bf16 data is carried as uint16 bit patterns (numpy has no
bf16 type); fp16 as float16; fp32 as float32.  All tensors use the layouts
of the C ABI: K/V [B, Hkv, T, D], q [B, Hq, D], appended tokens
[steps, B, Hkv, D] and per-step queries [steps, B, Hq, D].
"""
from __future__ import annotations

import dataclasses
import numpy as np

DTYPES = ("f32", "f16", "bf16")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_tokens: int          # tokens in the cache before any streaming step
    dtype: str             # "f32" | "f16" | "bf16"
    bits: int
    group: int             # G: tokens per key quantization group
    residual: int          # R: most recent tokens kept in full precision
    sink: int              # S: first tokens kept in full precision
    n_outlier: int         # outlier channels per KV head
    outlier_scale: float
    steps: int             # streaming decode steps (append + attention)
    seed: int
    window: int = 0        # sliding window in tokens (0: attend to everything)
    outliers: int = 0      # 1: dense-and-sparse side tables
    rope_base: float = 0.0 # > 0: keys cached before RoPE, rotated in decode

    @property
    def gqa(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def capacity(self) -> int:
        return self.n_tokens + self.steps


# The five workloads.  Outlier counts per KV head: 4 fixed channels (tiny),
# 3% of 64 channels -> 2 (GPT-2-shaped), 4 (7B-MHA-shaped), 2% of 128
# channels -> 3 (Mistral-shaped), 4 (70B-shaped).  seed = 1000 * index.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 64, 256, "f32", 4, 32, 32, 4, 4, 20.0, 0, 1000),
    "gpt2": Workload("gpt2", 1, 12, 12, 64, 1024, "f16", 8, 32, 32, 4, 2, 15.0, 64, 2000),
    "mha7b": Workload("mha7b", 8, 32, 32, 128, 4096, "f16", 4, 32, 128, 4, 4, 25.0, 0, 3000),
    "mistral": Workload("mistral", 4, 32, 8, 128, 32768, "bf16", 2, 32, 128, 4, 3, 20.0, 0, 4000),
    "llama70b": Workload("llama70b", 1, 64, 8, 128, 131072, "bf16", 4, 64, 128, 4, 4, 30.0, 128, 5000),
    # the Mistral-shaped layer with a 4096-token sliding window (the tract
    # PR's example pairs a 4096-token window with a quantized store):
    # bounded ring store, 64 streaming steps through evictions
    "mistral_swa": Workload("mistral_swa", 4, 32, 8, 128, 32768, "bf16", 2, 32, 128, 4, 3, 20.0, 64, 6000,
                            window=4096),
    # the 70B-shaped layer at 3-bit codes (codes straddle bytes), and with
    # dense-and-sparse side tables (one exact entry per key group channel
    # and per value token)
    "llama70b_3bit": Workload("llama70b_3bit", 1, 64, 8, 128, 131072, "bf16", 3, 64, 128, 4, 4, 30.0, 128,
                              7000),
    "llama70b_outliers": Workload("llama70b_outliers", 1, 64, 8, 128, 131072, "bf16", 4, 64, 128, 4, 4,
                                  30.0, 128, 8000, outliers=1),
    # and with keys cached before RoPE (base 500000, as the 70B-class
    # models use), rotated inside the decode
    "llama70b_rope": Workload("llama70b_rope", 1, 64, 8, 128, 131072, "bf16", 4, 64, 128, 4, 4, 30.0, 128,
                              9000, rope_base=500000.0),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def cast(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float32 draws to the storage representation of `dtype`."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def outlier_channels(rng: np.random.Generator, n_kv_heads: int, head_dim: int,
                     n_outlier: int) -> np.ndarray:
    """[Hkv, n_outlier] channel indices, drawn without replacement per head."""
    out = np.zeros((n_kv_heads, n_outlier), dtype=np.int64)
    for h in range(n_kv_heads):
        out[h] = np.sort(rng.choice(head_dim, size=n_outlier, replace=False))
    return out


def generate(w: Workload, n_tokens: int | None = None, steps: int | None = None):
    """Draw one workload.  Draw order: outlier channels, K, V, q, then per
    step (k_new, v_new, q_new).  Returns a dict of storage-dtype arrays."""
    T = w.n_tokens if n_tokens is None else n_tokens
    n_steps = w.steps if steps is None else steps
    rng = np.random.Generator(np.random.PCG64(w.seed))
    B, Hq, Hkv, D = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    chans = outlier_channels(rng, Hkv, D, w.n_outlier)
    scale = np.ones((Hkv, D), dtype=np.float32)
    for h in range(Hkv):
        scale[h, chans[h]] = np.float32(w.outlier_scale)

    K = _normal(rng, (B, Hkv, T, D))
    K *= scale[None, :, None, :]
    V = _normal(rng, (B, Hkv, T, D))
    q = _normal(rng, (B, Hq, D))
    k_new = _normal(rng, (n_steps, B, Hkv, D))
    k_new *= scale[None, None, :, :]
    v_new = _normal(rng, (n_steps, B, Hkv, D))
    q_new = _normal(rng, (n_steps, B, Hq, D))
    return {
        "K": cast(K, w.dtype), "V": cast(V, w.dtype), "q": cast(q, w.dtype),
        "k_new": cast(k_new, w.dtype), "v_new": cast(v_new, w.dtype),
        "q_new": cast(q_new, w.dtype), "outlier_channels": chans,
    }


def random_case(seed: int, B: int, Hq: int, Hkv: int, D: int, T: int, dtype: str,
                steps: int = 0, n_outlier: int = 2, outlier_scale: float = 20.0,
                value_scale: float = 1.0):
    """A small ad-hoc case with the same distribution family."""
    w = Workload("adhoc", B, Hq, Hkv, D, T, dtype, 4, 32, 0, 0, n_outlier,
                 outlier_scale, steps, seed)
    rng = np.random.Generator(np.random.PCG64(seed))
    chans = outlier_channels(rng, Hkv, D, n_outlier)
    scale = np.ones((Hkv, D), dtype=np.float32)
    for h in range(Hkv):
        scale[h, chans[h]] = np.float32(outlier_scale)
    K = _normal(rng, (B, Hkv, T, D)) * scale[None, :, None, :]
    V = _normal(rng, (B, Hkv, T, D)) * np.float32(value_scale)
    q = _normal(rng, (B, Hq, D))
    k_new = _normal(rng, (steps, B, Hkv, D)) * scale[None, None, :, :]
    v_new = _normal(rng, (steps, B, Hkv, D)) * np.float32(value_scale)
    q_new = _normal(rng, (steps, B, Hq, D))
    return {
        "K": cast(K, dtype), "V": cast(V, dtype), "q": cast(q, dtype),
        "k_new": cast(k_new, dtype), "v_new": cast(v_new, dtype),
        "q_new": cast(q_new, dtype), "outlier_channels": chans, "workload": w,
    }


def spiky_case(seed: int, B: int, Hq: int, Hkv: int, D: int, T: int, dtype: str,
               frac: float = 0.01, spike: float = 30.0):
    """random_case with about `frac` of the key and value entries scaled by
    `spike` (sparse outliers on top of the fixed outlier channels), the
    workload a dense-and-sparse side table is for."""
    case = random_case(seed, B, Hq, Hkv, D, T, "f32")
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    out = dict(case)
    for name in ("K", "V"):
        x = case[name].copy()
        x[rng.random(x.shape) < frac] *= np.float32(spike)
        out[name] = cast(x, dtype)
    out["q"] = cast(case["q"], dtype)
    return out
