"""ctypes binding of libkvq (the C ABI declared in include/kvq.h).

Argument marshalling only: torch supplies device memory and the stream,
every step of the path runs in the HIP kernels of libkvq.so.  The functions
carry the C names.  Loading fails loudly when the library is not built.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
STATUS = {0: "KVQ_OK", 1: "KVQ_EINVAL", 2: "KVQ_EUNSUPPORTED", 3: "KVQ_ECAPACITY",
          4: "KVQ_EWORKSPACE", 5: "KVQ_EHIP"}
MAX_SPLITS = 1024
NOALLOC_SCRATCH_BYTES = 16 << 20
EXPORTS = ("kvq_quantize_keys", "kvq_quantize_values", "kvq_append_token",
           "kvq_decode_attention", "kvq_decode_attention_noalloc")


class KvqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class c_config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group", ctypes.c_int32), ("sink", ctypes.c_int32),
                ("residual", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("capacity", ctypes.c_int64), ("window", ctypes.c_int64),
                ("outliers", ctypes.c_int32), ("rope_base", ctypes.c_float)]


class c_cache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero",
        "k_sink", "v_sink", "k_resid", "v_resid", "k_oidx", "k_oval", "v_oidx", "v_oval")]


class c_tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_t", ctypes.c_int64)]


_lib = None


def load_library(path: str | None = None):
    """Load libkvq.so (or the library at `path`) and declare its signatures
    (no GPU work).  The first library loaded stays bound."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.kvq_quantize_keys.argtypes = [P(c_config), P(c_cache), c_tensor, ctypes.c_int64, ctypes.c_void_p]
    lib.kvq_quantize_values.argtypes = [P(c_config), P(c_cache), c_tensor, ctypes.c_int64, ctypes.c_void_p]
    lib.kvq_append_token.argtypes = [P(c_config), P(c_cache), ctypes.c_int64, c_tensor, c_tensor,
                                     ctypes.c_void_p]
    lib.kvq_decode_attention.argtypes = [P(c_config), P(c_cache), ctypes.c_int64, ctypes.c_int32,
                                         c_tensor, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]
    lib.kvq_decode_attention_noalloc.argtypes = [P(c_config), P(c_cache), ctypes.c_int64,
                                                 ctypes.c_int32, c_tensor, ctypes.c_float,
                                                 ctypes.c_void_p, ctypes.c_void_p]
    for fn in EXPORTS:
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


@dataclasses.dataclass(frozen=True)
class Config:
    batch: int
    n_kv_heads: int
    head_dim: int
    bits: int
    group: int
    sink: int
    residual: int
    capacity: int
    dtype: str = "bf16"
    window: int = 0          # sliding window in tokens, 0 = none
    outliers: int = 0        # 1: one exact entry per quantization vector in side tables
    rope_base: float = 0.0   # > 0: keys stored before RoPE of this base, rotated in decode

    def c(self) -> c_config:
        """A new kvq_config struct of these fields."""
        return c_config(self.batch, self.n_kv_heads, self.head_dim, self.bits, self.group,
                        self.sink, self.residual, DTYPE_CODE[self.dtype], self.capacity,
                        self.window, self.outliers, self.rope_base)

    def _cref(self):
        """Pointer to this config's struct, built once (the dataclass is frozen)."""
        r = self.__dict__.get("_ref")
        if r is None:
            c = self.c()
            r = ctypes.byref(c)
            object.__setattr__(self, "_keep", c)
            object.__setattr__(self, "_ref", r)
        return r

    # closed-form sizes, as in include/kvq.h
    @property
    def qcap(self) -> int:
        step = max(64, self.group)
        n = max(0, self.capacity - self.sink)
        if self.window > 0:
            n = min(n, self.window + self.group)
        return -(-n // step) * step

    @property
    def row_bytes(self) -> int:
        return self.head_dim * self.bits // 8

    def workspace_bytes(self, n_q_heads: int, splits: int = MAX_SPLITS) -> int:
        """Room for `splits` partials per (batch, q head)."""
        return self.batch * n_q_heads * splits * (self.head_dim + 2) * 4


class Cache:
    """Device buffers of one cache in the layout of kvq.h, zero-filled (or
    every byte set to `fill`)."""

    def __init__(self, cfg: Config, device="cuda", fill: int | None = None):
        B, H, D, G = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.group
        qc = cfg.qcap
        td = TORCH_DTYPE[cfg.dtype]
        z = dict(device=device)
        self.cfg = cfg
        self.k_codes = torch.zeros((B, H, qc, cfg.row_bytes), dtype=torch.uint8, **z)
        self.v_codes = torch.zeros((B, H, qc * cfg.row_bytes), dtype=torch.uint8, **z)
        self.k_scale = torch.zeros((B, H, qc // G, D), dtype=torch.float32, **z)
        self.k_zero = torch.zeros((B, H, qc // G, D), dtype=torch.float32, **z)
        self.v_scale = torch.zeros((B, H, qc), dtype=torch.float32, **z)
        self.v_zero = torch.zeros((B, H, qc), dtype=torch.float32, **z)
        self.k_sink = torch.zeros((B, H, cfg.sink, D), dtype=td, **z)
        self.v_sink = torch.zeros((B, H, cfg.sink, D), dtype=td, **z)
        self.k_resid = torch.zeros((B, H, cfg.residual + G, D), dtype=td, **z)
        self.v_resid = torch.zeros((B, H, cfg.residual + G, D), dtype=td, **z)
        no = 1 if cfg.outliers else 0     # side tables only with outliers
        self.k_oidx = torch.zeros((B, H, no * qc // G, D), dtype=torch.uint8, **z)
        self.k_oval = torch.zeros((B, H, no * qc // G, D), dtype=td, **z)
        self.v_oidx = torch.zeros((B, H, no * qc), dtype=torch.uint8, **z)
        self.v_oval = torch.zeros((B, H, no * qc), dtype=td, **z)
        if fill is not None:
            for n in self.BUFFERS:
                t = getattr(self, n)
                if t.numel():
                    t.view(torch.uint8).fill_(fill)

    BUFFERS = ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero",
               "k_sink", "v_sink", "k_resid", "v_resid", "k_oidx", "k_oval", "v_oidx", "v_oval")

    def __setattr__(self, name, value):
        # a replaced buffer invalidates the cached kvq_cache struct
        super().__setattr__(name, value)
        if name in self.BUFFERS:
            super().__setattr__("_ref", None)

    def c(self) -> c_cache:
        """A new kvq_cache struct of the current buffers."""
        return c_cache(*[_ptr(getattr(self, n)) for n in self.BUFFERS])

    def _cref(self):
        """Pointer to the struct of the current buffers, rebuilt after a
        buffer is replaced."""
        r = self.__dict__.get("_ref")
        if r is None:
            c = self.c()
            r = ctypes.byref(c)
            super().__setattr__("_keep", c)
            super().__setattr__("_ref", r)
        return r

    def nbytes(self) -> int:
        return sum(getattr(self, n).numel() * getattr(self, n).element_size() for n in self.BUFFERS)


def _ptr(t: torch.Tensor):
    return t.data_ptr() if t.numel() else None


def tensor(t: torch.Tensor) -> c_tensor:
    """A [B][H][T][D] / [B][H][D] torch tensor as a kvq_tensor (strides in
    elements, last axis contiguous)."""
    if t.stride(-1) != 1:
        raise ValueError("last axis must be contiguous")
    st = t.stride()
    if t.dim() == 4:
        return c_tensor(t.data_ptr(), st[0], st[1], st[2])
    if t.dim() == 3:
        return c_tensor(t.data_ptr(), st[0], st[1], 0)
    raise ValueError("expected a 3-d or 4-d tensor")


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device: torch.device | None = None):
    if stream is None:
        if _raw_stream is not None and device is not None and device.index is not None:
            return _raw_stream(device.index)        # torch's current stream on that device
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(fn: str, status: int):
    if status != 0:
        raise KvqError(fn, status)


def kvq_quantize_keys(cfg: Config, cache: Cache, k: torch.Tensor, n_tokens: int, stream=None):
    lib = load_library()
    c, cc = cfg._cref(), cache._cref()
    _check("kvq_quantize_keys",
           lib.kvq_quantize_keys(c, cc, tensor(k), n_tokens, _stream(stream, k.device)))


def kvq_quantize_values(cfg: Config, cache: Cache, v: torch.Tensor, n_tokens: int, stream=None):
    lib = load_library()
    c, cc = cfg._cref(), cache._cref()
    _check("kvq_quantize_values",
           lib.kvq_quantize_values(c, cc, tensor(v), n_tokens, _stream(stream, v.device)))


def kvq_append_token(cfg: Config, cache: Cache, n_before: int, k_new: torch.Tensor,
                     v_new: torch.Tensor, stream=None):
    lib = load_library()
    c, cc = cfg._cref(), cache._cref()
    _check("kvq_append_token",
           lib.kvq_append_token(c, cc, n_before, tensor(k_new),
                                tensor(v_new), _stream(stream, k_new.device)))


def kvq_decode_attention(cfg: Config, cache: Cache, n_tokens: int, q: torch.Tensor,
                         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                         softmax_scale: float = 0.0, stream=None) -> torch.Tensor:
    lib = load_library()
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(cfg.workspace_bytes(Hq), dtype=torch.uint8, device=q.device)
    c, cc = cfg._cref(), cache._cref()
    _check("kvq_decode_attention",
           lib.kvq_decode_attention(c, cc, n_tokens, Hq, tensor(q),
                                    float(softmax_scale), out.data_ptr(), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), _stream(stream, q.device)))
    return out


def kvq_decode_attention_noalloc(cfg: Config, cache: Cache, n_tokens: int, q: torch.Tensor,
                                 out: torch.Tensor, softmax_scale: float = 0.0,
                                 stream=None) -> torch.Tensor:
    """Decode attention with the library's own split buffer; `out` is
    caller-provided ([B][Hq][D] fp32), so nothing is allocated here either."""
    lib = load_library()
    B, Hq, D = q.shape
    c, cc = cfg._cref(), cache._cref()
    _check("kvq_decode_attention_noalloc",
           lib.kvq_decode_attention_noalloc(c, cc, n_tokens, Hq, tensor(q), float(softmax_scale),
                                            out.data_ptr(), _stream(stream, q.device)))
    return out


def prefill(cfg: Config, cache: Cache, K: torch.Tensor, V: torch.Tensor, n_tokens: int, stream=None):
    """Both halves of the prefill."""
    kvq_quantize_keys(cfg, cache, K, n_tokens, stream)
    kvq_quantize_values(cfg, cache, V, n_tokens, stream)
