"""The streaming-read probe behind bench.py's read ceiling (libkvq_probe.so,
a measurement aid outside the kvq C ABI) reads every 32-bit word of its
buffers exactly once: the XOR of its per-thread outputs equals the XOR of
all words, for several launch shapes, buffer counts and ragged sizes."""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "kivi_quantized_kv_amd", "libkvq_probe.so")


@pytest.mark.gpu
@pytest.mark.parametrize("grid,u", [(256, 8), (256, 4), (1024, 4), (3, 8)])
def test_probe_reads_every_word_once(grid, u):
    import torch
    if not os.path.exists(PROBE):
        pytest.fail("libkvq_probe.so is not built")
    lib = ctypes.CDLL(PROBE)
    lib.kvqprobe_stream_read.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_int64),
                                         ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p]
    rng = np.random.default_rng(grid * 10 + u)
    # sizes in bytes: multiples of 16, ragged against the grid's stride
    sizes = [16 * int(n) for n in (rng.integers(1, 5000), 1, rng.integers(100000, 300000), 48)]
    host = [rng.integers(0, 2**32, size=s // 4, dtype=np.uint64).astype(np.uint32) for s in sizes]
    bufs = [torch.from_numpy(h.view(np.int32)).cuda() for h in host]
    out = torch.empty(grid * 512, dtype=torch.int32, device="cuda")
    ptrs = (ctypes.c_void_p * len(bufs))(*[b.data_ptr() for b in bufs])
    nb = (ctypes.c_int64 * len(bufs))(*sizes)
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.kvqprobe_stream_read(ptrs, nb, len(bufs), ctypes.c_void_p(out.data_ptr()), grid, u,
                                  ctypes.c_void_p(stream))
    assert rc == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.uint32(0)
    for h in host:
        want ^= np.bitwise_xor.reduce(h)
    assert got == want


@pytest.mark.gpu
def test_probe_rejects_bad_arguments():
    if not os.path.exists(PROBE):
        pytest.fail("libkvq_probe.so is not built")
    lib = ctypes.CDLL(PROBE)
    lib.kvqprobe_stream_read.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_int64),
                                         ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p]
    ptrs = (ctypes.c_void_p * 1)(16)
    nb = (ctypes.c_int64 * 1)(17)          # not a multiple of 16
    assert lib.kvqprobe_stream_read(ptrs, nb, 1, ctypes.c_void_p(16), 256, 4, None) != 0
    nb = (ctypes.c_int64 * 1)(16)
    assert lib.kvqprobe_stream_read(ptrs, nb, 0, ctypes.c_void_p(16), 256, 4, None) != 0   # no buffers
    assert lib.kvqprobe_stream_read(ptrs, nb, 1, ctypes.c_void_p(16), 256, 5, None) != 0   # bad u
