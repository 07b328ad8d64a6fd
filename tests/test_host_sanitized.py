"""The library's host code (argument checks, size arithmetic, the decode
split planning) built with AddressSanitizer and UndefinedBehaviorSanitizer
on the host pass, and driven on the CPU with every device hidden: every
bad-argument path of test_abi, and valid calls over a spread of
configurations (windows, side tables, RoPE, widths 1-8, capacities up to
2^40 tokens), which plan their launches and then fail with KVQ_EHIP for
want of a device.  No kernel can run: the driver checks that the runtime
sees no device before making any valid call."""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
sys.path.insert(0, ROOT)
from kivi_quantized_kv_amd import build_lib   # noqa: E402  (the list of translation units)

OBJS = [os.path.splitext(f)[0] + ".o" for f in build_lib.SOURCES if f != "kvq_api.hip"]

DRIVER = r'''
import ctypes, sys
sys.path.insert(0, ROOT)
from kivi_quantized_kv_amd import kvq
lib = kvq.load_library(LIB)
hip = ctypes.CDLL("libamdhip64.so")
n = ctypes.c_int(0)
hip.hipGetDeviceCount(ctypes.byref(n))
assert n.value == 0, "a device is visible: refusing to make valid calls"
fake = 1 << 20
P = ctypes.byref
def cache():
    return kvq.c_cache(*([fake] * 14))
def tens(st=64):
    return kvq.c_tensor(fake, 1 << 24, 1 << 20, st)
def qk(c, n_tok, cc=None, t=None):
    return lib.kvq_quantize_keys(P(c), P(cc or cache()), t or tens(), n_tok, None)
bad = 0
cfg = kvq.Config(1, 1, 64, 4, 32, 4, 32, 256, "f16")
for field, value, want in [("bits", 0, 2), ("bits", 9, 2), ("head_dim", 96, 2), ("group", 48, 2),
                           ("dtype", 7, 2), ("batch", 0, 1), ("outliers", 2, 1), ("rope_base", -1.0, 1),
                           ("rope_base", float("inf"), 1), ("rope_base", float("nan"), 1),
                           ("window", 10, 1), ("capacity", 0, 1), ("sink", -1, 1)]:
    c = cfg.c(); setattr(c, field, value)
    r = qk(c, 10)
    assert r == want, (field, value, r)
c = cfg.c()
assert qk(c, 257) == 3 and qk(c, -1) == 1
assert qk(c, 10, t=kvq.c_tensor(fake + 2, 0, 0, 64)) == 1
assert qk(c, 10, t=kvq.c_tensor(fake, 0, 0, 63)) == 1
# valid calls: plans are computed, launches fail (no device)
import itertools
n_calls = 0
for bits, D, G, dt, W, outl, rope, cap, T, hq in itertools.product(
        [1, 2, 3, 4, 8], [64, 128], [32, 128], ["f32", "bf16"], [0, 4096], [0, 1], [0.0, 500000.0],
        [300, 1 << 40], [1, 299], [8]):
    if W and W < 32 + G:
        continue
    cfgv = kvq.Config(2, 2, D, bits, G, 4, 32, cap, dt, W, outl, rope)
    c = cfgv.c()
    ws = ctypes.create_string_buffer(64)
    r1 = lib.kvq_quantize_keys(P(c), P(cache()), tens(), T, None)
    r2 = lib.kvq_append_token(P(c), P(cache()), T - 1, tens(0), tens(0), None)
    r3 = lib.kvq_decode_attention(P(c), P(cache()), T, hq, tens(0), 0.0, fake, fake, 1 << 30, None)
    r4 = lib.kvq_decode_attention_noalloc(P(c), P(cache()), T, hq, tens(0), 0.0, fake, None)
    for r in (r1, r2, r3, r4):
        assert r in (0, 5), (bits, D, G, dt, W, outl, rope, cap, T, r)
    n_calls += 4
print("ok", n_calls)
'''


def _asan_runtime():
    libs = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return libs[0] if libs else None


def test_host_code_under_address_and_undefined_behavior_sanitizers():
    build = os.path.join(ROOT, "_build")
    objs = [os.path.join(build, o) for o in OBJS]
    rt = _asan_runtime()
    if not os.path.exists(HIPCC) or rt is None or not all(os.path.exists(o) for o in objs):
        pytest.skip("needs hipcc, the ASan runtime and the objects of a library build")
    d = tempfile.mkdtemp()
    api = os.path.join(d, "kvq_api.o")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
             "-I", os.path.join(ROOT, "include"),
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all"]
    subprocess.run([HIPCC, *flags, "-c", os.path.join(ROOT, "kivi_quantized_kv_amd", "csrc", "kvq_api.hip"),
                    "-o", api], check=True, capture_output=True)
    lib = os.path.join(d, "libkvq_asan.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", api, *objs, "-o", lib], check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1", CUDA_VISIBLE_DEVICES="-1")
    script = "ROOT = %r\nLIB = %r\n" % (ROOT, lib) + DRIVER
    r = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert r.stdout.strip().startswith("ok"), r.stdout
