"""Host-side checks of the C ABI that need no GPU: the library loads, it
exports every entry point the header declares, the header's closed-form
sizes agree with the oracle's geometry, and argument validation rejects bad
calls before anything is launched (every call here fails validation, so no
kernel is ever enqueued)."""
import ctypes
import os
import re
import subprocess

import pytest

from oracle import kvq_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def _lib():
    from kivi_quantized_kv_amd import kvq
    if not os.path.exists(kvq.LIB_PATH):
        pytest.skip("libkvq.so not built")
    return kvq, kvq.load_library()


def test_library_exports_every_declared_entry_point():
    kvq, lib = _lib()
    text = open(HEADER).read()
    declared = re.findall(r"^kvq_status\s+(kvq_\w+)\s*\(", text, re.M)
    assert sorted(declared) == sorted(kvq.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for name in declared:
        assert re.search(rf"\bT {name}$", out, re.M), name
        assert hasattr(lib, name)


def test_probe_library_is_separate_from_the_abi():
    """The streaming-read probe the benchmark times lives in its own library:
    libkvq.so exports only kvq_* entry points, libkvq_probe.so its one call."""
    kvq, _ = _lib()
    probe = os.path.join(os.path.dirname(kvq.LIB_PATH), "libkvq_probe.so")
    if not os.path.exists(probe):
        pytest.skip("libkvq_probe.so not built")
    main = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH], capture_output=True,
                          text=True, check=True).stdout
    assert "kvqprobe_" not in main
    out = subprocess.run(["nm", "-D", "--defined-only", probe], capture_output=True, text=True,
                         check=True).stdout
    assert re.search(r"\bT kvqprobe_stream_read$", out, re.M)
    assert "kvq_decode_attention" not in out


def _header_sizes(cfg):
    """Compile a tiny C program against kvq.h and print its closed forms."""
    src = r"""
#include <stdio.h>
#include "kvq.h"
int main(int argc, char** argv) {
  kvq_config c = {%d, %d, %d, %d, %d, %d, %d, %d, %dLL, 0LL, %d};
  printf("%%lld %%lld %%lld %%lld %%lld %%lld %%lld %%lld %%lld\n", (long long)kvq_qcap(&c),
         (long long)kvq_k_codes_bytes(&c), (long long)kvq_v_codes_bytes(&c),
         (long long)kvq_k_params_count(&c), (long long)kvq_v_params_count(&c),
         (long long)kvq_sink_bytes(&c), (long long)kvq_resid_bytes(&c),
         (long long)kvq_k_side_count(&c), (long long)kvq_v_side_count(&c));
  return 0;
}
""" % cfg
    import tempfile
    d = tempfile.mkdtemp()
    with open(os.path.join(d, "t.c"), "w") as f:
        f.write(src)
    exe = os.path.join(d, "t")
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), os.path.join(d, "t.c"),
                    "-o", exe], check=True)
    return [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                           check=True).stdout.split()]


@pytest.mark.parametrize("B,H,D,bits,G,S,R,cap,dt", [
    (1, 1, 64, 4, 32, 4, 32, 256, "f32"),
    (1, 12, 64, 8, 32, 4, 32, 1088, "f16"),
    (4, 8, 128, 2, 32, 4, 128, 32768, "bf16"),
    (1, 8, 128, 4, 64, 4, 128, 131200, "bf16"),
    (2, 3, 128, 4, 128, 0, 0, 1000, "f16"),
    (1, 1, 64, 2, 32, 300, 0, 200, "f32"),
    (1, 2, 64, 3, 32, 4, 32, 300, "f16"),
    (2, 1, 128, 5, 64, 2, 64, 1000, "bf16"),
    (1, 1, 64, 1, 32, 0, 0, 100, "f32"),
    (1, 4, 128, 7, 128, 4, 128, 5000, "f16"),
    (1, 1, 64, 6, 32, 4, 32, 300, "bf16"),
])
@pytest.mark.parametrize("outl", [0, 1])
def test_header_sizes_match_oracle_geometry(B, H, D, bits, G, S, R, cap, dt, outl):
    code = {"f32": 0, "f16": 1, "bf16": 2}[dt]
    qcap, kc, vc, kp, vp, sink, resid, ks, vs = _header_sizes((B, H, D, bits, G, S, R, code, cap, outl))
    geo = O.CacheGeometry(B, H, D, bits, G, S, R, cap, dt, outliers=outl)
    st = geo.empty_state()
    assert ks == st["k_oidx"].size == st["k_oval"].size
    assert vs == st["v_oidx"].size == st["v_oval"].size
    assert qcap == geo.qcap
    assert kc == st["k_codes"].nbytes and vc == st["v_codes"].nbytes
    assert kp == st["k_scale"].size and vp == st["v_scale"].size
    assert sink == st["k_sink"].nbytes and resid == st["k_resid"].nbytes
    from kivi_quantized_kv_amd import kvq
    c = kvq.Config(B, H, D, bits, G, S, R, cap, dt)
    assert c.qcap == qcap and B * H * qcap * c.row_bytes == kc


def test_validation_rejects_bad_arguments_without_launching():
    kvq, lib = _lib()
    cfg = kvq.Config(1, 1, 64, 4, 32, 4, 32, 256, "f16")
    fake = 1 << 20   # aligned, never dereferenced: every call below fails validation
    cache = kvq.c_cache(*([fake] * 10))
    t = kvq.c_tensor(fake, 256 * 64, 256 * 64, 64)
    s = ctypes.c_void_p(0)

    def qk(c, cc=cache, tt=t, n=10):
        return lib.kvq_quantize_keys(ctypes.byref(c) if c is not None else None,
                                     ctypes.byref(cc) if cc is not None else None, tt, n, s)

    good = cfg.c()
    assert qk(None) == 1
    assert qk(good, cc=None) == 1
    bad = cfg.c(); bad.bits = 0
    assert qk(bad) == 2
    bad = cfg.c(); bad.bits = 9
    assert qk(bad) == 2
    bad = cfg.c(); bad.outliers = 2
    assert qk(bad) == 1
    bad = cfg.c(); bad.rope_base = -1.0
    assert qk(bad) == 1
    bad = cfg.c(); bad.rope_base = float("inf")
    assert qk(bad) == 1
    bad = cfg.c(); bad.rope_base = float("nan")
    assert qk(bad) == 1
    bad = cfg.c(); bad.outliers = 1           # side tables missing from the cache
    assert qk(bad) == 1
    bad = cfg.c(); bad.head_dim = 96
    assert qk(bad) == 2
    bad = cfg.c(); bad.group = 48
    assert qk(bad) == 2
    bad = cfg.c(); bad.dtype = 7
    assert qk(bad) == 2
    bad = cfg.c(); bad.batch = 0
    assert qk(bad) == 1
    assert qk(good, n=257) == 3
    assert qk(good, n=-1) == 1
    assert qk(good, tt=kvq.c_tensor(fake + 2, 0, 0, 64)) == 1        # misaligned
    assert qk(good, tt=kvq.c_tensor(fake, 0, 0, 63)) == 1            # row not 16-byte aligned
    assert qk(good, tt=kvq.c_tensor(None, 0, 0, 64)) == 1
    nulls = kvq.c_cache(*([fake] * 6 + [None] * 4))
    assert qk(good, cc=nulls) == 1
    # append
    assert lib.kvq_append_token(ctypes.byref(good), ctypes.byref(cache), 256, t, t, s) == 3
    assert lib.kvq_append_token(ctypes.byref(good), ctypes.byref(cache), -1, t, t, s) == 1
    # decode attention
    ws = cfg.workspace_bytes(4)

    def da(n_tok=100, hq=4, out=fake, wsb=ws, scale=0.0):
        return lib.kvq_decode_attention(ctypes.byref(good), ctypes.byref(cache), n_tok, hq, t,
                                        scale, out, fake, wsb, s)

    assert da(n_tok=0) == 1
    assert da(n_tok=257) == 3
    assert da(hq=0) == 1
    assert da(out=None) == 1
    assert da(wsb=1024) == 4
    assert da(scale=float("nan")) == 1
    cfg3 = kvq.Config(1, 3, 64, 4, 32, 4, 32, 256, "f16").c()
    assert lib.kvq_decode_attention(ctypes.byref(cfg3), ctypes.byref(cache), 10, 4, t, 0.0,
                                    fake, fake, ws, s) == 1   # 4 q heads over 3 KV heads
    # decode attention without a workspace: same checks, plus the limit of
    # the library's own split buffer (one split per row must fit)
    assert lib.kvq_decode_attention_noalloc(ctypes.byref(good), ctypes.byref(cache), 0, 4, t, 0.0,
                                            fake, s) == 1
    assert lib.kvq_decode_attention_noalloc(ctypes.byref(good), ctypes.byref(cache), 10, 4, t, 0.0,
                                            None, s) == 1
    big = kvq.Config(1000, 1, 128, 4, 32, 4, 32, 256, "f16")   # 1000 x 64 rows x 520 B > 16 MiB
    assert big.workspace_bytes(64, 1) > kvq.NOALLOC_SCRATCH_BYTES
    assert lib.kvq_decode_attention_noalloc(ctypes.byref(big.c()), ctypes.byref(cache), 10, 64,
                                            kvq.c_tensor(fake, 64 * 128, 128, 0), 0.0, fake, s) == 4


def test_noalloc_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define KVQ_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    from kivi_quantized_kv_amd import kvq
    assert m and int(m.group(1)) << int(m.group(2)) == kvq.NOALLOC_SCRATCH_BYTES
