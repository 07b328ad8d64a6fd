"""Build libkvq.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every source is compiled on each call; objects are compiled in parallel and
linked into kivi_quantized_kv_amd/libkvq.so.  The streaming-read probe that
the benchmark uses as a measured read ceiling is linked on its own into
kivi_quantized_kv_amd/libkvq_probe.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libkvq.so")
PROBE_OUT = os.path.join(HERE, "libkvq_probe.so")
PROBE_SOURCES = ["probe_read.hip"]
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["kvq_quant.hip", "kvq_quant_any.hip", "kvq_attn.hip", "kvq_attn_any.hip",
           "kvq_attn_rope.hip", "kvq_attn_rope_any.hip", "kvq_gqa.hip", "kvq_gqa_outl.hip",
           "kvq_gqa_rope.hip", "kvq_gqa_rope_outl.hip", "kvq_mfma.hip", "kvq_api.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division (the quantizer's codes depend on it), subnormals kept
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES + PROBE_SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES if s in objs], OUT)
    _link([objs[s] for s in PROBE_SOURCES if s in objs], PROBE_OUT)
    if verbose:
        print("built", OUT, "and", PROBE_OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
