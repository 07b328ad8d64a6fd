"""Decode benchmark of the quantized KV cache on one MI355X.

One step = one pass of the whole hot path for one layer: kvq_append_token
(write the new K/V token, freezing a key group when the residual window
fills) followed by kvq_decode_attention over the whole packed cache; for a
workload that does not stream (a fixed cache), the attention call alone.
The default workload is the long-context 70B-shaped layer (B 1, 64 q heads,
8 KV heads, head_dim 128, 131072 cached tokens, bf16 inputs, int4, G 64,
R 128, 4 sinks).  Steps rotate over several layer caches whose total size
exceeds the last-level cache, so every attention call streams its packed
cache from HBM as in a real multi-layer decode.

Before the warmup it times the prefill (both quantize entry points) and
the append on its own (a plain one and one that freezes a group); after the
timed steps it times the attention call alone.  Prints one JSON line
(metric, value, roofline, cpu_baseline, detail).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attn tokens/s + effective packed-KV HBM GB/s (% of peak), int4 GQA"
HBM_PEAK_GBS = 8000.0
PMC_PROFILE = os.path.join(ROOT, "profiles", "attn_mfma_llama70b_pmc.md")


def kernel_sources_sha256() -> str:
    """Hash of the library sources (kernels, host code, header): a traffic
    figure measured with hardware counters is only reported while the code
    it was measured on is unchanged."""
    import hashlib
    import glob
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kivi_quantized_kv_amd", "csrc")
    files = sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h")))
    files.append(os.path.join(ROOT, "include", "kvq.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per decode call from the committed counter summary, or None
    when it is missing, for another workload, or stale."""
    if workload != "llama70b" or not os.path.exists(PMC_PROFILE):
        return None
    fields = {}
    with open(PMC_PROFILE) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "|", "#")):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    try:
        return int(float(fields["traffic_bytes_per_call"]))
    except (KeyError, ValueError):
        return None


def uses_mfma(w) -> bool:
    """The library's routing: matrix cores for GQA groups of 4 and 8 with
    2/4-bit codes, no side tables and no pre-RoPE keys, the VALU kernel
    otherwise."""
    return w.gqa in (4, 8) and w.bits in (2, 4) and not w.outliers and not w.rope_base


def attn_kernel_name(w) -> str:
    if uses_mfma(w):
        return "k_attn_mfma"
    return "k_attn_gqa" if 2 <= w.gqa <= 8 else "k_attn_valu"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def partition(T, S, R, G):
    n_sink = min(T, S)
    n = max(0, T - S)
    Q = G * ((n - R) // G) if n >= R else 0
    return n_sink, Q, n - Q


def window_start(w, T: int) -> int:
    """First quantized token the query attends to (0 without a window)."""
    return max(0, T - w.window - w.sink) if w.window else 0


def algorithmic_bytes(w, T: int) -> int:
    """Bytes one decode-attention call must read: packed K and V codes, key
    group (delta, zero) pairs, value token (delta, zero) pairs and the
    full-precision sink + residual tokens of the tokens it attends to (the
    sinks and the last W tokens with a window), over all (batch, KV head)."""
    ns, Q, nr = partition(T, w.sink, w.residual, w.group)
    u_lo = window_start(w, T)
    nq = Q - u_lo
    ng = (Q - 1) // w.group - u_lo // w.group + 1 if nq > 0 else 0
    D, b = w.head_dim, w.bits
    eb = 4 if w.dtype == "f32" else 2
    per_head = (2 * nq * D * b // 8 + ng * D * 8 + nq * 8 + 2 * (ns + nr) * D * eb)
    if w.outliers:   # side tables: position byte and value per key group channel and value token
        per_head += (ng * D + nq) * (1 + eb)
    return per_head * w.batch * w.n_kv_heads


def prefill_bytes(w, T: int, qcap: int) -> int:
    """Bytes a prefill of T tokens moves: K and V read in the input dtype,
    packed codes, key group and value token (delta, zero) pairs and the
    exact sink / residual rows written.  With a window only the last qcap
    quantized tokens are quantized (older ones would be evicted)."""
    ns, Q, nr = partition(T, w.sink, w.residual, w.group)
    Q = min(Q, qcap)
    D, b = w.head_dim, w.bits
    eb = 4 if w.dtype == "f32" else 2
    per_head = (2 * (ns + Q + nr) * D * eb + 2 * Q * D * b // 8 + (Q // w.group) * D * 8 + Q * 8
                + 2 * (ns + nr) * D * eb)
    if w.outliers:
        per_head += ((Q // w.group) * D + Q) * (1 + eb)
    return per_head * w.batch * w.n_kv_heads


def decode_splits(w, T: int, cus: int, ws_splits: int = 1024) -> int:
    """Split count of one decode call, by the launch rule of the library's
    host code (matrix-core path: one round of one workgroup per CU over
    64-token chunks, at most min(64, 8 * (4096 // (2 * D * element bytes)))
    exact tokens per split; VALU path: see kvq_api.hip), for the
    split-partial byte count."""
    ns, Q, nr = partition(T, w.sink, w.residual, w.group)
    n_fp = ns + nr
    if uses_mfma(w) and Q > 0:
        nblk = -(-Q // 64) - window_start(w, T) // 64
        want = max(1, cus // (w.batch * w.n_kv_heads))
        want = min(want, nblk, ws_splits)
        bps = -(-nblk // want)
        n_split = -(-nblk // bps)
        eb = 4 if w.dtype == "f32" else 2
        xcap = min(64, 8 * (4096 // (2 * w.head_dim * eb)))
        return max(n_split, min(-(-n_fp // xcap), ws_splits), 1)
    return None


def cpu_baseline(w, data, sample_seconds: float):
    """Time the CPU oracle on a bounded sample of the same work, with BLAS
    pools pinned to one thread: the prefill and the appends (plain and
    freezing) of one KV head, and the decode attention of the q heads of
    one KV head, each scaled to the whole layer.  The reported value is
    tokens/s of one step (append + attention when the workload streams)."""
    from threadpoolctl import threadpool_limits
    from oracle import kvq_oracle as O

    T = w.n_tokens
    geo = O.CacheGeometry(w.batch, w.n_kv_heads, w.head_dim, w.bits, w.group, w.sink,
                          w.residual, w.capacity, w.dtype, w.window, w.outliers, w.rope_base)
    geo1 = O.CacheGeometry(w.batch, 1, w.head_dim, w.bits, w.group, w.sink, w.residual,
                           T + max(w.steps, 2 * w.group + w.residual + 1), w.dtype, w.window,
                           w.outliers, w.rope_base)
    g = w.gqa
    rows = [(0, h) for h in range(g)]          # the q heads of KV head 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        st1 = O.prefill(geo1, data["K"][:, :1], data["V"][:, :1], T)
        prefill_s = (time.perf_counter() - t0) * w.n_kv_heads
        # appends on the one-head state: plain ones up to the next freeze,
        # then the freezing one
        n = T
        plain, freeze = [], []
        while True:
            q0 = partition(n, w.sink, w.residual, w.group)[1]
            q1 = partition(n + 1, w.sink, w.residual, w.group)[1]
            kn = data["k_new"][(n - T) % len(data["k_new"])][:, :1]
            vn = data["v_new"][(n - T) % len(data["v_new"])][:, :1]
            t0 = time.perf_counter()
            st1 = O.append(geo1, st1, n, kn, vn)
            (freeze if q1 > q0 else plain).append(time.perf_counter() - t0)
            n += 1
            if freeze:
                break
        append_plain_s = sum(plain) / max(1, len(plain)) * w.n_kv_heads
        append_freeze_s = freeze[0] * w.n_kv_heads
        st = O.prefill(geo, data["K"], data["V"], T)
        times = []
        t_end = time.time() + sample_seconds
        while time.time() < t_end or not times:
            t0 = time.perf_counter()
            O.decode(geo, st, T, data["q"], w.n_q_heads, rows=rows)
            times.append(time.perf_counter() - t0)
    per_kv_head = sum(times) / len(times)
    decode_s = per_kv_head * w.n_kv_heads * w.batch
    # an append at the natural freeze rate (one freeze per G steps)
    append_s = (append_plain_s * (w.group - 1) + append_freeze_s) / w.group if w.steps else 0.0
    step_s = decode_s + append_s
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": w.batch / step_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
        "host_cpus": os.cpu_count(), "cpu_model": cpu_model,
        "prefill_s": round(prefill_s, 3), "append_plain_s": round(append_plain_s, 5),
        "append_freeze_s": round(append_freeze_s, 4), "decode_s": round(decode_s, 3),
        "sample": (f"oracle (fp32 quantize, fp64 dequantize then attend), one thread: prefill, "
                   f"{len(plain)} plain appends and one freezing append of KV head 0, scaled "
                   f"x{w.n_kv_heads}; decode attention for the {g} q heads of KV head 0 at T={T}, "
                   f"{len(times)} runs, mean {per_kv_head:.3f}s, scaled x{w.n_kv_heads * w.batch}; "
                   + ("step = decode + append at one freeze per G steps" if w.steps
                      else "step = decode (the workload does not stream)")),
    }


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)



def stream_read_ceiling(layers, n_calls: int):
    """A measured read ceiling for the decode call's bytes: the plain
    streaming-read kernel of libkvq_probe.so over each layer cache's own
    buffers (every byte of each, layer caches rotated as in the attention
    timing, so that each pass reads from HBM), for a few launch shapes; the
    fastest is reported.  None when the probe library is not built."""
    path = os.path.join(ROOT, "kivi_quantized_kv_amd", "libkvq_probe.so")
    if not os.path.exists(path):
        return None
    import ctypes
    import torch
    lib = ctypes.CDLL(path)
    lib.kvqprobe_stream_read.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_int64),
                                         ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p]
    sets = []
    for c in layers:
        bufs = [getattr(c, n) for n in type(c).BUFFERS if getattr(c, n).numel() > 0]
        ptrs = (ctypes.c_void_p * len(bufs))(*[b.data_ptr() for b in bufs])
        sizes = (ctypes.c_int64 * len(bufs))(*[b.numel() * b.element_size() for b in bufs])
        sets.append((ptrs, sizes, len(bufs), sum(sizes)))
    grids = (256, 512, 1024)
    out = torch.empty(max(grids) * 512, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    best = None
    for grid, u in ((256, 8), (256, 4), (512, 4), (1024, 4)):
        def run(count):
            for i in range(count):
                ptrs, sizes, n, _ = sets[i % len(sets)]
                rc = lib.kvqprobe_stream_read(ptrs, sizes, n, ctypes.c_void_p(out.data_ptr()), grid, u,
                                              ctypes.c_void_p(stream))
                if rc != 0:
                    raise RuntimeError(f"kvqprobe_stream_read failed: {rc}")
        run(20)
        e0, e1 = _events()
        torch.cuda.synchronize()
        e0.record()
        run(n_calls)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / n_calls * 1e3
        if best is None or us < best[0]:
            best = (us, grid, u)
    nbytes = sum(s[3] for s in sets) / len(sets)
    return {"us": round(best[0], 3), "bytes": int(nbytes), "GBps": round(nbytes / (best[0] * 1e3), 1),
            "launch": f"{best[1]} workgroups x 512 threads, {best[2]} 16-byte loads in flight per thread"}

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=400,
                    help="untimed steps first (the clocks settle within a few hundred)")
    ap.add_argument("--workload", default="llama70b")
    ap.add_argument("--layers", type=int, default=4,
                    help="layer caches the steps rotate over (1 = warm, cache-resident)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (a reference "
                         "kernel of known traffic for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    from kivi_quantized_kv_amd import kvq, synth

    kvq.load_library()
    w = synth.WORKLOADS[args.workload]
    streaming = w.steps > 0
    n_layers = max(1, args.layers)
    per_layer_steps = -(-(args.steps + args.warmup) // n_layers) if streaming else 0
    n_gen = max(w.steps, 64)                    # distinct appended tokens / queries
    # room for the timed steps and for the append timings (up to two freezes ahead)
    steps_cap = max(n_gen, per_layer_steps, 2 * w.group + w.residual + 2)
    t0 = time.time()
    data = synth.generate(w, steps=n_gen)
    log(f"inputs generated in {time.time() - t0:.1f}s")
    cfg = kvq.Config(w.batch, w.n_kv_heads, w.head_dim, w.bits, w.group, w.sink, w.residual,
                     w.n_tokens + steps_cap, w.dtype, w.window, w.outliers, w.rope_base)
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def dev(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    K, V = dev(data["K"]), dev(data["V"])
    kn, vn, qn = dev(data["k_new"]), dev(data["v_new"]), dev(data["q_new"])
    T0 = w.n_tokens
    layers = [kvq.Cache(cfg)]
    # prefill of the first layer cache, timed (both halves; the first run
    # also settles the clocks)
    pre_ms = []
    for _ in range(4):
        e0, e1 = _events()
        torch.cuda.synchronize()
        e0.record()
        kvq.prefill(cfg, layers[0], K, V, T0)
        e1.record()
        torch.cuda.synchronize()
        pre_ms.append(e0.elapsed_time(e1))
    prefill_ms = float(np.median(pre_ms[1:]))
    for _ in range(1, n_layers):
        c = kvq.Cache(cfg)
        for name in kvq.Cache.BUFFERS:
            getattr(c, name).copy_(getattr(layers[0], name))
        layers.append(c)
    del K, V
    torch.cuda.synchronize()
    log(f"{n_layers} layer caches of {layers[0].nbytes() / 2**20:.1f} MiB prefilled "
        f"(prefill {prefill_ms * 1e3:.1f} us)")
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    ws = torch.empty(cfg.workspace_bytes(w.n_q_heads), dtype=torch.uint8, device="cuda")

    # Append timings on a scratch copy of the first cache: a plain append and
    # a freezing one, each repeated back to back (a repeated append rewrites
    # the same slot and group with the same data).
    scratch = kvq.Cache(cfg)
    for name in kvq.Cache.BUFFERS:
        getattr(scratch, name).copy_(getattr(layers[0], name))
    n = T0
    while partition(n + 1, w.sink, w.residual, w.group)[1] == partition(n, w.sink, w.residual, w.group)[1]:
        kvq.kvq_append_token(cfg, scratch, n, kn[(n - T0) % n_gen], vn[(n - T0) % n_gen])
        n += 1
    n_freeze, n_plain = n, n - 1

    def time_appends(nb, reps):
        j = (nb - T0) % n_gen
        e0, e1 = _events()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            kvq.kvq_append_token(cfg, scratch, nb, kn[j], vn[j])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    append_plain_us = time_appends(n_plain, 200) if n_plain >= T0 else None
    append_freeze_us = time_appends(n_freeze, 100)
    del scratch
    torch.cuda.synchronize()

    n_tok = [T0] * n_layers

    def step(i):
        li = i % n_layers
        j = (n_tok[li] - T0) % n_gen
        if streaming:
            kvq.kvq_append_token(cfg, layers[li], n_tok[li], kn[j], vn[j])
            n_tok[li] += 1
        kvq.kvq_decode_attention(cfg, layers[li], n_tok[li], qn[j], out=out, workspace=ws)
        return n_tok[li]

    if args.copy_probe_mib > 0:
        nn = args.copy_probe_mib * 2**20 // 4
        src_probe = torch.ones(nn, dtype=torch.float32, device="cuda")
        dst_probe = torch.empty_like(src_probe)
        torch.cuda.synchronize()
        dst_probe.copy_(src_probe)
        torch.cuda.synchronize()
        del src_probe, dst_probe
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K_ = args.steps
    # Timed region: K whole steps back to back (append + attention, or
    # attention alone for a workload that does not stream), inputs resident
    # in HBM, bracketed by synchronizations.
    start, end = _events()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(K_):
        step(args.warmup + i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / K_
    value = w.batch * K_ / (total_ms / 1e3)
    # Per-call duration of kvq_decode_attention: at least 200 more calls back
    # to back (each layer cache at its current length, no appends between),
    # with HIP events on the launch stream around the loop only: an event
    # between two launches costs time of its own.  The spread: the same in
    # groups of 20 calls.
    n_calls = max(K_, 200)

    def attn_loop(count, offset):
        for i in range(count):
            li = (offset + i) % n_layers
            kvq.kvq_decode_attention(cfg, layers[li], n_tok[li], qn[(offset + i) % n_gen], out=out,
                                     workspace=ws)

    attn_T = [n_tok[i % n_layers] for i in range(n_calls)]
    a0, a1 = _events()
    torch.cuda.synchronize()
    a0.record()
    attn_loop(n_calls, 0)
    a1.record()
    torch.cuda.synchronize()
    mean_attn_ms = a0.elapsed_time(a1) / n_calls
    groups = []
    for gi in range(10):
        g0, g1 = _events()
        g0.record()
        attn_loop(20, 20 * gi)
        g1.record()
        torch.cuda.synchronize()
        groups.append(g0.elapsed_time(g1) / 20 * 1e3)
    bytes_per_call = sum(algorithmic_bytes(w, T) for T in attn_T) / n_calls
    achieved = bytes_per_call / (mean_attn_ms / 1e3) / 1e9
    read_ceiling = stream_read_ceiling(layers, n_calls)
    splits = decode_splits(w, n_tok[0], cus)
    pbytes = prefill_bytes(w, T0, cfg.qcap)
    detail = {
        "attn_us_mean": round(mean_attn_ms * 1e3, 3),
        "attn_us_groups_of_20": {"median": round(float(np.median(groups)), 3),
                                 "p10": round(float(np.percentile(groups, 10)), 3),
                                 "p90": round(float(np.percentile(groups, 90)), 3)},
        "attn_calls_timed": n_calls,
        # the same cache buffers read by a plain streaming kernel, and the
        # decode call's rate as a fraction of that measured ceiling
        "stream_read": read_ceiling,
        "attn_over_stream_read": (None if read_ceiling is None else
                                  round(achieved / read_ceiling["GBps"], 4)),
        "step_us_minus_attn_us": round(ms_per_step * 1e3 - mean_attn_ms * 1e3, 3),
        "append_plain_us": None if append_plain_us is None else round(append_plain_us, 3),
        "append_freeze_us": round(append_freeze_us, 3),
        "prefill_us": round(prefill_ms * 1e3, 1),
        "prefill_bytes": pbytes,
        "prefill_GBps": round(pbytes / (prefill_ms / 1e3) / 1e9, 1),
        "algorithmic_bytes_per_call": int(bytes_per_call),
        "cached_tokens_at_timing": sorted(set(n_tok)),
        "split_partial_bytes_per_call": (None if splits is None else
                                         2 * w.batch * w.n_q_heads * splits * (w.head_dim + 2) * 4),
        "splits_per_row": splits,
        "layer_caches": n_layers,
        "cache_mib_per_layer": round(layers[0].nbytes() / 2**20, 1),
        "host_wall_s": round(wall, 3),
        "kernel_sources_sha256": kernel_sources_sha256()[:16],
    }
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K_,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int%d-codes/fp32-accumulate" % w.bits,
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: layer B{w.batch} Hq{w.n_q_heads} Hkv{w.n_kv_heads} "
                        f"D{w.head_dim} T{w.n_tokens}{'+decode' if streaming else ''} {w.dtype} "
                        f"inputs int{w.bits} G{w.group} R{w.residual} S{w.sink}"
                        + (f" window {w.window}" if w.window else "")
                        + (" outlier side tables" if w.outliers else "")
                        + (f" pre-RoPE keys (base {w.rope_base:g})" if w.rope_base else ""),
            "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim, "cached_tokens": w.n_tokens, "bits": w.bits,
            "group": w.group, "residual": w.residual, "sink": w.sink, "input_dtype": w.dtype,
            "window": w.window, "outliers": w.outliers, "rope_base": w.rope_base,
            "step": ("append + decode attention, one layer" if streaming
                     else "decode attention, one layer"),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": (f"kvq_decode_attention: {attn_kernel_name(w)} (split-K attention) + the split merge; "
                       f"mean over {n_calls} back-to-back calls, HIP events on the launch stream"),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(w.name),
        },
        "detail": detail,
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, data, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
