#!/usr/bin/env python3
"""Throughput of row-wise ICL attention on one MI355X.

One step = one model call on the 512K-row FP8 workload: fit (FP8 scales,
K/V pack, scaled-query quantisation, context self-attention written to
out_ctx) + a 1,024-row query against the cache + cache release.  Inputs are
resident in HBM before the timed region.  value = algorithmic TFLOP/s of the
step, 4 n^2 D H + 4 R n D H with n the valid (unmasked) rows.

Also reported, on the 512K-row FP8 GatedLogScale cache: cached-prediction
GB/s of 128-row query batches (algorithmic bytes: the K/V codes once plus the
query rows, gate and outputs) and TFLOP/s of a 1,024-row batch; the roofline
of the dominant kernel (the context attention) from HIP events recorded
around its launches on its own stream during the timed region; and the
float64 oracle timed on this host on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA
PEAK_FP16_TFLOPS = 2500.0    # MI355X dense FP16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
# The FP8 attention kernels run QK^T on the FP8 pipe and PV on the FP16 pipe
# (P is fp16): half of the 4 n^2 D H FLOP at each peak, so the MFMA ceiling of
# that mix is 4 / (2 / 5000 + 2 / 2500) = 3333.3 TFLOP/s.
PEAK_MIXED_TFLOPS = 4.0 / (2.0 / PEAK_FP8_TFLOPS + 2.0 / PEAK_FP16_TFLOPS)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str, py: bool) -> str:
    """The source with its comments and blank lines removed, so that a change
    to a comment does not invalidate a measurement of the same code."""
    if py:
        text = re.sub(r"(?m)^\s*#.*$", "", text)
    else:
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash() -> str:
    """sha256 (first 16 hex digits) of the attention kernels' sources and of
    build_lib.py, which holds their compiler flags, comments excluded."""
    h = hashlib.sha256()
    for f in ("csrc/attention.hip", "csrc/prep.hip", "csrc/scaling.h", "build_lib.py"):
        with open(os.path.join(ROOT, "long_context_tabular_amd", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read(), f.endswith(".py")).encode())
    return h.hexdigest()[:16]


def counter_traffic(kernel: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    counters (calibrated against a plain copy) for this exact kernel source,
    or None if no measurement matches the current source."""
    path = os.path.join(ROOT, "profiles", "traffic_context_model512k.txt")
    rec = {}
    try:
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    rec[k.strip()] = v.strip()
    except OSError:
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    v = rec.get(f"{kernel}.bytes_per_launch")
    return None if v is None else int(float(v))


PEAKS_SRC = os.path.join(ROOT, "bench_peaks.hip")
PEAKS_LIB = os.path.join(ROOT, "bench_peaks.so")


def build_peaks() -> str:
    """Compile the peak probes (bench_peaks.hip) for gfx950 beside this file."""
    import shutil
    import subprocess
    hipcc = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
    tmp = PEAKS_LIB + ".tmp"
    cmd = [hipcc, "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", PEAKS_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building {PEAKS_SRC} failed:\n{r.stderr}")
    os.replace(tmp, PEAKS_LIB)
    return PEAKS_LIB


def measured_peaks() -> dict:
    """Dense MFMA TFLOP/s (FP8 and FP16 loops, two wavefronts per SIMD) and HBM
    streaming-read GB/s (0.5 and 4 GiB, once each, 32 workgroups per CU)
    sustained on this GPU; the best of three launches each."""
    import ctypes
    import torch
    if not os.path.exists(PEAKS_LIB):
        build_peaks()
    lib = ctypes.CDLL(PEAKS_LIB)
    lib.bench_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.bench_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def best_ms(go, reps=3):
        go()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            go()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        return min(times)

    res = {}
    blocks = cus * 2
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    for kind, name, flop, iters in ((0, "mfma_fp8_tflops", 131072, 20000), (1, "mfma_fp16_tflops", 32768, 40000)):
        def go():
            rc = lib.bench_peak_mfma(kind, blocks, iters, ctypes.c_void_p(out.data_ptr()), stream)
            if rc != 0:
                raise RuntimeError(f"bench_peak_mfma failed ({rc})")
        ms = best_ms(go)
        res[name] = round(blocks * 4 * iters * 4 * flop / (ms * 1e-3) / 1e12, 1)
    rblocks = cus * 32
    words = torch.empty(rblocks * 256, dtype=torch.int32, device="cuda")
    for gib in (0.5, 4):
        nbytes = int(gib * (1 << 30))
        buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

        def go():
            rc = lib.bench_peak_read(ctypes.c_void_p(buf.data_ptr()), nbytes // 16,
                                     ctypes.c_void_p(words.data_ptr()), rblocks, stream)
            if rc != 0:
                raise RuntimeError(f"bench_peak_read failed ({rc})")
        ms = best_ms(go)
        res[f"hbm_read_GB_per_s_{gib:g}GiB"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        del buf
    torch.cuda.synchronize()
    return res


def dev(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bench_model_call(B, gen, w, steps, warmup):
    import torch
    x = gen.make_inputs(w)
    gated = w.scale_mode == gen.SCALE_GATED_LOG
    q, k, v = dev(x.q_ctx), dev(x.k_ctx), dev(x.v_ctx)
    gate = dev(x.gate_ctx) if gated else None
    coef = x.head_coef if w.scale_mode != gen.SCALE_NONE else None
    qq = dev(x.q_query)
    gq = dev(x.gate_query) if gated else None
    out = torch.empty_like(q)
    qout = torch.empty_like(qq)
    lengths = w.length_list() if w.lengths else w.n_valid
    c = B.sdm_icl_attn_fit(q, k, v, lengths, w.scale_mode, w.precision, coef, gate, None)
    info = c.info()
    ws = torch.empty(B.sdm_icl_attn_query_workspace_size(c, w.n_query), dtype=torch.uint8, device="cuda")
    c.release()

    def step():
        cache = B.sdm_icl_attn_fit(q, k, v, lengths, w.scale_mode, w.precision, coef, gate, out)
        B.sdm_icl_attn_query(cache, qq, gq, out=qout, workspace=ws)
        cache.release()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    B.sdm_icl_timing_enable(True)
    for cls in range(5):
        B.sdm_icl_timing_read(cls)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    timings = {name: B.sdm_icl_timing_read(cls) for name, cls in
               (("context", B.SDM_ICL_TIMING_CONTEXT), ("query", B.SDM_ICL_TIMING_QUERY),
                ("combine", B.SDM_ICL_TIMING_COMBINE), ("scale", B.SDM_ICL_TIMING_SCALE),
                ("prep", B.SDM_ICL_TIMING_PREP))}
    B.sdm_icl_timing_enable(False)
    return x, info, (t1 - t0) / steps, timings


def bench_other_workload(B, gen, name, steps, warm_ms=60.0):
    """A model call of another workload (the 128K FP8, the 16K FP16 and the
    ragged 128K + 64K FP8 ones; a ragged call counts each element at its own length):
    warm-up calls adding up to about warm_ms of GPU work first (a few
    milliseconds leave the clocks below their steady state), then `steps`
    timed calls; the context kernel's time from the in-stream events."""
    import math
    w = gen.WORKLOADS[name]
    _, info, sec1, _ = bench_model_call(B, gen, w, 1, 1)
    warm = max(3, int(math.ceil(warm_ms / max(sec1 * 1e3, 1e-3))))
    _, info, sec, t = bench_model_call(B, gen, w, steps, warm)
    n, H, D, R = w.n_valid, w.heads, w.head_dim, w.n_query
    ns = w.length_list()                      # valid rows of each batch element
    ctx_flops = 4.0 * sum(m * m for m in ns) * D * H
    q_flops = 4.0 * R * sum(ns) * D * H
    ctx_ms = t["context"][0] / max(t["context"][1], 1)
    achieved = ctx_flops / (ctx_ms * 1e-3) / 1e12
    fp8 = info["precision"] == 1
    peak = PEAK_FP8_TFLOPS if fp8 else PEAK_FP16_TFLOPS
    mixed = PEAK_MIXED_TFLOPS if fp8 else PEAK_FP16_TFLOPS
    return {"n_valid": n if not w.lengths else list(ns), "n_query": R, "heads": H, "batch": w.batch,
            "precision": "fp8_e4m3" if fp8 else "fp16",
            "scale": ["none", "log", "gated_log"][w.scale_mode], "warmup": warm, "steps": steps,
            "ms_per_step": round(sec * 1e3, 4),
            "TFLOP_per_s_step": round((ctx_flops + q_flops) / sec / 1e12, 1),
            "context_kernel_ms": round(ctx_ms, 4), "context_TFLOP_per_s": round(achieved, 1),
            "peak": peak, "frac": round(achieved / peak, 4),
            "peak_mixed": round(mixed, 1), "frac_mixed": round(achieved / mixed, 4)}


def bench_cached(B, gen, w, reps, offload=True, warmup=300):
    import numpy as np
    import torch
    x = gen.make_inputs(w)
    gated = w.scale_mode == gen.SCALE_GATED_LOG
    q, k, v = dev(x.q_ctx), dev(x.k_ctx), dev(x.v_ctx)
    gate = dev(x.gate_ctx) if gated else None
    cache = B.sdm_icl_attn_fit(q, k, v, w.n_valid, w.scale_mode, w.precision, x.head_coef, gate, None)
    del q, k, v, gate
    qq = dev(x.q_query)
    gq = dev(x.gate_query) if gated else None
    res = {}
    n, H, D = w.n_valid, w.heads, w.head_dim
    for R in w.query_batches:
        ws = torch.empty(B.sdm_icl_attn_query_workspace_size(cache, R), dtype=torch.uint8, device="cuda")
        nb = max(1, w.n_query // R)                 # batches that cover the query set once
        qbs = [qq[:, i * R:(i + 1) * R].contiguous() for i in range(nb)]
        gbs = [gq[:, i * R:(i + 1) * R].contiguous() if gq is not None else None for i in range(nb)]
        obs = [torch.empty_like(qb) for qb in qbs]
        for _ in range(warmup):
            B.sdm_icl_attn_query(cache, qbs[0], gbs[0], out=obs[0], workspace=ws)
        torch.cuda.synchronize()
        # (1) one call at a time: the latency a single predict batch sees
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            a.record()
            B.sdm_icl_attn_query(cache, qbs[0], gbs[0], out=obs[0], workspace=ws)
            b.record()
        torch.cuda.synchronize()
        times = sorted(a.elapsed_time(b) for a, b in evs)
        med = times[len(times) // 2]
        # (2) the whole query set as nb batches of R rows issued back to back
        greps = max(3, reps // nb)
        gevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(greps)]
        for a, b in gevs:
            a.record()
            for qb, gb, ob in zip(qbs, gbs, obs):
                B.sdm_icl_attn_query(cache, qb, gb, out=ob, workspace=ws)
            b.record()
        torch.cuda.synchronize()
        gtimes = sorted(a.elapsed_time(b) for a, b in gevs)
        gmed = gtimes[len(gtimes) // 2] / nb
        # (3) per-kernel durations (library events around each launch)
        B.sdm_icl_timing_enable(True)
        for cls in range(5):
            B.sdm_icl_timing_read(cls)
        for _ in range(reps):
            B.sdm_icl_attn_query(cache, qbs[0], gbs[0], out=obs[0], workspace=ws)
        torch.cuda.synchronize()
        kt = {name: B.sdm_icl_timing_read(cls) for name, cls in
              (("scale", B.SDM_ICL_TIMING_SCALE), ("attention", B.SDM_ICL_TIMING_QUERY),
               ("combine", B.SDM_ICL_TIMING_COMBINE))}
        B.sdm_icl_timing_enable(False)
        kus = {k: ms / max(cnt, 1) * 1e3 for k, (ms, cnt) in kt.items()}
        alg_bytes = 2 * n * H * D + R * H * D * 2 * 2 + (R * H * 2 if gated else 0)
        flops = 4.0 * R * n * D * H
        res[R] = {"us_median": med * 1e3, "us_min": times[0] * 1e3, "us_max": times[-1] * 1e3,
                  "GB_per_s": alg_bytes / (med * 1e-3) / 1e9, "TFLOP_per_s": flops / (med * 1e-3) / 1e12,
                  "batches_in_sequence": nb, "us_per_batch_in_sequence": gmed * 1e3,
                  "GB_per_s_in_sequence": alg_bytes / (gmed * 1e-3) / 1e9,
                  "kernel_us": kus,
                  "attention_kernel_us": kus["attention"],
                  "attention_kernel_GB_per_s": alg_bytes / (kus["attention"] * 1e-6) / 1e9,
                  "algorithmic_bytes": alg_bytes}
    info = cache.info()
    if offload:
        # the same queries with the cache's K/V in pinned host memory, streamed
        # over PCIe in chunks (host-inclusive: not an HBM figure)
        B.sdm_icl_attn_cache_offload(cache)
        oinfo = cache.info()
        off = {"stream_chunk_splits": oinfo["stream_chunk_splits"], "device_bytes": oinfo["device_bytes"]}
        for R in w.query_batches:
            ws = torch.empty(B.sdm_icl_attn_query_workspace_size(cache, R), dtype=torch.uint8, device="cuda")
            qb = qq[:, :R].contiguous()
            gb = gq[:, :R].contiguous() if gq is not None else None
            ob = torch.empty_like(qb)
            for _ in range(2):
                B.sdm_icl_attn_query(cache, qb, gb, out=ob, workspace=ws)
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
            for a, b in evs:
                a.record()
                B.sdm_icl_attn_query(cache, qb, gb, out=ob, workspace=ws)
                b.record()
            torch.cuda.synchronize()
            med = sorted(a.elapsed_time(b) for a, b in evs)[2]
            n, H, D = w.n_valid, w.heads, w.head_dim
            off[str(R)] = {"us_median": round(med * 1e3, 1),
                           "host_GB_per_s": round(2 * n * H * D / (med * 1e-3) / 1e9, 1)}
        info["offloaded_queries"] = off
    cache.release()
    return res, info


def bench_projection(B, w, reps: int = 21, warmup: int = 10):
    """The fused Q/K/V projection at the model-call size: hidden rows
    [1, n_pad, H*64] times a [3*H*64, H*64] weight, LogScale on Q.  Median of
    `reps` calls after `warmup` (enough for the clock to settle after the
    cached leg's short bursts)."""
    import numpy as np
    import torch
    g = torch.Generator(device="cuda").manual_seed(w.seed)
    E = w.heads * w.head_dim
    x = (torch.randn((1, w.n_pad, E), generator=g, device="cuda") / 2).half()
    wt = (torch.randn((3 * E, E), generator=g, device="cuda") / (4 * E ** 0.5)).half()
    bias = (torch.randn((3 * E,), generator=g, device="cuda") / 16).half()
    coef = np.linspace(0.5, 1.5, w.heads).astype(np.float32)
    outs = tuple(torch.empty((1, w.n_pad, w.heads, w.head_dim), dtype=torch.float16, device="cuda") for _ in range(3))
    run = lambda: B.sdm_icl_qkv_project(x, wt, bias, heads=w.heads, key_length=w.n_valid, head_coef=coef,
                                        scale_mode=B.SDM_ICL_SCALE_LOG, outs=outs)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)[reps // 2]
    # reference point, not part of the path: torch's library GEMM (hipBLASLt)
    # on the same shape, fp16 in and out with the bias and without the scaling
    x2, y2 = x.view(w.n_pad, E), torch.empty((w.n_pad, 3 * E), dtype=torch.float16, device="cuda")
    lib = lambda: torch.addmm(bias, x2, wt.t(), out=y2)
    for _ in range(warmup):
        lib()
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        lib()
        b.record()
    torch.cuda.synchronize()
    lib_ms = sorted(a.elapsed_time(b) for a, b in evs)[reps // 2]
    flops = 2.0 * w.n_pad * 3 * E * E
    hbm = (w.n_pad * E + 3 * E * E + 3 * w.n_pad * E) * 2
    return {"rows": w.n_pad, "in_features": E, "out_features": 3 * E, "ms": round(ms, 4),
            "TFLOP_per_s": round(flops / (ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_FP16_TFLOPS, 4),
            "GB_per_s": round(hbm / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(hbm / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "library_gemm_ms": round(lib_ms, 4),
            "library_gemm": "torch.addmm (hipBLASLt), same shape, fp16, bias, no query scaling"}


def cpu_baseline(gen, x, w, sample_rows: int):
    """The float64 oracle (as it stands) on a bounded sample of the same workload."""
    import numpy as np
    from oracle import icl
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    gated = w.scale_mode == gen.SCALE_GATED_LOG
    t_fit0 = time.perf_counter()
    cache = icl.fit(x.q_ctx, x.k_ctx, x.v_ctx, w.n_valid, w.scale_mode, w.precision,
                    x.head_coef if w.scale_mode != gen.SCALE_NONE else None,
                    x.gate_ctx if gated else None)
    t_fit = time.perf_counter() - t_fit0
    rows = gen.sample_rows(w.n_valid, sample_rows, w.seed)
    qrows = np.arange(sample_rows)
    t0 = time.perf_counter()
    icl.context_outputs(cache, x.q_ctx, x.gate_ctx if gated else None, rows)
    icl.attend(cache, x.q_query[0, qrows], x.gate_query[0, qrows] if gated else None)
    dt = time.perf_counter() - t0
    flops = 4.0 * (rows.size + qrows.size) * w.n_valid * w.head_dim * w.heads
    rows_per_s = (rows.size + qrows.size) / dt
    # every row costs the same (all keys, all heads), so the whole model call's
    # rows (n context + R query) take n_rows / rows_per_s at this rate
    full_rows = w.n_valid + w.n_query
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3), "fit_seconds_untimed": round(t_fit, 3),
            "rows_per_s": round(rows_per_s, 2),
            "extrapolated_full_call_s": round(full_rows / rows_per_s, 1),
            "extrapolation": (f"linear in rows: {full_rows} rows (the {w.n_valid} valid context rows and {w.n_query} "
                              f"queries) at the sampled rows/s, excluding the fit"),
            "host_cpus": len(os.sched_getaffinity(0)),
            "sample": (f"{rows.size} context rows (incl. first/last 8 valid) + {qrows.size} query rows of "
                       f"{w.name}, each against all {w.n_valid} keys x {w.heads} heads, float64; the "
                       f"oracle's fit (scales + e4m3 codes of all K/V, {t_fit:.1f} s) ran before the timed part")}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="model512k_fp8_log")
    ap.add_argument("--cached-workload", default="cached512k_fp8_gated")
    ap.add_argument("--cached-reps", type=int, default=30)
    ap.add_argument("--cached-warmup", type=int, default=300,
                    help="untimed query calls per batch size before its timed calls (ten 128-row calls, about "
                         "2 ms of GPU work, leave the clocks below their steady state)")
    ap.add_argument("--no-cached", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-projection", action="store_true",
                    help="skip timing the fused Q/K/V projection")
    ap.add_argument("--no-offload", action="store_true",
                    help="skip the host-offloaded (PCIe-streamed) cached queries")
    ap.add_argument("--no-model-call", action="store_true",
                    help="skip the model-call measurement (only the cached-prediction leg runs)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the sustained MFMA and HBM-read peaks")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the 128K FP8 and 16K FP16 model calls")
    ap.add_argument("--other-workloads", default="ctx128k_fp8,ctx16k_log_fp16,ctx16k_gated_fp16,ragged128k_fp8")
    ap.add_argument("--cpu-sample-rows", type=int, default=384)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times) and exit; "
                         "the reference for scaling FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this engine runs on a single MI355X "
              "(multi-GPU sharding is a design note, not an implemented path).", file=sys.stderr)
        return 2

    import torch
    from long_context_tabular_amd import binding as B
    from long_context_tabular_amd import inputs as gen
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        nbytes = args.calibrate_copy << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": nbytes}), flush=True)
        return 0
    B.lib()

    if args.no_model_call:
        wc = gen.WORKLOADS[args.cached_workload]
        cres, cinfo = bench_cached(B, gen, wc, args.cached_reps, offload=not args.no_offload,
                                   warmup=args.cached_warmup)
        print(json.dumps({"cached": {"workload": wc.name, "kv_splits": cinfo["kv_splits"],
                                     "batches": {str(k): v for k, v in cres.items()}}}), flush=True)
        return 0
    w = gen.WORKLOADS[args.workload]
    log(f"[bench] model call {w.name}: n_pad={w.n_pad} n={w.n_valid} R={w.n_query} H={w.heads}")
    x, info, sec, t = bench_model_call(B, gen, w, args.steps, args.warmup)
    n, H, D, R = w.n_valid, w.heads, w.head_dim, w.n_query
    ctx_flops = 4.0 * n * n * D * H
    q_flops = 4.0 * R * n * D * H
    value = (ctx_flops + q_flops) / sec / 1e12
    ctx_ms, ctx_n = t["context"]
    ctx_avg = ctx_ms / max(ctx_n, 1)
    achieved = ctx_flops / (ctx_avg * 1e-3) / 1e12
    prec_name = "fp8_e4m3" if info["precision"] == 1 else "fp16"
    peak = PEAK_FP8_TFLOPS if info["precision"] == 1 else PEAK_FP16_TFLOPS
    peak_mixed = PEAK_MIXED_TFLOPS if info["precision"] == 1 else PEAK_FP16_TFLOPS
    log(f"[bench] step {sec * 1e3:.2f} ms, {value:.1f} TFLOP/s; context kernel {ctx_avg:.3f} ms "
        f"({achieved:.1f} TFLOP/s)")
    line = {
        "metric": "ICL attention TFLOP/s at 128K-512K context rows (% MFMA peak); cached GB/s",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prec_name,
        "data": "synthetic",
        "config": {"workload": w.name, "n_pad": w.n_pad, "n_valid": n, "n_query": R, "heads": H,
                   "head_dim": D, "precision": prec_name, "scale": ["none", "log", "gated_log"][w.scale_mode],
                   "qk_operands": prec_name, "pv_operands": "fp16", "softmax": "fp32",
                   "kv_splits": info["kv_splits"]},
        "roofline": {"bound": "mfma", "kernel": "attention_kernel (context pass)",
                     "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     # the MFMA ceiling of FP8 QK^T + FP16 PV (see PEAK_MIXED_TFLOPS)
                     "peak_mixed": round(peak_mixed, 1), "frac_mixed": round(achieved / peak_mixed, 4),
                     # the committed counter record is for the 512K model call only
                     "traffic": counter_traffic("context") if w.name == "model512k_fp8_log" else None,
                     "launch_ms": round(ctx_avg, 4), "launches": ctx_n},
        "step_breakdown_ms": {k: round(v[0] / max(v[1], 1), 4) for k, v in t.items() if v[1]},
    }
    peaks = None
    if not args.no_peaks:
        peaks = measured_peaks()
        line["measured_peaks"] = peaks
        mp = peaks["mfma_fp8_tflops" if info["precision"] == 1 else "mfma_fp16_tflops"]
        line["roofline"]["measured_peak"] = mp
        line["roofline"]["frac_of_measured"] = round(achieved / mp, 4)
        log(f"[bench] measured peaks: {json.dumps(peaks)}")
    if not args.no_cached:
        wc = gen.WORKLOADS[args.cached_workload]
        log(f"[bench] cached prediction {wc.name}: n={wc.n_valid} batches {wc.query_batches}")
        cres, cinfo = bench_cached(B, gen, wc, args.cached_reps, offload=not args.no_offload,
                                   warmup=args.cached_warmup)
        r128 = cres.get(128)
        line["cached"] = {"workload": wc.name, "kv_splits": cinfo["kv_splits"],
                          "GB_per_s": round(r128["GB_per_s"], 1) if r128 else None,
                          "hbm_frac": round(r128["GB_per_s"] / PEAK_HBM_GBS, 4) if r128 else None,
                          "batches": {str(k): {kk: (round(vv, 3) if isinstance(vv, float) else vv)
                                               for kk, vv in v.items()} for k, v in cres.items()},
                          "offloaded": cinfo.get("offloaded_queries")}
        if peaks and r128:
            line["cached"]["hbm_frac_of_measured"] = round(r128["GB_per_s"] / peaks["hbm_read_GB_per_s_4GiB"], 4)
        log(f"[bench] cached: {json.dumps(line['cached'])}")
    if not args.no_other:
        line["other_workloads"] = {}
        for name in [s for s in args.other_workloads.split(",") if s]:
            log(f"[bench] model call {name}")
            line["other_workloads"][name] = bench_other_workload(B, gen, name, 20 if "16k" in name else 8)
            log(f"[bench] {name}: {json.dumps(line['other_workloads'][name])}")
    if not args.no_projection:
        line["projection"] = bench_projection(B, w)
        if peaks:
            line["projection"]["mfma_frac_of_measured"] = round(
                line["projection"]["TFLOP_per_s"] / peaks["mfma_fp16_tflops"], 4)
        log(f"[bench] projection: {json.dumps(line['projection'])}")
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (float64 oracle)")
        line["cpu_baseline"] = cpu_baseline(gen, x, w, args.cpu_sample_rows)
    torch.cuda.synchronize()
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
