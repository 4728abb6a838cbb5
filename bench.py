"""Benchmark: fused exact attention forward on one MI355X.

A step is one call of the fused forward (attn_fwd: scores, online softmax and
value weighting in one kernel) on the dense 8k workload: B=8, H=32, N=8192,
d=128, bf16, non-causal, Q/K/V iid N(0,1) (seed 0).  Inputs are resident in
device memory before timing starts.  FLOP convention: 4*B*H*N^2*d (halved
when causal).

Prints ONE JSON line.  Besides the headline value it carries:
  roofline      -- the fused kernel against the bf16 dense MFMA peak, its
                   average launch time from HIP events on the launch stream,
                   and HBM traffic from rocprofv3 counters when the committed
                   counter record matches the current kernel source;
  cpu_baseline  -- the fp64 CPU oracle timed on a bounded sample of the same
                   workload (the host cores of this machine);
  sweep         -- the same fused forward on the other workloads;
  unfused       -- the three-launch standard path on the same workload, with
                   its algorithmic HBM bytes per second;
  backward      -- attn_bwd (dQ, dK, dV) on the dense 8k and causal 32k
                   workloads;
  fp8           -- attn_fwd_fp8 (e4m3 Q, K, V, bf16 O) on the dense 8k and
                   causal 32k shapes, and with e5m2 inputs on dense 8k,
                   against the fp8 dense MFMA peak;
  masked        -- attn_fwd_masked: dense 8k with an [N, N] fp32 bias, and
                   causal 32k with a 4096-key sliding window (FLOPs counted
                   over allowed (query, key) pairs only);
  fusion        -- the elementwise chain relu(scale*x + bias) on a 512 MiB
                   bf16 tensor, fused vs three launches, against HBM peak.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--quick]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused attention fwd TFLOP/s (bf16) + % of MFMA peak, B·H·N²·d sweep"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 bf16 FLOP/clk/CU (dense)
PEAK_FP8_TFLOPS = 5033.2    # twice the bf16 rate (32x32x64 fp8 MFMA)
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ["exact_attention_124_amd/csrc/attn_fwd_bf16.hip",
                  "exact_attention_124_amd/csrc/attn_fwd_bf16_dense.hip",
                  "exact_attention_124_amd/csrc/attn_fwd_bf16_persistent.hip",
                  "exact_attention_124_amd/csrc/common.h",
                  "exact_attention_124_amd/build.py"]
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "attn_fwd_bf16_dense_8k_traffic.json")
HEADLINE = "dense_8k_bf16"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_record():
    """HBM bytes per launch from the committed rocprofv3 counter record, or None
    if there is none or the kernel changed since the counters were taken."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, "no counter record"
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None, "kernel changed since counters were taken"
    return float(rec["bytes_per_launch"]), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated"


def time_launches(fn, steps, warmup, stream):
    """Warm up, then time exactly `steps` calls; returns (total_ms, per-launch ms list)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    total_ms = (time.perf_counter() - t0) * 1e3
    per = [a.elapsed_time(b) for a, b in evs]
    return total_ms, per


def time_graph(fn, calls, replays):
    """GPU time per call with no host work in between: `calls` back-to-back
    calls captured in one HIP graph, replayed `replays` times between two
    events.  For launches of a few microseconds, a per-launch event pair adds
    its own GPU time (and any host time while the queue is empty); this
    does not."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / (calls * replays)
    del graph
    return ms


def bench_fused_raw(ea, w, steps, warmup):
    """time_launches around direct C-ABI calls (ctypes, arguments computed
    once) instead of binding calls: the per-launch figure with the Python
    binding's checks and marshalling taken out."""
    import math
    import torch
    from exact_attention_124_amd.workloads import workload_inputs
    q, k, v = workload_inputs(w, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()
    fn = getattr(ea.load_library(), "attn_fwd" if w.dtype == torch.bfloat16 else "attn_fwd_f32")
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.H, w.N, w.d,
            1.0 / math.sqrt(w.d), 1 if w.causal else 0, stream.cuda_stream)
    assert fn(*args) == 0
    _, per = time_launches(lambda: fn(*args), steps, warmup, stream)
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return sum(per) / len(per)


def bench_fused_back_to_back(ea, w, calls=200):
    """GPU time per call for `calls` binding calls issued back to back
    between two events (no event pair around each call, no graph): if the
    binding's host time per call is below the kernel's, the queue never runs
    dry and this is the kernel's own rate."""
    import torch
    from exact_attention_124_amd.workloads import workload_inputs
    q, k, v = workload_inputs(w, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fn = getattr(ea, "attn_fwd" if w.dtype == torch.bfloat16 else "attn_fwd_f32")
    stream = torch.cuda.current_stream()
    for _ in range(10):
        fn(q, k, v, o, lse, causal=w.causal, stream=stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(calls):
        fn(q, k, v, o, lse, causal=w.causal, stream=stream)
    b.record(stream)
    host_us = (time.perf_counter() - t0) / calls * 1e6
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / calls
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return ms, host_us


def bench_fused_graph(ea, w, calls=20, replays=5):
    import torch
    from exact_attention_124_amd.workloads import workload_inputs
    q, k, v = workload_inputs(w, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fn = getattr(ea, "attn_fwd" if w.dtype == torch.bfloat16 else "attn_fwd_f32")
    ms = time_graph(lambda: fn(q, k, v, o, lse, causal=w.causal), calls, replays)
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return ms


def bench_fused_cold(ea, w, calls=10, flush_bytes=512 << 20):
    """Per-call time with a 512 MiB buffer written between calls, so the
    inputs are not served from L2 or the MALL; the event pair brackets only
    the attention call."""
    import torch
    from exact_attention_124_amd.workloads import workload_inputs
    q, k, v = workload_inputs(w, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device=q.device)
    fn = getattr(ea, "attn_fwd" if w.dtype == torch.bfloat16 else "attn_fwd_f32")
    stream = torch.cuda.current_stream()
    fn(q, k, v, o, lse, causal=w.causal, stream=stream)
    per = []
    for _ in range(calls):
        flush.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn(q, k, v, o, lse, causal=w.causal, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b))
    del q, k, v, o, lse, flush
    torch.cuda.empty_cache()
    return sorted(per)[len(per) // 2]


def device_info():
    import torch
    props = torch.cuda.get_device_properties(0)
    return {"name": props.name, "gcn_arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hip_runtime": torch.version.hip,
            "memory_GiB": round(props.total_memory / (1 << 30), 1)}


def bench_fused(ea, w, steps, warmup):
    import torch
    from exact_attention_124_amd.workloads import workload_inputs
    q, k, v = workload_inputs(w, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()
    fn_name = "attn_fwd" if w.dtype == torch.bfloat16 else "attn_fwd_f32"
    fn = getattr(ea, fn_name)
    call = lambda: fn(q, k, v, o, lse, causal=w.causal, stream=stream)  # noqa: E731
    total_ms, per = time_launches(call, steps, warmup, stream)
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return total_ms, per


def bench_unfused(ea, w, steps, warmup):
    import torch
    from exact_attention_124_amd.workloads import workload_inputs
    q, k, v = workload_inputs(w, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    ws = torch.empty(ea.attn_unfused_workspace_bytes(w.B, w.H, w.N, 2), dtype=torch.uint8,
                     device=q.device)
    stream = torch.cuda.current_stream()
    call = lambda: ea.attn_fwd_unfused(q, k, v, o, lse, ws, causal=w.causal, stream=stream)  # noqa
    total_ms, per = time_launches(call, steps, warmup, stream)
    del q, k, v, o, lse, ws
    torch.cuda.empty_cache()
    return total_ms, per


def bench_backward(ea, w, steps, warmup):
    """Time attn_bwd (statistics, dK/dV and dQ launches) on workload `w`."""
    import torch
    from exact_attention_124_amd.workloads import make_grad, workload_inputs
    q, k, v = workload_inputs(w, device="cuda")
    g = make_grad(w.B, w.H, w.N, w.d, w.dtype, w.seed, device="cuda")
    o, lse = ea.attention(q, k, v, causal=w.causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(w.B, w.H, w.N), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    call = lambda: ea.attn_bwd(q, k, v, o, lse, g, dq, dk, dv, ws, causal=w.causal, stream=stream)  # noqa
    total_ms, per = time_launches(call, steps, warmup, stream)
    del q, k, v, g, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return total_ms, per


def bench_fp8(ea, w, steps, warmup, fmt="e4m3"):
    """Time attn_fwd_fp8 on the shape of workload `w` (inputs quantised to
    `fmt`, e4m3 or e5m2, all three tensors)."""
    import torch
    from exact_attention_124_amd.workloads import make_qkv_fp8
    q8, k8, v8, qd, kd, vd = make_qkv_fp8(w.B, w.H, w.N, w.d, w.seed, w.q_mult, device="cuda",
                                          formats=(fmt,) * 3)
    o = torch.empty(q8.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(q8.shape[:3], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    call = lambda: ea.attn_fwd_fp8(q8, k8, v8, o, lse, qd, kd, vd, causal=w.causal, stream=stream)  # noqa
    total_ms, per = time_launches(call, steps, warmup, stream)
    del q8, k8, v8, o, lse
    torch.cuda.empty_cache()
    return total_ms, per


def backward_legs(ea, workloads, steps, warmup):
    bwd = []
    for name in (HEADLINE, "causal_32k_qx8_bf16"):
        ww = workloads[name]
        tot, pl = bench_backward(ea, ww, steps, warmup)
        bm = sum(pl) / len(pl)
        alg = 2.5 * ww.flops  # five products of 2*N^2*d per (b, h), halved when causal
        bwd.append({"workload": name, "ms": round(bm, 3),
                    "TFLOP/s": round(alg / (bm * 1e-3) / 1e12, 2),
                    "frac_bf16_peak": round(alg / (bm * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "flop_convention": "10*B*H*N^2*d (halved when causal); the kernels execute "
                                       "14*B*H*N^2*d (S and dP are recomputed for dQ)"})
        log(f"[bench] backward {name}: {bm:.3f} ms, {bwd[-1]['TFLOP/s']} TFLOP/s")
    return bwd


def fp8_legs(ea, workloads, steps, warmup):
    out = []
    for name, fmt in ((HEADLINE, "e4m3"), ("causal_32k_qx8_bf16", "e4m3"), (HEADLINE, "e5m2")):
        ww = workloads[name]
        tot, pl = bench_fp8(ea, ww, steps, warmup, fmt)
        fm = sum(pl) / len(pl)
        tf = ww.flops / (fm * 1e-3) / 1e12
        tag = "_fp8" if fmt == "e4m3" else "_fp8_e5m2"
        out.append({"workload": name.replace("_bf16", tag), "shape": ww.describe().replace("bf16", fmt),
                    "ms": round(fm, 4), "TFLOP/s": round(tf, 2),
                    "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4)})
        log(f"[bench] fp8 {fmt} {name}: {fm:.4f} ms, {out[-1]['TFLOP/s']} TFLOP/s")
    return out


def masked_legs(ea, workloads, steps, warmup):
    import torch
    from exact_attention_124_amd.workloads import make_bias, workload_inputs
    out = []
    stream = torch.cuda.current_stream()
    for name, window, with_bias in ((HEADLINE, (-1, -1), True), ("causal_32k_qx8_bf16", (4096, -1), False)):
        w = workloads[name]
        q, k, v = workload_inputs(w, device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        bias = make_bias(1, 1, w.N, seed=w.seed, device="cuda").expand(w.B, w.H, w.N, w.N) if with_bias else None
        call = lambda: ea.attn_fwd_masked(q, k, v, o, lse, causal=w.causal, window=window, bias=bias,  # noqa
                                          stream=stream)
        tot, pl = time_launches(call, steps, warmup, stream)
        ms = sum(pl) / len(pl)
        wl = window[0]
        if w.causal and wl >= 0:
            pairs = sum(min(i, wl) + 1 for i in range(w.N))
        elif w.causal:
            pairs = w.N * (w.N + 1) // 2
        else:
            pairs = w.N * w.N
        fl = 4.0 * w.B * w.H * pairs * w.d
        rec = {"workload": name, "window": list(window), "bias": "[N,N] fp32" if with_bias else None,
               "ms": round(ms, 4), "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 2),
               "flop_convention": "4*B*H*d per allowed (query, key) pair"}
        if with_bias:
            rec["bias_bytes_read"] = w.B * w.H * w.N * w.N * 4
            rec["bias_GB/s"] = round(rec["bias_bytes_read"] / (ms * 1e-3) / 1e9, 1)
        out.append(rec)
        log(f"[bench] masked {name} window={window} bias={with_bias}: {ms:.4f} ms, {rec['TFLOP/s']} TFLOP/s")
        del q, k, v, o, lse, bias
        torch.cuda.empty_cache()
    return out


def fusion_leg(ea, steps, warmup):
    import torch
    from exact_attention_124_amd.workloads import make_chain
    rows, cols = 65536, 4096
    x, b = make_chain(rows, cols, seed=0, device="cuda")
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    nbytes = x.numel() * 2
    out = {"shape": [rows, cols], "dtype": "bf16", "tensor_bytes": nbytes}
    for name, fn, crossings in (("fused", ea.ew_chain_fused, 2), ("unfused", ea.ew_chain_unfused, 6)):
        tot, pl = time_launches(lambda: fn(x, y, b, 1.7, stream=stream), steps, warmup, stream)  # noqa
        ms = sum(pl) / len(pl)
        gbs = crossings * nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 4), "algorithmic_bytes": crossings * nbytes, "GB/s": round(gbs, 1),
                     "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"[bench] fusion {name}: {ms * 1e3:.1f} us, {gbs:.0f} GB/s")
    out["fused_speedup"] = round(out["unfused"]["ms"] / out["fused"]["ms"], 2)
    del x, y, b
    torch.cuda.empty_cache()
    return out


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device copy of known size (for scaling the byte counters)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def cpu_baseline(w, target_s=15.0):
    """Time the fp64 oracle on a bounded sample of workload `w` -- every query row
    of a seeded subset of (b, h) slices, sized for about `target_s` seconds --
    and scale to TFLOP/s with the same FLOP convention."""
    import torch
    import oracle
    from exact_attention_124_amd.workloads import make_qkv
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.q_mult)
    order = torch.randperm(w.B * w.H, generator=torch.Generator().manual_seed(w.seed + 1)).tolist()
    q = q.reshape(-1, w.N, w.d)
    k = k.reshape(-1, w.N, w.d)
    v = v.reshape(-1, w.N, w.d)
    threads = oracle.max_threads()
    # calibration: a strided eighth of one slice's rows
    rows = list(range(0, w.N, 8))
    s0 = order[:1]
    t0 = time.perf_counter()
    oracle.attention(q[s0], k[s0], v[s0], w.scale, w.causal, rows=rows, threads=threads)
    per_slice = (time.perf_counter() - t0) * 8
    n_sl = int(max(1, min(len(order), round(target_s / max(per_slice, 1e-6)))))
    sl = order[:n_sl]
    t0 = time.perf_counter()
    oracle.attention(q[sl], k[sl], v[sl], w.scale, w.causal, threads=threads)
    secs = time.perf_counter() - t0
    keys = (w.N * (w.N + 1) // 2) if w.causal else w.N * w.N
    flops = 4.0 * w.d * keys * n_sl
    # The fp32 1x1x128x64 workload whole, on one thread (median of 5 runs).
    from exact_attention_124_amd.workloads import WORKLOADS
    ws = WORKLOADS["small_fp32"]
    qs, ks, vs = make_qkv(ws.B, ws.H, ws.N, ws.d, ws.dtype, ws.seed, ws.q_mult)
    ts = []
    for _ in range(5):
        t0 = time.perf_counter()
        oracle.attention(qs, ks, vs, ws.scale, ws.causal, threads=1)
        ts.append(time.perf_counter() - t0)
    small_ms = sorted(ts)[2] * 1e3
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"{w.name}: all {w.N} query rows of {n_sl} seeded (b,h) slices of {w.B * w.H}, "
                       f"fp64, {secs:.1f} s"),
            "seconds": round(secs, 3), "flop": flops,
            "small_fp32_one_thread_ms": round(small_ms, 3)}


def n_sweep(ea):
    """One fused and one unfused forward per sequence length, B=1 H=32 d=128
    non-causal, then a 1 GiB copy: a profiler's per-dispatch byte counters then
    show how each path's HBM traffic grows with N."""
    import dataclasses
    import torch
    from exact_attention_124_amd.workloads import WORKLOADS
    for N in (1024, 2048, 4096, 8192, 16384):
        w = dataclasses.replace(WORKLOADS[HEADLINE], name=f"n_sweep_{N}", B=1, H=32, N=N)
        bench_fused(ea, w, 1, 0)
        bench_unfused(ea, w, 1, 0)
        torch.cuda.synchronize()
        log(f"[bench] n-sweep N={N} done")
    copy_calibration(reps=2)


HEADLINE_KERNEL = "attn::fwd_bf16::persistent_kernel<128, false>"
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def write_traffic_record(fetch_csv: str, write_csv: str) -> dict:
    """Turn two rocprofv3 ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` counter
    CSVs of ``bench.py --quick --calibrate-copy`` into the traffic record read
    by the roofline entry: per-dispatch KiB of the headline kernel, each scaled
    by what the same counter reads for the 1 GiB device copy (2**30 bytes read
    and written).  Host-only; writes profiles/attn_fwd_bf16_dense_8k_traffic.json."""
    import collections
    import csv

    def per_dispatch(path):
        kern = collections.defaultdict(float)
        copies = []
        names = {}
        copy_acc = collections.defaultdict(float)
        for r in csv.DictReader(open(path)):
            d = int(r["Dispatch_Id"])
            if HEADLINE_KERNEL in r["Kernel_Name"]:
                kern[d] += float(r["Counter_Value"])
                names[d] = r["Kernel_Name"]
            elif COPY_KERNEL in r["Kernel_Name"]:
                copy_acc[d] += float(r["Counter_Value"])
        copies = [copy_acc[d] for d in sorted(copy_acc)]
        return [kern[d] for d in sorted(kern)], copies, next(iter(names.values()), None)

    fetch, fcopy, kname = per_dispatch(fetch_csv)
    write, wcopy, _ = per_dispatch(write_csv)
    if not fetch or not write or not fcopy or not wcopy:
        raise SystemExit("no headline-kernel or copy dispatches in the counter files")
    # the 1 GiB copy dominates: take the largest copy dispatch of each run
    fscale = (1 << 30) / 1024 / max(fcopy)
    wscale = (1 << 30) / 1024 / max(wcopy)
    fk = sum(fetch) / len(fetch)
    wk = sum(write) / len(write)
    w = __import__("exact_attention_124_amd.workloads", fromlist=["WORKLOADS"]).WORKLOADS[HEADLINE]
    rec = {
        "kernel": kname,
        "kernel_source_sha256": kernel_source_hash(),
        "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
        "fetch_kib_per_dispatch_each": fetch, "write_kib_per_dispatch_each": write,
        "copy_fetch_kib_per_GiB": max(fcopy), "copy_write_kib_per_GiB": max(wcopy),
        "fetch_scale": fscale, "write_scale": wscale,
        "read_bytes_per_launch": fk * 1024 * fscale, "write_bytes_per_launch": wk * 1024 * wscale,
        "bytes_per_launch": fk * 1024 * fscale + wk * 1024 * wscale,
        "algorithmic_read_bytes": 3 * w.B * w.H * w.N * w.d * 2,
        "algorithmic_write_bytes": w.B * w.H * w.N * w.d * 2 + w.B * w.H * w.N * 4,
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o pmc -- "
            "python3 bench.py --quick --steps 3 --warmup 1 --calibrate-copy",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o pmc -- "
            "python3 bench.py --quick --steps 3 --warmup 1 --calibrate-copy",
            f"python3 bench.py --write-traffic-record {fetch_csv} {write_csv}",
        ],
    }
    with open(TRAFFIC_RECORD, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--quick", action="store_true", help="headline only: no sweep, unfused or CPU leg")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--bwd-only", action="store_true",
                    help="only the backward legs (for kernel traces of the backward launches)")
    ap.add_argument("--masked-only", action="store_true",
                    help="only the masked / biased forward legs")
    ap.add_argument("--fp8-only", action="store_true",
                    help="only the fp8 forward legs (for kernel traces of that kernel)")
    ap.add_argument("--fused-only", metavar="WORKLOAD", default=None,
                    help="only time the fused forward on the named workload (for counter runs on it)")
    ap.add_argument("--n-sweep", action="store_true",
                    help="only run fused and unfused once each at B=1 H=32 d=128 for N = 1k..16k "
                         "(for HBM byte counters), plus the copy calibration")
    ap.add_argument("--write-traffic-record", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="host only: write the headline kernel's HBM byte record from two rocprofv3 "
                         "counter CSVs (FETCH_SIZE, WRITE_SIZE) of `--quick --calibrate-copy` runs")
    args = ap.parse_args()

    if args.write_traffic_record:
        rec = write_traffic_record(*args.write_traffic_record)
        print(json.dumps({k: rec[k] for k in ("kernel", "read_bytes_per_launch", "write_bytes_per_launch",
                                              "bytes_per_launch", "fetch_scale", "write_scale")}))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the kernel on one GPU's share of the work); "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_124_amd as ea
    from exact_attention_124_amd.workloads import ORDER, WORKLOADS

    ea.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.n_sweep:
        n_sweep(ea)
        return
    if args.bwd_only:
        print(json.dumps({"backward": backward_legs(ea, WORKLOADS, args.steps, args.warmup)}), flush=True)
        return
    if args.masked_only:
        print(json.dumps({"masked": masked_legs(ea, WORKLOADS, args.steps, args.warmup)}), flush=True)
        return
    if args.fused_only:
        ww = WORKLOADS[args.fused_only]
        tot, pl = bench_fused(ea, ww, args.steps, args.warmup)
        lm = sum(pl) / len(pl)
        print(json.dumps({"fused": {"workload": ww.name, "desc": ww.describe(), "launch_ms": round(lm, 4),
                                    "TFLOP/s": round(ww.flops / (lm * 1e-3) / 1e12, 2)}}), flush=True)
        return
    if args.fp8_only:
        print(json.dumps({"fp8": fp8_legs(ea, WORKLOADS, args.steps, args.warmup)}), flush=True)
        return

    w = WORKLOADS[HEADLINE]
    log(f"[bench] headline: {w.describe()}, warmup {args.warmup}, steps {args.steps}")
    total_ms, per = bench_fused(ea, w, args.steps, args.warmup)
    ms_step = total_ms / args.steps
    launch_ms = sum(per) / len(per)
    value = w.flops / (ms_step * 1e-3) / 1e12
    achieved = w.flops / (launch_ms * 1e-3) / 1e12
    traffic, traffic_src = traffic_from_record()
    log(f"[bench] {ms_step:.3f} ms/step, launch {launch_ms:.3f} ms, {achieved:.1f} TFLOP/s")

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1) Q, K, V, rounded to bf16)",
        "device": device_info(),
        "config": {"workload": f"{w.name}: {w.describe()}", "B": w.B, "H": w.H, "N": w.N,
                   "d": w.d, "causal": w.causal, "parallelism": "single GPU"},
        "pct_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "traffic_source": traffic_src,
                     "kernel": HEADLINE_KERNEL,
                     "avg_launch_ms": round(launch_ms, 4),
                     "flop_per_launch": w.flops},
    }

    if args.calibrate_copy:
        copy_calibration()

    if not args.quick:
        sweep = []
        for name in ORDER:
            if name == HEADLINE:
                continue
            ww = WORKLOADS[name]
            tot, pl = bench_fused(ea, ww, max(5, args.steps // 2), 3)
            pm = sum(pl) / len(pl)
            if pm < 0.05:  # launches of a few microseconds: average many more
                tot, pl = bench_fused(ea, ww, 200, 20)
                pm = sum(pl) / len(pl)
            # Per-call time of back-to-back binding calls between two events;
            # a per-launch event pair adds its own GPU time, which matters for
            # calls of a few microseconds.
            calls = 200 if pm < 1.0 else max(5, args.steps // 2)
            lm, host_us = bench_fused_back_to_back(ea, ww, calls)
            gm = bench_fused_graph(ea, ww) if lm < 1.0 else None
            sweep.append({"workload": name, "desc": ww.describe(), "launch_ms": round(lm, 4),
                          "TFLOP/s": round(ww.flops / (lm * 1e-3) / 1e12, 2),
                          "frac_bf16_peak": round(ww.flops / (lm * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "event_pair_launch_ms": round(pm, 4),
                          "binding_host_us_per_call": round(host_us, 2)})
            if gm is not None:
                sweep[-1].update({"graph_ms_per_call": round(gm, 4),
                                  "graph_TFLOP/s": round(ww.flops / (gm * 1e-3) / 1e12, 2)})
                if pm < 0.05:
                    sweep[-1]["raw_c_abi_event_pair_launch_ms"] = round(bench_fused_raw(ea, ww, 200, 20), 4)
            if name in ("gpt2_heads_bf16", "causal_2k_bf16"):
                cm = bench_fused_cold(ea, ww)
                sweep[-1].update({"cold_launch_ms": round(cm, 4),
                                  "cold_note": "median of 10 calls, each after a 512 MiB buffer write"})
            log(f"[bench] sweep {name}: {lm:.4f} ms per call back to back, {pm:.4f} ms per launch"
                " between its own events"
                + (f", {gm:.4f} ms per call in a graph" if gm is not None else "")
                + f", {sweep[-1]['TFLOP/s']} TFLOP/s")
        sweep.insert(3, {"workload": HEADLINE, "desc": w.describe(), "launch_ms": round(launch_ms, 4),
                         "TFLOP/s": round(achieved, 2),
                         "frac_bf16_peak": round(achieved / PEAK_BF16_TFLOPS, 4)})
        result["sweep"] = sweep

        tot, pl = bench_unfused(ea, w, 5, 2)
        um = sum(pl) / len(pl)
        s_bytes = w.B * w.H * w.N * w.N * 2
        io_bytes = 4 * w.B * w.H * w.N * w.d * 2 + 4 * w.B * w.H * w.N
        alg = 4 * s_bytes + io_bytes
        result["unfused"] = {"ms": round(um, 3), "algorithmic_bytes": alg,
                             "GB/s": round(alg / (um * 1e-3) / 1e9, 1),
                             "frac_hbm_peak": round(alg / (um * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                             "TFLOP/s": round(w.flops / (um * 1e-3) / 1e12, 2),
                             "fused_speedup": round(um / launch_ms, 2)}
        log(f"[bench] unfused: {um:.3f} ms, {result['unfused']['GB/s']} GB/s")

        result["backward"] = backward_legs(ea, WORKLOADS, 5, 2)
        result["fp8"] = fp8_legs(ea, WORKLOADS, 10, 3)
        result["masked"] = masked_legs(ea, WORKLOADS, 10, 3)
        result["fusion"] = fusion_leg(ea, 20, 5)

        if not args.no_cpu:
            log("[bench] timing the CPU oracle on a bounded sample")
            result["cpu_baseline"] = cpu_baseline(w)
            log(f"[bench] cpu: {result['cpu_baseline']['value']:.6f} TFLOP/s")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
