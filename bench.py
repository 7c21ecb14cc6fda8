"""Benchmark of the exact-attention forward on one MI355X.

One step = one ``attn_fwd`` call over the long-context causal workload
(B=1, H=16, N=8192, d=128, bf16, scale 1/sqrt(128)) with seeded synthetic
N(0, 1) inputs already resident in device memory.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-bwd]
                    [--no-window] [--no-sparse] [--no-variants] [--no-kv-outer]

The reported throughput counts algorithmic FLOPs only: 4 * d * (visible query-key
pairs) * B * H, i.e. the two matrix products over the causal triangle.

The same line carries, under "attn_bwd", the backward pass timed the same way
on its own workload (B=4, H=16, N=4096, d=128, bf16, causal), counted as
10 * d * pairs * B * H algorithmic FLOPs (S and dP recomputed, dV, dQ, dK), and
under "attn_fwd_window" the forward of the long-context head with a causal
sliding window of 1024 keys (4 * d * windowed pairs * B * H FLOPs), and under
"attn_fwd_kv_outer" the bench workload run in the original key/value-outer loop
order (the comparison of the two orders' memory traffic; same FLOP count),
and under "attn_fwd_block_sparse" the head under a band + global + random
64x64 block mask (4 * d * visible pairs FLOPs).  "variants" times the head in
the library's other forms, and "configs" the forward on each of the five
parity workloads at full size.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (bf16, causal, T=8192, d=128) and % of MFMA peak"
WORKLOAD = "long_causal_bf16"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, published
# graph replays after the requested warm-up calls, so the timed calls run at
# the clock the GPU holds under sustained load
WARMUP_FLOOR_S = 0.5
KERNEL_SOURCES = ("fwd_mfma.hip", "mfma_common.hpp")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "fwd_long_causal_bf16_traffic.md")
COUNTER_PROFILE = os.path.join(ROOT, "profiles", "fwd_long_causal_bf16_counters.md")
NOMINAL_SCLK_MHZ = 2400.0       # the clock the published peaks are quoted at


def progress(msg):
    """A progress line on stderr (stdout carries the one JSON line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def code_of(text: str) -> str:
    """A C++ source without its comments and blank lines, so that a comment edit
    leaves the kernel's identity unchanged."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "io_aware_exact_12_amd", "csrc", f)) as fh:
            h.update(code_of(fh.read()).encode())
    return h.hexdigest()[:16]


def _profile_fields(path, keys):
    """Machine-readable ``key: value`` lines of a committed rocprofv3 summary.

    Returns None when the file is missing, lacks a key, or was taken on a
    different version of the kernel source than the one being benchmarked.
    """
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m_hash or m_hash.group(1) != kernel_source_hash():
        return None
    out = {}
    for k in keys:
        m = re.search(rf"^{k}:\s*([0-9.eE+-]+)\s*$", text, flags=re.M)
        if not m:
            return None
        out[k] = float(m.group(1))
    return out


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by the copy-kernel calibration)."""
    f = _profile_fields(TRAFFIC_PROFILE, ["hbm_bytes_per_launch"])
    return None if f is None else f["hbm_bytes_per_launch"]


def measured_counters():
    """MFMA busy share, shader clock and VALU / LDS instructions per MFMA of the
    bench kernel, from the committed rocprofv3 SQ counter summary."""
    return _profile_fields(COUNTER_PROFILE, ["mfma_busy_share", "sclk_mhz", "valu_insts_per_mfma",
                                             "lds_insts_per_mfma"])


def cpu_baseline(w, x, budget_s=12.0):
    """Time the float64 oracle on the host on whole heads of the same workload."""
    import numpy as np

    import oracle
    blas = "unknown"
    try:
        import threadpoolctl
        info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        threads = max(int(i.get("num_threads", 1)) for i in info) if info else 1
        blas = ", ".join(sorted({str(i.get("internal_api")) for i in info})) or blas
    except Exception:  # threadpoolctl missing or no BLAS pool found
        threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    heads = 0
    pairs = w.N * (w.N + 1) // 2 if w.causal else w.N * w.N
    # whole heads in order, starting over after the last one, until the budget is spent
    while time.perf_counter() - t0 < budget_s:
        h = heads % (w.B * w.H)
        b, h = divmod(h, w.H)
        oracle.dense_fwd(x["q"][b, h], x["k"][b, h], x["v"][b, h], causal=w.causal, scale=w.scale)
        heads += 1
    dt = time.perf_counter() - t0
    flops = 4.0 * w.d * pairs * heads
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"dense float64 oracle on {heads} head evaluations, {heads / (w.B * w.H):.2f} "
                      f"passes over the {w.B * w.H} heads (all {w.N} rows each, full N x N scores "
                      f"computed, causal-visible FLOPs counted), {dt:.1f} s",
            "seconds": round(dt, 3), "blas": blas, "affinity_cores": len(os.sched_getaffinity(0))}


def time_graph(step, steps, warmup, torch, floor_s=WARMUP_FLOOR_S):
    """Capture `steps` calls of step() in one HIP graph and time one replay.

    Warm-up: exactly `warmup` eager calls, then graph replays until at least
    `floor_s` seconds of load have passed (sustained load lowers the shader
    clock, so a short warm-up would time a cold GPU).  Returns ms per call of
    the timed replay and a dict describing the warm-up actually run.
    """
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n_rep = 0
    while True:
        graph.replay()
        n_rep += 1
        if n_rep % 4 == 0 or floor_s <= 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= floor_s:
                break
    torch.cuda.synchronize()
    floor_dt = time.perf_counter() - t0
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    graph.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, {"calls": warmup, "floor_calls": n_rep * steps,
                                             "floor_s": round(floor_dt, 3)}


def bwd_record(fa, workloads, torch, steps, warmup):
    """Backward pass on its own workload, timed like the forward."""
    w = workloads.WORKLOADS["fwd_bwd_causal_bf16"]
    x = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (torch.from_numpy(x[n]).to(dev).to(torch.bfloat16).contiguous()
                   for n in ("q", "k", "v", "do"))
    o, lse = fa.attn_fwd(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.bwd_workspace_bytes(w.B, w.H, w.N, w.d, fa.BF16), dtype=torch.uint8,
                     device=dev)

    def step():
        fa.attn_bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv,
                    workspace=ws, stream=torch.cuda.current_stream(dev))

    ms, warm = time_graph(step, steps, warmup, torch)
    assert all(torch.isfinite(t).all().item() for t in (dq, dk, dv))
    flops = w.bwd_flops()
    tflops = flops / (ms * 1e-3) / 1e12
    return {"metric": "attention bwd TFLOP/s (bf16, causal, T=4096, d=128)",
            "value": round(tflops, 2), "unit": "TFLOP/s", "steps": steps, "warmup": warm["calls"],
            "warmup_floor": {"calls": warm["floor_calls"], "seconds": warm["floor_s"]},
            "ms_per_step": round(ms, 5),
            "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                       "mask": "causal", "scale": w.scale,
                       "inputs": "Q, K, V, dO i.i.d. N(0,1) rounded to bf16, seed 5"},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                         "kernels": "bwd_dq_pair + bwd_dkdv_pair (one call)",
                         "algorithmic_flops_per_launch": flops}}


def window_record(fa, workloads, torch, steps, warmup):
    """Sliding-window forward on its own workload, timed like the forward."""
    w = workloads.WORKLOADS["long_window_bf16"]
    x = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(torch.bfloat16).contiguous() for n in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    def step():
        fa.attn_fwd(q, k, v, causal=True, window=w.window, scale=w.scale, out=o, lse=lse,
                    stream=torch.cuda.current_stream(dev))

    ms, warm = time_graph(step, steps, warmup, torch)
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    flops = w.fwd_flops()
    tflops = flops / (ms * 1e-3) / 1e12
    return {"metric": f"attention fwd TFLOP/s (bf16, causal sliding window {w.window}, "
                      f"T={w.N}, d={w.d})",
            "value": round(tflops, 2), "unit": "TFLOP/s", "steps": steps, "warmup": warm["calls"],
            "warmup_floor": {"calls": warm["floor_calls"], "seconds": warm["floor_s"]},
            "ms_per_step": round(ms, 5),
            "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                       "mask": "causal", "window": w.window, "scale": w.scale,
                       "inputs": "Q, K, V i.i.d. N(0,1) rounded to bf16, seed 6"},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                         "kernel": "fwd_kernel<bf16, d=128, causal, window>",
                         "algorithmic_flops_per_launch": flops}}


def sparse_record(fa, workloads, torch, steps, warmup):
    """Block-sparse forward on its own workload (the bench head under a band +
    global + random block mask), timed like the forward."""
    w = workloads.WORKLOADS["long_sparse_bf16"]
    x = workloads.make_inputs(w)
    mask = workloads.block_sparse_mask(w.N, w.H, *w.sparse)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(torch.bfloat16).contiguous() for n in "qkv")
    bm = torch.from_numpy(mask).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    def step():
        fa.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, block_mask=bm,
                    stream=torch.cuda.current_stream(dev))

    ms, warm = time_graph(step, steps, warmup, torch)
    assert torch.isfinite(o).all().item()
    flops = 4 * w.d * workloads.sparse_pairs(mask, w.N, w.causal) * w.B
    tflops = flops / (ms * 1e-3) / 1e12
    band, n_global, n_random, _ = w.sparse
    return {"metric": f"attention fwd TFLOP/s (bf16, block-sparse {100 * float(mask.mean()):.1f} % of "
                      f"64x64 blocks, T={w.N}, d={w.d})",
            "value": round(tflops, 2), "unit": "TFLOP/s", "steps": steps, "warmup": warm["calls"],
            "warmup_floor": {"calls": warm["floor_calls"], "seconds": warm["floor_s"]},
            "ms_per_step": round(ms, 5),
            "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                       "mask": "causal" if w.causal else "none",
                       "block_mask": f"band {band}, {n_global} global, {n_random} random blocks per "
                                     f"query block, per head",
                       "scale": w.scale, "inputs": "Q, K, V i.i.d. N(0,1) rounded to bf16, seed 7"},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                         "kernel": "fwd_kernel<bf16, d=128, block-sparse>",
                         "algorithmic_flops_per_launch": flops}}


def variants_record(fa, workloads, torch, steps, warmup):
    """The bench head (B=1, H=16, N=8192, causal, bf16) in the other forms the
    library takes, each timed like the forward: a [B, N, H, d] view (strided
    call), d = 96, d = 256 (also with a window of 1024 keys) and d_v = 64 with
    d = 128 (forward and backward), and the
    backward of the block-sparse and sliding-window workloads (10 d FLOPs per
    visible pair)."""
    dev = torch.device("cuda:0")
    out = {}
    w = workloads.WORKLOADS[WORKLOAD]

    def rec(name, step, flops, s=steps, wm=warmup):
        ms, _ = time_graph(step, s, wm, torch)
        tf = flops / (ms * 1e-3) / 1e12
        out[name] = {"ms_per_step": round(ms, 5), "TFLOP/s": round(tf, 2),
                     "frac_of_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)}

    def dev_bf16(a):
        return torch.from_numpy(a).to(dev).to(torch.bfloat16)

    # strided: q, k, v as [B, H, N, d] views of [B, N, H, d] memory
    x = workloads.make_inputs(w)
    qb, kb, vb = (dev_bf16(x[n].transpose(0, 2, 1, 3).copy()).transpose(1, 2) for n in "qkv")
    ob = torch.empty_like(qb)
    rec("fwd_bshd_d128", lambda: fa.attn_fwd(qb, kb, vb, causal=True, out=ob), w.fwd_flops())
    # d = 96
    x96 = workloads.random_inputs(1, 16, 8192, 96, "bf16", seed=11)
    q96, k96, v96 = (dev_bf16(x96[n]).contiguous() for n in "qkv")
    o96 = torch.empty_like(q96)
    rec("fwd_d96", lambda: fa.attn_fwd(q96, k96, v96, causal=True, out=o96),
        4 * 96 * (8192 * 8193 // 2) * 16)
    # d = 256 (its own kernel)
    x256 = workloads.random_inputs(1, 16, 8192, 256, "bf16", seed=13)
    q256, k256, v256 = (dev_bf16(x256[n]).contiguous() for n in "qkv")
    del x256
    o256 = torch.empty_like(q256)
    rec("fwd_d256", lambda: fa.attn_fwd(q256, k256, v256, causal=True, out=o256),
        4 * 256 * (8192 * 8193 // 2) * 16)
    lse256 = torch.empty((1, 16, 8192), dtype=torch.float32, device=dev)
    fa.attn_fwd(q256, k256, v256, causal=True, out=o256, lse=lse256)
    do256 = torch.randn_like(o256)
    g256 = [torch.empty_like(q256) for _ in range(3)]
    ws256 = torch.empty(fa.bwd_workspace_bytes(1, 16, 8192, 256, fa.BF16), dtype=torch.uint8, device=dev)
    rec("bwd_d256", lambda: fa.attn_bwd(q256, k256, v256, o256, lse256, do256, causal=True, dq=g256[0],
                                        dk=g256[1], dv=g256[2], workspace=ws256),
        10 * 256 * (8192 * 8193 // 2) * 16, s=10, wm=3)
    # d = 256 with the sliding window of 1024 keys: W (W + 1) / 2 + (N - W) W pairs per head
    wpairs = (1024 * 1025 // 2 + (8192 - 1024) * 1024) * 16
    rec("fwd_d256_window", lambda: fa.attn_fwd(q256, k256, v256, causal=True, window=1024, out=o256),
        4 * 256 * wpairs)
    lse256w = torch.empty_like(lse256)
    fa.attn_fwd(q256, k256, v256, causal=True, window=1024, out=o256, lse=lse256w)
    rec("bwd_d256_window", lambda: fa.attn_bwd(q256, k256, v256, o256, lse256w, do256, causal=True,
                                               window=1024, dq=g256[0], dk=g256[1], dv=g256[2],
                                               workspace=ws256),
        10 * 256 * wpairs, s=10, wm=3)
    # d_v = 64 with d = 128: 2 d + 2 d_v FLOPs per visible pair
    xv = workloads.random_inputs(1, 16, 8192, 64, "bf16", seed=12)
    q, k = (dev_bf16(x[n]).contiguous() for n in "qk")
    v64 = dev_bf16(xv["v"]).contiguous()
    o64 = torch.empty((1, 16, 8192, 64), dtype=torch.bfloat16, device=dev)
    rec("fwd_d128_dv64", lambda: fa.attn_fwd(q, k, v64, causal=True, out=o64),
        2 * (128 + 64) * (8192 * 8193 // 2) * 16)
    # its backward: S, dQ, dK over d, dP, dV over d_v (6 d + 4 d_v FLOPs per visible pair)
    lse64 = torch.empty((1, 16, 8192), dtype=torch.float32, device=dev)
    fa.attn_fwd(q, k, v64, causal=True, out=o64, lse=lse64)
    do64 = torch.randn_like(o64)
    g64 = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v64)]
    ws64 = torch.empty(fa.bwd_workspace_bytes(1, 16, 8192, 128, fa.BF16), dtype=torch.uint8, device=dev)
    rec("bwd_d128_dv64", lambda: fa.attn_bwd(q, k, v64, o64, lse64, do64, causal=True, dq=g64[0],
                                             dk=g64[1], dv=g64[2], workspace=ws64),
        (6 * 128 + 4 * 64) * (8192 * 8193 // 2) * 16, s=20, wm=5)
    # backward of the block-sparse and the sliding-window workloads
    for name, wl in (("bwd_block_sparse", "long_sparse_bf16"), ("bwd_window", "long_window_bf16")):
        ww = workloads.WORKLOADS[wl]
        xw = workloads.make_inputs(ww)
        qq, kk, vv = (dev_bf16(xw[n]).contiguous() for n in "qkv")
        do = torch.randn_like(qq)
        kw = {}
        if ww.sparse is not None:
            mask = workloads.block_sparse_mask(ww.N, ww.H, *ww.sparse)
            kw["block_mask"] = torch.from_numpy(mask).to(dev)
            pairs = workloads.sparse_pairs(mask, ww.N, ww.causal)
        else:
            kw["window"] = ww.window
            pairs = ww.pairs() * ww.H
        oo, ll = fa.attn_fwd(qq, kk, vv, causal=ww.causal, **kw)
        g = [torch.empty_like(qq) for _ in range(3)]
        wsq = fa.bwd_block_sparse_workspace_bytes if ww.sparse is not None else fa.bwd_workspace_bytes
        ws = torch.empty(wsq(ww.B, ww.H, ww.N, ww.d, fa.BF16), dtype=torch.uint8,
                         device=dev)
        rec(name, lambda: fa.attn_bwd(qq, kk, vv, oo, ll, do, causal=ww.causal, dq=g[0], dk=g[1],
                                      dv=g[2], workspace=ws, **kw),
            10 * ww.d * pairs * ww.B, s=20, wm=5)
    return out


def configs_record(fa, workloads, torch, steps, warmup):
    """The forward on each of the five parity workloads, at full size, timed
    like the bench head: tiny fp32 (B=1, H=1, N=256, d=64, unmasked), the
    GPT-2-small shape (B=8, H=12, T=1024, d=64, causal, bf16), the bench head,
    the ragged sharp fp16 case (B=2, H=8, N=4097, d=128, unmasked) and the
    forward of the fwd+bwd case (B=4, H=16, T=4096, d=128, causal, bf16).
    fp32 inputs run on the fp64-VALU path; their share of the bf16 MFMA peak
    is not meaningful and is left out."""
    dev = torch.device("cuda:0")
    tdt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
    out = {}
    for name in ("tiny_fp32_full", "gpt2s_causal_bf16", "long_causal_bf16", "ragged_sharp_fp16",
                 "fwd_bwd_causal_bf16"):
        w = workloads.WORKLOADS[name]
        x = workloads.make_inputs(w)
        q, k, v = (torch.from_numpy(x[n]).to(dev).to(tdt[w.dtype]).contiguous() for n in "qkv")
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

        def step():
            fa.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse,
                        stream=torch.cuda.current_stream(dev))

        ms, _ = time_graph(step, steps, warmup, torch)
        tf = w.fwd_flops() / (ms * 1e-3) / 1e12
        out[name] = {"dtype": w.dtype, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                     "mask": "causal" if w.causal else "none", "ms_per_step": round(ms, 5),
                     "TFLOP/s": round(tf, 2),
                     "frac_of_mfma_peak": None if w.dtype == "fp32" else round(tf / PEAK_BF16_TFLOPS, 4)}
    return out


def kv_outer_record(fa, workloads, torch, steps, warmup):
    """The bench workload in the key/value-outer loop order (attn_fwd_kv_outer),
    timed over a few calls: each is tens of milliseconds."""
    w = workloads.WORKLOADS[WORKLOAD]
    x = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(torch.bfloat16).contiguous() for n in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.kv_outer_workspace_bytes(w.B, w.H, w.N, w.d, fa.BF16), dtype=torch.uint8,
                     device=dev)

    def step():
        fa.attn_fwd_kv_outer(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=ws,
                             stream=torch.cuda.current_stream(dev))

    ms, warm = time_graph(step, steps, warmup, torch)
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    flops = w.fwd_flops()
    tflops = flops / (ms * 1e-3) / 1e12
    return {"metric": "attention fwd TFLOP/s, key/value-outer loop order (bf16, causal, T=8192, d=128)",
            "value": round(tflops, 2), "unit": "TFLOP/s", "steps": steps, "warmup": warm["calls"],
            "warmup_floor": {"calls": warm["floor_calls"], "seconds": warm["floor_s"]},
            "ms_per_step": round(ms, 5),
            "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "mask": "causal",
                       "order": "kv_outer", "workgroups": w.B * w.H},
            "kernel": "fwd_kv_outer_kernel<bf16, d=128, causal>",
            "algorithmic_flops_per_launch": flops}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # untimed eager calls; graph replays then add at least WARMUP_FLOOR_S of
    # load, which the GPU needs to reach its sustained clock
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward measurement")
    ap.add_argument("--bwd-steps", type=int, default=40)
    ap.add_argument("--bwd-warmup", type=int, default=10)
    ap.add_argument("--no-window", action="store_true",
                    help="skip the sliding-window forward measurement")
    ap.add_argument("--window-steps", type=int, default=200)
    ap.add_argument("--window-warmup", type=int, default=10)
    ap.add_argument("--no-sparse", action="store_true",
                    help="skip the block-sparse forward measurement")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the strided / d = 96 / d_v = 64 / sparse and window backward timings "
                         "and the per-workload forward timings")
    ap.add_argument("--no-kv-outer", action="store_true",
                    help="skip the key/value-outer loop-order measurement")
    ap.add_argument("--kv-steps", type=int, default=3)
    ap.add_argument("--kv-warmup", type=int, default=2)
    ap.add_argument("--kv-only", action="store_true",
                    help="run only the key/value-outer measurement (for profiling its kernel)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (3 times), "
                         "the reference kernel for scaling HBM byte counters, and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(attention shards over (batch, head) with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import io_aware_exact_12_amd as fa
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy_mb:
        n = args.calibrate_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n * 4, "launches": 3}), flush=True)
        return
    if args.kv_only:
        print(json.dumps({"attn_fwd_kv_outer": kv_outer_record(fa, workloads, torch, args.kv_steps,
                                                               args.kv_warmup)}), flush=True)
        return
    w = workloads.WORKLOADS[WORKLOAD]
    x = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(torch.bfloat16).contiguous() for n in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    # The timed steps are replayed from a HIP graph so that host launch overhead
    # (Python, and a profiler's per-dispatch hooks) cannot open gaps between
    # kernels: the events then bracket back-to-back forward kernels only.
    def step():
        fa.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse,
                    stream=torch.cuda.current_stream(dev))

    ms, warm = time_graph(step, args.steps, args.warmup, torch)
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    progress(f"forward {w.name}: {ms * 1e3:.1f} us per call")

    flops = w.fwd_flops()
    tflops = flops / (ms * 1e-3) / 1e12
    traffic = measured_traffic()
    counters = measured_counters()
    record = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_floor": {"calls": warm["floor_calls"], "seconds": warm["floor_s"]},
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "mask": "causal" if w.causal else "none", "scale": w.scale,
                   "inputs": "Q, K, V i.i.d. N(0,1) rounded to bf16, seed 3"},
        "pct_of_mfma_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     # HBM bytes per launch measured by FETCH_SIZE / WRITE_SIZE, over
                     # this run's launch time
                     "hbm_gbs": None if traffic is None else round(traffic / (ms * 1e-3) / 1e9, 1),
                     "hbm_peak_gbs": PEAK_HBM_GBS,
                     # MFMA pipe busy share and shader clock from the SQ counters
                     # (SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE) of the same kernel
                     "mfma_busy": None if counters is None else counters["mfma_busy_share"],
                     "sclk_mhz": None if counters is None else counters["sclk_mhz"],
                     "frac_at_sclk": None if counters is None else round(
                         tflops / (PEAK_BF16_TFLOPS * counters["sclk_mhz"] / NOMINAL_SCLK_MHZ), 4),
                     "valu_insts_per_mfma": None if counters is None else counters["valu_insts_per_mfma"],
                     "lds_insts_per_mfma": None if counters is None else counters["lds_insts_per_mfma"],
                     "kernel": "fwd_kernel<bf16, d=128, causal>",
                     "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": w.fwd_bytes(),
                     "kernel_source_sha256_16": kernel_source_hash()},
    }
    if not args.no_bwd:
        record["attn_bwd"] = bwd_record(fa, workloads, torch, args.bwd_steps, args.bwd_warmup)
        progress("backward done")
    if not args.no_window:
        record["attn_fwd_window"] = window_record(fa, workloads, torch, args.window_steps,
                                                  args.window_warmup)
        progress("window forward done")
    if not args.no_sparse:
        record["attn_fwd_block_sparse"] = sparse_record(fa, workloads, torch, args.window_steps,
                                                        args.window_warmup)
        progress("block-sparse forward done")
    if not args.no_variants:
        record["variants"] = variants_record(fa, workloads, torch, 50, 10)
        progress("variants done")
        record["configs"] = configs_record(fa, workloads, torch, 50, 10)
        progress("per-workload forwards done")
    if not args.no_kv_outer:
        record["attn_fwd_kv_outer"] = kv_outer_record(fa, workloads, torch, args.kv_steps,
                                                      args.kv_warmup)
        progress("key/value-outer forward done")
    if not args.no_cpu_baseline:
        record["cpu_baseline"] = cpu_baseline(w, x)
        progress("cpu baseline done")
        record["cpu_baseline"]["gpu_over_cpu"] = round(record["value"] / record["cpu_baseline"]["value"], 1)
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
