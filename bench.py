#!/usr/bin/env python3
"""Benchmark of the rotated 1-bit GEMV (decode) and GEMM (prefill) on one GPU.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

A step is one pass of the whole hot path over one input: for the headline
workload (decode ffn_gate, M=1, K=5120, N=17408) that is the head
permutation (none for this width), the signs, the 1024-block transform, the
bit unpack, the per-group partial sums times their scales and the row
reduction -- one activation in, y out.  Every step reads a different copy of
the weights (the copies together exceed the 256 MB last-level cache), so the
timed traffic comes from HBM.  Inputs are resident in device memory before
timing starts.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "1-bit GEMV HBM GB/s (% of peak) at M=1; prefill TFLOP/s (% MFMA) at M=1024"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
CACHE_BYTES = 256 << 20      # last-level (Infinity) cache to defeat


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemv_bytes(N, K):
    """Algorithmic bytes of one GEMV: 1-bit weights, fp32 scales, x', y."""
    return N * K // 8 + N * (K // 128) * 4 + K * 4 + N * 4


def graph_time(torch, fn, iters, warmup, dev, check=None):
    """Average ms per call of fn(i) over `iters` calls.

    The calls are captured once into a HIP graph (so the host's launch cost
    does not starve the GPU on microsecond kernels) and replayed; the time is
    taken with HIP events recorded on the stream the graph runs on, with a
    device synchronization before and after the timed region.  `check`, if
    given, is called after the warmup replay and after the timed replay to
    compare the graph's results with eager ones."""
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        for i in range(max(warmup, 2)):   # eager warmup; allocates workspaces for s
            fn(i)
    torch.cuda.synchronize()
    g_warm = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_warm, stream=s):
        for i in range(max(warmup, 1)):
            fn(i)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(iters):
            fn(i)
    torch.cuda.synchronize()
    g_warm.replay()
    torch.cuda.synchronize()
    if check is not None:
        check()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    start.record(cur)
    g.replay()
    stop.record(cur)
    torch.cuda.synchronize()
    if check is not None:
        check()
    return start.elapsed_time(stop) / iters


def decode_bench(torch, pq1, wl, dev, steps, warmup):
    import numpy as np
    d = wl.make("ffn_gate")
    N, K = d["N"], d["K"]
    wbytes = d["bits"].nbytes + d["scales"].nbytes
    copies = max(2, -(-2 * CACHE_BYTES // wbytes))
    log(f"[decode] ffn_gate N={N} K={K}: {copies} weight copies ({copies * wbytes / 2**20:.0f} MiB)")
    bits0 = torch.from_numpy(d["bits"].view(np.int32)).to(dev)
    sc0 = torch.from_numpy(d["scales"]).to(dev)
    bits = [bits0.clone() for _ in range(copies)]
    scs = [sc0.clone() for _ in range(copies)]
    x = torch.from_numpy(d["x"][0].copy()).to(dev)
    signs = torch.from_numpy(d["signs"]).to(dev)
    xr = torch.empty(K, dtype=torch.float32, device=dev)
    y = torch.empty(N, dtype=torch.float32, device=dev)

    # load-time repack into the band-interleaved layout (not timed)
    packed = [pq1.pq1_pack_weights(bits[c], scs[c]) for c in range(copies)]
    torch.cuda.synchronize()

    def fused(i):
        pq1.pq1_rotate_gemv(x, signs, bits[i % copies], scs[i % copies], out=y)

    def packed_fused(i):
        pq1.pq1_rotate_gemv_packed(x, signs, packed[i % copies], out=y)

    def packed_split(i):
        pq1.pq1_rotate(x, signs, out=xr)
        pq1.pq1_gemv_packed(xr, packed[i % copies], out=y)

    def packed_gemv_only(i):
        pq1.pq1_gemv_packed(xr, packed[i % copies], out=y)

    def split(i):
        pq1.pq1_rotate(x, signs, out=xr)
        pq1.pq1_gemv(xr, bits[i % copies], scs[i % copies], out=y)

    def gemv_only(i, algo=pq1.PQ1_GEMV_AUTO):
        pq1.pq1_gemv_ex(xr, bits[i % copies], scs[i % copies], algo=algo, out=y)

    def rotate_only(i):
        pq1.pq1_rotate(x, signs, out=xr)

    res = {}
    for name, fn in (("packed_fused", packed_fused), ("packed_split", packed_split),
                     ("fused", fused), ("split", split)):
        # eager reference of this path (all copies hold the same data)
        fn(0)
        torch.cuda.synchronize()
        y_ref = y.clone()

        def check():
            assert torch.allclose(y, y_ref, rtol=0, atol=1e-4 * float(y_ref.abs().max())), \
                "graph replay result differs from the eager result"

        res[name] = graph_time(torch, fn, steps, warmup, dev, check)
        log(f"[decode] step path {name}: {res[name] * 1e3:.3f} us/step")
    pq1.pq1_rotate(x, signs, out=xr)
    kern = {}
    for name, fn in (("gemv_packed", packed_gemv_only),
                     ("gemv_lut", lambda i: gemv_only(i, pq1.PQ1_GEMV_LUT)),
                     ("gemv_expand", lambda i: gemv_only(i, pq1.PQ1_GEMV_EXPAND)),
                     ("rotate", rotate_only)):
        kern[name] = graph_time(torch, fn, steps, warmup, dev)
        log(f"[decode] kernel {name}: {kern[name] * 1e3:.3f} us/launch")
    torch.cuda.synchronize()
    return dict(N=N, K=K, steps=res, kernels=kern, copies=copies)


def prefill_bench(torch, pq1, wl, dev, steps, warmup):
    import numpy as np
    d = wl.make("prefill")
    M, N, K = d["M"], d["N"], d["K"]
    per_copy = d["bits"].nbytes + d["scales"].nbytes + d["x"].nbytes
    copies = max(2, -(-2 * CACHE_BYTES // (per_copy + M * N * 4)))
    log(f"[prefill] M={M} N={N} K={K}: {copies} input copies")
    bits0 = torch.from_numpy(d["bits"].view(np.int32)).to(dev)
    sc0 = torch.from_numpy(d["scales"]).to(dev)
    x0 = torch.from_numpy(d["x"]).to(dev)
    bits = [bits0.clone() for _ in range(copies)]
    scs = [sc0.clone() for _ in range(copies)]
    xs = [x0.clone() for _ in range(copies)]
    signs = torch.from_numpy(d["signs"]).to(dev)
    xb = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)

    # the rotation writes x' as bf16 in the GEMM's operand K order
    def step(i):
        c = i % copies
        pq1.pq1_rotate(xs[c], signs, out_dtype=torch.bfloat16, out=xb, gemm_order=True)
        pq1.pq1_gemm(xb, bits[c], scs[c], out=y, gemm_order=True)

    def gemm_only(i):
        c = i % copies
        pq1.pq1_gemm(xb, bits[c], scs[c], out=y, gemm_order=True)

    def rotate_only(i):
        pq1.pq1_rotate(xs[i % copies], signs, out_dtype=torch.bfloat16, out=xb, gemm_order=True)

    t_step = graph_time(torch, step, steps, warmup, dev)
    t_gemm = graph_time(torch, gemm_only, steps, warmup, dev)
    t_rot = graph_time(torch, rotate_only, steps, warmup, dev)
    flops = 2.0 * M * N * K
    log(f"[prefill] step {t_step:.3f} ms, gemm {t_gemm:.3f} ms ({flops / t_gemm / 1e9:.0f} TFLOP/s), "
        f"rotate {t_rot * 1e3:.1f} us")
    return dict(M=M, N=N, K=K, step_ms=t_step, gemm_ms=t_gemm, rotate_ms=t_rot, flops=flops)


def cpu_baseline(budget_s=12.0):
    """The oracle as it stands, on this host's cores, over a bounded sample of
    the decode ffn_gate step (whole steps, repeated until ~budget_s)."""
    import numpy as np
    import oracle.pq1_oracle as orc
    from gemm_hadamard_rotated_amd import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = 1
    d = wl.make("ffn_gate")
    t0 = time.perf_counter()
    n = 0
    while True:
        xr = orc.rotate(d["x"][0], d["signs"], d["perm"])
        orc.gemv(xr, d["bits"], d["scales"])
        n += 1
        if time.perf_counter() - t0 > budget_s or n >= 20:
            break
    dt = (time.perf_counter() - t0) / n
    b = gemv_bytes(d["N"], d["K"]) + d["K"] * 4
    return dict(value=b / dt / 1e9, unit="GB/s", cores=int(threads), kind="oracle",
                sample=f"{n} whole decode ffn_gate steps (rotate + GEMV, fp64 numpy), "
                       f"{dt:.2f} s per step")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--prefill-steps", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the GEMV shards by output rows with no exchange; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from gemm_hadamard_rotated_amd import pq1, workloads as wl
    dev = torch.device("cuda:0")
    pq1.load_library()

    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))
        return

    dec = decode_bench(torch, pq1, wl, dev, args.steps, args.warmup)
    N, K = dec["N"], dec["K"]
    best_path = min(dec["steps"], key=dec["steps"].get)
    ms = dec["steps"][best_path]
    step_bytes = gemv_bytes(N, K) + K * 4  # + the sign vector
    value = step_bytes / (ms * 1e-3) / 1e9

    # dominant kernel: the GEMV (fused paths: the single rotate+GEMV kernel)
    if best_path == "packed_fused":
        dom_name, dom_ms, dom_bytes = "gemv_packed_kernel<fused>", ms, step_bytes
    elif best_path == "fused":
        dom_name, dom_ms, dom_bytes = "rotate_gemv_lut_kernel", ms, step_bytes
    elif best_path == "packed_split":
        dom_name, dom_ms, dom_bytes = ("gemv_packed_kernel", dec["kernels"]["gemv_packed"],
                                       gemv_bytes(N, K))
    else:
        dom_name, dom_ms, dom_bytes = "gemv_lut_kernel", dec["kernels"]["gemv_lut"], gemv_bytes(N, K)
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode ffn_gate: M=1, K=5120, N=17408, 1-bit weights, "
                               "fp32 scales per 128, signs + WHT-1024 rotation",
                   "path": best_path, "weight_copies": dec["copies"]},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_ms * 1e3, 3)},
        "decode_us": {k: round(v * 1e3, 3) for k, v in dec["steps"].items()},
        "decode_kernel_us": {k: round(v * 1e3, 3) for k, v in dec["kernels"].items()},
    }
    if not args.no_prefill:
        pf = prefill_bench(torch, pq1, wl, dev, args.prefill_steps, max(3, args.prefill_steps // 5))
        tflops = pf["flops"] / (pf["gemm_ms"] * 1e-3) / 1e12
        out["prefill"] = {
            "workload": "prefill: M=1024, K=5120, N=17408, x' rounded to bf16, bf16 MFMA",
            "step_ms": round(pf["step_ms"], 4),
            "step_tflops": round(pf["flops"] / (pf["step_ms"] * 1e-3) / 1e12, 1),
            "gemm_ms": round(pf["gemm_ms"], 4),
            "gemm_tflops": round(tflops, 1),
            "rotate_us": round(pf["rotate_ms"] * 1e3, 2),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)},
        }
    if not args.no_cpu_baseline:
        log("[cpu] timing the oracle ...")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
