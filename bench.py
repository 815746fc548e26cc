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
timing starts.  The steps are timed with HIP events around one graph replay
that holds at least --steps of them and, for microsecond kernels, at least
1000 (`timed_launches` in the output line): every replay starts with a gap of
a few microseconds on this stack, which a 20-step replay would charge to its
steps.  The timed replay runs right behind about 60 ms of untimed steps that
keep the GPU busy, so it sees the steady-state clock.

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
COPY_CAL_BYTES = 256 << 20   # plain copy used to calibrate the byte counters

# The decode step is the single rotate + GEMV kernel on the packed layout.
STEP_PATH = "packed_fused"
STEP_KERNEL_MATCH = "gemv_packed_kernel"
STEP_KERNEL_SOURCES = ["gemm_hadamard_rotated_amd/csrc/gemv_packed.hip",
                       "gemm_hadamard_rotated_amd/csrc/gemv_common.h",
                       "gemm_hadamard_rotated_amd/csrc/pq1_device.h",
                       "gemm_hadamard_rotated_amd/csrc/pq1_internal.h"]
TRAFFIC_FILE = "profiles/traffic_gemv_packed_fused_{}.txt"      # per decode config
STEP_COUNTER_FILE = "profiles/counters_gemv_packed_fused_{}.txt"  # per decode config
DECODE_SHAPES = {"tiny": (256, 1024), "ffn_gate": (17408, 5120), "ffn_down": (5120, 17408),
                 "ssm_out": (5120, 6144)}  # N, K
STEP_SQ_COUNTERS = ["SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_ACTIVE_INST_VALU",
                    "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_WAVES", "SQ_BUSY_CYCLES",
                    "GRBM_GUI_ACTIVE"]

# The prefill GEMM (GEMM-order X) and its counter summary.
GEMM_KERNEL_MATCH = "gemm_xg_kernel"
SKINNY_KERNEL_MATCH = "gemm_skinny_kernel"
SKINNY_KERNEL_SOURCES = ["gemm_hadamard_rotated_amd/csrc/gemm_skinny.hip",
                         "gemm_hadamard_rotated_amd/csrc/gemm_common.h",
                         "gemm_hadamard_rotated_amd/csrc/pq1_internal.h"]
GEMM_KERNEL_SOURCES = ["gemm_hadamard_rotated_amd/csrc/gemm.hip",
                       "gemm_hadamard_rotated_amd/csrc/gemm_common.h",
                       "gemm_hadamard_rotated_amd/csrc/pq1_internal.h"]
GEMM_COUNTER_FILE = "profiles/counters_gemm_xg_prefill.txt"
GEMM_SQ_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS",
                    "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_LDS",
                    "GRBM_GUI_ACTIVE"]
BENCH_LIB = os.path.join(ROOT, "gemm_hadamard_rotated_amd", "libpq1_bench.so")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemv_bytes(N, K, scale_bytes=4):
    """Algorithmic bytes of one GEMV: 1-bit weights, scales (fp32, or f16 with
    scale_bytes=2), x', y."""
    return N * K // 8 + N * (K // 128) * scale_bytes + K * 4 + N * 4


WARM_MS = 60.0      # untimed GPU time run back to back right before every timed region
WARM_BATCH = 200    # launches per replay of the warm graph (at least)
MIN_TIMED = 1000    # launches per timed replay (at least; fewer only past MAX_TIMED_S)
MAX_TIMED_S = 0.25  # ... unless that many would take longer than this
_marks = None


def _mark(torch, dev):
    """Enqueue the empty marker kernel on the current stream (bench library):
    a kernel trace of the run is cut down to the dispatches between a pair."""
    global _marks
    if _marks is None:
        _marks = load_bench_lib()
    rc = _marks.pq1b_mark(ctypes_stream(torch, dev))
    if rc != 0:
        raise RuntimeError(f"marker kernel: HIP error {rc}")


def ctypes_stream(torch, dev):
    import ctypes
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def timed_launches(iters, per_launch_s):
    """Calls in one timed replay: at least `iters`, and at least MIN_TIMED
    unless those would run past MAX_TIMED_S.  Every graph replay starts with
    a gap of several microseconds on this stack (measured: 5.81 us per call
    with 20 calls per replay against 5.36 with 1000 on the decode step), so a
    short replay would charge that gap to each of its calls."""
    return max(iters, min(MIN_TIMED, int(MAX_TIMED_S / max(per_launch_s, 1e-9))))


def graph_time_n(torch, fn, iters, warmup, dev, check=None, warm_ms=WARM_MS, label="timed"):
    """Average ms per call of fn(i) over the calls of one timed replay.

    After `warmup` eager calls the calls are captured into HIP graphs: a warm
    graph of max(iters, WARM_BATCH) calls and the timed graph of
    timed_launches(iters, ...) calls.  Warm replays worth at least `warm_ms`
    of GPU time are enqueued back to back, followed -- with no host
    synchronization in between -- by a marker kernel, a start event, the
    timed replay, a stop event and a marker: the timed calls start while the
    GPU is still busy with warm ones, so a clock that has not ramped up does
    not land on them.  The events are recorded on the graph's stream, with a
    device synchronization before and after.  `check`, if given, is called
    after a warm replay and after the timed replay to compare the graph's
    results with eager ones.  Returns (ms per call, calls timed)."""
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        for i in range(max(warmup, 2)):   # eager warmup; allocates workspaces for s
            fn(i)
    torch.cuda.synchronize()
    n_warm = max(iters, WARM_BATCH)
    g_warm = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_warm, stream=s):
        for i in range(n_warm):
            fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_warm.replay()
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t0, 1e-6)
    if check is not None:
        check()
    n_timed = timed_launches(iters, one / n_warm)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(n_timed):
            fn(i)
    reps = max(1, int(warm_ms * 1e-3 / one + 0.999))
    # the timed regions of a run, in order: --summarize-trace names them from these lines
    log(f"[timed region] {label}")
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for _ in range(reps):
            g_warm.replay()
        _mark(torch, dev)
        start.record(s)
        g.replay()
        stop.record(s)
        _mark(torch, dev)
    torch.cuda.synchronize()
    if check is not None:
        check()
    return start.elapsed_time(stop) / n_timed, n_timed


def graph_time(torch, fn, iters, warmup, dev, check=None, warm_ms=WARM_MS, label="timed"):
    """graph_time_n without the call count."""
    return graph_time_n(torch, fn, iters, warmup, dev, check, warm_ms, label)[0]


def decode_setup(torch, pq1, wl, dev, name="ffn_gate"):
    """Decode inputs of one config (ffn_gate by default): the activation, the
    signs and enough weight copies (canonical and packed) that together they
    exceed the last-level cache.  The packed copies are made by the load-time
    repack (not timed)."""
    import numpy as np
    d = wl.make(name)
    N, K = d["N"], d["K"]
    wbytes = d["bits"].nbytes + d["scales"].nbytes
    copies = max(2, -(-2 * CACHE_BYTES // wbytes))
    log(f"[decode] {name} N={N} K={K}: {copies} weight copies ({copies * wbytes / 2**20:.0f} MiB)")
    bits0 = torch.from_numpy(d["bits"].view(np.int32)).to(dev)
    sc0 = torch.from_numpy(d["scales"]).to(dev)
    bits = [bits0.clone() for _ in range(copies)]
    scs = [sc0.clone() for _ in range(copies)]
    packed = [pq1.pq1_pack_weights(bits[c], scs[c]) for c in range(copies)]
    x = torch.from_numpy(d["x"][0].copy()).to(dev)
    signs = torch.from_numpy(d["signs"]).to(dev)
    torch.cuda.synchronize()
    return dict(N=N, K=K, copies=copies, bits=bits, scs=scs, packed=packed, x=x, signs=signs,
                perm=d["perm"])


def decode_bench(torch, pq1, wl, dev, steps, warmup):
    s = decode_setup(torch, pq1, wl, dev)
    N, K, copies = s["N"], s["K"], s["copies"]
    bits, scs, packed, x, signs = s["bits"], s["scs"], s["packed"], s["x"], s["signs"]
    xr = torch.empty(K, dtype=torch.float32, device=dev)
    y = torch.empty(N, dtype=torch.float32, device=dev)

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

    res, timed = {}, {}
    for name, fn in ((STEP_PATH, packed_fused), ("packed_split", packed_split),
                     ("fused", fused), ("split", split)):
        # eager reference of this path (all copies hold the same data)
        fn(0)
        torch.cuda.synchronize()
        y_ref = y.clone()

        def check():
            assert torch.allclose(y, y_ref, rtol=0, atol=1e-4 * float(y_ref.abs().max())), \
                "graph replay result differs from the eager result"

        res[name], timed[name] = graph_time_n(torch, fn, steps, warmup, dev, check,
                                              label=f"decode ffn_gate step: {name}")
        log(f"[decode] step path {name}: {res[name] * 1e3:.3f} us/step")
    pq1.pq1_rotate(x, signs, out=xr)
    kern = {}
    for name, fn in (("gemv_packed", packed_gemv_only),
                     ("gemv_lut", lambda i: gemv_only(i, pq1.PQ1_GEMV_LUT)),
                     ("gemv_expand", lambda i: gemv_only(i, pq1.PQ1_GEMV_EXPAND)),
                     ("rotate", rotate_only)):
        kern[name] = graph_time(torch, fn, steps, warmup, dev, label=f"decode ffn_gate kernel: {name}")
        log(f"[decode] kernel {name}: {kern[name] * 1e3:.3f} us/launch")
    torch.cuda.synchronize()
    return dict(N=N, K=K, steps=res, kernels=kern, copies=copies, timed=timed)


def traffic_probe(torch, pq1, wl, dev, name="ffn_gate"):
    """Launches for the HBM-traffic counters: the decode step kernel of one
    config on every weight copy in turn (each launch reads a copy that is not
    cache-resident), then three plain 256 MiB device copies whose counter
    readings calibrate the byte counts.  Nothing is timed."""
    s = decode_setup(torch, pq1, wl, dev, name)
    y = torch.empty(s["N"], dtype=torch.float32, device=dev)
    for i in range(2 * s["copies"]):
        pq1.pq1_rotate_gemv_packed(s["x"], s["signs"], s["packed"][i % s["copies"]],
                                   perm=s["perm"], out=y)
    torch.cuda.synchronize()
    n = COPY_CAL_BYTES
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"step_launches": 2 * s["copies"], "copy_bytes": n, "copy_launches": 3}),
          flush=True)


def kernel_source_digest(sources=None):
    """SHA-256 over the sources of a kernel (the decode step kernel by
    default): a recorded counter figure is only reported while these are
    unchanged."""
    import hashlib
    h = hashlib.sha256()
    for rel in (sources or STEP_KERNEL_SOURCES):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _counter_rows(d):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def summarize_pmc(fetch_dir, write_dir, out_path, name="ffn_gate"):
    """Turn two counter runs of --traffic-probe (FETCH_SIZE, then WRITE_SIZE)
    into HBM bytes per launch of the decode step kernel.  Each counter is
    scaled by bytes / reading of the plain copies (the last three copy
    dispatches of the run)."""
    import statistics
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(d) if r["Counter_Name"] == counter]
        per = {}
        for r in rows:  # one value per dispatch (sum over instances if split)
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        copies = sorted((k for k in per if "copyBuffer" in k[1]), key=lambda k: k[0])[-3:]
        step = [per[k] for k in per if STEP_KERNEL_MATCH in k[1]]
        if len(copies) < 3 or not step:
            raise SystemExit(f"{counter}: copy or step-kernel dispatches missing under {d}")
        copy_kib = statistics.median(per[k] for k in copies)
        factor = COPY_CAL_BYTES / (copy_kib * 1024.0)
        step_kib = statistics.median(step)
        res[counter] = dict(copy_kib=copy_kib, factor=factor, step_kib=step_kib,
                            step_bytes=step_kib * 1024.0 * factor, dispatches=len(step),
                            kernel=next(k[1] for k in per if STEP_KERNEL_MATCH in k[1]))
    with open(out_path, "w") as f:
        N, K = DECODE_SHAPES[name]
        f.write(f"# HBM traffic of the decode step kernel ({name}: M=1, K={K}, N={N})\n")
        f.write(f"# kernel: {res['FETCH_SIZE']['kernel']}\n")
        f.write("# commands (run from /tmp with TMPDIR=/tmp, repository at /root/repo):\n")
        for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
            f.write(f"#   timeout -s KILL 150 rocprofv3 --pmc {c} -d {d} -o run "
                    f"--output-format csv -- python3 /root/repo/bench.py --traffic-probe {name}\n")
        f.write(f"#   python bench.py --summarize-pmc {fetch_dir} {write_dir} "
                f"profiles/{os.path.basename(out_path)} {name}\n")
        f.write(f"# calibration: {COPY_CAL_BYTES} bytes read and written per plain copy\n")
        for c, r in res.items():
            f.write(f"# {c}: copy {r['copy_kib']:.1f} KiB -> factor {r['factor']:.4f}; step kernel "
                    f"median {r['step_kib']:.1f} KiB over {r['dispatches']} dispatches\n")
        f.write(f"source_sha256: {kernel_source_digest()}\n")
        f.write(f"fetch_bytes_per_launch: {res['FETCH_SIZE']['step_bytes']:.0f}\n")
        f.write(f"write_bytes_per_launch: {res['WRITE_SIZE']['step_bytes']:.0f}\n")
    print(open(out_path).read())


def recorded_traffic(name="ffn_gate"):
    """HBM bytes per launch of the step kernel on one decode config from the
    committed counter summary, or None if there is none or the kernel's
    sources changed since."""
    path = os.path.join(ROOT, TRAFFIC_FILE.format(name))
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_digest():
        return None
    return int(float(kv["fetch_bytes_per_launch"])) + int(float(kv["write_bytes_per_launch"]))


def summarize_step_sq(sq_dir, out_path, name="ffn_gate"):
    """SQ counters of the decode step kernel from one counter run of
    --traffic-probe: VALU lane operations per weight (the VALU budget of the
    table walk), VALU busy and LDS activity as rocprof's VALUBusy / LdsUtil
    define them (busy cycles / (GRBM_GUI_ACTIVE per XCC x SIMDs or CUs)),
    and LDS bank-conflict cycles per launch."""
    import statistics
    med = statistics.median
    rows = [r for r in _counter_rows(sq_dir) if STEP_KERNEL_MATCH in r["Kernel_Name"]]
    if not rows:
        raise SystemExit(f"no {STEP_KERNEL_MATCH} dispatches under {sq_dir}")
    agent = _agent(sq_dir)
    simds, xcc, cus = int(agent["Simd_Count"]), int(agent["Num_Xcc"]), int(agent["Cu_Count"])
    kernel = rows[0]["Kernel_Name"]
    per = {c: _per_dispatch(rows, c) for c in STEP_SQ_COUNTERS}
    disp = sorted({int(r["Dispatch_Id"]) for r in rows})

    def val(c, i):
        return next(v for k, v in per[c].items() if k[0] == i)
    N, K = DECODE_SHAPES[name]
    weights = N * K
    gui = [val("GRBM_GUI_ACTIVE", i) / xcc for i in disp]  # cycles per XCC
    valu_ops = med(val("SQ_INSTS_VALU", i) * 64.0 / weights for i in disp)
    salu = med(val("SQ_INSTS_SALU", i) * 64.0 / weights for i in disp)
    lds_ops = med(val("SQ_INSTS_LDS", i) * 64.0 / weights for i in disp)
    # SQ_ACTIVE_INST_VALU counts issue cycles of one quarter-wave: x 4 per instruction
    valu_busy = med(4.0 * val("SQ_ACTIVE_INST_VALU", i) / (g * simds) for i, g in zip(disp, gui))
    lds_util = med(val("SQ_LDS_IDX_ACTIVE", i) / (g * cus) for i, g in zip(disp, gui))
    conflicts = med(val("SQ_LDS_BANK_CONFLICT", i) for i in disp)
    waves = med(val("SQ_WAVES", i) for i in disp)
    with open(out_path, "w") as f:
        f.write(f"# SQ counters of the decode step kernel ({name}: M=1, K={K}, N={N})\n")
        f.write(f"# kernel: {kernel}\n")
        f.write("# command (run from /tmp with TMPDIR=/tmp, repository at /root/repo):\n")
        f.write(f"#   timeout -s KILL 150 rocprofv3 --pmc {' '.join(STEP_SQ_COUNTERS)} "
                f"-d {sq_dir} -o run --output-format csv -- python3 "
                f"/root/repo/bench.py --traffic-probe {name}\n")
        f.write(f"#   python bench.py --summarize-step-sq {sq_dir} profiles/{os.path.basename(out_path)} "
                f"{name}\n")
        f.write(f"# device: {cus} CUs, {simds} SIMDs, {xcc} XCCs; medians over {len(disp)} "
                "dispatches, each reading a weight copy that is not cache-resident\n")
        f.write("# *_per_weight: lane operations (wave instructions x 64) per weight; the walk's\n"
                "# budget at 70 % of the HBM peak is 1.1 VALU lane operations per weight\n")
        f.write(f"source_sha256: {kernel_source_digest()}\n")
        f.write(f"valu_ops_per_weight: {valu_ops:.3f}\n")
        f.write(f"salu_ops_per_weight: {salu:.3f}\n")
        f.write(f"lds_ops_per_weight: {lds_ops:.3f}\n")
        f.write(f"valu_busy_frac: {valu_busy:.4f}\n")
        f.write(f"lds_active_frac: {lds_util:.4f}\n")
        f.write(f"lds_bank_conflict_cycles: {conflicts:.0f}\n")
        f.write(f"waves_per_launch: {waves:.0f}\n")
    print(open(out_path).read())


def _read_kv(path, sources):
    """key: value lines of a committed counter summary, or None if there is
    none or the kernel's sources changed since it was taken."""
    full = os.path.join(ROOT, path)
    if not os.path.exists(full):
        return None
    kv = {}
    with open(full) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_digest(sources):
        return None
    return kv


def summarize_trace(trace_dir, out_path, title, log_path=None):
    """Per-kernel duration percentiles (p10 / p50 / p90, mean, count) of this
    library's kernels and the measurement microkernels, from a rocprofv3
    --kernel-trace run of bench.py, over the timed dispatches only: those
    between the two marker kernels bench.py launches around every timed
    region (eager warm-ups, warm stretches and reference launches are left
    out)."""
    import csv
    import glob
    import numpy as np
    files = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *kernel_trace.csv under {trace_dir}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    labels = []
    if log_path:  # the bench's stderr: one "[timed region] label" line per region, in order
        with open(log_path) as f:
            labels = [l.split("] ", 1)[1].strip() for l in f if l.startswith("[timed region] ")]
    dur, inside, regions, all_calls = {}, False, 0, {}
    for t0, t1, name in rows:
        if "mark_kernel" in name:
            inside = not inside
            regions += inside
            continue
        if "pq1::" not in name and "read_kernel" not in name and "read_chunks" not in name \
                and "mfma_loop" not in name and "empty_kernel" not in name:
            continue
        all_calls[name] = all_calls.get(name, 0) + 1
        if inside:
            region = labels[regions - 1] if regions - 1 < len(labels) else f"region {regions}"
            dur.setdefault((region, name), []).append((t1 - t0) * 1e-3)
    with open(out_path, "w") as f:
        f.write(f"# Kernel durations: {title}\n")
        f.write("# command (run from /tmp with TMPDIR=/tmp, repository at /root/repo):\n")
        f.write(f"#   rocprofv3 --kernel-trace --stats -d {trace_dir} -o bench "
                "--output-format csv -- python3 /root/repo/bench.py --steps 20 --warmup 5\n")
        f.write(f"#   python bench.py --summarize-trace {trace_dir} profiles/{os.path.basename(out_path)}"
                f"{' ' + os.path.basename(log_path) if log_path else ''}\n")
        f.write(f"# timed dispatches only: those inside the {regions} marked timed regions (all "
                "dispatches of the run\n# in the last column); microseconds from the trace's "
                "start and end timestamps\n\n")
        f.write("| timed region | kernel | timed calls | p10 us | p50 us | p90 us | mean us |\n"
                "|---|---|---:|---:|---:|---:|---:|\n")
        for (region, name), v in dur.items():  # in the order the regions ran
            a = np.array(v)
            short = name.replace("pq1::(anonymous namespace)::", "").replace(
                "(anonymous namespace)::", "").split("(")[0]
            f.write(f"| {region} | `{short}` | {len(a)} | {np.percentile(a, 10):.3f} | "
                    f"{np.percentile(a, 50):.3f} | {np.percentile(a, 90):.3f} | {a.mean():.3f} |\n")
    print(open(out_path).read())


SMALL_M = (1, 8, 16, 24, 32, 48, 64)  # short prompts: M rows of X against the prefill weights


def prefill_bench(torch, pq1, wl, dev, steps, warmup):
    s = gemm_setup(torch, pq1, wl, dev)
    M, N, K, copies = s["M"], s["N"], s["K"], s["copies"]
    log(f"[prefill] M={M} N={N} K={K}: {copies} input copies")
    bits, scs, xs, signs, y = s["bits"], s["scs"], s["xs"], s["signs"], s["y"]
    xbs, xrms = s["xbs"], s["xrms"]
    for c in range(copies):  # x' of every copy, in both layouts
        pq1.pq1_rotate(xs[c], signs, out_dtype=torch.bfloat16, out=xbs[c], gemm_order=True)
        pq1.pq1_rotate(xs[c], signs, out_dtype=torch.bfloat16, out=xrms[c])

    # the rotation writes x' as bf16 in the GEMM's operand K order
    def step(i):
        c = i % copies
        pq1.pq1_rotate(xs[c], signs, out_dtype=torch.bfloat16, out=xbs[c], gemm_order=True)
        pq1.pq1_gemm_ex(xbs[c], bits[c], scs[c], out=y, gemm_order=True)

    def gemm_only(i):
        c = i % copies
        pq1.pq1_gemm_ex(xbs[c], bits[c], scs[c], out=y, gemm_order=True)

    def rotate_only(i):
        c = i % copies
        pq1.pq1_rotate(xs[c], signs, out_dtype=torch.bfloat16, out=xbs[c], gemm_order=True)

    # the same GEMM on row-major X (natural K order: pq1_gemm), for comparison
    def gemm_row_major(i):
        c = i % copies
        pq1.pq1_gemm(xrms[c], bits[c], scs[c], out=y)

    # (every timed region follows about 60 ms of untimed steps: the MFMA
    # clock ramps up over the first tens of milliseconds of sustained load)
    t_step = graph_time(torch, step, steps, warmup, dev, label="prefill step (rotate + GEMM)")
    t_gemm = graph_time(torch, gemm_only, steps, warmup, dev, label="prefill GEMM (GEMM order)")
    t_rot = graph_time(torch, rotate_only, steps, warmup, dev, label="prefill rotate")
    t_rm = graph_time(torch, gemm_row_major, steps, warmup, dev, label="prefill GEMM (row-major)")
    flops = 2.0 * M * N * K
    log(f"[prefill] step {t_step:.3f} ms, gemm {t_gemm:.3f} ms ({flops / t_gemm / 1e9:.0f} TFLOP/s), "
        f"rotate {t_rot * 1e3:.1f} us, gemm on row-major X {t_rm:.3f} ms")
    # algorithmic bytes of one GEMM launch: 1-bit weights, fp32 scales, bf16 X, fp32 Y
    gbytes = N * K // 8 + N * (K // 128) * 4 + M * K * 2 + M * N * 4
    # short prompts: the same weights, M rows of row-major X; the weights
    # alone are 14 MB, so they get copies of their own that together exceed
    # twice the last-level cache (the prefill copies above would stay in it)
    small = {}
    wbytes = N * K // 8 + N * (K // 128) * 4
    wcopies = max(2, -(-2 * CACHE_BYTES // wbytes))
    wbits = [bits[0].clone() for _ in range(wcopies)]
    wscs = [scs[0].clone() for _ in range(wcopies)]
    for m in SMALL_M:
        xm = xrms[0][:m].contiguous()
        xg = xbs[0][:m].contiguous()  # the same rows in the GEMM K order
        ym = torch.empty((m, N), dtype=torch.float32, device=dev)
        t = graph_time(torch, lambda i: pq1.pq1_gemm(xm, wbits[i % wcopies], wscs[i % wcopies],
                                                     out=ym), max(steps, 200), warmup, dev,
                       label=f"short prompt M={m}")
        tg = graph_time(torch, lambda i: pq1.pq1_gemm_ex(xg, wbits[i % wcopies], wscs[i % wcopies],
                                                         out=ym, gemm_order=True),
                        max(steps, 200), warmup, dev, label=f"short prompt M={m} (GEMM order)")
        b = wbytes + m * K * 2 + m * N * 4
        small[f"M{m}"] = {"us": round(t * 1e3, 3), "gbs": round(b / t / 1e6, 1),
                          "weight_gbs": round(wbytes / t / 1e6, 1),
                          "tflops": round(2.0 * m * N * K / t / 1e9, 2),
                          "us_gemm_order_x": round(tg * 1e3, 3)}
        log(f"[prefill] M={m}: {t * 1e3:.2f} us, {b / t / 1e6:.0f} GB/s; "
            f"X in the GEMM order {tg * 1e3:.2f} us")
        del xm, xg, ym
    del wbits, wscs
    return dict(M=M, N=N, K=K, step_ms=t_step, gemm_ms=t_gemm, rotate_ms=t_rot,
                gemm_row_major_ms=t_rm, flops=flops, bytes=gbytes, small_m=small)


def _per_dispatch(rows, counter):
    """{(dispatch id, kernel name): value} for one counter (instances summed)."""
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return per


def _copy_factor(per, counter, d):
    """Bytes per KiB of counter reading, from the last three plain copies."""
    import statistics
    copies = sorted((k for k in per if "copyBuffer" in k[1]), key=lambda k: k[0])[-3:]
    if len(copies) < 3:
        raise SystemExit(f"{counter}: the calibration copies are missing under {d}")
    kib = statistics.median(per[k] for k in copies)
    return kib, COPY_CAL_BYTES / (kib * 1024.0)


def _agent(d):
    import csv
    import glob
    for fn in sorted(glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True)):
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Name", "").startswith("gfx"):
                    return r
    raise SystemExit(f"no GPU agent in an agent_info.csv under {d}")


def gemm_setup(torch, pq1, wl, dev):
    """Prefill inputs: `copies` copies of (bits, scales, x, and x' as bf16 in
    the GEMM K order and row-major) that together exceed twice the last-level
    cache, so every launch reads its inputs from HBM; the signs, and the
    output (one buffer, written by every launch)."""
    import numpy as np
    d = wl.make("prefill")
    M, N, K = d["M"], d["N"], d["K"]
    per_copy = d["bits"].nbytes + d["scales"].nbytes + d["x"].nbytes + 2 * M * K * 2
    copies = max(2, -(-2 * CACHE_BYTES // per_copy))
    bits0 = torch.from_numpy(d["bits"].view(np.int32)).to(dev)
    sc0 = torch.from_numpy(d["scales"]).to(dev)
    x0 = torch.from_numpy(d["x"]).to(dev)
    return dict(M=M, N=N, K=K, copies=copies,
                bits=[bits0.clone() for _ in range(copies)],
                scs=[sc0.clone() for _ in range(copies)],
                xs=[x0.clone() for _ in range(copies)],
                signs=torch.from_numpy(d["signs"]).to(dev),
                xbs=[torch.empty((M, K), dtype=torch.bfloat16, device=dev) for _ in range(copies)],
                xrms=[torch.empty((M, K), dtype=torch.bfloat16, device=dev) for _ in range(copies)],
                y=torch.empty((M, N), dtype=torch.float32, device=dev))


def gemm_probe(torch, pq1, wl, dev, m=None):
    """Launches for the prefill GEMM's counters: the rotation (bf16, GEMM
    order) and the GEMM on each input copy in turn, then three plain 256 MiB
    copies that calibrate the byte counters.  With `m`, the short-prompt
    GEMM instead: m rows of row-major X against each of enough weight copies
    to exceed twice the last-level cache.  Nothing is timed."""
    if m:
        import numpy as np
        d = wl.make("prefill")
        N, K = d["N"], d["K"]
        wbytes = d["bits"].nbytes + d["scales"].nbytes
        copies = max(2, -(-2 * CACHE_BYTES // wbytes))
        b0 = torch.from_numpy(d["bits"].view(np.int32)).to(dev)
        s0 = torch.from_numpy(d["scales"]).to(dev)
        wbits = [b0.clone() for _ in range(copies)]
        wscs = [s0.clone() for _ in range(copies)]
        xm = pq1.pq1_rotate(torch.from_numpy(d["x"][:m].copy()).to(dev),
                            torch.from_numpy(d["signs"]).to(dev), out_dtype=torch.bfloat16)
        ym = torch.empty((m, N), dtype=torch.float32, device=dev)
        for c in range(copies):
            pq1.pq1_gemm(xm, wbits[c], wscs[c], out=ym)
        launches = copies
    else:
        s = gemm_setup(torch, pq1, wl, dev)
        for c in range(s["copies"]):
            pq1.pq1_rotate(s["xs"][c], s["signs"], out_dtype=torch.bfloat16, out=s["xbs"][c],
                           gemm_order=True)
            pq1.pq1_gemm(s["xbs"][c], s["bits"][c], s["scs"][c], out=s["y"], gemm_order=True)
        launches = s["copies"]
    torch.cuda.synchronize()
    src = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"gemm_launches": launches, "copy_bytes": COPY_CAL_BYTES}), flush=True)


def summarize_gemm_pmc(fetch_dir, write_dir, sq_dir, out_path, m=None):
    """Counter summary of the prefill GEMM from three runs of --gemm-probe
    (with `m`: of the short-prompt GEMM, runs of --gemm-probe-m m):
    FETCH_SIZE, WRITE_SIZE (each scaled by the plain copies' reading) and the
    SQ/GRBM counters, normalised as rocprof's derived metrics do
    (MfmaUtil = MFMA busy cycles / (GRBM_GUI_ACTIVE per XCC * SIMDs),
    LdsUtil = LDS active cycles / (GRBM_GUI_ACTIVE per XCC * CUs))."""
    import statistics
    med = statistics.median
    match = SKINNY_KERNEL_MATCH if m else GEMM_KERNEL_MATCH
    probe = f"--gemm-probe-m {m}" if m else "--gemm-probe"
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _per_dispatch(_counter_rows(d), counter)
        kib, factor = _copy_factor(per, counter, d)
        g = [v for k, v in per.items() if match in k[1]]
        if not g:
            raise SystemExit(f"{counter}: no {match} dispatches under {d}")
        res[counter] = dict(copy_kib=kib, factor=factor, kib=med(g), bytes=med(g) * 1024.0 * factor,
                            n=len(g))
    rows = [r for r in _counter_rows(sq_dir) if match in r["Kernel_Name"]]
    agent = _agent(sq_dir)
    simds, xcc, cus = int(agent["Simd_Count"]), int(agent["Num_Xcc"]), int(agent["Cu_Count"])
    kernel = rows[0]["Kernel_Name"]
    per = {c: _per_dispatch(rows, c) for c in GEMM_SQ_COUNTERS}
    dur = {}
    for r in rows:
        dur[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    disp = sorted(dur)
    def val(c, i):
        return next(v for k, v in per[c].items() if k[0] == i)
    gui = [val("GRBM_GUI_ACTIVE", i) / xcc for i in disp]  # cycles per XCC
    mfma_util = med(val("SQ_VALU_MFMA_BUSY_CYCLES", i) / (g * simds) for i, g in zip(disp, gui))
    lds_util = med(val("SQ_LDS_IDX_ACTIVE", i) / (g * cus) for i, g in zip(disp, gui))
    clock = med(g / dur[i] / 1e9 for i, g in zip(disp, gui))
    valu = med(val("SQ_INSTS_VALU", i) / val("SQ_INSTS_MFMA", i) for i in disp)
    lds_per_mfma = med(val("SQ_INSTS_LDS", i) / val("SQ_INSTS_MFMA", i) for i in disp)
    conflicts = med(val("SQ_LDS_BANK_CONFLICT", i) for i in disp)
    with open(out_path, "w") as f:
        f.write(f"# Short-prompt GEMM counters (M={m}, K=5120, N=17408, X bf16 row-major, weights "
                f"not cache-resident)\n" if m else
                "# Prefill GEMM counters (M=1024, K=5120, N=17408, X bf16 in the GEMM K order)\n")
        f.write(f"# kernel: {kernel}\n")
        f.write("# commands (run from /tmp with TMPDIR=/tmp, repository at /root/repo):\n")
        for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir),
                     (" ".join(GEMM_SQ_COUNTERS), sq_dir)):
            f.write(f"#   timeout -s KILL 150 rocprofv3 --pmc {c} -d {d} -o run "
                    f"--output-format csv -- python3 /root/repo/bench.py {probe}\n")
        f.write(f"#   python bench.py --summarize-gemm-pmc {fetch_dir} {write_dir} {sq_dir} "
                f"profiles/{os.path.basename(out_path)}" + (f" {m}" if m else "") + "\n")
        f.write(f"# device: {cus} CUs, {simds} SIMDs, {xcc} XCCs, max engine clock "
                f"{agent.get('Max_Engine_Clk_Fcompute', '?')} MHz\n")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            r = res[c]
            f.write(f"# {c}: copy {r['copy_kib']:.1f} KiB -> factor {r['factor']:.4f}; GEMM median "
                    f"{r['kib']:.1f} KiB over {r['n']} dispatches\n")
        f.write(f"# SQ counters: medians over {len(disp)} dispatches; kernel duration under the "
                f"counters {med(dur.values()) * 1e6:.1f} us\n")
        f.write(f"source_sha256: "
                f"{kernel_source_digest(SKINNY_KERNEL_SOURCES if m else GEMM_KERNEL_SOURCES)}\n")
        f.write(f"fetch_bytes_per_launch: {res['FETCH_SIZE']['bytes']:.0f}\n")
        f.write(f"write_bytes_per_launch: {res['WRITE_SIZE']['bytes']:.0f}\n")
        f.write(f"mfma_busy_frac: {mfma_util:.4f}\n")
        f.write(f"lds_active_frac: {lds_util:.4f}\n")
        f.write(f"lds_bank_conflict_cycles: {conflicts:.0f}\n")
        f.write(f"valu_insts_per_mfma (MFMA included): {valu:.3f}\n")
        f.write(f"lds_insts_per_mfma: {lds_per_mfma:.3f}\n")
        if m:
            f.write(f"# no effective clock: GRBM_GUI_ACTIVE spans {clock / 2.4:.2f}x this short "
                    f"kernel's duration at 2.4 GHz, so the busy fractions above are of that "
                    f"longer window\n")
        else:
            f.write(f"effective_clock_ghz: {clock:.3f}\n")
    print(open(out_path).read())


def recorded_gemm_counters():
    """The committed GEMM counter summary as a dict, or None if there is none
    or the GEMM's sources changed since it was taken."""
    path = os.path.join(ROOT, GEMM_COUNTER_FILE)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_digest(GEMM_KERNEL_SOURCES):
        return None
    return kv


def load_bench_lib():
    import ctypes
    if not os.path.exists(BENCH_LIB):
        raise SystemExit(f"{BENCH_LIB} is missing: build it with "
                         "`python -m gemm_hadamard_rotated_amd.build`")
    lib = ctypes.CDLL(BENCH_LIB)
    lib.pq1b_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.pq1b_mfma_loop.restype = ctypes.c_int
    lib.pq1b_mfma_loop_random.argtypes = lib.pq1b_mfma_loop.argtypes
    lib.pq1b_mfma_loop_random.restype = ctypes.c_int
    lib.pq1b_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                              ctypes.c_int, ctypes.c_void_p]
    lib.pq1b_read.restype = ctypes.c_int
    lib.pq1b_read_chunks.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p]
    lib.pq1b_read_chunks.restype = ctypes.c_int
    lib.pq1b_mark.argtypes = [ctypes.c_void_p]
    lib.pq1b_mark.restype = ctypes.c_int
    lib.pq1b_empty.argtypes = [ctypes.c_void_p]
    lib.pq1b_empty.restype = ctypes.c_int
    return lib


READ_LOADS = (2, 4, 8, 16)        # 16-byte loads per lane in flight
READ_GRIDS = (None, 256, 512, 768, 1024)  # None: one pass (one chunk per workgroup)


def measured_peaks(torch, dev, same_bytes, copies, steps, warmup, extra=None):
    """What this GPU sustains, timed like the kernels (graph replay after a
    warm stretch): a bf16 MFMA loop with no memory traffic; the fastest of a
    set of streaming reads of `same_bytes` per launch over `copies` buffers
    (the decode step's bytes, cold in the caches; plain and non-temporal
    loads, 2-16 loads in flight per lane, one-pass and 1-4 workgroups per CU
    grids); a 1 GiB streaming read; and an empty launch.  `extra` maps a name
    to (bytes, copies): the same-bytes read of each, fastest of the six
    shapes that were fastest on `same_bytes`."""
    lib = load_bench_lib()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count

    def stream():
        return ctypes_stream(torch, dev)

    def ok(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: HIP error {rc}")

    iters, blocks = 2048, 4 * cus
    t = graph_time(torch, lambda i: ok(lib.pq1b_mfma_loop(None, blocks, iters, 0, stream()),
                                       "mfma loop"), 10, 3, dev, label="MFMA loop")
    mfma_tflops = blocks * 4 * iters * 8 * (2 * 32 * 32 * 16) / (t * 1e-3) / 1e12
    t = graph_time(torch, lambda i: ok(lib.pq1b_mfma_loop_random(None, blocks, iters, 0, stream()),
                                       "mfma loop (random operands)"), 10, 3, dev,
                   label="MFMA loop, random operands")
    mfma_rand_tflops = blocks * 4 * iters * 8 * (2 * 32 * 32 * 16) / (t * 1e-3) / 1e12
    t_empty = graph_time(torch, lambda i: ok(lib.pq1b_empty(stream()), "empty"), steps, warmup, dev,
                         label="empty launch")
    # the same-bytes reads: every shape of the sweep, the fastest reported
    n = -(-same_bytes // 16) * 16
    bufs = [torch.zeros(n // 4, dtype=torch.float32, device=dev) for _ in range(copies)]
    sweep = {}
    for nt in (1, 0):
        for loads in READ_LOADS:
            for grid in READ_GRIDS:
                nb = -(-n // (16 * 256 * loads)) if grid is None else grid // 256 * cus
                t = graph_time(torch, lambda i: ok(lib.pq1b_read_chunks(
                    bufs[i % copies].data_ptr(), n, None, loads, nb, nt, 0, stream()), "read"),
                    steps, warmup, dev, warm_ms=20.0,
                    label=f"same-bytes read {'nt' if nt else 'plain'} L{loads} grid{nb}")
                sweep[f"{'nt' if nt else 'plain'} L{loads} grid{nb}"] = t
    best = min(sweep, key=sweep.get)
    t_small = sweep[best]
    del bufs
    by_config = {}
    top = sorted(sweep, key=sweep.get)[:6]
    for name, (nbytes, ncopies) in (extra or {}).items():
        ne = -(-nbytes // 16) * 16
        ebufs = [torch.zeros(ne // 4, dtype=torch.float32, device=dev) for _ in range(ncopies)]
        res = {}
        for shape in top:
            kind, lf, gf = shape.split()
            nt, loads, grid = int(kind == "nt"), int(lf[1:]), int(gf[4:])
            one_pass = grid == -(-n // (16 * 256 * loads))  # the one-pass shape of the sweep
            nb = -(-ne // (16 * 256 * loads)) if one_pass else grid
            t = graph_time(torch, lambda i: ok(lib.pq1b_read_chunks(
                ebufs[i % ncopies].data_ptr(), ne, None, loads, nb, nt, 0, stream()), "read"),
                steps, warmup, dev, warm_ms=20.0,
                label=f"{name} same-bytes read {kind} L{loads} grid{nb}")
            res[f"{kind} L{loads} grid{nb}"] = t
        b = min(res, key=res.get)
        by_config[name] = {"bytes": ne, "us": round(res[b] * 1e3, 3),
                           "gbs": round(ne / res[b] / 1e6, 1), "shape": b}
        del ebufs
    big_n = 1 << 30
    big = torch.zeros(big_n // 4, dtype=torch.float32, device=dev)
    t_big, big_blocks = None, None
    for per_cu in (2, 4, 128):
        blocks = per_cu * cus
        t = graph_time(torch, lambda i: ok(lib.pq1b_read(big.data_ptr(), big_n, None, blocks, 0,
                                                         stream()), "read"), 20, 3, dev,
                       label=f"1 GiB read grid{blocks}")
        if t_big is None or t < t_big:
            t_big, big_blocks = t, blocks
    del big
    torch.cuda.synchronize()
    log(f"[peaks] MFMA loop {mfma_tflops:.0f} TFLOP/s ({mfma_rand_tflops:.0f} on random operands); empty launch {t_empty * 1e3:.3f} us; read "
        f"{n} B cold {n / t_small / 1e6:.0f} GB/s ({t_small * 1e3:.3f} us, {best}); read 1 GiB "
        f"{big_n / t_big / 1e6:.0f} GB/s ({big_blocks} workgroups)")
    return {"mfma_bf16_loop_tflops": round(mfma_tflops, 1),
            "mfma_bf16_loop_random_tflops": round(mfma_rand_tflops, 1),
            "empty_launch_us": round(t_empty * 1e3, 3),
            "hbm_read_same_bytes_gbs": round(n / t_small / 1e6, 1),
            "hbm_read_same_bytes_us": round(t_small * 1e3, 3),
            "hbm_read_same_bytes_shape": best,
            "hbm_read_same_bytes_sweep_us": {k: round(v * 1e3, 3) for k, v in sweep.items()},
            "hbm_read_1gib_gbs": round(big_n / t_big / 1e6, 1),
            "hbm_read_same_bytes_by_config": by_config,
            "how": f"graph-replayed microkernels, each after a warm stretch: 8 independent "
                   f"v_mfma_f32_32x32x16_bf16 chains per wave on {4 * cus} workgroups, on "
                   f"constant operands and on operands that change every MFMA (random bf16 A, "
                   f"random +-1 B, like the GEMM's); an empty "
                   f"one-wave kernel; streaming reads of {n} B per launch over {copies} buffers "
                   f"(fastest of {len(sweep)} shapes: plain / non-temporal 16-byte loads, "
                   f"{READ_LOADS} loads in flight per lane, one-pass or 1-4 workgroups per CU); "
                   f"a 1 GiB streaming read ({big_blocks} workgroups, fastest of 3 shapes)"}


def decode_configs_bench(torch, pq1, wl, dev, steps, warmup):
    """The fused packed step on every decode config besides the headline one
    (tiny, ffn_down, ssm_out with its head permutation), timed like the step:
    graph replay over enough weight copies to defeat the last-level cache."""
    import numpy as np
    out = {}
    for name in ("tiny", "ffn_down", "ssm_out"):
        d = wl.make(name)
        N, K = d["N"], d["K"]
        wbytes = d["bits"].nbytes + d["scales"].nbytes
        copies = max(2, -(-2 * CACHE_BYTES // wbytes))
        bits0 = torch.from_numpy(d["bits"].view(np.int32)).to(dev)
        sc0 = torch.from_numpy(d["scales"]).to(dev)
        packed = [pq1.pq1_pack_weights(bits0, sc0) for _ in range(copies)]
        del bits0, sc0
        x = torch.from_numpy(d["x"][0].copy()).to(dev)
        signs = torch.from_numpy(d["signs"]).to(dev)
        y = torch.empty(N, dtype=torch.float32, device=dev)
        t = graph_time(torch, lambda i: pq1.pq1_rotate_gemv_packed(x, signs, packed[i % copies],
                                                                   perm=d["perm"], out=y),
                       steps, warmup, dev, label=f"decode {name} step")
        b = gemv_bytes(N, K) + K * 4
        out[name] = {"M": 1, "K": K, "N": N, "perm": d["perm"], "us": round(t * 1e3, 3),
                     "gbs": round(b / t / 1e6, 1), "frac": round(b / t / 1e6 / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": b, "weight_copies": copies,
                     "traffic": recorded_traffic(name) if name in DECODE_SHAPES else None}
        log(f"[decode] {name}: {t * 1e3:.3f} us, {b / t / 1e6:.0f} GB/s")
        del packed
        torch.cuda.synchronize()
    return out


def widened_bench(torch, pq1, wl, dev, steps, warmup):
    """The rows beyond the headline step, timed the same way (graph replay,
    cold weight copies): ffn_gate + ffn_up stacked into one launch, the output
    head, the f16-scale weight format on ffn_gate and the output head, and the
    embedding lookup with the inverse rotation."""
    import numpy as np
    out = {}
    for name, sdt in (("gate_up", "f32"), ("lm_head", "f32"), ("ffn_gate", "f16"),
                      ("lm_head", "f16")):
        d = wl.make(name)
        N, K = d["N"], d["K"]
        sbytes = 2 if sdt == "f16" else 4
        wbytes = d["bits"].nbytes + d["scales"].nbytes * sbytes // 4
        copies = max(2, -(-2 * CACHE_BYTES // wbytes))
        bits0 = torch.from_numpy(d["bits"].view(np.int32)).to(dev)
        sc0 = torch.from_numpy(d["scales"]).to(dev)
        packed = []
        for _ in range(copies):
            if name == "gate_up":  # the two matrices packed one after the other
                n = N // 2
                packed.append(pq1.pq1_pack_weights_rows([(bits0[:n], sc0[:n]), (bits0[n:], sc0[n:])],
                                                        scale_dtype=sdt))
            else:
                packed.append(pq1.pq1_pack_weights(bits0, sc0, scale_dtype=sdt))
        del bits0, sc0
        x = torch.from_numpy(d["x"][0].copy()).to(dev)
        signs = torch.from_numpy(d["signs"]).to(dev)
        y = torch.empty(N, dtype=torch.float32, device=dev)
        n_steps = steps if N * K < 1e9 else max(20, steps // 10)
        t = graph_time(torch, lambda i: pq1.pq1_rotate_gemv_packed(x, signs, packed[i % copies],
                                                                   perm=d["perm"], out=y),
                       n_steps, min(warmup, n_steps), dev, label=f"{name} step, {sdt} scales")
        b = gemv_bytes(N, K, sbytes) + K * 4
        key = name if sdt == "f32" else f"{name}_f16_scales"
        out[key] = {"N": N, "K": K, "scale_dtype": sdt, "us": round(t * 1e3, 3),
                    "gbs": round(b / t / 1e6, 1), "bytes_per_launch": b, "weight_copies": copies}
        log(f"[widened] {key}: N={N} K={K} {t * 1e3:.3f} us, {b / t / 1e6:.0f} GB/s")
        del packed, x, y
        torch.cuda.synchronize()
    e = wl.make_embedding(M=1024)
    V, K = e["V"], e["K"]
    bits = torch.from_numpy(e["bits"].view(np.int32)).to(dev)
    sc = torch.from_numpy(e["scales"]).to(dev)
    signs = torch.from_numpy(e["signs"]).to(dev)
    toks = torch.from_numpy(e["tokens"]).to(dev)
    res = {}
    for M in (1, 1024):
        o = torch.empty((M, K), dtype=torch.float32, device=dev)
        t = graph_time(torch, lambda i: pq1.pq1_embed(toks[i % 1024:i % 1024 + 1] if M == 1 else toks,
                                                     bits, sc, signs, out=o), 200, 20, dev,
                       label=f"embedding lookup M={M}")
        res[f"M{M}_us"] = round(t * 1e3, 3)
        log(f"[widened] embed M={M}: {t * 1e3:.3f} us")
    out["embed"] = {"V": V, "K": K, **res}
    del bits, sc
    torch.cuda.synchronize()
    return out


def _host_facts():
    """CPU model, logical CPUs and NUMA nodes of this host."""
    model = "?"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nodes = len([d for d in os.listdir("/sys/devices/system/node") if d.startswith("node")
                     and d[4:].isdigit()])
    except OSError:
        nodes = None
    return dict(cpu_model=model, logical_cpus=os.cpu_count(),
                usable_cpus=len(os.sched_getaffinity(0)), numa_nodes=nodes)


_CPU_JOB = None  # inputs shared with the forked workers (they inherit them at the fork)


def _split_rows(N, parts):
    edges = [N * i // parts for i in range(parts + 1)]
    return [(edges[i], edges[i + 1]) for i in range(parts) if edges[i + 1] > edges[i]]


def _cpu_gemv_rows(args):
    """A worker's slice of decode output rows through the oracle (numpy
    single-threaded: the slices are the parallelism)."""
    import oracle.pq1_oracle as orc
    from threadpoolctl import threadpool_limits
    lo, hi, xr = args
    d = _CPU_JOB["decode"]
    with threadpool_limits(1):
        return orc.gemv(xr, d["bits"][lo:hi], d["scales"][lo:hi])


def _cpu_rotate_rows(bounds):
    """A worker's slice of prefill activation rows through the oracle's
    rotation, written into the shared x' buffer."""
    import numpy as np
    import oracle.pq1_oracle as orc
    from threadpoolctl import threadpool_limits
    lo, hi = bounds
    p = _CPU_JOB["prefill"]
    xr = np.frombuffer(_CPU_JOB["xr_shared"], dtype=np.float64).reshape(p["M"], p["K"])
    with threadpool_limits(1):
        xr[lo:hi] = orc.rotate(p["x"][lo:hi], p["signs"])
    return hi - lo


def _cpu_gemm_cols(bounds):
    """A worker's slice of prefill output columns (weight rows)."""
    import numpy as np
    import oracle.pq1_oracle as orc
    from threadpoolctl import threadpool_limits
    lo, hi = bounds
    p = _CPU_JOB["prefill"]
    xr = np.frombuffer(_CPU_JOB["xr_shared"], dtype=np.float64).reshape(p["M"], p["K"])
    with threadpool_limits(1):
        return orc.gemm(xr, p["bits"][lo:hi], p["scales"][lo:hi])


def cpu_baseline(budget_s=24.0):
    """The oracle as it stands, timed on this host's cores over bounded
    samples.  All-core: the work split into one slice of rows per usable CPU,
    each slice through the oracle in a forked worker (numpy single-threaded
    inside each); the workers stay alive across steps.  Whole decode ffn_gate
    steps (rotate + GEMV, fp64; the rotation of one activation in the parent,
    the GEMV's output rows over the workers), median of up to 3 after an
    untimed one; the same step on one thread; one full-size prefill (the 1024
    activation rows' rotations, then the GEMM's 17408 weight rows, over the
    workers).  `value` is the all-core decode figure in the decode unit."""
    import multiprocessing as mp
    import statistics
    import numpy as np
    import oracle.pq1_oracle as orc
    from gemm_hadamard_rotated_amd import workloads as wl
    from threadpoolctl import threadpool_limits
    global _CPU_JOB
    cores = len(os.sched_getaffinity(0))
    d = wl.make("ffn_gate")
    p = wl.make("prefill")
    N = d["N"]
    b = gemv_bytes(N, d["K"]) + d["K"] * 4
    _CPU_JOB = {"decode": d, "prefill": p,
                "xr_shared": mp.RawArray("d", p["M"] * p["K"])}
    t_all = time.perf_counter()

    def steps(step, limit):
        ts = []
        while len(ts) < 3 and (not ts or time.perf_counter() - t_all < limit):
            t0 = time.perf_counter()
            step()
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts), len(ts)

    dec_slices = _split_rows(N, cores)
    with mp.get_context("fork").Pool(processes=cores) as pool:
        def all_core_step():
            with threadpool_limits(1):
                xr = orc.rotate(d["x"][0], d["signs"], d["perm"])
            return np.concatenate(pool.map(_cpu_gemv_rows, [(lo, hi, xr) for lo, hi in dec_slices]))

        all_core_step()  # untimed: each worker touches its slice of the weights once
        t_all = time.perf_counter()
        dt_all, n_all = steps(all_core_step, budget_s * 0.25)
        t0 = time.perf_counter()
        pool.map(_cpu_rotate_rows, _split_rows(p["M"], cores))
        Y = np.concatenate(pool.map(_cpu_gemm_cols, _split_rows(p["N"], cores)), axis=1)
        dt_pf = time.perf_counter() - t0
        assert Y.shape == (p["M"], p["N"])
    flops = 2.0 * p["M"] * p["N"] * p["K"]
    _CPU_JOB = None
    del Y, p
    t_all = time.perf_counter()

    def one_thread_step():
        with threadpool_limits(1):
            orc.gemv(orc.rotate(d["x"][0], d["signs"], d["perm"]), d["bits"], d["scales"])

    dt_one, n_one = steps(one_thread_step, budget_s * 0.5)
    return dict(value=b / dt_all / 1e9, unit="GB/s", cores=cores, kind="oracle",
                sample=f"median of {n_all} whole decode ffn_gate steps after one untimed step "
                       f"(rotate + GEMV, fp64 numpy, {dt_all:.3f} s per step): the {N} output "
                       f"rows split into {len(dec_slices)} slices, one per usable CPU, each "
                       f"through the oracle in a forked worker with numpy single-threaded",
                single_thread={"value": b / dt_one / 1e9, "unit": "GB/s", "cores": 1,
                               "s_per_step": round(dt_one, 3), "steps": n_one},
                prefill={"value": flops / dt_pf / 1e12, "unit": "TFLOP/s", "cores": cores,
                         "s_per_step": round(dt_pf, 2),
                         "sample": "one full-size prefill: the 1024 rows' rotations, then the "
                                   "GEMM's 17408 weight rows, split over the same workers"},
                host=_host_facts())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--prefill-steps", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--traffic-probe", nargs="?", const="ffn_gate", default=None,
                    choices=sorted(DECODE_SHAPES), metavar="CONFIG",
                    help="only launch the step kernel on a decode config (default ffn_gate) and "
                         "a plain copy (for the byte counters)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="ARG",
                    help="FETCH_DIR WRITE_DIR OUT [CONFIG]: the traffic summary from two counter "
                         "runs of --traffic-probe")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="only launch the prefill rotate + GEMM and a plain copy (for counters)")
    ap.add_argument("--gemm-probe-m", type=int, default=0, metavar="M",
                    help="only launch the short-prompt GEMM with M rows and a plain copy "
                         "(for counters)")
    ap.add_argument("--summarize-gemm-pmc", nargs="+",
                    metavar="ARG",
                    help="FETCH_DIR WRITE_DIR SQ_DIR OUT [M]: write the GEMM counter summary "
                         "from three runs of --gemm-probe (or --gemm-probe-m M)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the MFMA-loop and streaming-read microkernels")
    ap.add_argument("--no-widened", action="store_true",
                    help="skip the gate+up, output-head and embedding figures")
    ap.add_argument("--summarize-step-sq", nargs="+", metavar="ARG",
                    help="SQ_DIR OUT [CONFIG]: the step kernel's SQ counter summary from a "
                         "--traffic-probe run")
    ap.add_argument("--summarize-trace", nargs="+", metavar="ARG",
                    help="TRACE_DIR OUT [BENCH_STDERR]: per-kernel duration percentiles of the "
                         "timed regions of a --kernel-trace run (named from the run's stderr)")
    args = ap.parse_args()

    if args.summarize_step_sq:
        summarize_step_sq(*args.summarize_step_sq)
        return
    if args.summarize_trace:
        a = args.summarize_trace
        summarize_trace(a[0], a[1], "every timed region of a bench.py run (headline: decode "
                        "ffn_gate, M=1, K=5120, N=17408; prefill M=1024, K=5120, N=17408)",
                        a[2] if len(a) > 2 else None)
        return

    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_gemm_pmc:
        a = args.summarize_gemm_pmc
        if len(a) not in (4, 5):
            raise SystemExit("--summarize-gemm-pmc takes FETCH_DIR WRITE_DIR SQ_DIR OUT [M]")
        summarize_gemm_pmc(*a[:4], m=int(a[4]) if len(a) == 5 else None)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: there is no multi-GPU path here "
              "(the GEMV would shard by output rows with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from gemm_hadamard_rotated_amd import pq1, workloads as wl
    dev = torch.device("cuda:0")
    pq1.load_library()

    if args.traffic_probe:
        traffic_probe(torch, pq1, wl, dev, args.traffic_probe)
        return
    if args.gemm_probe or args.gemm_probe_m:
        gemm_probe(torch, pq1, wl, dev, m=args.gemm_probe_m or None)
        return

    dec = decode_bench(torch, pq1, wl, dev, args.steps, args.warmup)
    N, K = dec["N"], dec["K"]
    ms = dec["steps"][STEP_PATH]
    step_bytes = gemv_bytes(N, K) + K * 4  # + the sign vector
    value = step_bytes / (ms * 1e-3) / 1e9
    # the step is one kernel launch, so the kernel's average launch time is
    # the per-step time of the replayed graph
    achieved = value
    traffic = recorded_traffic("ffn_gate")

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "timed_launches": dec["timed"][STEP_PATH],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode ffn_gate: M=1, K=5120, N=17408, 1-bit weights, "
                               "fp32 scales per 128, signs + WHT-1024 rotation",
                   "path": STEP_PATH, "weight_copies": dec["copies"]},
        "roofline": {"bound": "hbm", "kernel": "gemv_packed_kernel (fused rotate + GEMV)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": step_bytes, "avg_launch_us": round(ms * 1e3, 3)},
        "decode_us": {k: round(v * 1e3, 3) for k, v in dec["steps"].items()},
        "decode_kernel_us": {k: round(v * 1e3, 3) for k, v in dec["kernels"].items()},
    }
    sq = _read_kv(STEP_COUNTER_FILE.format("ffn_gate"), STEP_KERNEL_SOURCES)
    if sq is not None:
        for k in ("valu_ops_per_weight", "lds_ops_per_weight", "valu_busy_frac",
                  "lds_bank_conflict_cycles"):
            out["roofline"][f"{k}_counters"] = float(sq[k])
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
            "gemm_row_major_x_ms": round(pf["gemm_row_major_ms"], 4),
            "gemm_row_major_x_tflops": round(pf["flops"] / (pf["gemm_row_major_ms"] * 1e-3) / 1e12, 1),
            "small_m": {"workload": "short prompts: M rows of row-major bf16 X, K=5120, N=17408, "
                                    "cold weight copies (together twice the last-level cache); "
                                    "gbs counts weights + X + Y, weight_gbs the weights alone; "
                                    "us_gemm_order_x: the same rows stored in the GEMM K order",
                        **pf["small_m"]},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "kernel": "gemm_xg_kernel", "flops_per_launch": pf["flops"],
                         "algorithmic_bytes_per_launch": pf["bytes"], "traffic": None},
        }
        gc = recorded_gemm_counters()
        if gc is not None:
            out["prefill"]["roofline"]["traffic"] = (int(float(gc["fetch_bytes_per_launch"])) +
                                                     int(float(gc["write_bytes_per_launch"])))
            out["prefill"]["roofline"]["mfma_busy_frac_counters"] = float(gc["mfma_busy_frac"])
            out["prefill"]["roofline"]["effective_clock_ghz"] = float(gc["effective_clock_ghz"])
    out["decode_configs"] = decode_configs_bench(torch, pq1, wl, dev, min(args.steps, 1000),
                                                 min(args.warmup, 100))
    if not args.no_widened:
        out["widened"] = widened_bench(torch, pq1, wl, dev, min(args.steps, 1000),
                                       min(args.warmup, 100))
    if not args.no_peaks:
        extra = {k: (v["bytes_per_launch"], v["weight_copies"])
                 for k, v in out.get("decode_configs", {}).items() if k != "tiny"}
        pk = measured_peaks(torch, dev, step_bytes, dec["copies"], min(args.steps, 1000),
                            min(args.warmup, 100), extra=extra)
        out["measured_peaks"] = pk
        out["roofline"]["frac_of_measured_read"] = round(
            achieved / pk["hbm_read_same_bytes_gbs"], 4)
        for k, f in pk["hbm_read_same_bytes_by_config"].items():
            out["decode_configs"][k]["frac_of_measured_read"] = round(
                out["decode_configs"][k]["gbs"] / f["gbs"], 4)
        if "prefill" in out:
            out["prefill"]["roofline"]["frac_of_measured_mfma"] = round(
                out["prefill"]["gemm_tflops"] / pk["mfma_bf16_loop_tflops"], 4)
            out["prefill"]["roofline"]["frac_of_measured_mfma_random"] = round(
                out["prefill"]["gemm_tflops"] / pk["mfma_bf16_loop_random_tflops"], 4)
    if not args.no_cpu_baseline:
        log("[cpu] timing the oracle ...")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
