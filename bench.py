"""Benchmark of the Q8_0 decode matvec on one MI355X.

A step is one q8_matvec call (plan, activation staging, weight streaming,
convert, block partials, one scale per block and column, accumulate, split-K
combine, masked store) over one rotated copy of the synthetic workload's
weights and scales.  Default workload: the 70B-class MLP up-projection,
M=1, K=8192, N=28672, with 4 rotated W/S copies (about 1.06 GB) so that every
step reads its weights from HBM rather than the 256 MB Infinity Cache.

Prints ONE JSON line.  `value` is the effective HBM bandwidth on algorithmic
bytes (K*N + 4*ceil(K/32)*N + 4*M*K + 4*M*N per step) over the whole timed
region (host clock).  `roofline.achieved` divides the same bytes by the average
launch duration, taken from two HIP events recorded on the launch stream around
the timed region (one launch per step, issued back to back).  A second pass
records events around every single launch; its percentiles (`per_launch_us`)
show the spread but include the event packets' own overhead.

The warm-up is at least 400 launches and at least 20 ms of device time
(whichever is longer; `warmup_used` reports both) because the device needs
roughly 10 ms of sustained load before the kernel settles at its steady-state
duration.

`--graph` submits the timed steps as one captured HIP graph instead of one
call per step; it matters only for kernels shorter than a Python call.
`--workload` picks another workload of workloads.py.  The dense ones report
`value` in TFLOP/s of f32 products; their `roofline` is the bf16 matrix-core
issue rate the exact three-part split runs at (six bf16 part products per f32
product) against the bf16 peak, and `f32_equivalent` gives the f32 view.
Workloads on the matrix-core Q8_0 product (2-64 rows) add `bf16_mfma_issue`:
the bf16 MFMA work that product issues against the bf16 peak.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E peak
F32_MFMA_PEAK_TFLOPS = 157.3  # MI355X published dense f32 matrix peak
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 matrix peak
# The dense f32 products run on the bf16 matrix cores: every f32 product is
# six bf16 part products (an exact three-part split of each operand).
DENSE_BF16_PRODUCTS = 6
CSRC = os.path.join(ROOT, "quantized_decode_gemv_q8_amd", "csrc")
# Sources whose hash stamps a traffic measurement (the kernel code itself).
KERNEL_SRC = (os.path.join(CSRC, "q8_gemv_kernel.h"), os.path.join(CSRC, "q8_sum.h"), os.path.join(CSRC, "q8_xcd.h"),
              os.path.join(CSRC, "q8_common.h"))
DOT_SRC = (os.path.join(CSRC, "dot_t.hip"), os.path.join(CSRC, "q8_common.h"))
GEMM_SRC = (os.path.join(CSRC, "q8_gemm.hip"), os.path.join(CSRC, "q8_sum.h"), os.path.join(CSRC, "q8_xcd.h"),
            os.path.join(CSRC, "q8_common.h"))
DENSE_SRC = (os.path.join(CSRC, "dense_f32.hip"), os.path.join(CSRC, "q8_common.h"))
# Kernel-name prefix of each source set, as rocprofv3 reports it.
KERNEL_NAMES = {KERNEL_SRC: "q8_gemv_kernel", GEMM_SRC: "q8_gemm_kernel", DOT_SRC: "dot_t_",
                DENSE_SRC: "dense_split_kernel"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")



def source_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel_path):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None.

    profiles/traffic_counters.json holds FETCH_SIZE/WRITE_SIZE per dispatch,
    already scaled by the copy-kernel calibration, with the hash of the kernel
    source they were taken on; a changed kernel makes the record stale.
    """
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_sha") != source_hash(kernel_path):
        return None
    return rec.get("bytes_per_launch")


WARMUP_FLOOR_MS = 20.0  # the device needs about 10 ms of sustained load to settle


def warm_up(launch, warmup, n_copies, torch):
    """At least `warmup` untimed launches, and more until WARMUP_FLOOR_MS of
    device time have passed since the first (events on the launch stream);
    returns (launches, milliseconds)."""
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    n = 0
    for _ in range(warmup):
        launch(n % n_copies)
        n += 1
    while True:
        t1.record(stream)
        t1.synchronize()
        ms = t0.elapsed_time(t1)
        if ms >= WARMUP_FLOOR_MS:
            return n, ms
        for _ in range(16):
            launch(n % n_copies)
            n += 1


def time_steps(launch, steps, warmup, n_copies, torch):
    """Whole-job pass: the warm-up of warm_up(), then `steps` back-to-back
    launches bracketed by synchronisation; returns (wall seconds, HIP-event
    seconds, (warm-up launches, warm-up ms))."""
    stream = torch.cuda.current_stream()
    wu = warm_up(launch, warmup, n_copies, torch)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for i in range(steps):
        launch((wu[0] + i) % n_copies)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, t_start.elapsed_time(t_end) * 1e-3, wu


def time_steps_graph(launch, steps, warmup, n_copies, torch):
    """The same pass with the timed steps submitted as one HIP graph: the
    `steps` launches are captured once on a side stream (after eager warm-up
    launches there, which also allocate the workspace, for at least
    WARMUP_FLOOR_MS), replayed once untimed, then replayed once inside the
    timed region.  Returns (wall seconds, HIP-event seconds, (warm-up
    launches, warm-up ms)) of the timed replay."""
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        wu = warm_up(launch, max(warmup - steps, 1), n_copies, torch)
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for i in range(steps):
            launch(i % n_copies)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(side):
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        t_start.record(side)
        g.replay()
        t_end.record(side)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    del g
    return wall, t_start.elapsed_time(t_end) * 1e-3, wu


def time_kernels(launch, steps, n_copies, torch):
    """Per-launch pass: HIP events recorded around every launch on the launch
    stream; returns the per-launch durations in milliseconds."""
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        starts[i].record(stream)
        launch(i % n_copies)
        ends[i].record(stream)
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in zip(starts, ends)]


def _time_oracle(call, budget_s):
    call()  # warm-up (page-in of the f64 temporaries)
    times = []
    t_start = time.perf_counter()
    while len(times) < 3 or time.perf_counter() - t_start < budget_s:
        t0 = time.perf_counter()
        call()
        times.append(time.perf_counter() - t0)
    return len(times), sum(times)


def _blas_threads():
    from threadpoolctl import threadpool_info
    return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def device_memory_info(dev_index):
    """Memory clock and bus width as the HIP runtime reports them, and the peak
    they imply.  HIP reports the HBM3/HBM3E clock at a quarter of the per-pin
    data rate (MI300X: 1.3 GHz for 5.2 Gb/s pins, 5.3 TB/s), so the implied
    peak is clock x 4 x bus bytes.  The published 8 TB/s stays the roofline
    peak; this figure is reported beside it."""
    import ctypes

    try:
        hip = ctypes.CDLL("libamdhip64.so")
        clock, width = ctypes.c_int(0), ctypes.c_int(0)
        # hipDeviceAttributeMemoryClockRate (kHz) and hipDeviceAttributeMemoryBusWidth (bits)
        if hip.hipDeviceGetAttribute(ctypes.byref(clock), 60, dev_index) != 0 or \
                hip.hipDeviceGetAttribute(ctypes.byref(width), 59, dev_index) != 0:
            return None
    except OSError:
        return None
    return {"memory_clock_khz": clock.value, "bus_width_bits": width.value,
            "implied_peak_gbs": round(clock.value * 1e3 * 4 * width.value / 8 / 1e9, 1)}


def matrix_mfma_flops(M, K, N):
    """bf16 MFMA flops one launch of the matrix-core product issues: 2 x rows x
    K x N for each of A's three parts, with rows padded to the instance's 16,
    32 or 64 (per pass), K to whole 32-row blocks and N to 512-column tiles."""
    rt = 1 if M <= 16 else 2 if M <= 32 else 4
    rows = 16 * rt * math.ceil(M / (16 * rt))
    return 6 * rows * math.ceil(K / 32) * 32 * math.ceil(N / 512) * 512


def cpu_baseline(wl, A, W, S, budget_s=12.0):
    """The oracle as it stands, timed on the host: whole-workload calls on copy 0,
    repeated until about `budget_s` seconds of CPU work have been measured."""
    import oracle

    n, total = _time_oracle(lambda: oracle.q8_matvec(A, W, S), budget_s)
    threads = _blas_threads()
    return {
        "value": round(wl.algorithmic_bytes() * n / total / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": _cpu_model(),
        "sample": f"f64 factored oracle on the whole M={wl.M} K={wl.K} N={wl.N} workload (copy 0), "
                  f"{n} calls in {total:.1f} s; BLAS threads {threads}, numpy upcasts single-threaded",
    }


def cpu_baseline_fused(wl, A, Ws, Ss, budget_s=12.0):
    """The oracle's sibling projections on the whole fused workload (copy 0)."""
    import oracle

    sib = list(zip(Ws, Ss))
    n, total = _time_oracle(lambda: oracle.q8_matvec_fused(A, sib), budget_s)
    threads = _blas_threads()
    return {
        "value": round(wl.algorithmic_bytes() * n / total / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": _cpu_model(),
        "sample": f"f64 oracle of {wl.siblings} siblings on the whole M={wl.M} K={wl.K} N={wl.N} workload "
                  f"(copy 0), {n} calls in {total:.1f} s; BLAS threads {threads}",
    }


def cpu_baseline_dot_t(wl, A, W, budget_s=12.0):
    """The oracle's exact int64 dot_t on the whole workload (copy 0), in GB/s
    of the workload's algorithmic bytes.  numpy's integer matmul runs on one
    thread (it has no BLAS path)."""
    import oracle

    n, total = _time_oracle(lambda: oracle.dot_t(A, W), budget_s)
    return {
        "value": round(wl.algorithmic_bytes() * n / total / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "cpu_model": _cpu_model(),
        "sample": f"int64 oracle on the whole M={wl.M} K={wl.K} N={wl.N} dot_t (copy 0), {n} calls in {total:.1f} s; "
                  "numpy integer matmul, single-threaded",
    }


def cpu_baseline_dense(wl, A, B, alpha, rows=512, budget_s=12.0):
    """The dense oracle on a bounded sample: the first `rows` rows of A against
    all of B (copy 0), in TFLOP/s of the workload's arithmetic."""
    import oracle

    tr = wl.op == "dot_t_f32"
    As = np.ascontiguousarray(A[:rows])
    n, total = _time_oracle(lambda: oracle.dense_fused(As, B, tr, alpha), budget_s)
    threads = _blas_threads()
    flops = 2.0 * As.shape[0] * wl.N * wl.K
    return {
        "value": round(flops * n / total / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": _cpu_model(),
        "sample": f"f64 dense oracle on rows 0..{As.shape[0] - 1} of A against all of B (K={wl.K} N={wl.N}, "
                  f"copy 0), {n} calls in {total:.1f} s; BLAS threads {threads}",
    }


CALIB_BYTES = 256 << 20  # the calibration copy reads and writes this many bytes
CALIB_COPIES = 5         # calibration copies at the end of a --pmc-pass run


def ingest_pmc(fetch_csv, write_csv, workload, kernel_path):
    """Scales FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the workload's kernel by
    what the same counters read for a device copy of CALIB_BYTES, and records the
    HBM bytes per launch in profiles/traffic_counters.json."""
    import csv

    def per_kernel(path, counter):
        """Counter value per dispatch (summed over its instances), grouped by
        kernel name in dispatch order."""
        sums = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                key = (row["Kernel_Name"], int(row["Dispatch_Id"]))
                sums[key] = sums.get(key, 0.0) + float(row["Counter_Value"])
        by_name = {}
        for (name, did), v in sorted(sums.items(), key=lambda kv: kv[0][1]):
            by_name.setdefault(name, []).append(v)
        return by_name

    def pick(d, sub, last=None):
        hits = [v for k, v in d.items() if sub in k]
        if not hits:
            raise SystemExit(f"no kernel matching {sub!r} in {sorted(d)}")
        vals = hits[0] if last is None else hits[0][-last:]
        return float(np.mean(vals))

    kname = KERNEL_NAMES[kernel_path]
    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    f_k, w_k = pick(fetch, kname), pick(write, kname)
    # The calibration copies are the pass's last CALIB_COPIES copy dispatches
    # (earlier ones, if any, upload inputs).
    f_c, w_c = pick(fetch, "copyBuffer", CALIB_COPIES), pick(write, "copyBuffer", CALIB_COPIES)
    ff, fw = CALIB_BYTES / (f_c * 1024.0), CALIB_BYTES / (w_c * 1024.0)
    rec = {"kernel_sha": source_hash(kernel_path), "fetch_kib": f_k, "write_kib": w_k,
           "copy_fetch_kib": f_c, "copy_write_kib": w_c, "copy_bytes": CALIB_BYTES,
           "fetch_factor": ff, "write_factor": fw,
           "bytes_per_launch": round(f_k * 1024.0 * ff + w_k * 1024.0 * fw)}
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    data[workload] = rec
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps({workload: rec}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default="mlp_up_8192x28672")
    ap.add_argument("--copies", type=int, default=0, help="rotated W/S copies (0: workload default)")
    ap.add_argument("--plan", default="", help="vec,m_tile,workgroups[,kind] override, e.g. 8,1,224 or 0,0,0,2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="submit the timed steps as one captured HIP graph instead of one call each")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="short run for rocprofv3 --pmc: a few launches, then a device copy of known size")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="record HBM traffic per launch from two rocprofv3 --pmc counter CSVs")
    args = ap.parse_args()

    if args.ingest_pmc:
        import csv
        with open(args.ingest_pmc[0]) as f:
            names = [r["Kernel_Name"] for r in csv.DictReader(f)]
        counts = {src: sum(KERNEL_NAMES[src] in n for n in names) for src in KERNEL_NAMES}
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.workload, max(counts, key=counts.get))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import oracle
    from quantized_decode_gemv_q8_amd import binding, workloads

    wl = workloads.WORKLOADS[args.workload]
    n_copies = args.copies or workloads.COPIES.get(args.workload, 1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] workload {wl.name} M={wl.M} K={wl.K} N={wl.N} copies={n_copies}", file=sys.stderr, flush=True)

    plan = None
    if args.plan:
        fields = [int(x) for x in args.plan.split(",")]
        plan = dict(zip(("vec", "m_tile", "workgroups", "kind"), fields))

    # Inputs: copy j drawn with its own seed, uploaded once.
    host0 = workloads.make(wl.name, 0)
    if wl.op == "q8":
        A0, W0, S0 = host0
        A = torch.from_numpy(A0).to(dev)
        Ws, Ss = [], []
        for j in range(n_copies):
            _, Wj, Sj = host0 if j == 0 else workloads.make(wl.name, j)
            Ws.append(torch.from_numpy(Wj).to(dev))
            Ss.append(torch.from_numpy(Sj).to(dev))
        C = torch.empty((wl.M, wl.N), dtype=torch.float32, device=dev)

        if plan is None:
            def launch(j):
                binding.q8_matvec(A, Ws[j], Ss[j], out=C)
        else:
            def launch(j):
                binding.q8_matvec_with_plan(A, Ws[j], Ss[j], plan, out=C)
        used_plan = plan or binding.q8_matvec_choose_plan(wl.M, wl.K, wl.N, 256, 256,
                                                           torch.cuda.get_device_properties(dev).multi_processor_count)
        kernel_src = GEMM_SRC if used_plan.get("kind") == binding.PLAN_MATRIX else KERNEL_SRC
    elif wl.op == "q8_fused":
        A0, W0s, S0s = host0
        A = torch.from_numpy(A0).to(dev)
        Ws, Ss = [], []
        for j in range(n_copies):
            _, Wjs, Sjs = host0 if j == 0 else workloads.make(wl.name, j)
            Ws.append([torch.from_numpy(x).to(dev) for x in Wjs])
            Ss.append([torch.from_numpy(x).to(dev) for x in Sjs])
        Cs = [torch.empty((wl.M, wl.N), dtype=torch.float32, device=dev) for _ in range(wl.siblings)]
        C = Cs[0]

        def launch(j):
            binding.q8_matvec_fused(A, Ws[j], Ss[j], outs=Cs, plan=plan)

        def launch_unfused(j):
            for g in range(wl.siblings):
                binding.q8_matvec(A, Ws[j][g], Ss[j][g], out=Cs[g])
        kernel_src = KERNEL_SRC
        used_plan = plan
    elif wl.op in ("dot_f32", "dot_t_f32"):
        A0, B0 = host0
        tr = wl.op == "dot_t_f32"
        alpha = float(1.0 / np.sqrt(wl.K)) if tr else 1.0  # attention scores take 1/sqrt(head dim)
        As, Bs = [], []
        for j in range(n_copies):
            Aj, Bj = host0 if j == 0 else workloads.make(wl.name, j)
            As.append(torch.from_numpy(Aj).to(dev))
            Bs.append(torch.from_numpy(Bj).to(dev))
        C = torch.empty((wl.M, wl.N), dtype=torch.float32, device=dev)
        fn = binding.q8_dot_t_f32 if tr else binding.q8_dot_f32

        def launch(j):
            fn(As[j], Bs[j], out=C, alpha=alpha)
        kernel_src = DENSE_SRC
        used_plan = None
    else:
        A0, W0 = host0
        A = torch.from_numpy(A0).to(dev)
        Ws = [torch.from_numpy(W0).to(dev)] + [torch.from_numpy(workloads.make(wl.name, j)[1]).to(dev)
                                                for j in range(1, n_copies)]
        C = torch.empty((wl.M, wl.N), dtype=torch.int32, device=dev)

        def launch(j):
            binding.q8_dot_t(A, Ws[j], out=C)
        kernel_src = DOT_SRC
        used_plan = None

    # Parity of copy 0 on sampled columns before anything is timed.
    if not args.no_check:
        launch(0)
        torch.cuda.synchronize()
        cols = np.unique(np.random.default_rng(0).integers(0, wl.N, 512))
        Cg = C.cpu().numpy()[:, cols]
        if wl.op in ("dot_f32", "dot_t_f32"):
            rows = np.unique(np.random.default_rng(0).integers(0, wl.M, 64))
            Ar = np.ascontiguousarray(A0[rows])
            err = oracle.normalised_error(C.cpu().numpy()[rows], oracle.dense_fused(Ar, B0, tr, alpha),
                                          oracle.dense_fused_normaliser(Ar, B0, tr, alpha))
            if not err <= 1e-5:
                raise SystemExit(f"parity check failed: normalised error {err:.3e}")
            cols = rows  # reported below as the sample size
        elif wl.op in ("q8", "q8_fused"):
            pairs = [(W0, S0, Cg)] if wl.op == "q8" else \
                [(W0s[g], S0s[g], Cs[g].cpu().numpy()[:, cols]) for g in range(wl.siblings)]
            for Wg, Sg, Cgg in pairs:
                Wc, Sc = np.ascontiguousarray(Wg[:, cols]), np.ascontiguousarray(Sg[:, cols])
                err = oracle.normalised_error(Cgg, oracle.q8_matvec(A0, Wc, Sc), oracle.q8_normaliser(A0, Wc, Sc))
                if not err <= 1e-5:
                    raise SystemExit(f"parity check failed: normalised error {err:.3e}")
        else:
            if not np.array_equal(Cg, oracle.dot_t(A0, np.ascontiguousarray(W0[cols]))):
                raise SystemExit("parity check failed: dot_t differs from the oracle")
        what = "rows" if wl.op in ("dot_f32", "dot_t_f32") else "columns"
        print(f"[bench] parity ok on {len(cols)} sampled {what}", file=sys.stderr, flush=True)

    if args.pmc_pass:
        for i in range(args.warmup + args.steps):
            launch(i % n_copies)
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(CALIB_COPIES):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_pass": wl.name, "launches": args.warmup + args.steps, "copies": CALIB_COPIES,
                          "copy_bytes": CALIB_BYTES}), flush=True)
        return

    timer = time_steps_graph if args.graph else time_steps
    wall, gpu_s, (wu_n, wu_ms) = timer(launch, args.steps, args.warmup, n_copies, torch)
    per = time_kernels(launch, args.steps, n_copies, torch)
    nbytes = wl.algorithmic_bytes()
    ms_per_step = wall * 1e3 / args.steps
    value = nbytes * args.steps / wall / 1e9
    launch_s = gpu_s / args.steps
    achieved = nbytes / launch_s / 1e9
    print(f"[bench] launch avg {launch_s * 1e6:.2f} us (events over the timed region); "
          f"wall {ms_per_step * 1e3:.2f} us/step; per-launch events median {np.median(per) * 1e3:.2f}, "
          f"p10 {np.percentile(per, 10) * 1e3:.2f}, p90 {np.percentile(per, 90) * 1e3:.2f}",
          file=sys.stderr, flush=True)

    unfused = None
    if wl.op == "q8_fused":
        wall_u, gpu_u, _ = time_steps(launch_unfused, args.steps, args.warmup // 4, n_copies, torch)
        unfused = {"launches_per_step": wl.siblings, "step_us_events": round(gpu_u * 1e6 / args.steps, 3),
                   "value": round(nbytes * args.steps / wall_u / 1e9, 2)}
        print(f"[bench] unfused (one q8_matvec per sibling): {gpu_u * 1e6 / args.steps:.2f} us/step",
              file=sys.stderr, flush=True)

    traffic = measured_traffic(wl.name, kernel_src)
    dense = wl.op in ("dot_f32", "dot_t_f32")
    if dense:
        # The dense products are bound by the f32 matrix rate: value and roofline in TFLOP/s.
        flops = wl.algorithmic_flops()
        value = flops * args.steps / wall / 1e12
        achieved = flops / launch_s / 1e12
    headline = "Q8_0 GEMV effective HBM GB/s and % of peak at K=8192,N=28672, M=1"
    result = {
        "metric": headline if wl.name == "mlp_up_8192x28672" else
        (f"f32 TFLOP/s, {wl.name}" if dense else f"effective HBM GB/s, {wl.name}"),
        "value": round(value, 2),
        "unit": "TFLOP/s" if dense else "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_used": {"launches": wu_n, "device_ms": round(wu_ms, 2), "floor_ms": WARMUP_FLOOR_MS},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i32" if wl.op == "dot_t" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N, "siblings": wl.siblings,
                   "rotated_copies": n_copies,
                   "algorithmic_bytes_per_step": nbytes, "plan": used_plan,
                   **({"algorithmic_flops_per_step": wl.algorithmic_flops()} if dense else {})},
        "roofline": {"bound": "mfma", "achieved": round(DENSE_BF16_PRODUCTS * achieved, 2),
                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(DENSE_BF16_PRODUCTS * achieved / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": traffic,
                     "dtype": "bf16 (f32 operands split exactly into three bf16 parts, six part products each)"}
        if dense else
        {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
        "pct_of_peak": round(100.0 * (DENSE_BF16_PRODUCTS * value / BF16_MFMA_PEAK_TFLOPS if dense else
                                      value / HBM_PEAK_GBS), 2),
        "launch_us": round(launch_s * 1e6, 3),
        "submission": "one HIP graph of the timed steps" if args.graph else "one call per step",
        "per_launch_us": {"mean": round(float(np.mean(per)) * 1e3, 3), "median": round(float(np.median(per)) * 1e3, 3),
                      "p10": round(float(np.percentile(per, 10)) * 1e3, 3),
                      "p90": round(float(np.percentile(per, 90)) * 1e3, 3)},
    }
    props = torch.cuda.get_device_properties(dev)
    result["device"] = {"name": props.name, "arch": props.gcnArchName, "compute_units": props.multi_processor_count,
                        **(device_memory_info(dev.index or 0) or {})}
    if unfused is not None:
        result["unfused"] = unfused
    if wl.op == "q8" and used_plan.get("kind") == binding.PLAN_MATRIX:
        # The matrix-core product's own ceiling: the bf16 MFMA work it issues
        # (three parts of A per block; rows padded to the 16-, 32- or 64-row
        # instance and columns to 512-wide tiles) against the bf16 peak.
        flops = matrix_mfma_flops(wl.M, wl.K, wl.N)
        issue = flops / launch_s / 1e12
        result["bf16_mfma_issue"] = {"achieved": round(issue, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                     "frac": round(issue / BF16_MFMA_PEAK_TFLOPS, 4), "flops_per_launch": flops}
    if dense:
        # The same launches counted as f32 products: against the f32 matrix
        # peak, and against the ceiling of the bf16 split (bf16 peak / 6).
        result["f32_equivalent"] = {"achieved": round(achieved, 2), "unit": "TFLOP/s",
                                    "f32_matrix_peak": F32_MFMA_PEAK_TFLOPS,
                                    "vs_f32_matrix_peak": round(achieved / F32_MFMA_PEAK_TFLOPS, 4),
                                    "split_ceiling": round(BF16_MFMA_PEAK_TFLOPS / DENSE_BF16_PRODUCTS, 1),
                                    "bf16_products_per_f32_product": DENSE_BF16_PRODUCTS}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        if wl.op == "q8":
            result["cpu_baseline"] = cpu_baseline(wl, A0, W0, S0)
        elif wl.op == "q8_fused":
            result["cpu_baseline"] = cpu_baseline_fused(wl, A0, W0s, S0s)
        elif dense:
            result["cpu_baseline"] = cpu_baseline_dense(wl, A0, B0, alpha)
        else:
            result["cpu_baseline"] = cpu_baseline_dot_t(wl, A0, W0)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
