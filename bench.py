"""Benchmark of the Q8_0 decode matvec on one MI355X.

A step is one q8_matvec call (plan, activation staging, weight streaming,
convert, block partials, one scale per block and column, accumulate, split-K
combine, masked store) over one rotated copy of the synthetic workload's
weights and scales.  Default workload: the 70B-class MLP up-projection,
M=1, K=8192, N=28672, with 4 rotated W/S copies (about 1.06 GB) so that every
step reads its weights from HBM rather than the 256 MB Infinity Cache.

Prints ONE JSON line.  `value` is the effective HBM bandwidth on algorithmic
bytes (K*N + 4*ceil(K/32)*N + 4*M*K + 4*M*N per step) over the whole timed
region; `roofline.achieved` uses the average kernel duration from HIP events
recorded around each launch on the launch stream.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E peak
KERNEL_SRC = os.path.join(ROOT, "quantized_decode_gemv_q8_amd", "csrc", "q8_gemv.hip")
DOT_SRC = os.path.join(ROOT, "quantized_decode_gemv_q8_amd", "csrc", "dot_t.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")

# Rotated copies per workload: enough to exceed the Infinity Cache (>= 1 GiB).
COPIES = {"tiny": 1, "attn4096": 57, "mlp_up_8192x28672": 4, "mlp_down_28672x8192": 4,
          "ragged_m4": 47, "dot_t_16x4096x4096": 63}


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


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


def time_steps(launch, steps, warmup, n_copies, torch):
    """Whole-job pass: `warmup` untimed steps, then `steps` back-to-back launches
    bracketed by synchronisation; returns (wall seconds, HIP-event seconds)."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        launch(i % n_copies)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for i in range(steps):
        launch((warmup + i) % n_copies)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, t_start.elapsed_time(t_end) * 1e-3


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


def cpu_baseline(wl, A, W, S, budget_s=12.0):
    """The oracle as it stands, timed on the host on a column slice of the workload."""
    import oracle
    from threadpoolctl import threadpool_info

    n_cols = min(wl.N, 4096)
    Ws = np.ascontiguousarray(W[:, :n_cols])
    Ss = np.ascontiguousarray(S[:, :n_cols])
    from quantized_decode_gemv_q8_amd.workloads import Workload
    sample = Workload("sample", "q8", wl.M, wl.K, n_cols, wl.a_dist, wl.w_dist, wl.seed)
    oracle.q8_matvec(A, Ws, Ss)  # warm-up
    times = []
    t_start = time.perf_counter()
    while not times or (time.perf_counter() - t_start < budget_s and len(times) < 50):
        t0 = time.perf_counter()
        oracle.q8_matvec(A, Ws, Ss)
        times.append(time.perf_counter() - t0)
    med = float(np.median(times))
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {
        "value": round(sample.algorithmic_bytes() / med / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"f64 factored oracle on columns 0..{n_cols - 1} of the same M={wl.M} K={wl.K} inputs "
                  f"(copy 0), median of {len(times)} runs ({sum(times):.1f} s of CPU work); "
                  f"BLAS threads {threads}, numpy upcasts single-threaded",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mlp_up_8192x28672")
    ap.add_argument("--copies", type=int, default=0, help="rotated W/S copies (0: workload default)")
    ap.add_argument("--plan", default="", help="vec,m_tile,splits override, e.g. 16,1,12")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import oracle
    from quantized_decode_gemv_q8_amd import binding, workloads

    wl = workloads.WORKLOADS[args.workload]
    n_copies = args.copies or COPIES.get(args.workload, 1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] workload {wl.name} M={wl.M} K={wl.K} N={wl.N} copies={n_copies}", file=sys.stderr, flush=True)

    plan = None
    if args.plan:
        v, mt, sp = (int(x) for x in args.plan.split(","))
        plan = {"vec": v, "m_tile": mt, "splits": sp}

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
        kernel_src = KERNEL_SRC
        used_plan = plan or binding.q8_matvec_choose_plan(wl.M, wl.K, wl.N, 256, 256,
                                                           torch.cuda.get_device_properties(dev).multi_processor_count)
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
        if wl.op == "q8":
            ref = oracle.q8_matvec(A0, np.ascontiguousarray(W0[:, cols]), np.ascontiguousarray(S0[:, cols]))
            D = oracle.q8_normaliser(A0, np.ascontiguousarray(W0[:, cols]), np.ascontiguousarray(S0[:, cols]))
            err = oracle.normalised_error(Cg, ref, D)
            if not err <= 1e-5:
                raise SystemExit(f"parity check failed: normalised error {err:.3e}")
        else:
            if not np.array_equal(Cg, oracle.dot_t(A0, np.ascontiguousarray(W0[cols]))):
                raise SystemExit("parity check failed: dot_t differs from the oracle")
        print(f"[bench] parity ok on {len(cols)} sampled columns", file=sys.stderr, flush=True)

    wall, gpu_s = time_steps(launch, args.steps, args.warmup, n_copies, torch)
    per = time_kernels(launch, args.steps, n_copies, torch)
    nbytes = wl.algorithmic_bytes()
    ms_per_step = wall * 1e3 / args.steps
    value = nbytes * args.steps / wall / 1e9
    kern_ms = float(np.mean(per))
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    print(f"[bench] kernel avg {kern_ms * 1e3:.2f} us (median {np.median(per) * 1e3:.2f}, "
          f"p10 {np.percentile(per, 10) * 1e3:.2f}, p90 {np.percentile(per, 90) * 1e3:.2f}); "
          f"wall {ms_per_step * 1e3:.2f} us/step, events {gpu_s * 1e6 / args.steps:.2f} us/step",
          file=sys.stderr, flush=True)

    traffic = measured_traffic(wl.name, kernel_src)
    headline = "Q8_0 GEMV effective HBM GB/s and % of peak at K=8192,N=28672, M=1"
    result = {
        "metric": headline if wl.name == "mlp_up_8192x28672" else f"effective HBM GB/s, {wl.name}",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.op == "q8" else "i32",
        "data": "synthetic",
        "config": {"workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N, "rotated_copies": n_copies,
                   "algorithmic_bytes_per_step": nbytes, "plan": used_plan},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "step_us_events": round(gpu_s * 1e6 / args.steps, 3),
        "kernel_us": {"mean": round(kern_ms * 1e3, 3), "median": round(float(np.median(per)) * 1e3, 3),
                      "p10": round(float(np.percentile(per, 10)) * 1e3, 3),
                      "p90": round(float(np.percentile(per, 90)) * 1e3, 3)},
    }
    if not args.no_cpu_baseline and wl.op == "q8":
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, A0, W0, S0)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
