#!/usr/bin/env python3
"""Benchmark of the accurate float32 reduction path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * the variance of a [4096, 4096] float32 array along axis 1 (ddof 0,
    N(1e4, 1), seed 2) -- shift, compensated trees of y, d and d^2,
    two-term correction (the timing shape of the method page's §3);
  * the compensated tree sum of 10^8 float32 values (99% N(0,1), 1% large
    exactly cancelling +/- pairs, seed 3).
Inputs are resident in HBM before timing starts.  Several copies of each
input are cycled so that the 256 MB Infinity Cache cannot serve them
(6 x 64 MiB variance inputs, 2 x 400 MB sum inputs).

Prints ONE JSON line: whole-step throughput in GElem/s (10^9 input elements
per second), a roofline entry for the dominant kernel (the 10^8 sum; HBM
bound), the variance kernel's own entry, and the CPU oracle timed on the
host as a reported baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --calibrate-copy     (a plain 400 MB copy, for counter scaling)
       python bench.py --only KERNEL [--steps K] [--warmup W]
                                            (K launches of one kernel on the same inputs,
                                             for profiler runs: variance, variance_axis0,
                                             sum, adn, read)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GElem/s + % HBM peak: fp32 TwoSum-tree variance [4096,4096], 1e8-elem sum"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD datasheet
VALU_PEAK_TOPS = 39.3216       # 256 CU x 64 lanes x 2.4 GHz plain (non-packed) FP32 ops
VAR_ROWS, VAR_COLS = 4096, 4096
SUM_N = 100_000_000
N_VAR_COPIES, N_SUM_COPIES = 6, 2
# Algorithmic bytes per launch: every input value read once, outputs written once.
VAR_BYTES = VAR_ROWS * VAR_COLS * 4 + 2 * VAR_ROWS * 4
SUM_BYTES = SUM_N * 4 + 4
# Plain FP32 VALU operations the method needs per variance element, one tree
# node per element: shift 1, plain tree of y 1, centre 1, square 1,
# compensated tree of d 7 (TwoSum 6 + carry 1), of d^2 6 (Fast2Sum on
# non-negative operands 4 + carry 2).
VAR_OPS_PER_ELEM = 17
VAR_KERNEL = "k_var_rows_full<16, 4>"
VAR0_KERNEL = "k_cols_one<1, 16, 4, false, 64, 1>"
SUM_COUNTERS = os.path.join(ROOT, "profiles", "k_tree_sum_1e8_counters.txt")
VAR_COUNTERS = os.path.join(ROOT, "profiles", "k_var_rows_full_4096x4096_counters.txt")
VAR_VALU = os.path.join(ROOT, "profiles", "k_var_rows_full_4096x4096_valu.txt")
VAR0_COUNTERS = os.path.join(ROOT, "profiles", "k_cols_one_4096x4096_axis0_counters.txt")
ADN_COUNTERS = os.path.join(ROOT, "profiles", "k_adn_sum_1e8_counters.txt")
ADN_FOLD = 3
# float-sum throughput printed on the ADN page ("Scalar-sum throughput", GElements/s)
ADN_PAGE_FLOAT_GELEMS = {"NVIDIA GB10": 55.4, "NVIDIA RTX PRO 4500 Blackwell": 135.1,
                         "AMD Radeon Pro W7500": 16.0, "Intel Arc Pro B70": 54.2}


def source_digest() -> str:
    h = hashlib.sha256()
    for rel in ("stable_variance_amd/csrc/sv_lib.hip", "stable_variance_amd/csrc/sv_adn.hip",
                "stable_variance_amd/csrc/sv_f64.hip", "stable_variance_amd/csrc/sv_device.hpp",
                "stable_variance_amd/csrc/sv_index.hpp", "stable_variance_amd/csrc/sv_adn_kernel.hpp",
                "stable_variance_amd/csrc/sv_adn_folds_9_14.hip", "stable_variance_amd/csrc/sv_adn_folds_15_21.hip"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_summary(path, key):
    """One figure from a committed rocprofv3 counter summary, or None when
    the summary is absent or was taken on other kernel source."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest():
        return None
    try:
        return float(kv[key].split()[0])  # the figure, before any note
    except (KeyError, ValueError, IndexError):
        return None


def read_counter_traffic(path):
    """HBM bytes per launch (FETCH_SIZE and WRITE_SIZE scaled by a plain copy
    of known size) from a committed counter summary, or None."""
    return read_summary(path, "traffic_bytes_per_launch")


def calibrate_copy():
    import torch

    dev = torch.device("cuda:0")
    src = torch.ones(SUM_N, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": SUM_N * 4, "bytes_written": SUM_N * 4, "launches": 3}))


def cpu_baseline(c4_host, c5_host):
    """The oracle (single-threaded C, as it stands) on the same workload:
    the full [4096,4096] variance and the full 10^8 sum, repeated until about
    10 s have passed (at most 30 repetitions)."""
    import oracle

    oracle.lib()
    reps, t_total = 0, 0.0
    while reps < 30 and t_total < 10.0:
        t0 = time.perf_counter()
        oracle.variance(c4_host, axis=1)
        oracle.tree_sum(c5_host)
        t_total += time.perf_counter() - t0
        reps += 1
    elems = (VAR_ROWS * VAR_COLS + SUM_N) * reps
    return {"value": round(elems / t_total / 1e9, 5), "unit": "GElem/s", "cores": 1, "kind": "oracle",
            "sample": f"full workload ({VAR_ROWS}x{VAR_COLS} variance + {SUM_N} sum) x {reps} reps, "
                      f"{t_total:.1f} s, single-threaded C oracle"}


def cpu_oracle_all_cores(c4_host, c5_host):
    """The same oracle on every host core the process may use: slices of the
    variance in blocks, the sum cut into aligned subtrees (same bits),
    repeated until about 5 s have passed."""
    import oracle

    cores = min(len(os.sched_getaffinity(0)), 16)
    reps, t_total = 0, 0.0
    while reps < 30 and t_total < 5.0:
        t0 = time.perf_counter()
        oracle.variance_threads(c4_host, 1, cores)
        oracle.tree_sum_threads(c5_host, cores)
        t_total += time.perf_counter() - t0
        reps += 1
    elems = (VAR_ROWS * VAR_COLS + SUM_N) * reps
    return {"value": round(elems / t_total / 1e9, 5), "unit": "GElem/s", "cores": cores, "kind": "oracle",
            "sample": f"full workload x {reps} reps, {t_total:.1f} s, C oracle on {cores} threads"}


def only(kernel, steps, warmup):
    """K launches of one kernel on the benchmark's inputs (after W untimed
    ones), nothing else: the command the committed profiles are taken with."""
    import torch

    import stable_variance_amd as sv
    import workloads as W

    dev = torch.device("cuda:0")
    L = sv.capi()
    sh = torch.cuda.current_stream(dev).cuda_stream

    def check(st):
        if st != 0:
            raise RuntimeError(L.sv_last_error_message().decode())

    if kernel in ("variance", "variance_axis0"):
        c4 = [torch.from_numpy(W.c4_matrix()).to(dev)]
        for k in range(1, N_VAR_COPIES):
            c4.append(torch.roll(c4[0], shifts=97 * k, dims=1).contiguous())
        axis = 1 if kernel == "variance" else 0
        nsl = VAR_ROWS if axis == 1 else VAR_COLS
        ws_b = max(1, L.sv_variance_f32_workspace_size(VAR_ROWS, VAR_COLS, axis))
        ws = torch.zeros(ws_b, dtype=torch.uint8, device=dev)
        v = torch.empty(nsl, dtype=torch.float32, device=dev)
        m = torch.empty(nsl, dtype=torch.float32, device=dev)
        run = lambda i: check(L.sv_variance_f32(c4[i % N_VAR_COPIES].data_ptr(), VAR_ROWS, VAR_COLS, axis, 0,
                                                v.data_ptr(), m.data_ptr(), ws.data_ptr(), ws_b, sh))
        elems = VAR_ROWS * VAR_COLS
    else:
        c5 = [torch.from_numpy(W.sum_cancelling_pairs()).to(dev)]
        for k in range(1, N_SUM_COPIES):
            c5.append(torch.roll(c5[0], shifts=1_000_003 * k).contiguous())
        out = torch.empty((), dtype=torch.float32, device=dev)
        if kernel == "sum":
            ws_b = L.sv_tree_sum_f32_workspace_size(SUM_N)
            ws = torch.zeros(ws_b, dtype=torch.uint8, device=dev)
            run = lambda i: check(L.sv_tree_sum_f32(c5[i % N_SUM_COPIES].data_ptr(), SUM_N, out.data_ptr(),
                                                    ws.data_ptr(), ws_b, sh))
        elif kernel == "adn":
            ws_b = L.sv_adn_sum_f32_workspace_size(SUM_N)
            ws = torch.zeros(ws_b, dtype=torch.uint8, device=dev)
            run = lambda i: check(L.sv_adn_sum_f32(c5[i % N_SUM_COPIES].data_ptr(), SUM_N, ADN_FOLD, out.data_ptr(),
                                                   ws.data_ptr(), ws_b, sh))
        elif kernel == "read":
            run = lambda i: check(L.sv_probe_read_bandwidth(c5[i % N_SUM_COPIES].data_ptr(), SUM_N, out.data_ptr(),
                                                             sh))
        else:
            raise SystemExit(f"bench.py --only: unknown kernel {kernel!r}")
        elems = SUM_N
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"only": kernel, "launches": steps, "warmup": warmup, "avg_ms": round(ms, 5),
                      "gelem_s": round(elems / (ms * 1e-3) / 1e9, 2)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=60.0,
                    help="untimed steps run back to back for this long before the warm-up steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--only", default=None, help="run one kernel only (see the usage above)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; the benchmark runs on one GPU "
              f"(the method has no cross-GPU step).", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.only:
        only(args.only, args.steps, args.warmup)
        return

    import numpy as np
    import torch

    import stable_variance_amd as sv
    import workloads as W

    dev = torch.device("cuda:0")
    L = sv.capi()

    # ---------------- inputs (host generation, then resident in HBM)
    c4_host = W.c4_matrix()
    c5_host = W.sum_cancelling_pairs()
    c4 = [torch.from_numpy(c4_host).to(dev)]
    for k in range(1, N_VAR_COPIES):
        c4.append(torch.roll(c4[0], shifts=97 * k, dims=1).contiguous())
    c5 = [torch.from_numpy(c5_host).to(dev)]
    for k in range(1, N_SUM_COPIES):
        c5.append(torch.roll(c5[0], shifts=1_000_003 * k).contiguous())
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    ws_bytes = L.sv_tree_sum_f32_workspace_size(SUM_N)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    var_out = torch.empty(VAR_ROWS, dtype=torch.float32, device=dev)
    mean_out = torch.empty(VAR_ROWS, dtype=torch.float32, device=dev)
    sum_out = torch.empty((), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def check(st):
        if st != 0:
            raise RuntimeError(L.sv_last_error_message().decode())

    # launch arguments prepared once: the per-launch host cost is then the
    # ctypes call alone, well below the kernels' durations
    var_fn, sum_fn = L.sv_variance_f32, L.sv_tree_sum_f32
    var_args = [(a.data_ptr(), VAR_ROWS, VAR_COLS, 1, 0, var_out.data_ptr(), mean_out.data_ptr(), None, 0, sh)
                for a in c4]
    sum_args = [(b.data_ptr(), SUM_N, sum_out.data_ptr(), ws.data_ptr(), ws_bytes, sh) for b in c5]

    def run_var(i):
        if var_fn(*var_args[i % N_VAR_COPIES]):
            check(1)

    def run_sum(i):
        if sum_fn(*sum_args[i % N_SUM_COPIES]):
            check(1)

    # ---------------- clock settle: after an idle spell of even 20 ms the chip's
    # clocks take about 10 ms of sustained load to reach their steady state
    # (the tree sum runs ~10% slower meanwhile), so whole steps run back to
    # back for --settle-ms before the warm-up steps.
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for i in range(8):
            run_var(i)
            run_sum(i)
        settle_steps += 8
        torch.cuda.synchronize()

    # ---------------- warmup
    for i in range(args.warmup):
        run_var(i)
        run_sum(i)
    torch.cuda.synchronize()

    # ---------------- timed region: K steps.  The K variance launches run back to
    # back, then the K sum launches (each step's two parts are independent), with
    # HIP events on the launch stream between the two phases, so the per-kernel
    # average launch durations come from the timed region itself.
    K = args.steps
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        run_var(i)
    e1.record(stream)
    for i in range(K):
        run_sum(i)
    e2.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    var_avg = e0.elapsed_time(e1) / K
    sum_avg = e1.elapsed_time(e2) / K

    # ---------------- parity spot check at full size (the timed launch configuration)
    parity = None
    if not args.no_cpu_baseline:
        import oracle

        run_var(0)
        run_sum(0)
        torch.cuda.synchronize()
        rows = np.random.default_rng(0).choice(VAR_ROWS, 16, replace=False)
        ov, om = oracle.variance(c4_host[rows], axis=1)
        gv = var_out.cpu().numpy()[rows]
        gm = mean_out.cpu().numpy()[rows]
        ok_var = bool(np.array_equal(gv.view(np.uint32), ov.view(np.uint32)) and
                      np.array_equal(gm.view(np.uint32), om.view(np.uint32)))
        os_ = oracle.tree_sum(c5_host)
        ok_sum = bool(np.float32(sum_out.item()).view(np.uint32) == np.float32(os_).view(np.uint32))
        parity = {"variance_16_rows_bit_exact": ok_var, "sum_bit_exact": ok_sum}

    # ---------------- context: library reductions on the same buffers
    def time_op(fn, reps=20):
        for _ in range(3):
            fn(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # per-kernel batches after the timed steps: 7 batches of 50 launches each,
    # median / min / max of the per-launch time (the method page timed 7 runs)
    def batches(fn, n_batches=7, reps=50):
        t = sorted(time_op(fn, reps) for _ in range(n_batches))
        return {"median_ms": round(t[len(t) // 2], 5), "min_ms": round(t[0], 5), "max_ms": round(t[-1], 5),
                "batches": n_batches, "launches_per_batch": reps}

    var_batches = batches(run_var)
    sum_batches = batches(run_sum)
    torch_var_ms = time_op(lambda i: torch.var(c4[i % N_VAR_COPIES], dim=1, correction=0))
    # The step's two parts are independent: the VALU-bound variance and the
    # HBM-bound sum on two default-priority streams at once, each with its
    # own buffers.  Context only: `value` is the sequential step above.
    s_var, s_sum = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    ws2 = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    var2 = [(a.data_ptr(), VAR_ROWS, VAR_COLS, 1, 0, var_out.data_ptr(), mean_out.data_ptr(), None, 0,
             s_var.cuda_stream) for a in c4]
    sum2 = [(b.data_ptr(), SUM_N, sum_out.data_ptr(), ws2.data_ptr(), ws_bytes, s_sum.cuda_stream) for b in c5]

    def two_streams(k):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev_var, ev_sum = torch.cuda.Event(), torch.cuda.Event()
        torch.cuda.synchronize()
        start.record(stream)
        s_var.wait_event(start)
        s_sum.wait_event(start)
        for i in range(k):
            check(var_fn(*var2[i % N_VAR_COPIES]))
            check(sum_fn(*sum2[i % N_SUM_COPIES]))
        ev_var.record(s_var)
        ev_sum.record(s_sum)
        stream.wait_event(ev_var)
        stream.wait_event(ev_sum)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / k

    two_streams(5)
    overlap_ms = min(two_streams(K) for _ in range(3))
    overlap = {"ms_per_step": round(overlap_ms, 5),
               "gelem_s": round((VAR_ROWS * VAR_COLS + SUM_N) / (overlap_ms * 1e-3) / 1e9, 2),
               "over_sequential_step": round(overlap_ms / ((var_avg + sum_avg)), 3)}
    # the same buffers along axis 0 (4096 column slices of stride 4096: one
    # launch, sixteen whole columns per workgroup, the input read once)
    ws0 = torch.zeros(max(1, L.sv_variance_f32_workspace_size(VAR_ROWS, VAR_COLS, 0)), dtype=torch.uint8, device=dev)
    v0 = torch.empty(VAR_COLS, dtype=torch.float32, device=dev)
    m0 = torch.empty(VAR_COLS, dtype=torch.float32, device=dev)
    run_var0 = lambda i: check(L.sv_variance_f32(c4[i % N_VAR_COPIES].data_ptr(), VAR_ROWS, VAR_COLS, 0, 0,
                                                 v0.data_ptr(), m0.data_ptr(), ws0.data_ptr(), ws0.numel(), sh))
    var0_ms = time_op(run_var0, reps=400)  # about 10 ms of work: clocks at their steady state
    torch_var0_ms = time_op(lambda i: torch.var(c4[i % N_VAR_COPIES], dim=0, correction=0))
    var0_gbs = VAR_BYTES / (var0_ms * 1e-3) / 1e9
    axis0 = {"kernel": VAR0_KERNEL, "avg_ms": round(var0_ms, 5), "gb_s": round(var0_gbs, 1),
             "hbm_frac": round(var0_gbs / HBM_PEAK_GBS, 4), "traffic": read_counter_traffic(VAR0_COUNTERS),
             "torch_var_dim0_ms": round(torch_var0_ms, 5)}
    if parity is not None:
        run_var0(0)
        torch.cuda.synchronize()
        cols = np.random.default_rng(1).choice(VAR_COLS, 16, replace=False)
        ov0, om0 = oracle.variance(np.ascontiguousarray(c4_host[:, cols]), axis=0)
        axis0["bit_exact_16_columns"] = bool(
            np.array_equal(v0.cpu().numpy()[cols].view(np.uint32), ov0.view(np.uint32)) and
            np.array_equal(m0.cpu().numpy()[cols].view(np.uint32), om0.view(np.uint32)))
    torch_sum_ms = time_op(lambda i: torch.sum(c5[i % N_SUM_COPIES]))
    # practical HBM read ceiling: a plain non-temporal read of the same buffers
    probe_out = torch.empty(1, dtype=torch.float32, device=dev)
    # (the median of 7 batches, like the kernels' own batches: a single short
    # batch after the context measurements can run at unsettled clocks)
    read_sum_ms = batches(lambda i: check(L.sv_probe_read_bandwidth(c5[i % N_SUM_COPIES].data_ptr(), SUM_N,
                                                                     probe_out.data_ptr(), sh)))["median_ms"]
    read_var_ms = batches(lambda i: check(L.sv_probe_read_bandwidth(c4[i % N_VAR_COPIES].data_ptr(),
                                                                     VAR_ROWS * VAR_COLS, probe_out.data_ptr(), sh)),
                          reps=60)["median_ms"]
    read_sum_gbs = SUM_N * 4 / (read_sum_ms * 1e-3) / 1e9
    read_var_gbs = VAR_ROWS * VAR_COLS * 4 / (read_var_ms * 1e-3) / 1e9

    # the method page's ablation rows on the same [4096,4096] buffers: time of
    # each variant and its ratio to the two-term reference formula
    variant_ms = {}
    for name, code in sv.VARIANTS.items():
        variant_ms[name] = time_op(lambda i, c=code: check(L.sv_variance_variant_f32(
            c4[i % N_VAR_COPIES].data_ptr(), VAR_ROWS, VAR_COLS, 1, 0, c, var_out.data_ptr(), mean_out.data_ptr(),
            sh)), reps=60)
    variants = {k: {"ms": round(v, 5), "ratio_to_reference": round(v / variant_ms["reference"], 3)}
                for k, v in variant_ms.items()}

    # second workload: the ADN binned reproducible sum of the same 10^8 values
    adn_need = L.sv_adn_sum_f32_workspace_size(SUM_N)
    adn_ws = torch.zeros(adn_need, dtype=torch.uint8, device=dev)
    adn_out = torch.empty((), dtype=torch.float32, device=dev)
    adn_ms = time_op(lambda i: check(L.sv_adn_sum_f32(c5[i % N_SUM_COPIES].data_ptr(), SUM_N, ADN_FOLD,
                                                     adn_out.data_ptr(), adn_ws.data_ptr(), adn_need, sh)), reps=40)
    adn_gbs = SUM_BYTES / (adn_ms * 1e-3) / 1e9
    adn = {"kernel": f"k_adn_sum<{ADN_FOLD}, 16> (1e8 values)", "fold": ADN_FOLD, "avg_launch_ms": round(adn_ms, 5),
           "gelem_s": round(SUM_N / (adn_ms * 1e-3) / 1e9, 2),
           "hbm": {"achieved": round(adn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac": round(adn_gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": SUM_BYTES,
                   "traffic": read_counter_traffic(ADN_COUNTERS), "read_ceiling_gbs": round(read_sum_gbs, 1),
                   "frac_of_read_ceiling": round(adn_gbs / read_sum_gbs, 4)},
           "over_tree_sum": round(adn_ms / sum_avg, 3),
           "pages_float_sum_gelem_s": ADN_PAGE_FLOAT_GELEMS, "bit_exact": None, "cpu_oracle": None}
    if not args.no_cpu_baseline:
        from oracle import adn as oracle_adn

        check(L.sv_adn_sum_f32(c5[0].data_ptr(), SUM_N, ADN_FOLD, adn_out.data_ptr(), adn_ws.data_ptr(), adn_need, sh))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        want = oracle_adn.adn_sum(c5_host, ADN_FOLD)
        t_or = time.perf_counter() - t0
        adn["bit_exact"] = bool(np.float32(adn_out.item()).view(np.uint32) == np.float32(want).view(np.uint32))
        adn["cpu_oracle"] = {"value": round(SUM_N / t_or / 1e9, 5), "unit": "GElem/s", "cores": 1, "kind": "oracle",
                             "sample": f"the full 10^8 sum once, {t_or:.1f} s, numpy closed form (float64 steps, "
                                       f"integer sums)"}

    # carry variant: the same tree with double-word (renormalised) carries
    dw_ms = time_op(lambda i: check(L.sv_tree_sum_dw_f32(c5[i % N_SUM_COPIES].data_ptr(), SUM_N,
                                                        sum_out.data_ptr(), ws.data_ptr(), ws_bytes, sh)), reps=40)
    dw_gbs = SUM_BYTES / (dw_ms * 1e-3) / 1e9
    dw = {"kernel": "k_tree_sum<32, ..., NODE_DW> (1e8 values)", "avg_launch_ms": round(dw_ms, 5),
          "gelem_s": round(SUM_N / (dw_ms * 1e-3) / 1e9, 2),
          "hbm": {"achieved": round(dw_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(dw_gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": SUM_BYTES,
                  "frac_of_read_ceiling": round(dw_gbs / read_sum_gbs, 4)},
          "over_tree_sum": round(dw_ms / sum_avg, 3), "bit_exact": None, "accuracy": None, "cpu_oracle": None}
    if not args.no_cpu_baseline:
        check(L.sv_tree_sum_dw_f32(c5[0].data_ptr(), SUM_N, sum_out.data_ptr(), ws.data_ptr(), ws_bytes, sh))
        torch.cuda.synchronize()
        got_dw = np.float32(sum_out.item())
        t0 = time.perf_counter()
        want_dw = oracle.tree_sum_dw(c5_host)
        t_dw = time.perf_counter() - t0
        exact = oracle.exact_sum(c5_host)
        dw["bit_exact"] = bool(got_dw.view(np.uint32) == np.float32(want_dw).view(np.uint32))
        rel = lambda v: abs(float(v) - float(exact)) / abs(float(exact))
        dw["accuracy"] = {"exact_sum": float(exact), "dw_value": float(got_dw), "dw_rel_err": rel(got_dw),
                          "plain_value": float(os_), "plain_rel_err": rel(os_),
                          "dw_is_correctly_rounded": bool(got_dw == oracle.round_f32(exact))}
        dw["cpu_oracle"] = {"value": round(SUM_N / t_dw / 1e9, 5), "unit": "GElem/s", "cores": 1, "kind": "oracle",
                            "sample": f"the full 10^8 sum once, {t_dw:.2f} s, single-threaded C oracle"}

    # the float64 path: the same workloads in double (2 + 4 copies)
    c5d = [t.to(torch.float64) for t in c5]
    c4d = [c4[k].to(torch.float64) for k in range(4)]
    need64 = L.sv_tree_sum_f64_workspace_size(SUM_N)
    ws64 = torch.zeros(need64, dtype=torch.uint8, device=dev)
    out64 = torch.empty((), dtype=torch.float64, device=dev)
    var64 = torch.empty(VAR_ROWS, dtype=torch.float64, device=dev)
    mean64 = torch.empty(VAR_ROWS, dtype=torch.float64, device=dev)
    sum64_ms = time_op(lambda i: check(L.sv_tree_sum_f64(c5d[i % 2].data_ptr(), SUM_N, out64.data_ptr(),
                                                        ws64.data_ptr(), need64, sh)), reps=30)
    var64_ms = time_op(lambda i: check(L.sv_variance_f64(c4d[i % 4].data_ptr(), VAR_ROWS, VAR_COLS, 1, 0,
                                                        var64.data_ptr(), mean64.data_ptr(), None, 0, sh)), reps=40)
    read64_ms = time_op(lambda i: check(L.sv_probe_read_bandwidth(c5d[i % 2].data_ptr(), 2 * SUM_N,
                                                                   probe_out.data_ptr(), sh)), reps=20)
    # along axis 0: columns of 4096 doubles read once
    var64c = torch.empty(VAR_COLS, dtype=torch.float64, device=dev)
    ws64c_n = max(1, L.sv_variance_f64_workspace_size(VAR_ROWS, VAR_COLS, 0))
    ws64c = torch.zeros(ws64c_n, dtype=torch.uint8, device=dev)
    var64c_ms = time_op(lambda i: check(L.sv_variance_f64(c4d[i % 4].data_ptr(), VAR_ROWS, VAR_COLS, 0, 0,
                                                         var64c.data_ptr(), None, ws64c.data_ptr(), ws64c_n, sh)),
                        reps=40)
    top = torch.full((1, 3), 1e307, dtype=torch.float64, device=dev)
    top_var = torch.empty(1, dtype=torch.float64, device=dev)
    check(L.sv_variance_f64(top.data_ptr(), 1, 3, 1, 0, top_var.data_ptr(), None, None, 0, sh))
    torch.cuda.synchronize()
    f64 = {"sum_1e8": {"avg_launch_ms": round(sum64_ms, 5), "gb_s": round(8 * SUM_N / (sum64_ms * 1e-3) / 1e9, 1),
                       "hbm_frac": round(8 * SUM_N / (sum64_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "read_ceiling_gbs": round(8 * SUM_N / (read64_ms * 1e-3) / 1e9, 1)},
           "variance_4096x4096": {"avg_launch_ms": round(var64_ms, 5),
                                  "gb_s": round(8 * VAR_ROWS * VAR_COLS / (var64_ms * 1e-3) / 1e9, 1),
                                  "hbm_frac": round(8 * VAR_ROWS * VAR_COLS / (var64_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
           "variance_4096x4096_axis0": {"avg_launch_ms": round(var64c_ms, 5),
                                        "gb_s": round(8 * VAR_ROWS * VAR_COLS / (var64c_ms * 1e-3) / 1e9, 1),
                                        "hbm_frac": round(8 * VAR_ROWS * VAR_COLS / (var64c_ms * 1e-3) / 1e9 /
                                                          HBM_PEAK_GBS, 4)},
           "variance_of_1e307_x3": float(top_var.item()), "bit_exact": None}
    if not args.no_cpu_baseline:
        check(L.sv_tree_sum_f64(c5d[0].data_ptr(), SUM_N, out64.data_ptr(), ws64.data_ptr(), need64, sh))
        check(L.sv_variance_f64(c4d[0].data_ptr(), VAR_ROWS, VAR_COLS, 1, 0, var64.data_ptr(), mean64.data_ptr(), None, 0,
                                sh))
        torch.cuda.synchronize()
        rows = np.random.default_rng(1).choice(VAR_ROWS, 16, replace=False)
        ov64, om64 = oracle.variance_f64(c4_host[rows].astype(np.float64), axis=1)
        ok64 = (np.float64(out64.item()) == oracle.tree_sum_f64(c5_host.astype(np.float64)) and
                np.array_equal(var64.cpu().numpy()[rows].view(np.uint64), ov64.view(np.uint64)) and
                np.array_equal(mean64.cpu().numpy()[rows].view(np.uint64), om64.view(np.uint64)))
        f64["bit_exact"] = bool(ok64)
    del c5d, c4d

    # complex64: pairs of the [4096, 4096] float32 buffers as (re, im), two
    # 134 MB copies, along axis 1 (one pass, parts split in registers) and
    # axis 0 (the interleaved array as float32 [4096, 8192], then the pair add)
    zs = [torch.complex(c4[2 * k], c4[2 * k + 1]).contiguous() for k in range(2)]
    zvar = torch.empty(VAR_COLS, dtype=torch.float32, device=dev)
    zmean = torch.empty(2 * VAR_COLS, dtype=torch.float32, device=dev)
    zws = {ax: max(1, L.sv_variance_c64_workspace_size(VAR_ROWS, VAR_COLS, ax)) for ax in (0, 1)}
    zbuf = {ax: torch.zeros(zws[ax], dtype=torch.uint8, device=dev) for ax in (0, 1)}

    def run_c64(i, ax):
        check(L.sv_variance_c64(zs[i % 2].data_ptr(), VAR_ROWS, VAR_COLS, ax, 0, zvar.data_ptr(), zmean.data_ptr(),
                                zbuf[ax].data_ptr(), zws[ax], sh))

    c64 = {}
    for ax in (1, 0):
        ms = time_op(lambda i: run_c64(i, ax), reps=40)
        gbs = 8 * VAR_ROWS * VAR_COLS / (ms * 1e-3) / 1e9
        torch_ms = time_op(lambda i: torch.var(zs[i % 2], dim=ax, correction=0))
        c64[f"variance_4096x4096_axis{ax}"] = {"avg_launch_ms": round(ms, 5), "gb_s": round(gbs, 1),
                                               "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                                               "torch_var_ms": round(torch_ms, 5)}
    c64["bit_exact_16_rows"] = None
    if parity is not None:
        run_c64(0, 1)
        torch.cuda.synchronize()
        rows = np.random.default_rng(2).choice(VAR_ROWS, 16, replace=False)
        z_host = zs[0][rows].cpu().numpy()
        ovz, omz = oracle.variance_complex(z_host, axis=1)
        got_m = zmean.cpu().numpy().view(np.complex64)[rows]
        c64["bit_exact_16_rows"] = bool(np.array_equal(zvar.cpu().numpy()[rows].view(np.uint32), ovz.view(np.uint32))
                                        and np.array_equal(got_m.view(np.uint64), omz.view(np.uint64)))
    del zs

    elems = VAR_ROWS * VAR_COLS + SUM_N
    value = elems * K / wall / 1e9
    sum_gbs = SUM_BYTES / (sum_avg * 1e-3) / 1e9
    var_gbs = VAR_BYTES / (var_avg * 1e-3) / 1e9
    var_tops = VAR_ROWS * VAR_COLS * VAR_OPS_PER_ELEM / (var_avg * 1e-3) / 1e12
    traffic = read_counter_traffic(SUM_COUNTERS)
    var_traffic = read_counter_traffic(VAR_COUNTERS)
    var_valu = read_summary(VAR_VALU, "valu_instructions_issued_per_element")
    sum_frac, var_frac = sum_gbs / HBM_PEAK_GBS, var_gbs / HBM_PEAK_GBS

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GElem/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "variance [4096,4096] axis 1 ddof 0 N(1e4,1) seed 2 + tree sum of 1e8 "
                               "(99% N(0,1), 1% +/-U(1e6,1e8) cancelling pairs, seed 3)",
                   "variance_shape": [VAR_ROWS, VAR_COLS], "sum_n": SUM_N,
                   "input_copies": {"variance": N_VAR_COPIES, "sum": N_SUM_COPIES}},
        "roofline": {"bound": "hbm", "kernel": "k_tree_sum (1e8 values)", "achieved": round(sum_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(sum_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "avg_launch_ms": round(sum_avg, 5),
                     "algorithmic_bytes_per_launch": SUM_BYTES,
                     "read_ceiling_gbs": round(read_sum_gbs, 1),
                     "frac_of_read_ceiling": round(sum_gbs / read_sum_gbs, 4),
                     # both kernels of the step against the same HBM peak
                     "step_kernels": {"k_tree_sum": round(sum_frac, 4), VAR_KERNEL: round(var_frac, 4)},
                     "min_frac": round(min(sum_frac, var_frac), 4)},
        "variance_kernel": {"kernel": f"{VAR_KERNEL} (4096x4096, axis 1, four waves per row)",
                            "avg_launch_ms": round(var_avg, 5),
                            "gelem_s": round(VAR_ROWS * VAR_COLS / (var_avg * 1e-3) / 1e9, 2),
                            "hbm": {"achieved": round(var_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                    "frac": round(var_gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": VAR_BYTES,
                                    "traffic": var_traffic, "read_ceiling_gbs": round(read_var_gbs, 1),
                                    "frac_of_read_ceiling": round(var_gbs / read_var_gbs, 4)},
                            "alu": {"achieved": round(var_tops, 2), "peak": VALU_PEAK_TOPS, "unit": "Tops/s",
                                    "frac": round(var_tops / VALU_PEAK_TOPS, 4),
                                    "ops_per_element": VAR_OPS_PER_ELEM,
                                    "valu_instructions_issued_per_element": var_valu},
                            "batches": var_batches},
        "sum_kernel": {"avg_launch_ms": round(sum_avg, 5), "gelem_s": round(SUM_N / (sum_avg * 1e-3) / 1e9, 2),
                       "batches": sum_batches},
        "context": {"torch_var_correction0_ms": round(torch_var_ms, 5),
                    "step_on_two_streams": overlap,
                    "variance_axis0_4096x4096": axis0,
                    "kernel_over_torch_var": round(var_avg / torch_var_ms, 3),
                    "torch_sum_ms": round(torch_sum_ms, 5),
                    "torch_sum_gbs": round(SUM_BYTES / (torch_sum_ms * 1e-3) / 1e9, 1),
                    "kernel_over_reference_formula": round(var_avg / variant_ms["reference"], 3),
                    "pages_kernel_over_reference": {"kaggle_cpu": 2.27, "kaggle_gpu": 2.19},
                    "ablation_4096x4096": variants},
        "tree_sum_dw_carry": dw,
        "float64_path": f64,
        "complex64_path": c64,
        "adn_sum": adn,
        "parity": parity,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(c4_host, c5_host)
        out["context"]["cpu_oracle_all_cores"] = cpu_oracle_all_cores(c4_host, c5_host)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
