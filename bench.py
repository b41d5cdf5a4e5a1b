#!/usr/bin/env python3
"""Throughput of dynamic block-scaled quantization on one MI355X.

Headline: dense BF16 -> MXFP8 quantization of an [8192, 7168] activation
matrix (N(0, 1) rows scaled by 2^U(-8, 8), 0.1% outliers x100), block 32, E8M0
scales.  One step = one call of the whole hot path (load, block amax, scale,
quantize, pack, store codes and scales) over that matrix.  Metric: achieved
HBM GB/s counting algorithmic bytes (BF16 read + codes + scales written), as a
fraction of the 8 TB/s HBM3E peak.

Protocol: inputs are resident in HBM before timing starts.  The timed loop
rotates over several copies of the input/output buffers whose combined size is
well above the 256 MB last-level (MALL) cache, so each step streams from HBM
(no warm-cache reuse).  One pair of HIP events, recorded on the stream the
kernels run on, brackets the K back-to-back launches: their elapsed time / K
is the mean launch duration the roofline figure uses; the headline ``value``
uses the host wall clock of the same loop.  The CPU oracle is timed on a bounded
sample of the same workload on the host's cores (``cpu_baseline``), and its
output doubles as a parity check of that sample.

Usage: python bench.py [--gpus 1] [--steps 500] [--warmup 20]
       [--workload dense_mxfp8] [--no-secondary] [--no-cpu-baseline]
       python bench.py --copy-bytes N   (plain copy kernel, for counter calibration)
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20
METRIC = "achieved HBM GB/s (% of 8 TB/s) for BF16→MXFP4/MXFP8/NVFP4 quant, 1 GPU"
KERNEL_SRC = os.path.join(ROOT, "fp8_quantization_amd", "csrc", "bsq_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ workloads

def load_workload(name):
    import workloads as W
    table = {
        "dense_mxfp4": W.dense_mxfp4_small,
        "dense_mxfp8": W.dense_mxfp8_scaled_rows,
        "dense_nvfp4": W.dense_nvfp4_scaled_rows,
        "grouped_nvfp4": W.grouped_nvfp4_prefill,
        # the same routing quantized to the MX formats (large grouped MX path)
        "grouped_mxfp8": lambda: W.grouped_mx_prefill(W.MXFP8),
        "grouped_mxfp4": lambda: W.grouped_mx_prefill(W.MXFP4),
        "grouped_mxfp4_decode": lambda: W.grouped_mx_decode(W.MXFP4),
        "grouped_mxfp8_decode": lambda: W.grouped_mx_decode(W.MXFP8),
        # dequantization of codes and scales of the dense MXFP8 / NVFP4 sizes
        "dequant_mxfp8": lambda: W.dequant_random_bytes(W.MXFP8, 8192, 7168, seed=1102),
        "dequant_nvfp4": lambda: W.dequant_random_bytes(W.NVFP4, 16384, 7168, seed=1103,
                                                        tensor_sf=0.0123),
        # the matrix-core consumer of the MFMA scale layout
        "mfma_gemm_mxfp8": lambda: W.gemm_random_operands(W.MXFP8, 4096, 4096, 7168, seed=1202),
        "mfma_gemm_mxfp4": lambda: W.gemm_random_operands(W.MXFP4, 4096, 4096, 7168, seed=1201),
        # a dense layer at decode: 16 rows against 16384 x 7168 weights
        "mfma_gemm_mxfp4_m16": lambda: W.gemm_random_operands(W.MXFP4, 16, 16384, 7168,
                                                              seed=1205),
        "mfma_grouped_gemm_mxfp4": lambda: W.grouped_gemm_prefill(W.MXFP4),
        "mfma_grouped_gemm_mxfp4_decode": lambda: W.grouped_gemm_decode(W.MXFP4),
    }
    return table[name]()


def bytes_per_element(fmt):
    """BF16 read (2) + code bytes (1/2 or 1) + one scale byte per block."""
    bs = 16 if fmt == 2 else 32
    return 2.0 + (1.0 if fmt == 1 else 0.5) + 1.0 / bs


# NVFP4 tensor-scale producer steps, measured on the named quantizer input
PRODUCERS = {"tsf_dense_nvfp4": "dense_nvfp4", "tsf_grouped_nvfp4": "grouped_nvfp4"}


def producer_bytes(case):
    """Bytes one producer step must move: the BF16 rows it reduces (each
    distinct source row once), the grouping metadata and the fp32 results."""
    import workloads as W
    K = case.x.shape[1]
    if isinstance(case, W.DenseCase):
        M = case.x.shape[0]
        return M * K * 2 + 4, M * K
    lo, hi = int(case.row_offsets[0]), int(case.row_offsets[-1])
    src = (hi - lo) if case.row_indices is None else np.unique(case.row_indices[lo:hi]).size
    meta = (case.row_offsets.size + case.expert_ids.size) * 4 + case.tensor_sf.size * 4
    if case.row_indices is not None:
        meta += (hi - lo) * 4
    return int(src * K * 2 + meta), (hi - lo) * K


# dense matrix-core peaks of MI355X (TFLOP/s) for the GEMM's operand format
PEAK_MFMA_TFLOPS = {0: 10100.0, 1: 5000.0}


def gemm_flops(case):
    import workloads as W
    if isinstance(case, W.GroupedGemmCase):
        routed = int(case.row_offsets[-1]) - int(case.row_offsets[0])
        return 2 * routed * (case.b_codes.shape[0] // case.num_experts) * case.K
    return 2 * case.a_codes.shape[0] * case.b_codes.shape[0] * case.K


def dequant_bytes(case):
    """Codes and scales read, fp32 values written."""
    M = case.codes.shape[0]
    return int(case.codes.nbytes + case.scales.nbytes + 4 * M * case.K), M * case.K


def algorithmic_bytes(case):
    """Bytes one launch must move at minimum (read + written)."""
    import workloads as W
    if isinstance(case, W.DequantCase):
        return dequant_bytes(case)
    if isinstance(case, W.GroupedGemmCase):
        # routed A, its scale records and the metadata read once; the weights
        # and scale records of each expert that owns rows read once (an
        # expert with no rows is never read); c written
        N = case.b_codes.shape[0] // case.num_experts
        E = case.num_experts
        meta = 4 * (case.row_offsets.size + case.scales_offsets.size + case.expert_ids.size)
        counts = np.diff(case.row_offsets.astype(np.int64))
        used = np.unique(case.expert_ids[counts > 0]).size
        return int(case.a_codes.nbytes + case.a_scales.nbytes +
                   used * (case.b_codes.nbytes + case.b_scales.nbytes) // E +
                   meta + 4 * case.max_rows * N), case.max_rows * N
    if isinstance(case, W.GemmCase):    # operands read once + c written
        M, N = case.a_codes.shape[0], case.b_codes.shape[0]
        return int(case.a_codes.nbytes + case.a_scales.nbytes + case.b_codes.nbytes +
                   case.b_scales.nbytes + 4 * M * N), M * N
    if isinstance(case, W.DenseCase):
        M, K = case.x.shape
        return int(M * K * bytes_per_element(case.fmt)), M * K
    K = case.x.shape[1]
    routed = int(case.row_offsets[-1]) - int(case.row_offsets[0])
    fmt = case.fmt
    out = routed * K * (bytes_per_element(fmt) - 2.0)
    if case.row_indices is None:
        src_read = routed * K * 2
    else:  # each distinct source row must be read once
        used = np.unique(case.row_indices[int(case.row_offsets[0]):int(case.row_offsets[-1])])
        src_read = used.size * K * 2
    meta = (case.row_offsets.size + case.scales_offsets.size + case.expert_ids.size) * 4
    if case.tensor_sf is not None:
        meta += case.tensor_sf.size * 4
    if case.row_indices is not None:
        meta += routed * 4
    return int(src_read + out + meta), routed * K


class Runner:
    """Holds NB resident copies of one workload's buffers and launches one
    step on copy i: the quantizer; with ``producer`` the NVFP4 tensor-scale
    producer on the same input; for a DequantCase the dequantization."""

    def __init__(self, case, nb, producer=False):
        import torch

        import fp8_quantization_amd as bsq
        import workloads as W
        self.bsq, self.torch, self.case = bsq, torch, case
        self.dequant = isinstance(case, W.DequantCase)
        self.gemm = isinstance(case, (W.GemmCase, W.GroupedGemmCase))
        self.grouped_gemm = isinstance(case, W.GroupedGemmCase)
        self.grouped = isinstance(case, W.GroupedCase)
        self.producer = producer
        self.sets = []
        if self.gemm:
            t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
            n_out = case.b_codes.shape[0] // (case.num_experts if self.grouped_gemm else 1)
            s = {"aq": t(case.a_codes), "as": t(case.a_scales), "bq": t(case.b_codes),
                 "bs": t(case.b_scales),
                 "c": torch.empty((case.a_codes.shape[0], n_out), dtype=torch.float32,
                                  device="cuda")}
            if self.grouped_gemm:
                s["ro"] = t(case.row_offsets.view(np.int32))
                s["so"] = t(case.scales_offsets.view(np.int32))
                s["ids"] = t(case.expert_ids)
            self.sets.append(s)
            torch.cuda.synchronize()
            return
        if self.dequant:
            codes, scales = torch.from_numpy(case.codes).cuda(), torch.from_numpy(case.scales).cuda()
            for i in range(nb):
                self.sets.append({"q": codes if i == 0 else codes.clone(),
                                  "s": scales if i == 0 else scales.clone(),
                                  "out": torch.empty((case.codes.shape[0], case.K),
                                                     dtype=torch.float32, device="cuda")})
            torch.cuda.synchronize()
            return
        xd = torch.from_numpy(np.ascontiguousarray(case.x).view(np.int16)).cuda()
        K = case.x.shape[1]
        bs = bsq.BLOCK_SIZE[case.fmt]
        for i in range(nb):
            s = {"x": xd if i == 0 else xd.clone()}
            if self.grouped:
                t = lambda a, dt: None if a is None else torch.from_numpy(
                    np.ascontiguousarray(a).view(dt)).cuda()
                s["ro"] = t(case.row_offsets, np.int32)
                s["so"] = t(case.scales_offsets, np.int32)
                s["ids"] = t(case.expert_ids, np.int32)
                s["sf"] = t(case.tensor_sf, np.float32)
                s["ri"] = t(case.row_indices, np.int32)
                if producer:
                    s["tsf"] = torch.empty(case.tensor_sf.size, dtype=torch.float32,
                                           device="cuda")
                    self.sets.append(s)
                    continue
                s["q"] = torch.empty((case.max_rows, bsq.code_width(case.fmt, K)),
                                     dtype=torch.uint8, device="cuda")
                s["s"] = torch.empty((case.num_scale_rows, K // bs), dtype=torch.uint8,
                                     device="cuda")
            elif producer:
                s["tsf"] = torch.empty(1, dtype=torch.float32, device="cuda")
            else:
                M = case.x.shape[0]
                s["q"] = torch.empty((M, bsq.code_width(case.fmt, K)), dtype=torch.uint8,
                                     device="cuda")
                s["s"] = torch.empty((M, K // bs), dtype=torch.uint8, device="cuda")
            self.sets.append(s)
        torch.cuda.synchronize()

    def step(self, i):
        s = self.sets[i % len(self.sets)]
        c = self.case
        if self.grouped_gemm:
            self.bsq.grouped_block_scaled_matmul_mfma(
                s["aq"], s["as"], s["ro"], s["so"], s["ids"], c.max_rows, c.num_scale_rows,
                s["bq"], s["bs"], c.num_experts, c.fmt, c.K, out=s["c"])
        elif self.gemm:
            self.bsq.block_scaled_matmul_mfma(s["aq"], s["as"], s["bq"], s["bs"], c.fmt, c.K,
                                              out=s["c"])
        elif self.dequant:
            self.bsq.dequantize_block_scaled(s["q"], s["s"], c.fmt, c.K, c.tensor_sf, out=s["out"])
        elif self.producer and self.grouped:
            self.bsq.grouped_tensor_scale_nvfp4(s["x"], s["ro"], s["ids"], c.tensor_sf.size,
                                                c.max_rows, row_indices=s["ri"], out=s["tsf"])
        elif self.producer:
            self.bsq.tensor_scale_nvfp4(s["x"], out=s["tsf"])
        elif self.grouped:
            self.bsq.grouped_quantize_block_scaled(
                s["x"], c.fmt, s["ro"], s["so"], s["ids"], s["sf"], c.max_rows,
                c.num_scale_rows, row_indices=s["ri"], codes=s["q"], scales=s["s"])
        else:
            self.bsq.quantize_block_scaled(s["x"], c.fmt, c.tensor_sf, codes=s["q"],
                                           scales=s["s"])


def time_steps(runner, steps, warmup):
    """Wall time of `steps` back-to-back launches, and the mean launch
    duration from one pair of HIP events recorded on the launch stream around
    the whole timed loop."""
    torch = runner.torch
    for i in range(warmup):
        runner.step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        runner.step(warmup + i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) / steps


def launch_percentiles(runner, n, offset):
    """Per-launch durations (µs) of n further launches, each bracketed by its
    own HIP event pair on the launch stream, still rotating over the buffer
    sets: median, p10 and p90."""
    torch = runner.torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record()
        runner.step(offset + i)
        b.record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return {"median": round(float(np.median(us)), 3), "p10": round(float(np.percentile(us, 10)), 3),
            "p90": round(float(np.percentile(us, 90)), 3), "n": n}


def graph_launch_us(runner, n_launch=64, replays=20):
    """Mean duration per launch (µs) when n_launch launches, rotating over the
    buffer sets, are replayed from one captured HIP graph: no host launch cost
    sits between the kernels, so for a small problem this is the kernel's own
    time plus the dispatch gap, where the eager loop measures the host."""
    torch = runner.torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_launch):
            runner.step(i)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return round(a.elapsed_time(b) / (n_launch * replays) * 1e3, 3)


# below this many bytes per launch the host's launch cost exceeds the kernel's
# time, and the graph replay figure is the one that describes the kernel
LATENCY_BOUND_BYTES = 16 << 20


def measure(name, steps, warmup, rotate=True):
    import workloads as W
    producer = name in PRODUCERS
    case = load_workload(PRODUCERS.get(name, name))
    nbytes, elems = producer_bytes(case) if producer else algorithmic_bytes(case)
    rotate = rotate and not isinstance(case, (W.GemmCase, W.GroupedGemmCase))  # reuse is the point
    nb = max(2, -(-3 * MALL_BYTES // max(nbytes, 1)) + 1) if rotate else 1
    nb = min(nb, 64)
    runner = Runner(case, nb, producer)
    wall, kern = time_steps(runner, steps, warmup)
    runner.percentiles = launch_percentiles(runner, steps, warmup + steps)
    runner.graph_us = graph_launch_us(runner) if nbytes < LATENCY_BOUND_BYTES else None
    return case, runner, nbytes, elems, nb, wall, kern


def summary(name, nbytes, elems, wall, launch_ms, steps, nb, percentiles=None, graph_us=None):
    k = launch_ms * 1e-3
    out = {
        "workload": name,
        "bytes_per_launch": nbytes,
        "elements": elems,
        "buffer_sets": nb,
        "launch_us_mean": round(k * 1e6, 3),
        "launch_us_each": percentiles,
        "GBps": round(nbytes / k / 1e9, 1),
        "frac_of_8TBps": round(nbytes / k / 1e9 / PEAK_HBM_GBS, 4),
        "Gelem_per_s": round(elems / k / 1e9, 1),
        "wall_GBps": round(nbytes * steps / wall / 1e9, 1),
    }
    if graph_us is not None:  # latency-bound: the kernel's time without the host's launch cost
        out.update({"graph_us_mean": graph_us, "graph_GBps": round(nbytes / graph_us / 1e3, 1),
                    "graph_Gelem_per_s": round(elems / graph_us / 1e3, 1)})
    return out


# ------------------------------------------------------------------ CPU baseline

def cpu_baseline(case, runner, target_cpu_seconds=12.0, max_wall_seconds=20.0):
    """Time the oracle (as it stands) on the same input on the host's cores:
    whole passes over the leading rows (all of them when the input is small)
    until about target_cpu_seconds of CPU work (wall x threads) are done;
    check the GPU's output for those rows."""
    import oracle
    torch = runner.torch
    threads = max(1, min(16, os.cpu_count() or 1))
    M, K = case.x.shape
    probe = min(M, 64)
    t = time.perf_counter()
    oracle.quantize(case.x[:probe], case.fmt, case.tensor_sf, nthreads=threads)
    per_row = (time.perf_counter() - t) / probe           # wall seconds per row
    want_rows = target_cpu_seconds / threads / max(per_row, 1e-9)
    rows = int(min(M, max(probe, want_rows)))
    # whole passes over those rows until the CPU work (wall x threads) reaches the target
    reps, dt = 0, 0.0
    while reps == 0 or (dt * threads < target_cpu_seconds and dt < max_wall_seconds):
        t = time.perf_counter()
        qh, sh = oracle.quantize(case.x[:rows], case.fmt, case.tensor_sf, nthreads=threads)
        dt += time.perf_counter() - t
        reps += 1
    nbytes = reps * rows * K * bytes_per_element(case.fmt)
    runner.step(0)
    torch.cuda.synchronize()
    s0 = runner.sets[0]
    ok = bool(np.array_equal(s0["q"][:rows].cpu().numpy(), qh) and
              np.array_equal(s0["s"][:rows].cpu().numpy(), sh))
    # the same oracle on one thread, over a smaller leading sample (a few seconds at most)
    rows1 = int(min(M, max(1, 3.0 / max(per_row * threads, 1e-9))))
    t = time.perf_counter()
    oracle.quantize(case.x[:rows1], case.fmt, case.tensor_sf, nthreads=1)
    dt1 = time.perf_counter() - t
    return {
        "value": round(nbytes / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "one_thread": {"value": round(rows1 * K * bytes_per_element(case.fmt) / dt1 / 1e9, 3),
                       "sample": f"first {rows1} rows, {dt1:.2f} s wall on 1 thread"},
        "sample": f"first {rows} of {M} rows of the {case.name} input, {reps} pass(es) "
                  f"({reps * rows * K} elements, {nbytes / 1e6:.1f} MB algorithmic), "
                  f"{dt:.2f} s wall on {threads} thread(s)",
        "parity_of_sample": "identical" if ok else "MISMATCH",
    }


def traffic_from_counters(nbytes_per_launch):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    counters, valid only while the kernel source is the one they were taken
    on (sha256 recorded beside them)."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None, "no counter file"
    sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != sha:
        return None, "kernel changed since the counters were taken"
    return int(rec["hbm_bytes_per_launch"]), rec.get("note", "")


# ------------------------------------------------------------------ main

def vendor_cast_context(runner, steps, warmup):
    """Context for the headline: torch's own elementwise cast of the same BF16
    buffers to float8_e4m3fn (2 bytes read and 1 written per element, the
    MXFP8 byte mix without the scales), rotated and timed like the quantizer.
    A vendor streaming kernel of this mix shows what such a stream reaches on
    this chip; it computes no block scales."""
    torch = runner.torch
    if not hasattr(torch, "float8_e4m3fn"):
        return None
    xs = [st["x"].view(torch.bfloat16) for st in runner.sets]
    outs = [torch.empty(x.shape, dtype=torch.float8_e4m3fn, device="cuda") for x in xs]
    for i in range(warmup):
        outs[i % len(xs)].copy_(xs[i % len(xs)])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        outs[i % len(xs)].copy_(xs[i % len(xs)])
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / steps * 1e3
    nbytes = xs[0].numel() * 3
    return {"kernel": "torch bf16 -> float8_e4m3fn cast (same inputs, same rotation)",
            "bytes_per_launch": nbytes, "launch_us_mean": round(us, 3),
            "GBps": round(nbytes / us / 1e3, 1)}


def copy_calibration(nbytes, steps):
    import torch
    n = nbytes // 4
    a = torch.empty(n, dtype=torch.int32, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "steps": steps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dense_mxfp8")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0)
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (each GPU would "
              "quantize its own shard with no exchange); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_bytes:
        copy_calibration(args.copy_bytes, args.steps)
        return

    import fp8_quantization_amd as bsq

    case, runner, nbytes, elems, nb, wall, kern = measure(args.workload, args.steps, args.warmup)
    head = summary(args.workload, nbytes, elems, wall, kern, args.steps, nb, runner.percentiles,
                   runner.graph_us)
    log("[bench] headline", json.dumps(head))
    achieved = nbytes / (kern * 1e-3) / 1e9
    quantizer = args.workload not in PRODUCERS and not args.workload.startswith(
        ("dequant_", "mfma_gemm", "mfma_grouped_gemm"))
    if not quantizer:
        traffic, traffic_note = None, "counters are taken on the quantizer only"
    else:
        traffic, traffic_note = traffic_from_counters(nbytes)

    context = None
    if args.workload == "dense_mxfp8":
        context = vendor_cast_context(runner, args.steps, args.warmup)
        log("[bench] context", json.dumps(context))

    secondary = []
    if not args.no_secondary:
        for name in ("dense_nvfp4", "grouped_nvfp4", "dense_mxfp4", "grouped_mxfp4_decode",
                     "grouped_mxfp8_decode", "grouped_mxfp8", "grouped_mxfp4",
                     "tsf_dense_nvfp4", "tsf_grouped_nvfp4", "dequant_mxfp8", "dequant_nvfp4",
                     "mfma_gemm_mxfp8", "mfma_gemm_mxfp4", "mfma_gemm_mxfp4_m16",
                     "mfma_grouped_gemm_mxfp4", "mfma_grouped_gemm_mxfp4_decode"):
            if name == args.workload:
                continue
            c2, r2, nb2, el2, nbs2, w2, k2 = measure(name, args.steps, args.warmup)
            s = summary(name, nb2, el2, w2, k2, args.steps, nbs2, r2.percentiles, r2.graph_us)
            if name.startswith(("mfma_gemm", "mfma_grouped_gemm")):
                tf = gemm_flops(c2) / (k2 * 1e-3) / 1e12
                peak = PEAK_MFMA_TFLOPS[c2.fmt]
                # the bound is whichever ideal time is longer: flops at the peak or bytes at 8 TB/s
                hbm_bound = nb2 / PEAK_HBM_GBS / 1e9 > gemm_flops(c2) / peak / 1e12
                s.update({"bound": "hbm" if hbm_bound else "mfma", "TFLOPs": round(tf, 1),
                          "peak_TFLOPs": peak, "frac_of_peak": round(tf / peak, 4)})
            log("[bench] secondary", json.dumps(s))
            secondary.append(s)
            del r2, c2
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline and quantizer:
        cpu = cpu_baseline(case, runner)
        log("[bench] cpu_baseline", json.dumps(cpu))

    fmt_name = {0: "MXFP4", 1: "MXFP8", 2: "NVFP4"}[case.fmt]
    if hasattr(case, "a_codes"):
        rows, K = case.a_codes.shape[0], case.K
    elif hasattr(case, "codes"):
        rows, K = case.codes.shape[0], case.K
    else:
        rows, K = case.x.shape
    line = {
        "metric": METRIC,
        "value": round(nbytes * args.steps / wall / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": case.name, "format": fmt_name, "rows": int(rows),
                   "K": int(K), "block": bsq.BLOCK_SIZE[case.fmt],
                   "bytes_per_step": nbytes, "buffer_sets_rotated": nb,
                   "version": bsq.version()},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "traffic_note": traffic_note,
                     "launch_us_mean": head["launch_us_mean"],
                     "launch_us_each": head["launch_us_each"]},
        "cpu_baseline": cpu,
        "stream_context": context,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
