#!/usr/bin/env python3
"""Throughput of dynamic block-scaled quantization on one MI355X.

Headline: grouped per-expert BF16 -> NVFP4 quantization of the MoE prefill
routing -- 16384 routed rows x 7168 of N(0, 1) activations over 128 experts
(Dirichlet(0.3) counts, empty experts kept), uint32 row and scale offsets
(scale rows padded to 128 per expert), int32 expert ids and fp32 per-expert
tensor scales.  One step = one call of the whole hot path over that input:
load, group search, block amax, scale, quantize, pack, store codes and
scales.  Metric: achieved HBM GB/s counting algorithmic bytes (BF16 read +
codes + scales written + routing metadata), as a fraction of the 8 TB/s HBM3E
peak.  The other workloads (dense MXFP4 [128, 4096], dense MXFP8 [8192, 7168],
dense NVFP4 [16384, 7168], the MXFP4 / MXFP8 decode gather) are measured in
the same run, each with its own figures.

Protocol.  Inputs are resident in HBM before timing starts.  Each workload's
loop rotates over several copies of its buffers whose combined size is well
above the 256 MB last-level (MALL) cache, so every step streams from HBM.
The timed region is K back-to-back launches between two device
synchronisations; the headline ``value`` is its host wall clock.  The same K
launches then run again, each with a pair of HIP events bound to its kernel's
dispatch (``bsq_time_next_launch``, hipExtLaunchKernel on the launch stream;
kept out of the timed region because binding adds a few µs between
launches): their elapsed time is the kernel's own execution, the figure
rocprofv3's kernel trace reports, and the roofline fraction is computed from
it (mean, and median beside it).  For the large dense and grouped quantizer
workloads and the two dequantizations the same job also times the
same-byte-mix trivial stream of ``libbsq_ceiling.so`` on the same buffers
(``ceiling``).  The CPU oracle is timed on a bounded sample
of every quantizer workload on the host's cores, on one thread and on all of
them, and its output is compared with the GPU's for that sample.

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 10]
       [--workload grouped_nvfp4] [--no-secondary] [--no-cpu-baseline] [--no-ceiling]
       python bench.py --copy-bytes N          (plain copy, for counter calibration)
       python bench.py --pmc-summary DIR       (counters of rocprofv3 --pmc runs -> traffic)
       python bench.py --pmc-gemm-summary DIR  (matrix-core counters of the GEMM workloads)
       python bench.py --trace-summary DIR [--bench-line FILE]
                                               (a rocprofv3 kernel trace of this script)
"""
import argparse
import glob
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
CSRC = os.path.join(ROOT, "fp8_quantization_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
HEADLINE = "grouped_nvfp4"
# the host's CPU share for one GPU on the measurement box
CPU_THREADS = max(1, min(16, os.cpu_count() or 1))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ workloads

# quantizer workloads: name -> (builder, chunks per wave of the dense byte-mix
# stream that prices it, or None)
def quantizer_table():
    import workloads as W
    return {
        "grouped_nvfp4": (W.grouped_nvfp4_prefill, 4),
        "dense_mxfp4": (W.dense_mxfp4_small, None),
        "dense_mxfp8": (W.dense_mxfp8_scaled_rows, 2),
        "dense_nvfp4": (W.dense_nvfp4_scaled_rows, 4),
        "grouped_mxfp4_decode": (lambda: W.grouped_mx_decode(W.MXFP4), None),
        "grouped_mxfp8_decode": (lambda: W.grouped_mx_decode(W.MXFP8), None),
        # the prefill routing quantized to the MX formats
        "grouped_mxfp8": (lambda: W.grouped_mx_prefill(W.MXFP8), 2),
        "grouped_mxfp4": (lambda: W.grouped_mx_prefill(W.MXFP4), 4),
    }


def consumer_table():
    import workloads as W
    return {
        # the NVFP4 tensor-scale producer on the dense and grouped 16384 x 7168 inputs
        "tsf_dense_nvfp4": W.dense_nvfp4_scaled_rows,
        "tsf_grouped_nvfp4": W.grouped_nvfp4_prefill,
        # dequantization of random codes and scales of the dense MXFP8 / NVFP4 sizes
        "dequant_mxfp8": lambda: W.dequant_random_bytes(W.MXFP8, 8192, 7168, seed=1102),
        "dequant_nvfp4": lambda: W.dequant_random_bytes(W.NVFP4, 16384, 7168, seed=1103,
                                                        tensor_sf=0.0123),
        # the matrix-core consumers of the MFMA scale layout
        "mfma_gemm_mxfp8": lambda: W.gemm_random_operands(W.MXFP8, 4096, 4096, 7168, seed=1202),
        "mfma_gemm_mxfp4": lambda: W.gemm_random_operands(W.MXFP4, 4096, 4096, 7168, seed=1201),
        "mfma_grouped_gemm_mxfp4": lambda: W.grouped_gemm_prefill(W.MXFP4),
        "mfma_grouped_gemm_mxfp4_decode": lambda: W.grouped_gemm_decode(W.MXFP4),
    }


def load_workload(name):
    q = quantizer_table()
    if name in q:
        return q[name][0]()
    return consumer_table()[name]()


def bytes_per_element(fmt):
    """BF16 read (2) + code bytes (1/2 or 1) + one scale byte per block."""
    bs = 16 if fmt == 2 else 32
    return 2.0 + (1.0 if fmt == 1 else 0.5) + 1.0 / bs


def producer_bytes(case):
    """Bytes one tensor-scale step must move: the BF16 rows it reduces (each
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
    producer on the same input; for a DequantCase the dequantization; for a
    GEMM case the matrix-core GEMM."""

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


# ------------------------------------------------------------------ timing

def recorded_events(torch, n):
    """n pairs of timing events, each recorded once so that it exists."""
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n)]
    for a, b in pairs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    return pairs


def spread(us):
    us = np.asarray(us, np.float64)
    return {"mean": round(float(us.mean()), 3), "median": round(float(np.median(us)), 3),
            "p10": round(float(np.percentile(us, 10)), 3),
            "p90": round(float(np.percentile(us, 90)), 3), "n": int(us.size)}


def timed_region(torch, arm, launch, steps, warmup):
    """Warm up, then two passes of `steps` launches.

    The timed region: the launches between two device synchronisations, with
    one event pair around them -- its wall time and the events' span per
    launch (kernel time plus the gap between launches).

    Then the same launches with a recorded event pair bound to each kernel's
    dispatch (arm(start_i, stop_i) before launch i): every kernel's own time
    in µs.  Binding events to a dispatch adds a few µs between launches on
    this runtime, so this pass is kept out of the timed region."""
    for i in range(warmup):
        launch(i)
    outer = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    outer[0].record()
    for i in range(steps):
        launch(warmup + i)
    outer[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    span = outer[0].elapsed_time(outer[1]) * 1e3 / steps
    pairs = recorded_events(torch, steps)
    for i in range(steps):
        arm(*pairs[i])
        launch(warmup + steps + i)
    torch.cuda.synchronize()
    kernel_us = [a.elapsed_time(b) * 1e3 for a, b in pairs]
    return wall, span, kernel_us


COLD_FLUSH_BYTES = 1 << 30


def cold_launches(runner, nbytes, flush_kind, launches=50, warmup=5):
    """The cold-cache protocol: before each launch a kernel on the same stream
    streams a 1 GiB buffer (more than the 256 MB MALL and the L2 together),
    then the launch runs with an event pair bound to its dispatch; `warmup`
    such pairs untimed, then `launches` timed.  flush_kind "read" reads the
    buffer (a reduction): every line the launch uses is evicted and the caches
    hold clean lines.  "write" fills it (a memset): the caches then hold up to
    the MALL's size in dirty lines, whose write-back to HBM falls inside the
    next launch.  Returns the kernel times' spread and the bandwidth of their
    median."""
    torch = runner.torch
    flush = torch.ones(COLD_FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty((), dtype=torch.int64, device="cuda")
    pairs = recorded_events(torch, launches)
    for i in range(warmup + launches):
        if flush_kind == "read":
            torch.sum(flush, dim=0, out=sink)
        else:
            flush.fill_(i)
        if i >= warmup:
            runner.bsq.time_next_launch(*pairs[i - warmup])
        runner.step(i)
    torch.cuda.synchronize()
    k = spread([a.elapsed_time(b) * 1e3 for a, b in pairs])
    del flush
    return {"kernel_us": k, "GBps_median": round(nbytes / k["median"] / 1e3, 1),
            "frac_median": round(nbytes / k["median"] / 1e3 / PEAK_HBM_GBS, 4),
            "flush": f"1 GiB {'read (a reduction)' if flush_kind == 'read' else 'fill (memset)'}"
                     " on the launch stream before each launch",
            "launches": launches, "warmup": warmup}


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


def rotation(nbytes):
    """Buffer sets to rotate over: together more than three times the MALL."""
    return min(64, max(2, -(-3 * MALL_BYTES // max(nbytes, 1)) + 1))


def measure(name, steps, warmup, ceiling_u=None):
    """One workload: its runner, algorithmic bytes and elements per launch,
    its timing summary, and (with ceiling_u) the same-byte-mix stream timed on
    its buffers just before it."""
    import workloads as W
    producer = name.startswith("tsf_")
    case = load_workload(name)
    nbytes, elems = producer_bytes(case) if producer else algorithmic_bytes(case)
    reuse = isinstance(case, (W.GemmCase, W.GroupedGemmCase))   # one set: reuse is the point
    nb = 1 if reuse else rotation(nbytes)
    runner = Runner(case, nb, producer)
    ceil = ceiling(runner, ceiling_u, steps, warmup) if ceiling_u else None
    wall, region_us, kernel_us = timed_region(runner.torch, runner.bsq.time_next_launch,
                                              runner.step, steps, warmup)
    s = summary(name, nbytes, elems, nb, wall, region_us, kernel_us, steps)
    if nbytes < LATENCY_BOUND_BYTES:
        g = graph_launch_us(runner)
        s.update({"graph_us_mean": g, "graph_GBps": round(nbytes / g / 1e3, 1),
                  "graph_Gelem_per_s": round(elems / g / 1e3, 1)})
    return case, runner, nbytes, s, ceil


def summary(name, nbytes, elems, nb, wall, region_us, kernel_us, steps):
    k = spread(kernel_us)
    return {
        "workload": name,
        "bytes_per_launch": nbytes,
        "elements": elems,
        "buffer_sets": nb,
        "kernel_us": k,
        "timed_region_us_per_launch": round(region_us, 3),
        "GBps": round(nbytes / k["mean"] / 1e3, 1),
        "frac_of_8TBps": round(nbytes / k["mean"] / 1e3 / PEAK_HBM_GBS, 4),
        "GBps_median": round(nbytes / k["median"] / 1e3, 1),
        "Gelem_per_s": round(elems / k["mean"] / 1e3, 1),
        "wall_GBps": round(nbytes * steps / wall / 1e9, 1),
        "wall_s": round(wall, 6),
    }


def ceiling(runner, u, steps, warmup):
    """The same-byte-mix trivial stream on the workload's own buffers (its
    BF16 input and, as dense [M, K] outputs, the first rows of its code and
    scale buffers), timed like the quantizer, at the quantizer's own tile of u
    chunks per wave and at the other tile sizes; the fastest is the
    ceiling.  It runs right before the quantizer's own timing."""
    bsq, torch, case = runner.bsq, runner.torch, runner.case
    fmt = case.fmt
    if runner.dequant:                   # the dequantizer's mix: codes and scales in, fp32 out
        M, K = case.codes.shape[0], case.K
        nbytes = algorithmic_bytes(case)[0]
        kernel = "bsq::expand_kernel"
        what = "dequantizer"

        def run(st, uu, a, b):
            bsq.ceiling_expand(st["q"], st["s"], fmt, K, uu, out=st["out"], start=a, stop=b)
    else:
        M, K = case.x.shape
        nbytes = int(M * K * bytes_per_element(fmt))
        kernel = "bsq::ceiling_kernel"
        what = "quantizer"

        def run(st, uu, a, b):
            bsq.ceiling_stream(st["x"], fmt, uu, codes=st["q"][:M], scales=st["s"][:M],
                               start=a, stop=b)
    # at least 300 launches per tile size: together about 50 ms of streaming,
    # which also brings the GPU to its steady clocks before the kernel
    steps = max(steps, 300)
    by_u = {}
    for uu in (1, 2, 4):
        armed = {}

        def arm(a, b):
            armed["ev"] = (a, b)

        def launch(i):
            a, b = armed.pop("ev", (None, None))
            run(runner.sets[i % len(runner.sets)], uu, a, b)

        _, _, kernel_us = timed_region(torch, arm, launch, steps, warmup)
        by_u[uu] = spread(kernel_us)
    best = min(by_u, key=lambda k: by_u[k]["mean"])
    k = by_u[best]
    return {"kernel": f"{kernel}, {M}x{K}, {['MXFP4', 'MXFP8', 'NVFP4'][fmt]} {what} "
                      f"byte mix, best of 1 / 2 / 4 chunks per wave",
            "bytes_per_launch": nbytes, "chunks_per_wave": best, "kernel_us": k,
            "GBps": round(nbytes / k["mean"] / 1e3, 1),
            "frac_of_8TBps": round(nbytes / k["mean"] / 1e3 / PEAK_HBM_GBS, 4),
            "kernel_us_mean_by_chunks_per_wave": {str(a): b["mean"] for a, b in by_u.items()},
            f"{what}_chunks_per_wave": u}


def roofline(s, traffic, traffic_note, ceil=None):
    k = s["kernel_us"]
    r = {"bound": "hbm", "achieved": s["GBps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
         "frac": s["frac_of_8TBps"],
         "frac_median": round(s["GBps_median"] / PEAK_HBM_GBS, 4),
         "kernel_us_mean": k["mean"], "kernel_us_median": k["median"],
         # back to back, one event pair around the timed region: kernels plus the gaps
         "frac_timed_region": round(s["bytes_per_launch"] / s["timed_region_us_per_launch"] / 1e3
                                    / PEAK_HBM_GBS, 4),
         "bytes_per_launch": s["bytes_per_launch"],
         "timing": "per-launch HIP events bound to the kernel dispatch (hipExtLaunchKernel) "
                   "over the timed region",
         "traffic": traffic, "traffic_note": traffic_note,
         # the counters' HBM bytes over the same kernel time, beside the algorithmic rate
         "traffic_GBps": round(traffic / k["mean"] / 1e3, 1) if traffic else None}
    if ceil is not None:
        r["ceiling"] = ceil
        # the kernel's speed as a fraction of the trivial stream's (above 1: faster than it)
        r["of_ceiling"] = round(ceil["kernel_us"]["mean"] / k["mean"], 4)
    return r


# ------------------------------------------------------------------ CPU baseline

def _oracle_sample(case, rows, threads):
    """The oracle on a leading sample of the workload: the first `rows`
    routed rows (groups cut at that row).  Returns the codes and scale rows it
    wrote, the index arrays of those rows, and their algorithmic bytes."""
    import oracle
    import workloads as W
    if isinstance(case, W.DenseCase):
        q, s = oracle.quantize(case.x[:rows], case.fmt, case.tensor_sf, nthreads=threads)
        K = case.x.shape[1]
        return q, s, np.arange(rows), np.arange(rows), rows * K * bytes_per_element(case.fmt)
    ro = np.minimum(case.row_offsets.astype(np.int64), rows).astype(np.uint32)
    q, s = oracle.grouped_quantize(case.x, case.fmt, ro, case.scales_offsets, case.expert_ids,
                                   case.tensor_sf, case.max_rows, case.num_scale_rows,
                                   row_indices=case.row_indices, nthreads=threads)
    code_rows = np.arange(int(ro[0]), int(ro[-1]))
    scale_rows = np.concatenate([np.arange(int(so), int(so) + int(hi - lo)) for lo, hi, so in
                                 zip(ro[:-1], ro[1:], case.scales_offsets[:-1])]
                                + [np.zeros(0, np.int64)])
    K = case.x.shape[1]
    if case.row_indices is None:
        reads = code_rows.size
    else:
        reads = np.unique(case.row_indices[code_rows]).size
    nbytes = reads * K * 2 + code_rows.size * K * (bytes_per_element(case.fmt) - 2.0)
    return q[code_rows], s[scale_rows], code_rows, scale_rows, nbytes


def cpu_baseline(case, runner, cpu_seconds):
    """Time the oracle (as it stands) on the workload's own input on the
    host's cores: all threads over a leading sample sized for about
    `cpu_seconds` of CPU work (wall x threads), in whole passes; then one
    thread over a smaller leading sample.  The GPU's output for the sample
    must equal the oracle's."""
    import workloads as W
    torch = runner.torch
    total = case.x.shape[0] if isinstance(case, W.DenseCase) else int(case.row_offsets[-1])
    probe = min(total, 64)
    t = time.perf_counter()
    _oracle_sample(case, probe, CPU_THREADS)
    per_row = max((time.perf_counter() - t) / probe, 1e-9)      # wall per row on all threads
    rows = int(min(total, max(probe, cpu_seconds / CPU_THREADS / per_row)))
    reps, dt, nbytes = 0, 0.0, 0.0
    while reps == 0 or (dt * CPU_THREADS < cpu_seconds and dt < 2 * cpu_seconds / CPU_THREADS):
        t = time.perf_counter()
        q, s, code_rows, scale_rows, b = _oracle_sample(case, rows, CPU_THREADS)
        dt += time.perf_counter() - t
        nbytes += b
        reps += 1
    runner.step(0)
    torch.cuda.synchronize()
    s0 = runner.sets[0]
    idx_q = torch.from_numpy(code_rows).cuda()
    idx_s = torch.from_numpy(scale_rows).cuda()
    same = bool(np.array_equal(s0["q"][idx_q].cpu().numpy(), q) and
                np.array_equal(s0["s"][idx_s].cpu().numpy(), s))
    # one thread, on a leading sample sized for about a second
    rows1 = int(min(total, max(1, 1.0 / (per_row * CPU_THREADS))))
    t = time.perf_counter()
    _, _, _, _, b1 = _oracle_sample(case, rows1, 1)
    dt1 = time.perf_counter() - t
    return {
        "value": round(nbytes / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": CPU_THREADS,
        "kind": "oracle",
        "sample": f"first {rows} of {total} rows of the {case.name} input, {reps} pass(es), "
                  f"{nbytes / 1e6:.1f} MB algorithmic, {dt:.2f} s wall on {CPU_THREADS} threads",
        "one_thread": {"value": round(b1 / dt1 / 1e9, 4), "cores": 1,
                       "sample": f"first {rows1} rows, {dt1:.2f} s wall"},
        "host_cpus_seen": os.cpu_count(),
        "parity_of_sample": "identical" if same else "MISMATCH",
    }


# ------------------------------------------------------------------ counters

# the sources each workload's kernels are built from (host launch code included)
FAMILY_SOURCES = {
    "quantize": ("bsq_kernels.hip", "bsq_internal.h", "bsq_api.cpp"),
    "consume": ("bsq_consume.hip", "bsq_internal.h", "bsq_api.cpp"),
}


def family(name):
    return "consume" if name.startswith(("dequant_", "mfma_")) else "quantize"


def source_hash(fam):
    """sha256 over the sources of one kernel family: counters taken on other
    sources do not describe the kernels that run."""
    h = hashlib.sha256()
    for f in FAMILY_SOURCES[fam]:
        h.update(f.encode())
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def traffic_from_counters(name):
    """HBM bytes per launch of workload `name` from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, valid only while its kernel family's
    sources are the ones they were taken on."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None, "no counter file"
    fam = rec.get(family(name), {})
    if fam.get("source_sha256") != source_hash(family(name)):
        return None, "the kernels changed since the counters were taken"
    v = fam.get("hbm_bytes_per_launch", {}).get(name)
    if v is None:
        return None, f"no counters for {name}"
    return int(v), ("committed measurement (profiles/pmc_traffic.json), not taken in this "
                    "run: " + fam.get("note", ""))


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


def _pmc_rows(path, counter):
    """(kernel name, value, duration ns) of every dispatch in a rocprofv3
    counter_collection.csv for one counter."""
    import csv
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], float(r["Counter_Value"]),
                            int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return out


def _main_kernel(rows):
    """The library kernel with the most GPU time in a run (the workload's own)."""
    tot = {}
    for name, _, ns in rows:
        if "bsq::" in name:
            tot[name] = tot.get(name, 0) + ns
    return max(tot, key=tot.get) if tot else None


# each workload's main kernel in a trace of this script, by name
TRACE_KERNELS = {
    "grouped_nvfp4": "quantize_kernel<2, true, 4>", "dense_nvfp4": "quantize_kernel<2, false, 4>",
    "dense_mxfp8": "quantize_kernel<1, false, 2>", "grouped_mxfp4": "quantize_kernel<0, true, 4>",
    "grouped_mxfp8": "quantize_kernel<1, true, 4>", "tsf_dense_nvfp4": "tsf_amax_kernel<false>",
    "tsf_grouped_nvfp4": "tsf_amax_kernel<true>", "dequant_mxfp8": "dequant_kernel<1, 1>",
    "dequant_nvfp4": "dequant_kernel<2, 1>",
    "mfma_grouped_gemm_mxfp4": "mfma_gemm_grouped_kernel<0>",
    "mfma_grouped_gemm_mxfp4_decode": "mfma_gemm_grouped_skinny_kernel<0, 1>"}


def trace_summary(d, bench_line=None):
    """Markdown tables of a rocprofv3 --kernel-trace --stats run of this
    script in d (output name "bench"): per library kernel, calls and average /
    median / min / max duration; then, per large workload, the mean duration
    of its main kernel's back-to-back dispatches (the timed region) and of its
    event-bound ones, beside the events' own mean from the bench line printed
    under the profiler (bench_line, optional)."""
    import csv
    by = {}
    with open(os.path.join(d, "bench_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            by.setdefault(r["Kernel_Name"], []).append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    print("| kernel | calls | average us | median us | min us | max us |")
    print("|---|---|---|---|---|---|")
    with open(os.path.join(d, "bench_kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            n = r["Name"]
            if "bsq::" not in n and "ceiling_kernel" not in n and "expand_kernel" not in n:
                continue                                 # library and ceiling kernels only
            med = float(np.median([(e - b) / 1e3 for b, e in by[n]]))
            short = n.replace("(anonymous namespace)::", "").replace("bsq::", "")
            print(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {med:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    ev = {}
    if bench_line:
        line = json.loads(open(bench_line).read().strip().splitlines()[-1])
        ev[HEADLINE] = line["roofline"]["kernel_us_mean"]     # a run with the default headline
        for n, w in line.get("workloads", {}).items():
            ev[n] = w["kernel_us"]["mean"]
    print("\n| workload | trace, dispatches 11-110 (back to back) | trace, dispatches 111-210 "
          "(event-bound) | events under the profiler |")
    print("|---|---|---|---|")
    for w, k in TRACE_KERNELS.items():
        names = [n for n in by if k in n]
        if not names:
            continue
        t = np.array([(e - b) / 1e3 for b, e in sorted(by[names[0]])])
        e = f"{ev[w]:.2f}" if w in ev else ""
        print(f"| {w} | {t[10:110].mean():.2f} | {t[110:210].mean():.2f} | {e} |")


GEMM_COUNTERS = ("SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS",
                 "SQ_LDS_BANK_CONFLICT", "SQ_VALU_MFMA_BUSY_CYCLES")


def pmc_gemm_summary(d):
    """A markdown table of the matrix-core counters of each GEMM workload's
    run in d (rocprofv3 --kernel-trace --pmc output named <workload>_p1):
    means per dispatch after the first, the kernel's duration under the
    profiler, and the committed HBM bytes (profiles/pmc_traffic.json) against
    the algorithmic bytes."""
    import csv
    traffic = {}
    try:
        traffic = json.load(open(TRAFFIC_FILE)).get("consume", {}).get("hbm_bytes_per_launch", {})
    except (OSError, ValueError):
        pass
    print("| workload | kernel | kernel µs (profiled) | GRBM_GUI_ACTIVE / µs | " +
          " | ".join(GEMM_COUNTERS) + " | HBM bytes | algorithmic bytes | ratio |")
    print("|" + "---|" * (len(GEMM_COUNTERS) + 7))
    for p in sorted(glob.glob(os.path.join(d, "*_p1_counter_collection.csv"))):
        w = os.path.basename(p)[:-len("_p1_counter_collection.csv")]
        per, dur = {}, {}
        with open(p) as f:
            for r in csv.DictReader(f):
                if "bsq::" not in r["Kernel_Name"]:
                    continue
                key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
                c = per.setdefault(key, {})
                c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                dur[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        keys = sorted(per, key=lambda k: k[1])[1:]       # after the first profiled dispatch
        if not keys:
            continue
        us = float(np.mean([dur[k] for k in keys]))
        mean = {c: float(np.mean([per[k].get(c, 0.0) for k in keys]))
                for c in GEMM_COUNTERS + ("GRBM_GUI_ACTIVE",)}
        alg = algorithmic_bytes(load_workload(w))[0]
        hbm = traffic.get(w)
        tail = f"{hbm:,} | {alg:,} | {hbm / alg:.3f}" if hbm else f"| {alg:,} |"
        print(f"| {w} | `{keys[0][0]}` | {us:.1f} | {mean['GRBM_GUI_ACTIVE'] / us:.0f} | " +
              " | ".join(f"{mean[c]:.4g}" for c in GEMM_COUNTERS) + f" | {tail} |")


def pmc_summary(d, copy_bytes):
    """Turn rocprofv3 --pmc runs into HBM bytes per launch: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) of each workload's main kernel, each scaled
    by what the counter reads for a plain copy of copy_bytes bytes.  Writes
    profiles/pmc_traffic.json and prints a markdown table."""
    def mean_of(stem, counter, pick=None):
        rows = _pmc_rows(os.path.join(d, f"{stem}_counter_collection.csv"), counter)
        k = pick or _main_kernel(rows)
        v = [x for n, x, _ in rows if n == k]
        return k, float(np.mean(v)), len(v)
    _, cf, _ = mean_of("copy_fetch", "FETCH_SIZE", "__amd_rocclr_copyBuffer")
    _, cw, _ = mean_of("copy_write", "WRITE_SIZE", "__amd_rocclr_copyBuffer")
    ff, wf = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    table, out = [], {}
    for p in sorted(glob.glob(os.path.join(d, "*_fetch_counter_collection.csv"))):
        w = os.path.basename(p)[:-len("_fetch_counter_collection.csv")]
        if w == "copy":
            continue
        k, f, n = mean_of(f"{w}_fetch", "FETCH_SIZE")
        _, wr, _ = mean_of(f"{w}_write", "WRITE_SIZE", k)
        hbm = int(round(f * 1024 * ff + wr * 1024 * wf))
        case = load_workload(w)
        alg = (producer_bytes(case) if w.startswith("tsf_") else algorithmic_bytes(case))[0]
        out[w] = hbm
        table.append(f"| {w} | `{k}` | {n} | {f:.1f} | {wr:.1f} | {hbm:,} | {alg:,} | "
                     f"{hbm / alg:.4f} |")
        # the run's other library kernels (the tensor scale's zero and finish passes)
        others = {x for x, _, _ in _pmc_rows(p, "FETCH_SIZE") if "bsq::" in x and x != k}
        for k2 in sorted(others):
            _, f2, n2 = mean_of(f"{w}_fetch", "FETCH_SIZE", k2)
            _, w2, _ = mean_of(f"{w}_write", "WRITE_SIZE", k2)
            table.append(f"| {w} | `{k2}` | {n2} | {f2:.2f} | {w2:.2f} | "
                         f"{int(round(f2 * 1024 * ff + w2 * 1024 * wf)):,} | | |")
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        rec = {}
    note = (f"FETCH_SIZE x {ff:.4f} + WRITE_SIZE x {wf:.4f} per dispatch of the workload's main "
            f"kernel; factors from a plain copy of {copy_bytes} bytes")
    for fam in FAMILY_SOURCES:      # replace what this run measured, keep the other family
        mine = {w: b for w, b in out.items() if family(w) == fam}
        if mine:
            rec[fam] = {"source_sha256": source_hash(fam), "hbm_bytes_per_launch": mine,
                        "fetch_factor": ff, "write_factor": wf, "note": note}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(f"copy of {copy_bytes} bytes: FETCH_SIZE {cf:.1f} KiB (factor {ff:.4f}), "
          f"WRITE_SIZE {cw:.1f} KiB (factor {wf:.4f})\n")
    print("| workload | kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes "
          "(calibrated) | algorithmic bytes | ratio |")
    print("|---|---|---|---|---|---|---|---|")
    print("\n".join(table))
    sq = sorted(glob.glob(os.path.join(d, "*_sq_counter_collection.csv")))
    if sq:
        print("\n| workload | kernel | dispatches | counters (mean per dispatch) | per wave |")
        print("|---|---|---|---|---|")
    for p in sq:
        w = os.path.basename(p)[:-len("_sq_counter_collection.csv")]
        import csv
        per = {}
        with open(p) as f:
            for r in csv.DictReader(f):
                if "bsq::" in r["Kernel_Name"]:
                    per.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(
                        float(r["Counter_Value"]))
        for k, cs in sorted(per.items()):
            means = {c: float(np.mean(v)) for c, v in cs.items()}
            n = max(len(v) for v in cs.values())
            waves = means.get("SQ_WAVES", 0.0)
            pw = ", ".join(f"{c[8:] if c.startswith('SQ_INSTS') else c} {v / waves:.1f}"
                           for c, v in sorted(means.items())
                           if waves and c.startswith("SQ_INSTS"))
            print(f"| {w} | `{k}` | {n} | " +
                  ", ".join(f"{c} {v:.0f}" for c, v in sorted(means.items())) + f" | {pw} |")


# ------------------------------------------------------------------ main

LARGE = ("grouped_nvfp4", "dense_mxfp8", "dense_nvfp4")
# the dequantizations, timed against their own trivial stream; the library's
# dequantizer takes one 512-element chunk per wave
DEQUANT = {"dequant_mxfp8": 1, "dequant_nvfp4": 1}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--pmc-summary", default="")
    ap.add_argument("--pmc-gemm-summary", default="")
    ap.add_argument("--trace-summary", default="")
    ap.add_argument("--bench-line", default="")
    args = ap.parse_args()

    if args.trace_summary:
        trace_summary(args.trace_summary, args.bench_line or None)
        return
    if args.pmc_gemm_summary:
        pmc_gemm_summary(args.pmc_gemm_summary)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary, args.copy_bytes or 268435456)
        return
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

    quant = quantizer_table()
    # The headline is measured last: the GPU needs tens of milliseconds of
    # sustained work to reach its steady clocks, and the other workloads (and
    # the headline's own ceiling legs, on its buffers, right before it)
    # provide them without adding warm-up launches beyond --warmup.
    names = []
    if not args.no_secondary:
        names += [n for n in list(quant) + list(consumer_table()) if n != args.workload]
    names.append(args.workload)
    results, head = {}, None
    for name in names:
        u = None if args.no_ceiling else (quant[name][1] if name in quant and name in LARGE
                                          else DEQUANT.get(name))
        case, runner, nbytes, s, ceil = measure(name, args.steps, args.warmup, u)
        if ceil is not None:
            log("[bench] ceiling", name, json.dumps(ceil))
        if name.startswith(("mfma_gemm", "mfma_grouped_gemm")):
            tf = gemm_flops(case) / s["kernel_us"]["mean"] / 1e6
            peak = PEAK_MFMA_TFLOPS[case.fmt]
            # the bound is whichever ideal time is longer: flops at the peak or bytes at 8 TB/s
            hbm_bound = nbytes / PEAK_HBM_GBS / 1e9 > gemm_flops(case) / peak / 1e12
            s.update({"bound": "hbm" if hbm_bound else "mfma", "TFLOPs": round(tf, 1),
                      "peak_TFLOPs": peak, "frac_of_peak": round(tf / peak, 4)})
        if name in DEQUANT:
            s["roofline"] = roofline(s, *traffic_from_counters(name), ceil)
        if name in quant:
            if name in LARGE:
                s["roofline"] = roofline(s, *traffic_from_counters(name), ceil)
                # the cold-cache protocol beside the rotated buffers (one flush per launch)
                s["roofline"]["cold"] = cold_launches(runner, nbytes, "read")
                s["roofline"]["cold_after_fill"] = cold_launches(runner, nbytes, "write")
            if not args.no_cpu_baseline:
                s["cpu_baseline"] = cpu_baseline(case, runner, 12.0 if name == args.workload
                                                 else 4.0)
        log("[bench]", json.dumps(s))
        if name == args.workload:
            head = (case, s)
        results[name] = s
        del runner, case
        torch.cuda.empty_cache()

    case, s = head
    fmt_name = {0: "MXFP4", 1: "MXFP8", 2: "NVFP4"}[case.fmt]
    config = {"workload": getattr(case, "name", args.workload), "format": fmt_name,
              "input": "bf16", "bytes_per_step": s["bytes_per_launch"],
              "buffer_sets_rotated": s["buffer_sets"], "version": bsq.version()}
    if hasattr(case, "x"):
        config.update({"rows": int(case.x.shape[0]), "K": int(case.x.shape[1]),
                       "block": bsq.BLOCK_SIZE[case.fmt]})
    if hasattr(case, "expert_ids"):
        config["groups"] = int(case.expert_ids.shape[0])
    rl = s.get("roofline") or roofline(s, None, "counters are taken on the large quantizers")
    line = {
        "metric": METRIC,
        "value": s["wall_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(s["wall_s"] / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32" if case.fmt == 2 else "int32",
        "data": "synthetic",
        "config": config,
        "roofline": rl,
        "cpu_baseline": s.get("cpu_baseline"),
        "workloads": {n: r for n, r in results.items() if n != args.workload},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
