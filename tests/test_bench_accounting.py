"""The byte and flop counts behind bench.py's achieved GB/s and TFLOP/s,
pinned to the per-element figures stated for each workload: BF16 read (2
bytes) plus codes (1 byte FP8, 1/2 FP4) plus one scale byte per block, times
the elements a launch processes, plus the grouping metadata; each distinct
gathered source row is read once.  CPU only: no kernel runs."""
import numpy as np
import pytest

import bench
import workloads as W


def test_dense_workloads():
    assert bench.algorithmic_bytes(W.dense_mxfp8_scaled_rows()) == (177_995_776, 8192 * 7168)
    assert bench.algorithmic_bytes(W.dense_nvfp4_scaled_rows()) == (300_941_312, 16384 * 7168)
    assert bench.algorithmic_bytes(W.dense_mxfp4_small()) == (1_327_104, 128 * 4096)
    for fmt, per in ((W.MXFP4, 2.53125), (W.MXFP8, 3.03125), (W.NVFP4, 2.5625)):
        assert bench.bytes_per_element(fmt) == per


def test_grouped_workloads():
    c = W.grouped_nvfp4_prefill()
    # 16384 x 7168 x 2.5625 + (129 + 129 + 128 + 128) x 4 bytes of offsets, ids and scales
    assert bench.algorithmic_bytes(c) == (300_943_368, 16384 * 7168)
    assert 16384 * 7168 * 2.5625 + (129 + 129 + 128 + 128) * 4 == 300_943_368
    for fmt, want in ((W.MXFP4, 824_328), (W.MXFP8, 1_348_616)):
        d = W.grouped_mx_decode(fmt)
        distinct = np.unique(d.row_indices).size
        assert distinct == 64                    # every token is routed
        assert bench.algorithmic_bytes(d)[0] == want


def test_tensor_scale_producer_bytes():
    assert bench.producer_bytes(W.dense_nvfp4_scaled_rows()) == (16384 * 7168 * 2 + 4,
                                                                16384 * 7168)
    nb, elems = bench.producer_bytes(W.grouped_nvfp4_prefill())
    assert nb == 16384 * 7168 * 2 + (129 + 128 + 128) * 4 and elems == 16384 * 7168


def test_dequantize_and_gemm_accounting():
    d = W.dequant_random_bytes(W.MXFP8, 256, 7168, seed=1)
    assert bench.algorithmic_bytes(d) == (256 * 7168 * (1 + 4) + 256 * 224, 256 * 7168)
    g = W.gemm_random_operands(W.MXFP4, 256, 512, 1024, seed=2)
    nb, _ = bench.algorithmic_bytes(g)
    rec = 256 * (1024 // 512)                    # MFMA-layout bytes per 16 rows
    assert nb == 256 * 512 + 512 * 512 + (256 // 16 + 512 // 16) * rec + 4 * 256 * 512
    assert bench.gemm_flops(g) == 2 * 256 * 512 * 1024


@pytest.mark.parametrize("name", ["mfma_gemm_mxfp8", "mfma_gemm_mxfp4"])
def test_measured_gemm_flops(name):
    c = bench.load_workload(name)
    assert bench.gemm_flops(c) == 2 * 4096 * 4096 * 7168


def test_grouped_gemm_bytes_count_only_experts_with_rows():
    """Routed A and its scale records, the weights of each expert that owns
    rows (an expert with no rows is never read), the metadata, and c."""
    for c in (W.grouped_gemm_prefill(W.MXFP4, rows=512, K=256, N=64, experts=16),
              W.grouped_gemm_decode(W.MXFP4, tokens=8, K=256, N=32, experts=64, topk=2)):
        E, K = c.num_experts, c.K
        N = c.b_codes.shape[0] // E
        counts = np.diff(c.row_offsets.astype(np.int64))
        used = int(np.count_nonzero(counts))             # expert_ids = arange: one group each
        assert 0 < used < E                              # some experts are empty
        per_expert = N * K // 2 + ((N + 15) // 16) * ((K // 32 + 15) // 16) * 256
        want = (c.a_codes.nbytes + c.a_scales.nbytes + used * per_expert +
                4 * (2 * (E + 1) + E) + 4 * c.max_rows * N)
        assert bench.algorithmic_bytes(c) == (want, c.max_rows * N)


def test_dense_decode_gemm_bytes():
    """16 rows against 16384 x 7168 MXFP4 weights: operands and their scale
    records read once, c written; HBM-bound (bytes at 8 TB/s outlast the
    flops at the fp4 matrix peak)."""
    c = W.gemm_random_operands(W.MXFP4, 16, 16384, 7168, seed=1205)
    nb, elems = bench.algorithmic_bytes(c)
    rec = (7168 // 512) * 256
    assert nb == 16 * 3584 + 16384 * 3584 + (1 + 1024) * rec + 4 * 16 * 16384
    assert elems == 16 * 16384
    assert nb / bench.PEAK_HBM_GBS / 1e9 > bench.gemm_flops(c) / bench.PEAK_MFMA_TFLOPS[0] / 1e12


def test_headline_is_the_grouped_nvfp4_prefill():
    """The line's headline is the largest single-GPU workload: grouped NVFP4
    prefill, 16384 routed rows x 7168 over 128 experts."""
    assert bench.HEADLINE == "grouped_nvfp4"
    c = bench.load_workload(bench.HEADLINE)
    assert c.fmt == W.NVFP4 and c.x.shape == (16384, 7168) and c.G == 128
    for name in ("dense_mxfp8", "dense_nvfp4", "grouped_nvfp4"):
        assert name in bench.LARGE and bench.quantizer_table()[name][1] in (2, 4)


def test_oracle_sample_of_a_grouped_workload():
    """The CPU baseline's sample of a grouped workload: the first R routed
    rows, each group cut at R; the codes rows and scale rows it reports are
    exactly those the oracle wrote, and its bytes count them."""
    c = W.grouped_mx_decode(W.MXFP4)
    R = 100
    q, s, code_rows, scale_rows, nbytes = bench._oracle_sample(c, R, 1)
    assert np.array_equal(code_rows, np.arange(R))
    counts = np.diff(np.minimum(c.row_offsets.astype(np.int64), R))
    assert scale_rows.size == R and q.shape[0] == R and s.shape[0] == R
    starts = c.scales_offsets[:-1].astype(np.int64)
    want = np.concatenate([np.arange(a, a + n) for a, n in zip(starts, counts)])
    assert np.array_equal(scale_rows, want)
    distinct = np.unique(c.row_indices[:R]).size
    assert nbytes == distinct * 2048 * 2 + R * 2048 * (bench.bytes_per_element(W.MXFP4) - 2)


def test_rotation_exceeds_the_last_level_cache():
    for nb in (1_327_104, 177_995_776, 300_943_368):
        sets = bench.rotation(nb)
        assert sets >= 2 and (sets * nb > 3 * bench.MALL_BYTES or sets == 64)


@pytest.mark.parametrize("n", [2, 8])
def test_bench_refuses_more_than_one_gpu(n):
    """bench.py measures one GPU: --gpus N > 1 exits with status 2 and a
    message, before touching torch or the library."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", str(n)],
                         capture_output=True, text=True, timeout=120, cwd=root)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def _write_csv(path, header, rows):
    import csv
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_summary_tables(tmp_path, capsys):
    """--trace-summary: per-kernel calls and durations of the library and ceiling
    kernels only, and per workload the means over the back-to-back and the
    event-bound dispatch windows (dispatches 11-110 and 111-210)."""
    k = "void bsq::(anonymous namespace)::quantize_kernel<2, true, 4>(bsq::KernelArgs)"
    rows = [[k, 1000 * i, 1000 * i + (40_000 if i < 110 else 41_000)] for i in range(210)]
    rows += [["__amd_rocclr_copyBuffer", 0, 5000]]
    _write_csv(tmp_path / "bench_kernel_trace.csv",
               ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    _write_csv(tmp_path / "bench_kernel_stats.csv",
               ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
               [[k, 210, 40476.2, 40000, 41000], ["__amd_rocclr_copyBuffer", 1, 5000, 5000, 5000]])
    bench.trace_summary(str(tmp_path))
    out = capsys.readouterr().out
    assert "quantize_kernel<2, true, 4>" in out and "rocclr" not in out
    assert "| 210 | 40.48 |" in out
    assert "| grouped_nvfp4 | 40.00 | 41.00 |" in out


def test_pmc_gemm_summary_table(tmp_path, capsys, monkeypatch):
    """--pmc-gemm-summary: means per dispatch after the first, against the
    committed HBM bytes and the workload's algorithmic bytes."""
    k = "void bsq::(anonymous namespace)::mfma_gemm_grouped_kernel<0>(x)"
    rows = []
    for d in range(1, 4):
        for c, v in (("SQ_INSTS_MFMA", 100.0 * d), ("GRBM_GUI_ACTIVE", 2000.0)) + tuple(
                (c, 1.0) for c in bench.GEMM_COUNTERS if c != "SQ_INSTS_MFMA"):
            rows.append([k, d, c, v, 0, 2000 * 1000])          # 2000 us each
    _write_csv(tmp_path / "mfma_grouped_gemm_mxfp4_p1_counter_collection.csv",
               ["Kernel_Name", "Dispatch_Id", "Counter_Name", "Counter_Value", "Start_Timestamp",
                "End_Timestamp"], rows)
    alg = bench.algorithmic_bytes(W.grouped_gemm_prefill(W.MXFP4))[0]
    tf = tmp_path / "traffic.json"
    tf.write_text('{"consume": {"hbm_bytes_per_launch": {"mfma_grouped_gemm_mxfp4": %d}}}'
                  % (2 * alg))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    bench.pmc_gemm_summary(str(tmp_path))
    out = capsys.readouterr().out
    line = [ln for ln in out.splitlines() if ln.startswith("| mfma_grouped_gemm_mxfp4 |")][0]
    cells = [c.strip() for c in line.split("|")]
    assert cells[3] == "2000.0"                   # kernel µs, dispatches 2 and 3
    assert cells[5] == "250"                      # SQ_INSTS_MFMA: mean of 200 and 300
    assert cells[-2] == "2.000"                   # HBM over algorithmic bytes
