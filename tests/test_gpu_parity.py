"""GPU parity: the HIP library against the CPU oracle, byte for byte.

Every comparison covers whole output buffers that both sides pre-fill with
the sentinel 0xA5, padding columns and rows no group owns included, so a
stray or missing write fails as surely as a wrong code.  Inputs are the
seeded workloads (full sizes, in the launch configuration the benchmark
times), every BF16 pattern at every block position, hand-worked blocks, and
ragged / degenerate shapes.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

SENT = 0xA5
NTHREADS = max(1, min(16, os.cpu_count() or 1))
GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


@pytest.fixture(scope="module")
def bsq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantization_amd as m
    return m


def dev(x_bits):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda()


def dense_pair(bsq, x_bits, fmt, tsf=1.0, pad_x=0, pad_q=0, pad_s=0):
    """Run GPU and oracle on the same bytes; return (gpu, oracle) buffers."""
    M, K = x_bits.shape
    bs = oracle.BLOCK[fmt]
    wq, ws = oracle.code_width(fmt, K), K // bs
    xh = np.zeros((M, K + pad_x), np.uint16)
    xh[:, :K] = x_bits
    xd = dev(xh)
    qd = torch.full((M, wq + pad_q), SENT, dtype=torch.uint8, device="cuda")
    sd = torch.full((M, ws + pad_s), SENT, dtype=torch.uint8, device="cuda")
    bsq.quantize_block_scaled(xd[:, :K], fmt, tsf, codes=qd[:, :wq], scales=sd[:, :ws])
    qh = np.full((M, wq + pad_q), SENT, np.uint8)
    sh = np.full((M, ws + pad_s), SENT, np.uint8)
    oracle.quantize(xh[:, :K], fmt, tsf, codes=qh[:, :wq], scales=sh[:, :ws], nthreads=NTHREADS)
    torch.cuda.synchronize()
    return (qd.cpu().numpy(), sd.cpu().numpy()), (qh, sh)


def assert_same(gpu, ref, what=""):
    for name, g, r in (("codes", gpu[0], ref[0]), ("scales", gpu[1], ref[1])):
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            i = tuple(bad[0])
            raise AssertionError(f"{what} {name}: {len(bad)} bytes differ, first at {i}: "
                                 f"gpu={g[i]:#04x} oracle={r[i]:#04x}")


# ------------------------------------------------------------------ hand-worked blocks

@pytest.mark.parametrize("case", GOLDEN["blocks"], ids=[b["name"] for b in GOLDEN["blocks"]])
def test_hand_examples(bsq, case):
    x = np.zeros((1, case["bs"]), np.uint16)
    for k, v in case["x"].items():
        x[0, int(k)] = int(v, 16)
    q, s = bsq.quantize_block_scaled(dev(x), case["fmt"], case["tsf"])
    torch.cuda.synchronize()
    assert s.cpu().numpy()[0, 0] == int(case["scale"], 16), case["why"]
    assert q.cpu().numpy()[0].tobytes().hex().upper() == case["codes"], case["why"]


# ------------------------------------------------------------------ exhaustive sweeps

MX_BG = [("zeros", 0), ("anchor", 0x3F80), ("anchor", 0x7180), ("anchor", 0x0380),
         ("anchor", 0x4260), ("normal", 0)]
NV_TSF = [1.0, 2.0 ** -10, float(np.float32(1.0) / np.float32(2688.0)), 3.0]


def sweep_case(bsq, fmt, tsf, bg, anchor):
    bs = oracle.BLOCK[fmt]
    x = W.sweep_matrix(bs, bg, anchor, seed=41)
    # one block per row (K = bs: only the first lanes of each wave work) ...
    g, r = dense_pair(bsq, x, fmt, tsf, pad_q=16, pad_s=4)
    assert_same(g, r, f"K={bs}")
    # ... and the same blocks laid out 16 to a row (every lane of a chunk)
    wide = x.reshape(-1, 16 * bs)
    g, r = dense_pair(bsq, wide, fmt, tsf)
    assert_same(g, r, f"K={16 * bs}")


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8], ids=["mxfp4", "mxfp8"])
@pytest.mark.parametrize("bg", MX_BG, ids=lambda b: f"{b[0]}_{b[1]:04x}")
def test_mx_sweep_every_pattern_every_position(bsq, fmt, bg):
    sweep_case(bsq, fmt, 1.0, bg[0], bg[1])


@pytest.mark.parametrize("tsf", NV_TSF, ids=["tsf1", "tsf2^-10", "tsf1/2688", "tsf3"])
@pytest.mark.parametrize("bg", [("zeros", 0), ("anchor", 0x3F80), ("anchor", 0x7180),
                                ("normal", 0)], ids=lambda b: f"{b[0]}_{b[1]:04x}")
def test_nvfp4_sweep_every_pattern_every_position(bsq, tsf, bg):
    sweep_case(bsq, oracle.NVFP4, tsf, bg[0], bg[1])


# ------------------------------------------------------------------ full-size workloads

def test_dense_mxfp4_128x4096(bsq):
    c = W.dense_mxfp4_small()
    assert_same(*dense_pair(bsq, c.x, c.fmt), c.name)


def test_dense_mxfp8_8192x7168(bsq):
    c = W.dense_mxfp8_scaled_rows()
    assert_same(*dense_pair(bsq, c.x, c.fmt), c.name)


def test_dense_nvfp4_16384x7168(bsq):
    c = W.dense_nvfp4_scaled_rows()
    assert_same(*dense_pair(bsq, c.x, c.fmt, c.tensor_sf), c.name)


def grouped_pair(bsq, c, pad_rows=0, pad_scale_rows=0):
    K = c.x.shape[1]
    bs = oracle.BLOCK[c.fmt]
    wq, ws = oracle.code_width(c.fmt, K), K // bs
    nq, ns = c.max_rows + pad_rows, c.num_scale_rows + pad_scale_rows
    qd = torch.full((nq, wq), SENT, dtype=torch.uint8, device="cuda")
    sd = torch.full((ns, ws), SENT, dtype=torch.uint8, device="cuda")
    t = lambda a, dt: None if a is None else torch.from_numpy(
        np.ascontiguousarray(a).view(dt)).cuda()
    bsq.grouped_quantize_block_scaled(
        dev(c.x), c.fmt, t(c.row_offsets, np.int32), t(c.scales_offsets, np.int32),
        t(c.expert_ids, np.int32), t(c.tensor_sf, np.float32), c.max_rows, ns,
        row_indices=t(c.row_indices, np.int32), codes=qd[:c.max_rows], scales=sd)
    qh = np.full((nq, wq), SENT, np.uint8)
    sh = np.full((ns, ws), SENT, np.uint8)
    oracle.grouped_quantize(c.x, c.fmt, c.row_offsets, c.scales_offsets, c.expert_ids,
                            c.tensor_sf, c.max_rows, ns, row_indices=c.row_indices,
                            codes=qh[:c.max_rows], scales=sh, nthreads=NTHREADS)
    torch.cuda.synchronize()
    return (qd.cpu().numpy(), sd.cpu().numpy()), (qh, sh)


def test_grouped_nvfp4_prefill_16384x7168(bsq):
    c = W.grouped_nvfp4_prefill()
    assert (c.extra["counts"] == 0).sum() > 0          # empty experts are present
    assert_same(*grouped_pair(bsq, c), c.name)


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8], ids=["mxfp4", "mxfp8"])
def test_grouped_mx_prefill_16384x7168(bsq, fmt):
    """The prefill routing quantized to the MX formats, as measured."""
    c = W.grouped_mx_prefill(fmt)
    assert_same(*grouped_pair(bsq, c), c.name)


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8], ids=["mxfp4", "mxfp8"])
def test_grouped_decode_gather_512x2048(bsq, fmt):
    c = W.grouped_mx_decode(fmt)
    assert_same(*grouped_pair(bsq, c, pad_rows=3, pad_scale_rows=5), c.name)


# ------------------------------------------------------------------ ragged and degenerate

@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8, oracle.NVFP4],
                         ids=["mxfp4", "mxfp8", "nvfp4"])
@pytest.mark.parametrize("M,K", [(1, 32), (3, 64), (1, 512), (7, 544), (129, 1056), (5, 4096),
                                 (33, 7168), (2, 9216), (300, 160)])
def test_ragged_shapes_padded_strides(bsq, fmt, M, K):
    if K % oracle.BLOCK[fmt]:
        pytest.skip("K must be a multiple of the block")
    x = W.random_bf16((M, K), seed=M * 7919 + K, scale_log2_range=(-20, 20), special_frac=0.002)
    tsf = 0.01 if fmt == oracle.NVFP4 else 1.0
    assert_same(*dense_pair(bsq, x, fmt, tsf, pad_x=24, pad_q=16, pad_s=3), f"{M}x{K}")


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8, oracle.NVFP4],
                         ids=["mxfp4", "mxfp8", "nvfp4"])
@pytest.mark.parametrize("M,K", [(1000, 4544), (1001, 4608), (600, 7200)])
def test_dense_large_problem_path(bsq, fmt, M, K):
    """Over 2^22 elements dense rows go in tiles of 2 (MXFP8) or 4 (FP4)
    chunks of 512 elements, and FP4 codes take the write-through stores.
    K = 4544 is 9 chunks, the last holding 448 elements, so every row ends in
    a partly empty tile with a partial chunk; K = 4608 is 9 whole chunks;
    K = 7200 is 14 whole chunks and a 32-element one.  Strides are padded."""
    assert M * K > (1 << 22)
    x = W.random_bf16((M, K), seed=M + K + 100 * fmt, scale_log2_range=(-20, 20),
                      special_frac=0.001)
    tsf = 0.01 if fmt == oracle.NVFP4 else 1.0
    assert_same(*dense_pair(bsq, x, fmt, tsf, pad_x=40, pad_q=16, pad_s=5), f"{M}x{K}")


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8, oracle.NVFP4],
                         ids=["mxfp4", "mxfp8", "nvfp4"])
def test_nvfp4_nk_16_not_32(bsq, fmt):
    # K = 16 * odd: NVFP4 accepts it (packed row is 8 * odd bytes); MX rejects it
    x = W.random_bf16((9, 48), seed=5)
    if fmt == oracle.NVFP4:
        assert_same(*dense_pair(bsq, x, fmt, 0.02), "K=48")
    else:
        with pytest.raises(Exception):
            bsq.quantize_block_scaled(dev(x), fmt)


def test_zero_rows_is_noop(bsq):
    x = torch.zeros((0, 256), dtype=torch.int16, device="cuda")
    q, s = bsq.quantize_block_scaled(x, oracle.MXFP4)
    assert q.shape == (0, 128) and s.shape == (0, 8)


@pytest.mark.parametrize("tsf", [2.0 ** -117, 2.0 ** 100, 1e-30, 7.5e25])
def test_nvfp4_extreme_tensor_scales(bsq, tsf):
    x = W.random_bf16((64, 512), seed=8, scale_log2_range=(-126, 126), special_frac=0.01)
    assert_same(*dense_pair(bsq, x, oracle.NVFP4, tsf), f"tsf={tsf}")


def test_all_special_patterns_dense(bsq):
    """NaN, Inf, signed zeros and subnormals in every mix within blocks."""
    rng = np.random.default_rng(9)
    pats = np.array([0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x807F, 0x7F7F,
                     0xFF7F, 0x0080, 0x7F81, 0x3F80], np.uint16)
    x = pats[rng.integers(0, len(pats), (256, 1024))]
    x[:128] = np.where(rng.random((128, 1024)) < 0.9, np.uint16(0x0001) * rng.integers(
        0, 0x80, (128, 1024)).astype(np.uint16), x[:128])
    for fmt, tsf in ((oracle.MXFP4, 1.0), (oracle.MXFP8, 1.0), (oracle.NVFP4, 2.0 ** -117),
                     (oracle.NVFP4, 1.0)):
        assert_same(*dense_pair(bsq, x, fmt, tsf), f"fmt={fmt}")


# ------------------------------------------------------------------ grouped edge cases

def make_grouped(fmt, S, K, G, E, rows, gather, seed, first_row=0, extra_rows=0, pad=8,
                 empty_frac=0.5):
    rng = np.random.default_rng(seed)
    x = W.random_bf16((S, K), seed=seed + 1, scale_log2_range=(-10, 10))
    w = rng.random(G) * (rng.random(G) > empty_frac)
    if w.sum() == 0:
        w[rng.integers(0, G)] = 1.0
    counts = rng.multinomial(rows, w / w.sum())
    ro, so = W.offsets_from_counts(counts, pad)
    ro = (ro + first_row).astype(np.uint32)
    ids = rng.integers(0, E, G).astype(np.int32)
    sf = None
    if fmt == oracle.NVFP4:
        sf = (np.exp2(rng.uniform(-12, 2, E)) * 0.37).astype(np.float32)
    max_rows = first_row + rows + extra_rows
    ri = rng.integers(0, S, max_rows).astype(np.int32) if gather else None
    if not gather:
        assert max_rows <= S
    return W.GroupedCase(f"g{G}_e{E}", fmt, x, ro, so, ids, sf, ri, max_rows=max_rows,
                         num_scale_rows=int(so[-1]) + 2)


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8, oracle.NVFP4],
                         ids=["mxfp4", "mxfp8", "nvfp4"])
@pytest.mark.parametrize("G,gather,first,extra", [(1, False, 0, 0), (5, True, 0, 0),
                                                   (64, False, 3, 5), (65, True, 0, 0),
                                                   (200, True, 7, 9), (300, False, 0, 4),
                                                   (1000, True, 0, 0)])
def test_grouped_random_offsets(bsq, fmt, G, gather, first, extra):
    K = 1024 if G < 300 else 256
    rows = 700
    c = make_grouped(fmt, S=max(800, first + rows + extra), K=K, G=G, E=G + 17, rows=rows,
                     gather=gather, seed=G * 31 + first, first_row=first, extra_rows=extra)
    assert_same(*grouped_pair(bsq, c, pad_rows=2, pad_scale_rows=3), c.name)


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8, oracle.NVFP4],
                         ids=["mxfp4", "mxfp8", "nvfp4"])
@pytest.mark.parametrize("G", [255, 256, 257, 511, 512, 513])
@pytest.mark.parametrize("gather", [False, True], ids=["direct", "gather"])
def test_grouped_search_round_boundaries(bsq, fmt, G, gather):
    """The group lookup counts row_offsets 256 entries at a time: G + 1 =
    256, 257, 258 entries (one round, a second round of one and of two
    entries) and 512, 513, 514.  Every group owns at least one row, so the
    last groups' rows sit at each round's edge, and 5 rows past the last group
    are owned by none (left as they were)."""
    rng = np.random.default_rng(G * 7 + fmt + gather)
    K = 512
    counts = 1 + rng.multinomial(G, np.full(G, 1.0 / G))
    rows = int(counts.sum())
    S = rows + 5
    x = W.random_bf16((S, K), seed=G + 3, scale_log2_range=(-10, 10))
    ro, so = W.offsets_from_counts(counts, 8)
    E = G + 5
    ids = rng.integers(0, E, G).astype(np.int32)
    sf = (np.exp2(rng.uniform(-12, 2, E)) * 0.37).astype(np.float32) \
        if fmt == oracle.NVFP4 else None
    ri = rng.integers(0, S, rows + 5).astype(np.int32) if gather else None
    c = W.GroupedCase(f"g{G}_boundary", fmt, x, ro, so, ids, sf, ri, max_rows=rows + 5,
                      num_scale_rows=int(so[-1]) + 2)
    assert_same(*grouped_pair(bsq, c, pad_rows=2, pad_scale_rows=3), c.name)


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.NVFP4], ids=["mxfp4", "nvfp4"])
@pytest.mark.parametrize("M,K,pad_q,pad_s", [(1100, 4032, 4, 1), (700, 6160, 8, 0),
                                             (700, 6144, 4, 2), (1030, 4096, 12, 3)])
def test_large_path_misaligned_rows_and_partial_tiles(bsq, fmt, M, K, pad_q, pad_s):
    """FP4 over 2^22 elements (tiles of 4 chunks, write-through code stores)
    into code rows only 4- or 8-byte aligned (strides K/2 + 4, + 8, + 12
    bytes) and scale rows at alternating even and odd addresses.  K = 4032 is
    7 whole chunks and a partial one, so a row's second tile is full but holds
    the partial chunk; K = 6160 (NVFP4 only) is 12 whole chunks and a
    16-element one."""
    if fmt == oracle.MXFP4 and K % 32:
        pytest.skip("MXFP4 needs K a multiple of 32")
    assert M * K > (1 << 22)
    x = W.random_bf16((M, K), seed=M + K + pad_q, scale_log2_range=(-20, 20),
                      special_frac=0.001)
    tsf = 0.02 if fmt == oracle.NVFP4 else 1.0
    assert_same(*dense_pair(bsq, x, fmt, tsf, pad_x=8, pad_q=pad_q, pad_s=pad_s), f"{M}x{K}")


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.NVFP4], ids=["mxfp4", "nvfp4"])
@pytest.mark.parametrize("K", [4048, 6144])
def test_grouped_large_path_odd_scale_rows_with_gather(bsq, fmt, K):
    """The grouped FP4 path over 2^22 elements with gather and unpadded scale
    offsets.  K = 4048 (NVFP4 only): 253 scale bytes per row, so scale rows
    alternate between even and odd addresses, and a row's second tile holds
    its partial chunk."""
    if fmt == oracle.MXFP4 and K % 32:
        pytest.skip("MXFP4 needs K a multiple of 32")
    rows = 1100
    assert rows * K > (1 << 22)
    c = make_grouped(fmt, S=1200, K=K, G=40, E=50, rows=rows, gather=True, seed=K + fmt,
                     first_row=3, extra_rows=4, pad=1)
    assert_same(*grouped_pair(bsq, c, pad_rows=1, pad_scale_rows=2), c.name)


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8, oracle.NVFP4],
                         ids=["mxfp4", "mxfp8", "nvfp4"])
@pytest.mark.parametrize("G,gather,K", [(5, False, 4608), (129, True, 4608), (600, False, 4608),
                                         (129, True, 4544), (7, False, 4544)])
def test_grouped_large_problem_path(bsq, fmt, G, gather, K):
    """Over 2^22 routed elements the library switches to 4-chunk tiles (and,
    for FP4 codes, write-through stores); K = 4608 leaves a ragged 1-chunk last
    tile, K = 4544 a last tile of one partial chunk (448 elements)."""
    rows = 1200
    assert rows * K > (1 << 22)
    c = make_grouped(fmt, S=1300, K=K, G=G, E=G + 3, rows=rows, gather=gather, seed=G + 7,
                     first_row=2, extra_rows=5)
    assert_same(*grouped_pair(bsq, c, pad_rows=1, pad_scale_rows=2), c.name)


def test_grouped_single_group_equals_dense(bsq):
    x = W.random_bf16((130, 2048), seed=77)
    for fmt, tsf in ((oracle.MXFP4, 1.0), (oracle.MXFP8, 1.0), (oracle.NVFP4, 0.004)):
        qd, sd = bsq.quantize_block_scaled(dev(x), fmt, tsf)
        ro = torch.tensor([0, 130], dtype=torch.int32, device="cuda")
        qg, sg = bsq.grouped_quantize_block_scaled(
            dev(x), fmt, ro, ro.clone(), torch.zeros(1, dtype=torch.int32, device="cuda"),
            torch.tensor([tsf], dtype=torch.float32, device="cuda"), 130, 130)
        torch.cuda.synchronize()
        assert torch.equal(qd, qg) and torch.equal(sd, sg)


# ------------------------------------------------------------------ streams and errors

def test_runs_on_a_side_stream(bsq):
    c = W.dense_mxfp4_small()
    s = torch.cuda.Stream()
    xd = dev(c.x)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        q, sc = bsq.quantize_block_scaled(xd, c.fmt)
    s.synchronize()
    qh, sh = oracle.quantize(c.x, c.fmt)
    assert np.array_equal(q.cpu().numpy(), qh) and np.array_equal(sc.cpu().numpy(), sh)


def test_bad_arguments_raise_before_launch(bsq):
    x = torch.zeros((4, 64), dtype=torch.int16, device="cuda")
    with pytest.raises(bsq.BsqError, match="INVALID"):
        bsq.quantize_block_scaled(x, oracle.NVFP4, tensor_sf=float("nan"))
    with pytest.raises(bsq.BsqError, match="INVALID"):
        bsq.quantize_block_scaled(x[:, :48], oracle.MXFP4)
    with pytest.raises(bsq.BsqError, match="INVALID"):
        bsq.quantize_block_scaled(x, oracle.MXFP8, codes=torch.empty(
            (4, 60), dtype=torch.uint8, device="cuda"))
