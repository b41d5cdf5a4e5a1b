"""The MFMA consumer: c = A B^T on gfx950's scaled matrix instruction, reading
MX codes row-major and scales in the MFMA layout -- the check that the
layout is what the hardware takes.

Every output is compared with the oracle's exact GEMM within the bound of
``gemm_bound`` (derived from the instruction's arithmetic: for E2M1 only the
float32 roundings of each 128-element K step and of the accumulation, about
2^-17.2 of sum |a b| at K = 7168, tight enough that one wrong element fails;
for E4M3 also 2^-11 of each step's largest product).  The worst error as a
fraction of the bound is printed.  At the measured sizes whole outputs are
compared: a full 256-row tile band (and the last one) of the dense GEMM, and
every routed row of the grouped prefill and decode GEMMs."""
import os

import numpy as np
import pytest
import torch

import gemm_bound
import oracle
import workloads as W

pytestmark = pytest.mark.gpu
NTHREADS = max(1, min(16, os.cpu_count() or 1))
MXFP4, MXFP8 = oracle.MXFP4, oracle.MXFP8


@pytest.fixture(scope="module")
def bsq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantization_amd as m
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def operand(fmt, rows, K, seed, span=(-8, 8)):
    x = W.random_bf16((rows, K), seed=seed, scale_log2_range=span)
    q, s = oracle.quantize(x, fmt, 1.0, nthreads=NTHREADS)
    return x, q, s


@pytest.mark.parametrize("fmt", [MXFP4, MXFP8])
@pytest.mark.parametrize("M,N,K", [(16, 16, 128), (37, 45, 1024), (128, 96, 2048),
                                   (33, 130, 7168), (1, 300, 640),
                                   # M <= 32: 16- / 32-row tiles streaming B (by default)
                                   (5, 1000, 1152), (24, 520, 2048), (32, 257, 256),
                                   (17, 130, 7168)])
def test_mfma_matmul_matches_oracle(bsq, fmt, M, N, K):
    _, qa, sa = operand(fmt, M, K, seed=M + K + fmt)
    _, qb, sb = operand(fmt, N, K, seed=N + K + fmt + 1)
    got = bsq.block_scaled_matmul_mfma(dev(qa), dev(oracle.scales_to_mfma16(sa)), dev(qb),
                                       dev(oracle.scales_to_mfma16(sb)), fmt, K)
    torch.cuda.synchronize()
    want = oracle.block_scaled_matmul(qa, sa, qb, sb, fmt, K)
    worst = gemm_bound.check(got.cpu().numpy(), qa, sa, qb, sb, fmt, K, want)
    print(f"format {fmt} {M}x{N}x{K}: worst |err| / bound = {worst:.3f}")


@pytest.mark.parametrize("fmt", [MXFP4, MXFP8])
def test_pipeline_quantize_into_layout_then_mfma(bsq, fmt):
    """BF16 -> GPU quantizer writing the MFMA layout -> MFMA GEMM, against the
    exact GEMM of the oracle's quantization (and the end-to-end error against
    the BF16 GEMM, which must match the naive pipeline's)."""
    K = 2048
    xa = W.random_bf16((128, K), seed=1, scale_log2_range=(-4, 4))
    xb = W.random_bf16((96, K), seed=11, scale_log2_range=(-4, 4))
    L = bsq.SCALES_MFMA16
    qa, la = bsq.quantize_block_scaled(dev(xa.view(np.int16)), fmt, scale_layout=L)
    qb, lb = bsq.quantize_block_scaled(dev(xb.view(np.int16)), fmt, scale_layout=L)
    c = bsq.block_scaled_matmul_mfma(qa, la, qb, lb, fmt, K)
    torch.cuda.synchronize()
    qa_h, sa_h = oracle.quantize(xa, fmt, 1.0, nthreads=NTHREADS)
    qb_h, sb_h = oracle.quantize(xb, fmt, 1.0, nthreads=NTHREADS)
    want = oracle.block_scaled_matmul(qa_h, sa_h, qb_h, sb_h, fmt, K)
    got = c.cpu().numpy().astype(np.float64)
    gemm_bound.check(got, qa_h, sa_h, qb_h, sb_h, fmt, K, want)
    ref = W.bf16_to_f32(xa).astype(np.float64) @ W.bf16_to_f32(xb).astype(np.float64).T
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    err_exact = np.linalg.norm(want - ref) / np.linalg.norm(ref)
    print(f"format {fmt}: end-to-end relative error {err:.4f} (exact sums {err_exact:.4f})")
    assert abs(err - err_exact) <= 1e-3 * err_exact


@pytest.mark.parametrize("fmt", [MXFP4, MXFP8])
def test_nan_scale_and_nan_code(bsq, fmt):
    """A block holding NaN or Inf gets the NaN scale 0xFF (and zero codes):
    the instruction must turn its row of c into NaN, as the oracle does."""
    K = 512
    x = W.random_bf16((20, K), seed=9 + fmt, scale_log2_range=(-4, 4))
    x[3, 100] = 0x7FC0                      # NaN in A row 3
    y = W.random_bf16((18, K), seed=10 + fmt, scale_log2_range=(-4, 4))
    y[7, 300] = 0xFF80                      # -Inf in B row 7
    qa, sa = oracle.quantize(x, fmt, 1.0)
    qb, sb = oracle.quantize(y, fmt, 1.0)
    got = bsq.block_scaled_matmul_mfma(dev(qa), dev(oracle.scales_to_mfma16(sa)), dev(qb),
                                       dev(oracle.scales_to_mfma16(sb)), fmt, K)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    want = oracle.block_scaled_matmul(qa, sa, qb, sb, fmt, K)
    assert np.isnan(want[3]).all() and np.isnan(want[:, 7]).all()
    gemm_bound.check(got, qa, sa, qb, sb, fmt, K, want)


def random_operand(fmt, rows, K, rng):
    """Random codes (E4M3 NaN codes replaced by 1.0) and row-major scale
    bytes in [120, 134]: any bytes are valid operands for the GEMM."""
    width = K if fmt == MXFP8 else K // 2
    q = rng.integers(0, 256, (rows, width), dtype=np.uint8)
    if fmt == MXFP8:
        q[(q & 0x7F) == 0x7F] = 0x38
    s = rng.integers(120, 135, (rows, K // 32), dtype=np.uint8)
    return q, s


@pytest.mark.parametrize("fmt", [MXFP4, MXFP8])
@pytest.mark.parametrize("M,N,K", [(4096, 4096, 7168), (4000, 4100, 1536)])
def test_full_size_tile_bands(bsq, fmt, M, N, K):
    """At the measured GEMM's size (and a ragged one), where the library takes
    its 256 x 256 tiles: the first 256-row tile band and the last (partial)
    one, every column, element by element against the oracle."""
    rng = np.random.default_rng(M + N + K + fmt)
    qa, sa = random_operand(fmt, M, K, rng)
    qb, sb = random_operand(fmt, N, K, rng)
    got = bsq.block_scaled_matmul_mfma(dev(qa), dev(oracle.scales_to_mfma16(sa)), dev(qb),
                                       dev(oracle.scales_to_mfma16(sb)), fmt, K)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    last = (M - 1) // 256 * 256
    for r0, r1 in ((0, 256), (last, M)):
        worst = gemm_bound.check(got[r0:r1], qa[r0:r1], sa[r0:r1], qb, sb, fmt, K)
        print(f"format {fmt} {M}x{N}x{K} rows {r0}..{r1}: worst |err| / bound = {worst:.3f}")


def mfma16_rows_to_row_major(lay, rows, nblk):
    """Row-major scales [len(rows), nblk] of the given rows of an MFMA-layout
    buffer, through the oracle's index map (offsets within a row group depend
    only on r % 16 and the block)."""
    lds = lay.shape[1]
    inner = np.array([[oracle.mfma16_scale_offset(r16, kb, lds) for kb in range(nblk)]
                      for r16 in range(16)], np.int64)
    rows = np.asarray(rows, np.int64)
    return lay.reshape(-1)[(rows // 16)[:, None] * lds + inner[rows % 16]]


def check_every_group(got, c, fmt, K, N):
    """Every routed row of every group of a grouped GEMM workload against the
    oracle; returns the worst |err| / bound."""
    nblk = K // 32
    ro, so, ids = c.row_offsets, c.scales_offsets, c.expert_ids
    worst = 0.0
    for g in range(len(c.expert_ids)):
        lo, hi, e = int(ro[g]), int(ro[g + 1]), int(ids[g])
        if hi == lo:
            continue
        rows = np.arange(lo, hi)
        sa = mfma16_rows_to_row_major(c.a_scales, int(so[g]) + rows - lo, nblk)
        brows = e * N + np.arange(N)
        sb = mfma16_rows_to_row_major(c.b_scales, brows, nblk)
        worst = max(worst, gemm_bound.check(got[lo:hi], c.a_codes[lo:hi], sa, c.b_codes[brows],
                                            sb, fmt, K))
    return worst


def test_grouped_gemm_prefill_full_size(bsq):
    """The measured grouped GEMM (prefill routing, 128 experts, N = 512,
    K = 7168, 128-row tiles): every routed row, element by element."""
    c = W.grouped_gemm_prefill(W.MXFP4)
    fmt, K, E = c.fmt, c.K, c.num_experts
    N = c.b_codes.shape[0] // E
    assert tile_rows(c.max_rows, E) == 128
    ro, so, ids = c.row_offsets, c.scales_offsets, c.expert_ids
    out = bsq.grouped_block_scaled_matmul_mfma(
        dev(c.a_codes), dev(c.a_scales), dev(ro.view(np.int32)), dev(so.view(np.int32)),
        dev(ids), c.max_rows, c.num_scale_rows, dev(c.b_codes), dev(c.b_scales), E, fmt, K)
    torch.cuda.synchronize()
    worst = check_every_group(out.cpu().numpy(), c, fmt, K, N)
    print(f"grouped prefill: worst |err| / bound = {worst:.3f}")


def test_grouped_gemm_decode_full_size(bsq):
    """The measured decode GEMM (64 tokens routed top-8 over 256 experts, N =
    7168, K = 2048, 16-row tiles): every routed row, element by element."""
    c = W.grouped_gemm_decode(W.MXFP4)
    fmt, K, E = c.fmt, c.K, c.num_experts
    N = c.b_codes.shape[0] // E
    assert tile_rows(c.max_rows, E) == 16
    ro, so, ids = c.row_offsets, c.scales_offsets, c.expert_ids
    out = bsq.grouped_block_scaled_matmul_mfma(
        dev(c.a_codes), dev(c.a_scales), dev(ro.view(np.int32)), dev(so.view(np.int32)),
        dev(ids), c.max_rows, c.num_scale_rows, dev(c.b_codes), dev(c.b_scales), E, fmt, K)
    torch.cuda.synchronize()
    worst = check_every_group(out.cpu().numpy(), c, fmt, K, N)
    print(f"grouped decode: worst |err| / bound = {worst:.3f}")


def grouped_case(fmt, G, E, N, K, rows, seed, misaligned=None):
    """Routed activations quantized by the oracle's grouped quantizer (scales
    then mapped into the MFMA layout) and E experts' [N, K] weights (one
    layout per expert, stacked)."""
    rng = np.random.default_rng(seed)
    S = rows + 10
    x = W.random_bf16((S, K), seed=seed, scale_log2_range=(-6, 6))
    w = rng.random(G) * (rng.random(G) > 0.3)
    w[0] += 1e-3
    counts = rng.multinomial(rows, w / w.sum())
    ro = np.concatenate([[0], np.cumsum(counts)]).astype(np.uint32)
    pads = -(-counts // 16) * 16 + 16 * rng.integers(0, 2, G)          # some extra padding
    so = np.concatenate([[0], np.cumsum(pads)]).astype(np.uint32)
    if misaligned is not None:                                          # shift one group's scales
        so[misaligned] += 8
    ids = rng.integers(0, E, G).astype(np.int32)
    max_rows, nsr = int(ro[-1]) + 7, int(so[-1]) + 16
    width = K if fmt == MXFP8 else K // 2
    qa, sa = oracle.grouped_quantize(x, fmt, ro, so, ids, None, max_rows, nsr,
                                     codes=np.zeros((max_rows, width), np.uint8),
                                     scales=np.zeros((nsr, K // 32), np.uint8), nthreads=NTHREADS)
    wb = W.random_bf16((E * N, K), seed=seed + 1, scale_log2_range=(-6, 6))
    qb, sb = oracle.quantize(wb, fmt, 1.0, nthreads=NTHREADS)
    lb = np.concatenate([oracle.scales_to_mfma16(sb[e * N:(e + 1) * N]) for e in range(E)])
    return dict(qa=qa, sa=sa, la=oracle.scales_to_mfma16(sa), ro=ro, so=so, ids=ids,
                max_rows=max_rows, nsr=nsr, qb=qb, sb=sb, lb=lb, counts=counts)


@pytest.mark.parametrize("fmt", [MXFP4, MXFP8])
@pytest.mark.parametrize("G,E,N,K,rows", [(1, 1, 128, 256, 128), (5, 3, 100, 512, 300),
                                          (40, 16, 160, 1024, 900), (9, 4, 256, 7168, 700),
                                          (130, 20, 96, 512, 3000), (200, 7, 48, 256, 9000),
                                          (3, 2, 200, 128, 400), (4, 3, 130, 384, 500),
                                          (6, 5, 272, 1664, 800), (256, 9, 48, 256, 9000),
                                          (257, 9, 48, 256, 9000), (300, 11, 64, 512, 10000)])
def test_grouped_mfma_matches_oracle(bsq, fmt, G, E, N, K, rows):
    """Groups of more than 16 rows on average: 128 x 128 tiles, both operands
    staged through LDS.  K = 128 and 384 end on a half stage in MXFP4 (256
    elements a stage); 1664 is 13 K steps.  Up to 256 groups the tile's group
    comes from one round of metadata loads held in registers; 257 and 300 take
    the search over 64 groups at a time."""
    d = grouped_case(fmt, G, E, N, K, rows, seed=G + N + K + fmt)
    assert d["max_rows"] > 16 * G
    check_grouped_run(bsq, fmt, d, G, E, N, K)


def tile_rows(max_rows, G):
    """The library's tile for a grouped GEMM, from the rows per group."""
    return 16 if max_rows <= 4 * G else 32 if max_rows <= 16 * G else 128


@pytest.mark.parametrize("fmt", [MXFP4, MXFP8])
@pytest.mark.parametrize("G,E,N,K,rows,tile", [
    (256, 32, 272, 256, 512, 16), (128, 16, 300, 2048, 400, 16), (100, 12, 96, 1152, 300, 16),
    (128, 8, 128, 512, 500, 16),
    (64, 16, 300, 2048, 400, 32), (40, 8, 96, 512, 300, 32), (100, 12, 512, 1152, 700, 32),
    (16, 4, 128, 7168, 240, 32), (200, 10, 144, 128, 500, 16), (50, 10, 144, 128, 500, 32)])
def test_grouped_mfma_few_rows_matches_oracle(bsq, fmt, G, E, N, K, rows, tile):
    """At most 16 rows per group on average (decode steps): 16-row tiles (at
    most 4 on average) or 32-row tiles, the weights streamed through LDS.
    N = 300, 96, 272 and 144 leave partial column tiles and idle waves;
    K = 1152, 256 and 128 end in a partial round of K steps (K = 128: a single
    step, most of the round's weight loads clamped); groups of up to 22 rows (16-row
    tiles, G = 128 with 500 rows) and up to 38-40 rows (32-row tiles, G = 40
    and 16) take several row tiles."""
    d = grouped_case(fmt, G, E, N, K, rows, seed=G + N + K + fmt + 11)
    assert tile_rows(d["max_rows"], G) == tile
    check_grouped_run(bsq, fmt, d, G, E, N, K)


@pytest.mark.parametrize("fmt", [MXFP4, MXFP8])
@pytest.mark.parametrize("rows,max_rows,tile", [(125, 128, 16), (125, 129, 32), (508, 512, 32),
                                                (508, 513, 128)])
def test_grouped_mfma_tile_choice_at_the_cuts(bsq, fmt, rows, max_rows, tile):
    """The tile follows max_rows / num_groups: exactly 4 rows per group on
    average still takes 16-row tiles and one more row 32-row tiles; exactly 16
    still takes 32-row tiles and one more row the 128-row tiles.  Every choice
    gives the oracle's results within the bound on the same data."""
    G, E, N, K = 32, 8, 160, 640
    d = grouped_case(fmt, G, E, N, K, rows, seed=rows + max_rows + fmt)
    assert int(d["ro"][-1]) == rows <= max_rows <= d["max_rows"]
    assert tile_rows(max_rows, G) == tile
    check_grouped_run(bsq, fmt, d, G, E, N, K, max_rows=max_rows)


def check_grouped_run(bsq, fmt, d, G, E, N, K, ids=None, max_rows=None, skipped=()):
    """Run the grouped GEMM on grouped_case data (optionally with other expert
    ids or a smaller max_rows) into a buffer of 7.0s; every group not in
    `skipped` must match the oracle within the bound, and every other row keep
    7.0."""
    ids = d["ids"] if ids is None else ids
    max_rows = d["max_rows"] if max_rows is None else max_rows
    out = torch.full((max_rows, N), 7.0, dtype=torch.float32, device="cuda")
    bsq.grouped_block_scaled_matmul_mfma(
        dev(d["qa"]), dev(d["la"]), dev(d["ro"].view(np.int32)), dev(d["so"].view(np.int32)),
        dev(ids), max_rows, d["nsr"], dev(d["qb"]), dev(d["lb"]), E, fmt, K, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    owned = np.zeros(max_rows, bool)
    worst = 0.0
    for g in range(G):
        lo, hi, so, e = int(d["ro"][g]), int(d["ro"][g + 1]), int(d["so"][g]), int(ids[g])
        if hi == lo or g in skipped:
            continue
        owned[lo:hi] = True
        qa, sa = d["qa"][lo:hi], d["sa"][so:so + hi - lo]
        qb, sb = d["qb"][e * N:(e + 1) * N], d["sb"][e * N:(e + 1) * N]
        want = oracle.block_scaled_matmul(qa, sa, qb, sb, fmt, K)
        worst = max(worst, gemm_bound.check(got[lo:hi], qa, sa, qb, sb, fmt, K, want))
    assert np.all(got[~owned] == 7.0)              # rows no group owns are not written
    print(f"format {fmt} G={G} N={N} K={K}: worst |err| / bound = {worst:.3f}")


@pytest.mark.parametrize("fmt", [MXFP4, MXFP8])
@pytest.mark.parametrize("rows,tile", [(100, 16), (150, 32)])
def test_grouped_mfma_few_rows_skips_bad_groups(bsq, fmt, rows, tile):
    """The 16- and 32-row kernels skip what the 128-row one skips: a group
    whose scale offset is not a multiple of 16, groups whose expert id is out
    of range either way, and a group running past max_rows."""
    G, E, N, K = 30, 5, 80, 512
    counts = grouped_case(fmt, G, E, N, K, rows, seed=79)["counts"]
    nonempty = [int(g) for g in np.nonzero(counts)[0] if g >= 1]
    mis, bad_hi, bad_lo = nonempty[0], nonempty[1], nonempty[2]
    last = [g for g in nonempty if counts[g] > 1][-1]
    d = grouped_case(fmt, G, E, N, K, rows, seed=79, misaligned=mis)
    ids = d["ids"].copy()
    ids[bad_hi], ids[bad_lo] = E, -1
    max_rows = int(d["ro"][last]) + int(counts[last]) // 2
    assert tile_rows(max_rows, G) == tile
    check_grouped_run(bsq, fmt, d, G, E, N, K, ids=ids, max_rows=max_rows,
                      skipped=(mis, bad_hi, bad_lo, last) + tuple(range(last + 1, G)))


def test_grouped_mfma_skips_a_misaligned_group(bsq):
    fmt, G, E, N, K = MXFP8, 6, 3, 64, 512
    d = grouped_case(fmt, G, E, N, K, 400, seed=77, misaligned=2)
    out = torch.full((d["max_rows"], N), 7.0, dtype=torch.float32, device="cuda")
    bsq.grouped_block_scaled_matmul_mfma(
        dev(d["qa"]), dev(d["la"]), dev(d["ro"].view(np.int32)), dev(d["so"].view(np.int32)),
        dev(d["ids"]), d["max_rows"], d["nsr"], dev(d["qb"]), dev(d["lb"]), E, fmt, K, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    lo, hi = int(d["ro"][2]), int(d["ro"][3])
    assert hi > lo and np.all(got[lo:hi] == 7.0)    # scale offset not a multiple of 16: skipped
    lo1, hi1 = int(d["ro"][1]), int(d["ro"][2])
    assert hi1 == lo1 or np.all(got[lo1:hi1] != 7.0)


def test_grouped_mfma_skips_bad_expert_ids_and_rows_past_max_rows(bsq):
    """Groups whose expert id is out of range, or whose rows run past
    max_rows, are skipped (their rows keep the caller's bytes); every other
    group matches the oracle."""
    fmt, G, E, N, K = MXFP4, 7, 3, 64, 256
    d = grouped_case(fmt, G, E, N, K, 500, seed=78)
    ro, ids = d["ro"], d["ids"].copy()
    ids[1], ids[3] = E, -1                                  # out of range both ways
    counts = np.diff(ro)
    assert counts[1] > 0 and counts[3] > 0 and counts[6] > 1
    max_rows = int(ro[6]) + int(counts[6]) // 2             # group 6 runs past it
    out = torch.full((max_rows, N), 7.0, dtype=torch.float32, device="cuda")
    bsq.grouped_block_scaled_matmul_mfma(
        dev(d["qa"]), dev(d["la"]), dev(ro.view(np.int32)), dev(d["so"].view(np.int32)),
        dev(ids), max_rows, d["nsr"], dev(d["qb"]), dev(d["lb"]), E, fmt, K, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    for g in range(G):
        lo, hi, so = int(ro[g]), int(ro[g + 1]), int(d["so"][g])
        if g in (1, 3, 6):
            assert np.all(got[lo:min(hi, max_rows)] == 7.0), g
            continue
        if hi == lo:
            continue
        e = int(ids[g])
        qa, sa = d["qa"][lo:hi], d["sa"][so:so + hi - lo]
        qb, sb = d["qb"][e * N:(e + 1) * N], d["sb"][e * N:(e + 1) * N]
        want = oracle.block_scaled_matmul(qa, sa, qb, sb, fmt, K)
        gemm_bound.check(got[lo:hi], qa, sa, qb, sb, fmt, K, want)


@pytest.mark.parametrize("fmt", [MXFP4, MXFP8])
@pytest.mark.parametrize("G,rows,pad", [(5, 300, 4), (5, 300, 3), (40, 100, 4), (40, 100, 3)])
def test_grouped_mfma_into_a_wider_output(bsq, fmt, G, rows, pad):
    """c as a view of a wider buffer (ldc = N + pad): 128-row tiles (5 groups,
    300 rows) and 16-row tiles (40 groups, 100 rows); with pad 4 the rows stay
    16-byte aligned and c leaves in 16-byte stores, with pad 3 in 4-byte ones.
    Every owned row matches the oracle within the bound, and the pad columns
    and the rows no group owns keep their 7.0."""
    E, N, K = 3, 100, 512
    d = grouped_case(fmt, G, E, N, K, rows, seed=G + rows + pad + fmt)
    max_rows = d["max_rows"]
    wide = torch.full((max_rows, N + pad), 7.0, dtype=torch.float32, device="cuda")
    out = wide[:, :N]
    bsq.grouped_block_scaled_matmul_mfma(
        dev(d["qa"]), dev(d["la"]), dev(d["ro"].view(np.int32)), dev(d["so"].view(np.int32)),
        dev(d["ids"]), max_rows, d["nsr"], dev(d["qb"]), dev(d["lb"]), E, fmt, K, out=out)
    torch.cuda.synchronize()
    got = wide.cpu().numpy().astype(np.float64)
    assert np.all(got[:, N:] == 7.0)
    owned = np.zeros(max_rows, bool)
    for g in range(G):
        lo, hi, so, e = int(d["ro"][g]), int(d["ro"][g + 1]), int(d["so"][g]), int(d["ids"][g])
        if hi == lo:
            continue
        owned[lo:hi] = True
        qa, sa = d["qa"][lo:hi], d["sa"][so:so + hi - lo]
        qb, sb = d["qb"][e * N:(e + 1) * N], d["sb"][e * N:(e + 1) * N]
        want = oracle.block_scaled_matmul(qa, sa, qb, sb, fmt, K)
        gemm_bound.check(got[lo:hi, :N], qa, sa, qb, sb, fmt, K, want)
    assert np.all(got[~owned, :N] == 7.0)


@pytest.mark.parametrize("rows", [300, 30])
def test_grouped_zero_k_writes_zeros(bsq, rows):
    """K = 0 with 128-row (300 rows over 2 groups) and 32-row tiles: every
    routed row of c is an empty sum, 0; rows no group owns keep 7.0.  No
    operand is read (none is passed)."""
    ro = np.array([0, rows // 3, rows - 5], np.uint32)
    so = np.array([0, -(-(rows // 3) // 16) * 16, 0], np.uint32)
    so[2] = so[1] + -(-(rows - 5 - rows // 3) // 16) * 16
    out = torch.full((rows, 96), 7.0, dtype=torch.float32, device="cuda")
    empty = torch.zeros((rows, 0), dtype=torch.uint8, device="cuda")
    bsq.grouped_block_scaled_matmul_mfma(
        empty, torch.zeros((int(so[2]) // 16, 0), dtype=torch.uint8, device="cuda"),
        dev(ro.view(np.int32)), dev(so.view(np.int32)), dev(np.array([1, 0], np.int32)), rows,
        int(so[2]), torch.zeros((2 * 96, 0), dtype=torch.uint8, device="cuda"),
        torch.zeros((2 * 96 // 16, 0), dtype=torch.uint8, device="cuda"), 2, MXFP4, 0, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[:rows - 5] == 0.0) and np.all(got[rows - 5:] == 7.0)


def test_zero_k_and_empty(bsq):
    z = bsq.block_scaled_matmul_mfma(torch.zeros((5, 0), dtype=torch.uint8, device="cuda"),
                                     torch.zeros((1, 0), dtype=torch.uint8, device="cuda"),
                                     torch.zeros((7, 0), dtype=torch.uint8, device="cuda"),
                                     torch.zeros((1, 0), dtype=torch.uint8, device="cuda"),
                                     MXFP8, 0)
    torch.cuda.synchronize()
    assert z.shape == (5, 7) and torch.all(z == 0)
