"""The matrix-core GEMM tests' error bound is tight enough to catch a single
wrong element: at K = 7168, corrupting one code of A (or one block scale)
moves the oracle's own exact result by more than the bound at every output
the corrupted element reaches.  CPU only."""
import numpy as np
import pytest

import oracle
import workloads as W
from gemm_bound import bound

MXFP4, MXFP8 = oracle.MXFP4, oracle.MXFP8


def operands(fmt, M, N, K, seed):
    xa = W.random_bf16((M, K), seed=seed, scale_log2_range=(-8, 8))
    xb = W.random_bf16((N, K), seed=seed + 1, scale_log2_range=(-8, 8))
    qa, sa = oracle.quantize(xa, fmt, 1.0)
    qb, sb = oracle.quantize(xb, fmt, 1.0)
    return qa, sa, qb, sb


def test_blas_oracle_equals_the_c_oracle():
    rng = np.random.default_rng(3)
    for fmt in (MXFP4, MXFP8):
        qa, sa, qb, sb = operands(fmt, 23, 19, 1024, seed=40 + fmt)
        sa[4, 7] = 0xFF                                  # a NaN block scale: row 4 is NaN
        c = oracle.block_scaled_matmul(qa, sa, qb, sb, fmt, 1024)
        d = oracle.block_scaled_matmul_blas(qa, sa, qb, sb, fmt, 1024)
        assert np.array_equal(np.isnan(c), np.isnan(d)) and np.isnan(c[4]).all()
        A = np.abs(oracle.dequantize(qa, sa, fmt, 1024))
        B = np.abs(oracle.dequantize(qb, sb, fmt, 1024))
        A[np.isnan(A)] = 0
        B[np.isnan(B)] = 0
        ok = ~np.isnan(c)
        assert np.all(np.abs(c - d)[ok] <= (2 * 1024 * 2.0 ** -53 * (A @ B.T))[ok])
    del rng


@pytest.mark.parametrize("k_star", [0, 3000, 7167])
def test_one_wrong_fp4_code_exceeds_the_bound(k_star):
    """Flip the top magnitude bit of one E2M1 code of A (the smallest such
    change is 1.5 units of the block scale): every output whose B element at
    that position is non-zero moves by more than the bound."""
    fmt, M, N, K = MXFP4, 6, 40, 7168
    qa, sa, qb, sb = operands(fmt, M, N, K, seed=11)
    want = oracle.block_scaled_matmul_blas(qa, sa, qb, sb, fmt, K)
    b = bound(qa, sa, qb, sb, fmt, K)
    for m in range(M):
        bad = qa.copy()
        byte, hi = divmod(k_star, 2)
        bad[m, byte] ^= np.uint8(0x40 if hi else 0x04)
        moved = oracle.block_scaled_matmul_blas(bad, sa, qb, sb, fmt, K)
        reach = oracle.dequantize(qb, sb, fmt, K)[:, k_star] != 0
        assert reach.sum() > N // 2
        assert np.all(np.abs(moved[m] - want[m])[reach] > b[m][reach])
        assert np.array_equal(moved[np.arange(M) != m], want[np.arange(M) != m])


def test_one_wrong_block_scale_exceeds_the_bound():
    """A block scale one binade off (a layout or opsel slip) doubles a whole
    block's contribution to its row: outside the bound at nearly every output
    (a block's signed sum of 32 products can nearly cancel at a few), for both
    formats."""
    for fmt in (MXFP4, MXFP8):
        qa, sa, qb, sb = operands(fmt, 4, 64, 7168, seed=21 + fmt)
        want = oracle.block_scaled_matmul_blas(qa, sa, qb, sb, fmt, 7168)
        b = bound(qa, sa, qb, sb, fmt, 7168)
        for kb in (0, 100, 223):
            bad = sa.copy()
            bad[2, kb] += 1
            moved = oracle.block_scaled_matmul_blas(qa, bad, qb, sb, fmt, 7168)
            caught = np.abs(moved[2] - want[2]) > b[2]
            assert caught.mean() >= 0.9, (fmt, kb, caught.mean())


def test_fp4_bound_is_far_below_the_old_one():
    """(2 T + 1) 2^-24 at T = 56 steps is 2^-17.2: about 140 times tighter
    than a flat 2^-10."""
    T = 7168 // 128
    assert (2 * T + 1) * 2.0 ** -24 < 2.0 ** -17
