"""Pins of the oracle's consumer side: dequantization and the naive
block-scaled GEMM.

The decoder below is written from the format definitions alone -- E2M1 from
its bit fields, E4M3 through torch's float8_e4m3fn view-cast, E8M0 as
2^(b - 127) -- and checked against ``oracle.dequantize`` over every code byte
and every scale byte.  The GEMM is checked against a float64 BLAS matmul of
those independently decoded operands (rounded to fp32, the operands a GEMM
consumes), within the rounding bound of a double summation, and against
closed forms."""
import numpy as np
import pytest

import oracle
from decode_ref import numpy_dequantize, same_f64

MXFP4, MXFP8, NVFP4 = oracle.MXFP4, oracle.MXFP8, oracle.NVFP4


@pytest.mark.parametrize("fmt,tsf", [(MXFP4, 1.0), (MXFP8, 1.0), (NVFP4, 1.0), (NVFP4, 0.0123),
                                     (NVFP4, 2.0 ** -117)])
def test_dequantize_every_code_and_scale_byte(fmt, tsf):
    bs = oracle.BLOCK[fmt]
    width = 256                                      # every code byte once per row
    K = width if fmt == MXFP8 else 2 * width
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], K // bs, axis=1)  # row r: byte r
    got = oracle.dequantize(codes, scales, fmt, K, tsf)
    want = numpy_dequantize(codes, scales, fmt, K, tsf)
    assert same_f64(got, want)


def random_operand(rng, rows, fmt, K, scale_range):
    bs = oracle.BLOCK[fmt]
    width = K if fmt == MXFP8 else K // 2
    codes = rng.integers(0, 256, (rows, width)).astype(np.uint8)
    if fmt == MXFP8:
        codes[(codes & 0x7F) == 0x7F] = 0x38                 # no NaN codes here
    scales = rng.integers(scale_range[0], scale_range[1], (rows, K // bs)).astype(np.uint8)
    return codes, scales


@pytest.mark.parametrize("fmt,tsfs", [(MXFP4, (1.0, 1.0)), (MXFP8, (1.0, 1.0)),
                                      (NVFP4, (0.0123, 3.5)), (NVFP4, (2.0 ** -20, 1.0 / 3))])
def test_matmul_matches_numpy_on_independent_decode(fmt, tsfs):
    rng = np.random.default_rng(fmt * 10 + 3)
    M, N, K = 37, 29, 512
    srange = (110, 145) if fmt != NVFP4 else (0x08, 0x7E)      # NVFP4: normal E4M3 scales
    a_c, a_s = random_operand(rng, M, fmt, K, srange)
    b_c, b_s = random_operand(rng, N, fmt, K, srange)
    if fmt == NVFP4:
        b_s[::3] |= 0x80                                          # negative block scales too
    got = oracle.block_scaled_matmul(a_c, a_s, b_c, b_s, fmt, K, *tsfs)
    A = numpy_dequantize(a_c, a_s, fmt, K, tsfs[0]).astype(np.float32).astype(np.float64)
    B = numpy_dequantize(b_c, b_s, fmt, K, tsfs[1]).astype(np.float32).astype(np.float64)
    want = A @ B.T
    bound = 2 * K * 2.0 ** -53 * (np.abs(A) @ np.abs(B).T) + 1e-300
    assert np.all(np.abs(got - want) <= bound)
    if fmt == NVFP4:   # the fp32 rounding of the operands is part of the definition
        A_exact = numpy_dequantize(a_c, a_s, fmt, K, tsfs[0])
        B_exact = numpy_dequantize(b_c, b_s, fmt, K, tsfs[1])
        assert not (np.array_equal(A_exact, A) and np.array_equal(B_exact, B))


def test_matmul_closed_forms():
    K = 1024
    ones = np.full((4, K), 0x38, np.uint8)                        # E4M3 1.0
    unit = np.full((4, K // 32), 127, np.uint8)                   # E8M0 2^0
    c = oracle.block_scaled_matmul(ones, unit, ones, unit, MXFP8, K)
    assert np.all(c == K)
    neg = ones.copy()
    neg[2] = 0xB8                                                 # -1.0
    c = oracle.block_scaled_matmul(ones, unit, neg, unit, MXFP8, K)
    assert np.all(c[:, 2] == -K) and np.all(np.delete(c, 2, axis=1) == K)
    halves = unit.copy()
    halves[1] = 126                                               # 2^-1 on A's row 1
    c = oracle.block_scaled_matmul(ones, halves, ones, unit, MXFP8, K)
    assert np.all(c[1] == K / 2) and np.all(c[0] == K)
    # NaN scale in A row 3: that row of c is NaN, nothing else
    nan_s = unit.copy()
    nan_s[3, 5] = 0xFF
    c = oracle.block_scaled_matmul(ones, nan_s, ones, unit, MXFP8, K)
    assert np.all(np.isnan(c[3])) and not np.any(np.isnan(c[:3]))
    # NVFP4: 1.0 codes under block scale 1.0 and tensor scales 2 and 0.25 give K/2
    fp4_ones = np.full((3, K // 2), 0x22, np.uint8)               # E2M1 1.0 in both nibbles
    s1 = np.full((3, K // 16), 0x38, np.uint8)                    # E4M3 1.0
    c = oracle.block_scaled_matmul(fp4_ones, s1, fp4_ones, s1, NVFP4, K, 2.0, 0.25)
    assert np.all(c == K / 2)
    # empty sizes
    assert oracle.block_scaled_matmul(ones[:0], unit[:0], ones, unit, MXFP8, K).shape == (0, 4)
