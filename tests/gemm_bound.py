"""Error bound of the matrix-core GEMMs against the oracle's exact GEMM, from
the arithmetic of gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 (test
infrastructure; the oracle computes the exact result, this module only says
how far a float32 matrix-core result may lie from it).

The kernels issue one instruction per 128-element K step t and accumulate
its result into float32 in ascending K.  Let S_t be the exact sum of the
step's products and P = sum over k of |a_k b_k|.
  * E2M1 (MXFP4): the products and their sums within a step come out as exact
    sums would, so the only roundings are float32 ones: at most two per step
    (the step's sum and the accumulation), each at most 2^-24 of a magnitude
    no larger than P.  Over T = K / 128 steps:
        |c - c_exact| <= (2 T + 1) 2^-24 P  (+ T float32 subnormal units).
  * E4M3 (MXFP8): the instruction sums a step's products at reduced precision,
    measured at up to about 2^-12 of the step's largest product in one-wave
    probes; the bound takes twice that, 2^-11 max_k |a_k b_k| per step, on
    top of the float32 accumulation above.  The largest product of a step is
    bounded by (max |a_k|) (max |b_k|) over the step, which keeps the bound a
    matrix product.
At K = 7168 the E2M1 bound is about 2^-17.2 P, where a single wrong element
moves c by a whole product, typically about P / K = 2^-12.8 P."""
import numpy as np

import oracle

U32 = 2.0 ** -24
FP8_STEP = 2.0 ** -11
SUBNORMAL = 2.0 ** -149


def fp32_operand(codes, scales, fmt, K):
    """The dequantized operand as the GEMM consumes it (float32 values, held
    in float64), NaN rows zeroed (their outputs are compared as NaN)."""
    A = oracle.dequantize(codes, scales, fmt, K).astype(np.float32).astype(np.float64)
    A[np.isnan(A).any(axis=1)] = 0.0
    return A


def bound(qa, sa, qb, sb, fmt, K):
    """Elementwise bound on |c_gpu - c_exact| for c = A B^T over row-major
    scales (float64 [M, N])."""
    A, B = np.abs(fp32_operand(qa, sa, fmt, K)), np.abs(fp32_operand(qb, sb, fmt, K))
    T = max(1, K // 128)
    b = (2 * T + 1) * U32 * (A @ B.T) + T * SUBNORMAL
    if fmt == oracle.MXFP8:
        ma = A.reshape(A.shape[0], T, -1).max(axis=2)
        mb = B.reshape(B.shape[0], T, -1).max(axis=2)
        b += FP8_STEP * (ma @ mb.T)
    return b


def check(got, qa, sa, qb, sb, fmt, K, want=None):
    """Assert that got (the GPU's c) equals the exact GEMM within the bound,
    NaN where the exact result is NaN; return the worst |err| / bound."""
    if want is None:
        want = oracle.block_scaled_matmul_blas(qa, sa, qb, sb, fmt, K)
    got = np.asarray(got, np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    b = bound(qa, sa, qb, sb, fmt, K)
    err = np.abs(got - want)
    ok = ~nan
    worst = float(np.max(err[ok] / b[ok])) if ok.any() else 0.0
    assert np.all(err[ok] <= b[ok]), f"error {worst:.3f} x the bound"
    return worst
