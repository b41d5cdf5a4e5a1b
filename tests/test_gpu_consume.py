"""GPU parity of the consumer side -- dequantization and the naive
block-scaled GEMM -- against the CPU oracle.

Dequantization is compared bit for bit (fp32 of the oracle's exact values;
NaN where the oracle has NaN).  The GEMM sums fp32 products in fp32, so it is
compared with the oracle's double sums within the bound of that arithmetic:
each of the K products and K - 1 additions rounds once, so
|c_gpu - c| <= gamma_K * sum |a||b| with gamma_K = K u / (1 - K u), u = 2^-24
(plus the oracle's own double rounding, and a few smallest subnormals for
products that underflow)."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu
NTHREADS = max(1, min(16, os.cpu_count() or 1))
MXFP4, MXFP8, NVFP4 = oracle.MXFP4, oracle.MXFP8, oracle.NVFP4


@pytest.fixture(scope="module")
def bsq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantization_amd as m
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def assert_same_f32(gpu, ref64):
    with np.errstate(over="ignore"):   # MX scale bytes near 0xFE overflow fp32 by design
        ref = ref64.astype(np.float32)
    nan_g, nan_r = np.isnan(gpu), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), np.argwhere(nan_g != nan_r)[:5]
    g = np.where(nan_g, 0, gpu).view(np.uint32)
    r = np.where(nan_r, 0, ref).view(np.uint32)
    bad = np.argwhere(g != r)
    assert bad.size == 0, [(tuple(i), gpu[tuple(i)], ref[tuple(i)]) for i in bad[:5]]


def dequant_gpu(bsq, codes, scales, fmt, K, tsf=1.0, ldo=None):
    out = None
    if ldo is not None:
        out = torch.full((codes.shape[0], ldo), 7.0, dtype=torch.float32, device="cuda")[:, :K]
    got = bsq.dequantize_block_scaled(dev(codes) if isinstance(codes, np.ndarray) else codes,
                                      dev(scales) if isinstance(scales, np.ndarray) else scales,
                                      fmt, K, tsf, out=out)
    torch.cuda.synchronize()
    return got.cpu().numpy()


@pytest.mark.parametrize("fmt,tsf", [(MXFP4, 1.0), (MXFP8, 1.0), (NVFP4, 1.0), (NVFP4, 0.0123),
                                     (NVFP4, 2.0 ** -117), (NVFP4, 2.0 ** 100)])
def test_dequantize_every_code_and_scale_byte(bsq, fmt, tsf):
    bs = oracle.BLOCK[fmt]
    K = 256 if fmt == MXFP8 else 512
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], K // bs, axis=1)
    assert_same_f32(dequant_gpu(bsq, codes, scales, fmt, K, tsf),
                    oracle.dequantize(codes, scales, fmt, K, tsf))


@pytest.mark.parametrize("fmt", [MXFP4, MXFP8, NVFP4])
@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (300, 1056), (17, 4128), (64, 7168)])
def test_dequantize_random_bytes_ragged_and_padded(bsq, fmt, M, K):
    if K % oracle.BLOCK[fmt]:
        pytest.skip("K not a multiple of the block")
    rng = np.random.default_rng(M * 7 + K + fmt)
    bs = oracle.BLOCK[fmt]
    width = K if fmt == MXFP8 else K // 2
    codes_full = rng.integers(0, 256, (M, width + 24)).astype(np.uint8)    # padded rows
    scales_full = rng.integers(0, 256, (M, K // bs + 5)).astype(np.uint8)
    codes, scales = codes_full[:, :width], scales_full[:, :K // bs]
    tsf = 0.37 if fmt == NVFP4 else 1.0
    got = bsq.dequantize_block_scaled(dev(codes_full)[:, :width], dev(scales_full)[:, :K // bs],
                                      fmt, K, tsf,
                                      out=torch.full((M, K + 12), 7.0, dtype=torch.float32,
                                                     device="cuda")[:, :K])
    torch.cuda.synchronize()
    assert_same_f32(got.cpu().numpy(), oracle.dequantize(codes, scales, fmt, K, tsf))


def test_dequantize_leaves_padding_alone(bsq):
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (9, 64)).astype(np.uint8)
    scales = rng.integers(100, 150, (9, 4)).astype(np.uint8)
    buf = torch.full((9, 136), 7.0, dtype=torch.float32, device="cuda")
    bsq.dequantize_block_scaled(dev(codes), dev(scales), MXFP4, 128, out=buf[:, :128])
    torch.cuda.synchronize()
    assert torch.all(buf[:, 128:] == 7.0)
    assert_same_f32(buf[:, :128].cpu().numpy(), oracle.dequantize(codes, scales, MXFP4, 128))


@pytest.mark.parametrize("fmt", [MXFP4, MXFP8, NVFP4])
def test_dequantize_quantizer_output(bsq, fmt):
    x = W.random_bf16((200, 2048), seed=31 + fmt, scale_log2_range=(-30, 30), special_frac=0.003)
    tsf = 0.0123 if fmt == NVFP4 else 1.0
    q, s = oracle.quantize(x, fmt, tsf, nthreads=NTHREADS)
    assert_same_f32(dequant_gpu(bsq, q, s, fmt, 2048, tsf), oracle.dequantize(q, s, fmt, 2048, tsf))


def test_dequantize_full_size_mxfp8(bsq):
    """[8192, 7168] MXFP8 codes and scales (random bytes), every element."""
    rng = np.random.default_rng(77)
    codes = rng.integers(0, 256, (8192, 7168)).astype(np.uint8)
    scales = rng.integers(0, 256, (8192, 224)).astype(np.uint8)
    assert_same_f32(dequant_gpu(bsq, codes, scales, MXFP8, 7168),
                    oracle.dequantize(codes, scales, MXFP8, 7168))


def gemm_bound(a_c, a_s, b_c, b_s, fmt, K, ta, tb):
    A = oracle.dequantize(a_c, a_s, fmt, K, ta).astype(np.float32).astype(np.float64)
    B = oracle.dequantize(b_c, b_s, fmt, K, tb).astype(np.float32).astype(np.float64)
    S = np.abs(A) @ np.abs(B).T
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    return gamma * S + 2 * K * 2.0 ** -53 * S + K * 2.0 ** -149


@pytest.mark.parametrize("fmt,tsfs", [(MXFP4, (1.0, 1.0)), (MXFP8, (1.0, 1.0)),
                                      (NVFP4, (0.0123, 0.5)), (NVFP4, (2.0 ** -30, 1.0 / 3))])
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (70, 45, 1056), (33, 130, 2048)])
def test_naive_matmul_matches_oracle(bsq, fmt, tsfs, M, N, K):
    if K % oracle.BLOCK[fmt]:
        pytest.skip("K not a multiple of the block")
    xa = W.random_bf16((M, K), seed=M + K + fmt, scale_log2_range=(-10, 10))
    xb = W.random_bf16((N, K), seed=N + K + fmt + 1, scale_log2_range=(-10, 10))
    qa, sa = oracle.quantize(xa, fmt, tsfs[0], nthreads=NTHREADS)
    qb, sb = oracle.quantize(xb, fmt, tsfs[1], nthreads=NTHREADS)
    got = bsq.block_scaled_matmul_naive(dev(qa), dev(sa), dev(qb), dev(sb), fmt, K, *tsfs)
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)
    want = oracle.block_scaled_matmul(qa, sa, qb, sb, fmt, K, *tsfs)
    bound = gemm_bound(qa, sa, qb, sb, fmt, K, *tsfs)
    assert np.all(np.abs(got - want) <= bound), np.max(np.abs(got - want) / bound)


def test_naive_matmul_nan_and_empty(bsq):
    rng = np.random.default_rng(3)
    K = 256
    a_c = rng.integers(0, 256, (5, K)).astype(np.uint8)
    a_c[(a_c & 0x7F) == 0x7F] = 0x38
    b_c = a_c[::-1].copy()
    a_s = rng.integers(115, 140, (5, K // 32)).astype(np.uint8)
    b_s = a_s.copy()
    a_s[2, 3] = 0xFF                              # NaN scale: row 2 of c is NaN
    b_c[4, 10] = 0x7F                             # NaN code: column 4 of c is NaN
    got = bsq.block_scaled_matmul_naive(dev(a_c), dev(a_s), dev(b_c), dev(b_s), MXFP8, K)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    want = oracle.block_scaled_matmul(a_c, a_s, b_c, b_s, MXFP8, K)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.isnan(got[2]).all() and np.isnan(got[:, 4]).all() and not np.isnan(got[0, 0])
    z = bsq.block_scaled_matmul_naive(dev(a_c[:, :0]), dev(a_s[:, :0]), dev(b_c[:, :0]),
                                      dev(b_s[:, :0]), MXFP8, 0)
    torch.cuda.synchronize()
    assert torch.all(z == 0)


# End-to-end: BF16 -> quantize (GPU) -> naive GEMM (GPU), against the exact
# GEMM of the BF16 inputs.  The relative Frobenius error is the format's
# quantization error seen through a GEMM (about 4% MXFP8, 13-14% NVFP4,
# 15-17% MXFP4 on these inputs); the GPU pipeline must reproduce the CPU
# oracle pipeline's error, and stay under loose ceilings.
@pytest.mark.parametrize("fmt,ceiling", [(MXFP8, 0.06), (NVFP4, 0.17), (MXFP4, 0.20)])
def test_end_to_end_error_metric(bsq, fmt, ceiling):
    A = W.random_bf16((128, 2048), seed=1, scale_log2_range=(-4, 4))
    B = W.random_bf16((96, 2048), seed=11, scale_log2_range=(-4, 4))
    ref = W.bf16_to_f32(A).astype(np.float64) @ W.bf16_to_f32(B).astype(np.float64).T
    ta = float(oracle.tensor_scale(A)) if fmt == NVFP4 else 1.0
    tb = float(oracle.tensor_scale(B)) if fmt == NVFP4 else 1.0
    qa, sa = bsq.quantize_block_scaled(dev(A.view(np.int16)), fmt, ta)
    qb, sb = bsq.quantize_block_scaled(dev(B.view(np.int16)), fmt, tb)
    c = bsq.block_scaled_matmul_naive(qa, sa, qb, sb, fmt, 2048, ta, tb)
    torch.cuda.synchronize()
    err_gpu = np.linalg.norm(c.cpu().numpy() - ref) / np.linalg.norm(ref)
    qa_h, sa_h = oracle.quantize(A, fmt, ta, nthreads=NTHREADS)
    qb_h, sb_h = oracle.quantize(B, fmt, tb, nthreads=NTHREADS)
    c_h = oracle.block_scaled_matmul(qa_h, sa_h, qb_h, sb_h, fmt, 2048, ta, tb)
    err_cpu = np.linalg.norm(c_h - ref) / np.linalg.norm(ref)
    print(f"format {fmt}: relative GEMM error {err_gpu:.4f} (oracle pipeline {err_cpu:.4f})")
    assert abs(err_gpu - err_cpu) <= 1e-5 * err_cpu
    assert err_gpu < ceiling
