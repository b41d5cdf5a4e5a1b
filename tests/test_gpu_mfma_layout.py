"""GPU parity of the MFMA 16x16x128 scale layout (MX formats): the
quantizers write their scales straight into it, and dequantization and the
naive GEMM read it.  Expected scales are the oracle's row-major scales put
through the oracle's index map; bytes no scale lands in must keep the
caller's fill."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu
NTHREADS = max(1, min(16, os.cpu_count() or 1))
MXFP4, MXFP8 = oracle.MXFP4, oracle.MXFP8
FILL = 0xEE


@pytest.fixture(scope="module")
def bsq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantization_amd as m
    return m


def dev(a, dt=None):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a if dt is None else a.view(dt)).cuda()


def layout_buffer(bsq, fmt, rows, K, extra=0):
    groups, width = bsq.scale_shape(fmt, rows, K, bsq.SCALES_MFMA16)
    return torch.full((groups, width + extra), FILL, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("fmt", [MXFP4, MXFP8])
@pytest.mark.parametrize("M,K,extra", [(1, 32, 0), (16, 512, 0), (37, 1056, 0), (300, 2048, 64),
                                       (129, 7168, 0), (5, 544, 256),
                                       # over 2^22 elements: tiles of 2 (MXFP8) or 4 (MXFP4)
                                       # chunks, ragged last tile
                                       (1000, 4544, 0), (1003, 4608, 32)])
def test_dense_quantize_writes_the_layout(bsq, fmt, M, K, extra):
    x = W.random_bf16((M, K), seed=M + K + fmt, scale_log2_range=(-30, 30), special_frac=0.002)
    buf = layout_buffer(bsq, fmt, M, K, extra)
    q, s = bsq.quantize_block_scaled(dev(x, np.int16), fmt, scales=buf,
                                     scale_layout=bsq.SCALES_MFMA16)
    torch.cuda.synchronize()
    qh, sh = oracle.quantize(x, fmt, 1.0, nthreads=NTHREADS)
    assert np.array_equal(q.cpu().numpy(), qh)
    want = oracle.scales_to_mfma16(sh, lds_out=buf.shape[1], fill=FILL)
    assert np.array_equal(buf.cpu().numpy(), want)


@pytest.mark.parametrize("fmt", [MXFP4, MXFP8])
@pytest.mark.parametrize("gather,pad16,K", [(False, True, 1024), (True, True, 1024),
                                            (True, False, 1024),
                                            # 350+ routed rows x 12544: over 2^22 elements
                                            # (tiles of 4 chunks), last tile 1 partial chunk
                                            (True, True, 12544), (False, False, 12544)])
def test_grouped_quantize_writes_the_layout(bsq, fmt, gather, pad16, K):
    rng = np.random.default_rng(fmt * 3 + gather + 2 * pad16)
    S, G = 400, 23
    x = W.random_bf16((S, K), seed=S + fmt, scale_log2_range=(-10, 10), special_frac=0.001)
    w = rng.random(G) * (rng.random(G) > 0.3)
    w[0] += 1e-3
    counts = rng.multinomial(350, w / w.sum())
    ro = np.concatenate([[0], np.cumsum(counts)]).astype(np.uint32)
    pad = 16 if pad16 else 1
    so = np.concatenate([[0], np.cumsum(-(-counts // pad) * pad + (0 if pad16 else 3))]).astype(np.uint32)
    nsr = int(so[-1]) + 5
    ids = np.arange(G, dtype=np.int32)
    max_rows = int(ro[-1]) + 4
    ri = rng.integers(0, S, max_rows).astype(np.int32) if gather else None
    buf = layout_buffer(bsq, fmt, nsr, K)
    q, s = bsq.grouped_quantize_block_scaled(
        dev(x, np.int16), fmt, dev(ro, np.int32), dev(so, np.int32), dev(ids), None, max_rows, nsr,
        row_indices=None if ri is None else dev(ri), scales=buf, scale_layout=bsq.SCALES_MFMA16,
        codes=torch.zeros((max_rows, bsq.code_width(fmt, K)), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    sh = np.full((nsr, K // 32), FILL, np.uint8)              # unowned rows keep the fill
    qh, sh = oracle.grouped_quantize(x, fmt, ro, so, ids, None, max_rows, nsr, row_indices=ri,
                                     scales=sh, codes=np.zeros((max_rows, bsq.code_width(fmt, K)),
                                                               np.uint8), nthreads=NTHREADS)
    assert np.array_equal(q.cpu().numpy(), qh)
    want = oracle.scales_to_mfma16(sh, lds_out=buf.shape[1], fill=FILL)
    assert np.array_equal(buf.cpu().numpy(), want)


def test_full_size_mxfp8_layout(bsq):
    c = W.dense_mxfp8_scaled_rows()
    M, K = c.x.shape
    buf = layout_buffer(bsq, MXFP8, M, K)
    bsq.quantize_block_scaled(dev(c.x, np.int16), MXFP8, scales=buf, scale_layout=bsq.SCALES_MFMA16)
    torch.cuda.synchronize()
    _, sh = oracle.quantize(c.x, MXFP8, 1.0, nthreads=NTHREADS)
    assert np.array_equal(buf.cpu().numpy(), oracle.scales_to_mfma16(sh, fill=FILL))


@pytest.mark.parametrize("fmt", [MXFP4, MXFP8])
def test_dequantize_and_naive_matmul_read_the_layout(bsq, fmt):
    K = 1056
    xa = W.random_bf16((45, K), seed=3 + fmt, scale_log2_range=(-8, 8))
    xb = W.random_bf16((19, K), seed=4 + fmt, scale_log2_range=(-8, 8))
    qa, sa = oracle.quantize(xa, fmt, 1.0, nthreads=NTHREADS)
    qb, sb = oracle.quantize(xb, fmt, 1.0, nthreads=NTHREADS)
    la, lb = oracle.scales_to_mfma16(sa), oracle.scales_to_mfma16(sb)
    got = bsq.dequantize_block_scaled(dev(qa), dev(la), fmt, K, scale_layout=bsq.SCALES_MFMA16)
    torch.cuda.synchronize()
    want = oracle.dequantize(qa, sa, fmt, K).astype(np.float32)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))
    c_layout = bsq.block_scaled_matmul_naive(dev(qa), dev(la), dev(qb), dev(lb), fmt, K,
                                             scale_layout=bsq.SCALES_MFMA16)
    c_rows = bsq.block_scaled_matmul_naive(dev(qa), dev(sa), dev(qb), dev(sb), fmt, K)
    torch.cuda.synchronize()
    assert torch.equal(c_layout, c_rows)            # same sums, scales read from either layout
