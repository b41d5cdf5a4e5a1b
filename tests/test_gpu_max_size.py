"""Maximum sizes: inputs past 2^31 elements (and past 4 GiB of BF16), where
any 32-bit element or byte offset would wrap.

The input repeats a seeded block of R0 rows (R0 = 4093, prime), row r being
block row r % R0, so the oracle can produce the expected bytes of any row
from the block alone.  A wrapped offset would land mid-row in another period
and read different bytes.  Checked rows include both sides of element 2^31
and the last rows; every check is bit-exact."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu
NTHREADS = max(1, min(16, os.cpu_count() or 1))
MXFP4, MXFP8, NVFP4 = oracle.MXFP4, oracle.MXFP8, oracle.NVFP4
R0, K = 4093, 7168
M = 300_007                                   # M * K = 2 150 450 176 > 2^31
EDGE = (1 << 31) // K                         # the row holding element 2^31


@pytest.fixture(scope="module")
def bsq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantization_amd as m
    return m


@pytest.fixture(scope="module")
def block():
    return W.random_bf16((R0, K), seed=2031, scale_log2_range=(-20, 20), special_frac=0.0005)


@pytest.fixture(scope="module")
def x_big(bsq, block):
    xb = torch.from_numpy(block.view(np.int16)).cuda()
    x = xb.repeat(-(-M // R0), 1)[:M]
    torch.cuda.synchronize()
    yield x
    del x
    torch.cuda.empty_cache()


def sample_rows(seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, R0 - 1, R0, EDGE - 1, EDGE, EDGE + 1, M - 2, M - 1]
    return np.unique(np.concatenate([fixed, rng.integers(0, M, 8)]))


def test_sizes_cross_the_boundary():
    assert M * K > 2**31 and 2 * M * K > 2**32
    assert EDGE * K < 2**31 <= (EDGE + 1) * K
    assert (2**31 % K) != 0                   # element 2^31 falls inside a row


@pytest.mark.parametrize("fmt", [MXFP8, MXFP4])
def test_dense_mx_past_2_31_elements(bsq, block, x_big, fmt):
    q, s = bsq.quantize_block_scaled(x_big, fmt)
    torch.cuda.synchronize()
    qh, sh = oracle.quantize(block, fmt, 1.0, nthreads=NTHREADS)
    rows = sample_rows(fmt)
    idx = torch.from_numpy(rows).cuda()
    assert np.array_equal(q[idx].cpu().numpy(), qh[rows % R0])
    assert np.array_equal(s[idx].cpu().numpy(), sh[rows % R0])
    if fmt == MXFP8:
        out = bsq.dequantize_block_scaled(q, s, fmt, K)
        torch.cuda.synchronize()
        want = oracle.dequantize(qh[rows % R0], sh[rows % R0], fmt, K).astype(np.float32)
        got = out[idx].cpu().numpy()
        del out
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_nvfp4_tensor_scale_and_dense_past_2_31_elements(bsq, block, x_big):
    tsf = bsq.tensor_scale_nvfp4(x_big)
    torch.cuda.synchronize()
    want_tsf = oracle.tensor_scale(block)      # every block row occurs in x
    assert tsf.cpu().numpy().view(np.uint32)[0] == np.float32(want_tsf).view(np.uint32)
    q, s = bsq.quantize_block_scaled(x_big, NVFP4, tensor_sf=float(want_tsf))
    torch.cuda.synchronize()
    qh, sh = oracle.quantize(block, NVFP4, want_tsf, nthreads=NTHREADS)
    rows = sample_rows(7)
    idx = torch.from_numpy(rows).cuda()
    assert np.array_equal(q[idx].cpu().numpy(), qh[rows % R0])
    assert np.array_equal(s[idx].cpu().numpy(), sh[rows % R0])


def test_grouped_nvfp4_gather_past_2_31_elements(bsq, block, x_big):
    """Three groups over all M routed rows (experts 0, 1, 0), each routed row
    gathering a source row far from its own index; per-expert tensor scales
    on the GPU, then the grouped quantizer."""
    ro = np.array([0, 150_000, 290_000, M], np.uint32)
    ids = np.array([0, 1, 0], np.int32)
    ri = ((np.arange(M, dtype=np.int64) * 7919 + 11) % M).astype(np.int32)
    d_ro = torch.from_numpy(ro.view(np.int32)).cuda()
    d_ids = torch.from_numpy(ids).cuda()
    d_ri = torch.from_numpy(ri).cuda()
    tsf = bsq.grouped_tensor_scale_nvfp4(x_big, d_ro, d_ids, 2, M, row_indices=d_ri)
    torch.cuda.synchronize()
    # source row i holds block row i % R0: the oracle sees the same routed values
    # through the block with the reduced indices
    want_tsf = oracle.grouped_tensor_scale(block, ro, ids, 2, row_indices=ri % R0)
    assert np.array_equal(tsf.cpu().numpy().view(np.uint32), want_tsf.view(np.uint32))
    q, s = bsq.grouped_quantize_block_scaled(x_big, NVFP4, d_ro, d_ro.clone(), d_ids, tsf, M, M,
                                             row_indices=d_ri)
    torch.cuda.synchronize()
    rows = sample_rows(11)
    idx = torch.from_numpy(rows).cuda()
    got_q, got_s = q[idx].cpu().numpy(), s[idx].cpu().numpy()
    for i, r in enumerate(rows):
        e = ids[np.searchsorted(ro, r, side="right") - 1]
        src = int(ri[r]) % R0
        qh, sh = oracle.quantize(block[src:src + 1], NVFP4, want_tsf[e])
        assert np.array_equal(got_q[i], qh[0]) and np.array_equal(got_s[i], sh[0]), r
