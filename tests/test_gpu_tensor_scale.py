"""GPU parity of the NVFP4 tensor-scale producer and of the device-only
pipeline it enables (tensor scales computed on the GPU feeding the grouped
quantizer with no host round trip), against the CPU oracle, bit for bit."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu
NTHREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module")
def bsq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantization_amd as m
    return m


def dev(a, dt=np.int16):
    return torch.from_numpy(np.ascontiguousarray(a).view(dt)).cuda()


def tame(x):
    """Keep the NaN/Inf/zero/subnormal specials but map +-max-finite BF16 to
    +-1.0: one such element would clamp its whole expert's scale to 2^100
    (covered on its own below), hiding the reduction's other results."""
    x = x.copy()
    x[x == 0x7F7F] = 0x3F80
    x[x == 0xFF7F] = 0xBF80
    return x


def varied(ref, n_nonempty):
    """The reference takes many distinct values, so a misrouted max shows."""
    assert len(np.unique(ref)) >= min(n_nonempty, 8) // 2


def same_bits(gpu_vals, ref_vals):
    g = np.asarray(gpu_vals, np.float32).view(np.uint32)
    r = np.asarray(ref_vals, np.float32).view(np.uint32)
    assert np.array_equal(g, r), [(i, float(np.float32(gpu_vals[i])), float(ref_vals[i]))
                                  for i in np.nonzero(g != r)[0][:5]]


@pytest.mark.parametrize("M,K,span,specials", [(1, 16, (-3, 3), 0.0), (3, 512, (-20, 20), 0.01),
                                               (300, 1056, (-60, 60), 0.002),
                                               (129, 7168, (-4, 4), 0.0)])
def test_dense_matches_oracle(bsq, M, K, span, specials):
    x = tame(W.random_bf16((M, K), seed=M + K, scale_log2_range=span, special_frac=specials))
    out = bsq.tensor_scale_nvfp4(dev(x))
    torch.cuda.synchronize()
    same_bits(out.cpu().numpy(), [oracle.tensor_scale(x)])


def test_dense_full_size_workload(bsq):
    c = W.dense_nvfp4_scaled_rows()
    out = bsq.tensor_scale_nvfp4(dev(c.x))
    torch.cuda.synchronize()
    same_bits(out.cpu().numpy(), [oracle.tensor_scale(c.x)])
    assert out.item() == np.float32(c.tensor_sf)   # the workload's own recipe agrees


def test_dense_special_cases(bsq):
    cases = [np.zeros((4, 64), np.uint16),
             np.array([[0x7FC0, 0xFF80] * 8], np.uint16),          # only NaN / Inf
             np.full((2, 32), 0x7F7F, np.uint16),                     # clamps at 2^100
             np.full((2, 32), 0x0001, np.uint16),                     # clamps at 2^-117
             np.concatenate([np.full((1, 16), 0x7F80, np.uint16),
                             np.full((1, 16), 0x3F80, np.uint16)], 0)]  # Inf row + 1.0 row
    for x in cases:
        out = bsq.tensor_scale_nvfp4(dev(x))
        torch.cuda.synchronize()
        same_bits(out.cpu().numpy(), [oracle.tensor_scale(x)])
    empty = bsq.tensor_scale_nvfp4(torch.zeros((0, 64), dtype=torch.int16, device="cuda"))
    torch.cuda.synchronize()
    assert empty.item() == 1.0


@pytest.mark.parametrize("G,E,gather,rows", [(1, 1, False, 64), (12, 9, True, 300),
                                             (200, 150, False, 900), (600, 40, True, 700)])
def test_grouped_matches_oracle(bsq, G, E, gather, rows):
    rng = np.random.default_rng(G * 7 + E)
    S, K = 1000, 512
    x = tame(W.random_bf16((S, K), seed=G + 3, scale_log2_range=(-12, 12), special_frac=0.001))
    w = rng.random(G) * (rng.random(G) > 0.4)
    w[0] += 1e-3
    counts = rng.multinomial(rows, w / w.sum())
    ro = np.concatenate([[2], 2 + np.cumsum(counts)]).astype(np.uint32)  # first group starts at 2
    ids = rng.integers(0, E, G).astype(np.int32)                          # repeats allowed
    max_rows = int(ro[-1]) + 3
    ri = rng.integers(0, S, max_rows).astype(np.int32) if gather else None
    out = bsq.grouped_tensor_scale_nvfp4(dev(x), dev(ro, np.int32), dev(ids, np.int32), E,
                                         max_rows, row_indices=None if ri is None else dev(ri, np.int32))
    torch.cuda.synchronize()
    ref = oracle.grouped_tensor_scale(x, ro, ids, E, row_indices=ri)
    varied(ref, len(np.unique(ids[np.diff(ro) > 0])))
    same_bits(out.cpu().numpy(), ref)


def routed_case(seed, S, K, G, E, rows, gather, empty_frac=0.4, first=2):
    rng = np.random.default_rng(seed)
    x = tame(W.random_bf16((S, K), seed=seed + 1, scale_log2_range=(-12, 12),
                           special_frac=0.0005))
    w = rng.random(G) * (rng.random(G) > empty_frac)
    w[0] += 1e-3
    counts = rng.multinomial(rows, w / w.sum())
    ro = np.concatenate([[first], first + np.cumsum(counts)]).astype(np.uint32)
    ids = rng.integers(0, E, G).astype(np.int32)
    max_rows = int(ro[-1]) + 5
    ri = rng.integers(0, S, max_rows).astype(np.int32) if gather else None
    return x, ro, ids, max_rows, ri


# Sizes at which every wave of the reduction walks several tiles (its range
# crosses rows and groups, starts mid-row, and flushes on expert changes), and
# with more than 4096 experts, where flushes go straight to device atomics.
@pytest.mark.parametrize("S,K,G,E,rows,gather", [(40000, 512, 600, 9, 39990, False),
                                                 (30000, 512, 2000, 300, 45000, True),
                                                 (5000, 7168, 37, 16, 4990, False),
                                                 (40000, 512, 700, 5000, 39990, False),
                                                 (20000, 1040, 3000, 6000, 26000, True)])
def test_grouped_multi_tile_waves(bsq, S, K, G, E, rows, gather):
    x, ro, ids, max_rows, ri = routed_case(S + G, S, K, G, E, rows, gather)
    out = bsq.grouped_tensor_scale_nvfp4(dev(x), dev(ro, np.int32), dev(ids, np.int32), E,
                                         max_rows, row_indices=None if ri is None else dev(ri, np.int32))
    torch.cuda.synchronize()
    ref = oracle.grouped_tensor_scale(x, ro, ids, E, row_indices=ri)
    varied(ref, len(np.unique(ids[np.diff(ro) > 0])))
    same_bits(out.cpu().numpy(), ref)


@pytest.mark.parametrize("M,K", [(9000, 7168), (5000, 1040), (70000, 512)])
def test_dense_multi_tile_waves(bsq, M, K):
    x = tame(W.random_bf16((M, K), seed=M, scale_log2_range=(-30, 30), special_frac=0.0001))
    out = bsq.tensor_scale_nvfp4(dev(x))
    torch.cuda.synchronize()
    same_bits(out.cpu().numpy(), [oracle.tensor_scale(x)])


def test_grouped_prefill_workload(bsq):
    c = W.grouped_nvfp4_prefill()
    out = bsq.grouped_tensor_scale_nvfp4(dev(c.x), dev(c.row_offsets, np.int32),
                                         dev(c.expert_ids, np.int32), 128, c.max_rows)
    torch.cuda.synchronize()
    ref = oracle.grouped_tensor_scale(c.x, c.row_offsets, c.expert_ids, 128)
    same_bits(out.cpu().numpy(), ref)
    same_bits(ref, c.tensor_sf)                       # the workload's own per-expert recipe


def test_device_pipeline_scale_then_quantize(bsq):
    """Tensor scales computed on the GPU feed the grouped NVFP4 quantizer
    directly; with one group over all rows this is the dense form reading its
    tensor scale from device memory.  Codes and scales match the oracle run
    with the oracle's own tensor scales."""
    x = W.random_bf16((700, 2048), seed=17, scale_log2_range=(-6, 6))
    xd = dev(x)
    tsf = bsq.tensor_scale_nvfp4(xd)
    ro = torch.tensor([0, 700], dtype=torch.int32, device="cuda")
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    q, s = bsq.grouped_quantize_block_scaled(xd, bsq.NVFP4, ro, ro.clone(), ids, tsf, 700, 700)
    torch.cuda.synchronize()
    qh, sh = oracle.quantize(x, oracle.NVFP4, oracle.tensor_scale(x), nthreads=NTHREADS)
    assert np.array_equal(q.cpu().numpy(), qh) and np.array_equal(s.cpu().numpy(), sh)

    c = W.grouped_nvfp4_prefill(rows=4096, K=2048)
    sf = bsq.grouped_tensor_scale_nvfp4(dev(c.x), dev(c.row_offsets, np.int32),
                                        dev(c.expert_ids, np.int32), 128, c.max_rows)
    q, s = bsq.grouped_quantize_block_scaled(dev(c.x), bsq.NVFP4, dev(c.row_offsets, np.int32),
                                             dev(c.scales_offsets, np.int32),
                                             dev(c.expert_ids, np.int32), sf, c.max_rows,
                                             c.num_scale_rows,
                                             scales=torch.full((c.num_scale_rows, 128), 0xA5,
                                                               dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    sf_ref = oracle.grouped_tensor_scale(c.x, c.row_offsets, c.expert_ids, 128)
    sh = np.full((c.num_scale_rows, 128), 0xA5, np.uint8)
    qh, sh = oracle.grouped_quantize(c.x, oracle.NVFP4, c.row_offsets, c.scales_offsets,
                                     c.expert_ids, sf_ref, c.max_rows, c.num_scale_rows,
                                     scales=sh, nthreads=NTHREADS)
    assert np.array_equal(q.cpu().numpy(), qh) and np.array_equal(s.cpu().numpy(), sh)
