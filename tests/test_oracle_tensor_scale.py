"""Pins of the oracle's NVFP4 tensor-scale producer (the step before the
quantizer, whose scale the pages take as an input).  Its value reduces to a
library reduction: numpy's max over the finite |x|, one float32 division by
2688 = 6 * 448, and the clamp to the quantizer's domain."""
import numpy as np
import pytest

import oracle
import workloads as W

LO, HI = np.float32(2.0 ** -117), np.float32(2.0 ** 100)


def numpy_tensor_scale(x_bits):
    f = W.bf16_to_f32(x_bits).astype(np.float64)
    f = np.abs(f[np.isfinite(f)])
    amax = f.max() if f.size else 0.0
    if amax == 0:
        return np.float32(1.0)
    return np.clip(np.float32(amax) / np.float32(2688.0), LO, HI)


@pytest.mark.parametrize("seed,span,specials", [(1, (-8, 8), 0.0), (2, (-60, 60), 0.01),
                                                (3, (-4, 4), 0.05)])
def test_dense_tensor_scale_matches_numpy(seed, span, specials):
    x = W.random_bf16((300, 512), seed=seed, scale_log2_range=span, special_frac=specials)
    assert oracle.tensor_scale(x) == numpy_tensor_scale(x)


def test_dense_tensor_scale_special_cases():
    z = np.zeros((4, 64), np.uint16)
    assert oracle.tensor_scale(z) == 1.0                       # all zero
    z[1, 3] = 0x7FC0
    z[2, 5] = 0xFF80
    assert oracle.tensor_scale(z) == 1.0                       # nothing finite and non-zero
    z[3, 7] = 0x40C0                                           # 6.0
    assert oracle.tensor_scale(z) == np.float32(6.0) / np.float32(2688.0)
    big = np.full((1, 16), 0x7F7F, np.uint16)                  # largest BF16: clamps high
    assert oracle.tensor_scale(big) == HI
    tiny = np.full((1, 16), 0x0001, np.uint16)                 # smallest subnormal: clamps low
    assert oracle.tensor_scale(tiny) == LO
    assert oracle.tensor_scale(np.zeros((0, 16), np.uint16)) == 1.0


def test_grouped_tensor_scale_matches_per_expert_numpy():
    rng = np.random.default_rng(8)
    S, K, G, E = 50, 256, 12, 9
    x = W.random_bf16((S, K), seed=9, scale_log2_range=(-10, 10), special_frac=0.01)
    counts = rng.integers(0, 6, G)
    counts[3] = 0
    ro = np.concatenate([[0], np.cumsum(counts)]).astype(np.uint32)
    ids = rng.integers(0, E - 2, G).astype(np.int32)          # experts E-2, E-1 get no rows
    ri = rng.integers(0, S, int(ro[-1])).astype(np.int32)
    out = oracle.grouped_tensor_scale(x, ro, ids, E, row_indices=ri)
    for e in range(E):
        rows = [ri[r] for g in range(G) if ids[g] == e for r in range(ro[g], ro[g + 1])]
        want = numpy_tensor_scale(x[rows]) if rows else np.float32(1.0)
        assert out[e] == want, e
    assert out[E - 1] == 1.0 and out[E - 2] == 1.0
