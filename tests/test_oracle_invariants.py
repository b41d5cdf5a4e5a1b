"""Pins of the oracle by properties the mathematics fixes:

* exact round trip of blocks made of representable values (MX and NVFP4);
* idempotence of quantize o dequantize for MX;
* the amax element lands in the top binade of the element format, and on the
  largest code exactly when its scaled value passes the last midpoint;
* dequantization error bounds (half a format ulp, or the saturation bound);
* sign, monotonicity and scale-range invariants;
* the grouped form reduces to the dense form (one group; per-group slices on
  gathered rows), and leaves every byte no group owns untouched.
"""
import numpy as np
import pytest

import oracle
import workloads as W

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])


def unpack(fmt, q):
    if fmt == oracle.MXFP8:
        return q.copy()
    out = np.empty((q.shape[0], q.shape[1] * 2), np.uint8)
    out[:, 0::2] = q & 0xF
    out[:, 1::2] = q >> 4
    return out


def magnitude_code(fmt, c):
    return c & (0x7F if fmt == oracle.MXFP8 else 0x7)


def sign_of_code(fmt, c):
    return (c >> (7 if fmt == oracle.MXFP8 else 3)) & 1


def f64_to_bf16_exact(v):
    """float64 values that are exactly BF16-representable -> uint16 patterns."""
    f = v.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), v)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0)
    return (b >> 16).astype(np.uint16)


# ------------------------------------------------------------------ round trips

@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8], ids=["mxfp4", "mxfp8"])
def test_mx_exact_round_trip(fmt):
    rng = np.random.default_rng(21)
    M, bs = 512, 32
    if fmt == oracle.MXFP4:
        mags = E2M1
        top = np.array([6, 7])                         # 4 and 6: the top binade
        ncodes = 8
    else:
        mags = np.array([oracle.e4m3_decode(c) for c in range(127)])
        top = np.arange(0x78, 0x7F)                    # exponent field 15
        ncodes = 127
    X = rng.integers(-118, 118, M)
    codes = rng.integers(0, ncodes, (M, bs))
    codes[np.arange(M), rng.integers(0, bs, M)] = rng.choice(top, M)
    sign = rng.integers(0, 2, (M, bs))
    vals = np.where(sign == 1, -1.0, 1.0) * mags[codes] * np.exp2(X)[:, None]
    x = f64_to_bf16_exact(vals)
    q, s = oracle.quantize(x, fmt)
    assert np.array_equal(s[:, 0].astype(np.int64), X + 127)
    back = oracle.dequantize(q, s, fmt, bs)
    assert np.array_equal(back, vals)


def test_nvfp4_exact_round_trip():
    """Power-of-two E4M3 block scale s and tensor scale tsf with block amax
    exactly 6 * s * tsf: every step is exact and the codes come back."""
    rng = np.random.default_rng(22)
    M, bs = 512, 16
    k_s = rng.integers(-6, 9, M)                        # s = 2^k, a normal E4M3 value
    k_t = rng.integers(-30, 30, M)
    codes = rng.integers(0, 8, (M, bs))
    codes[np.arange(M), rng.integers(0, bs, M)] = 7     # amax element: 6
    sign = rng.integers(0, 2, (M, bs))
    out_vals, rows_x = [], []
    for r in range(M):
        tsf = float(np.exp2(k_t[r]))
        vals = np.where(sign[r] == 1, -1.0, 1.0) * E2M1[codes[r]] * np.exp2(k_s[r]) * tsf
        x = f64_to_bf16_exact(vals)[None, :]
        q, s = oracle.quantize(x, oracle.NVFP4, tsf)
        assert oracle.e4m3_decode(int(s[0, 0])) == np.exp2(k_s[r])
        back = oracle.dequantize(q, s, oracle.NVFP4, bs, tsf)
        assert np.array_equal(back[0], vals), r
        out_vals.append(back)
        rows_x.append(x)


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8], ids=["mxfp4", "mxfp8"])
def test_mx_quantize_dequantize_idempotent(fmt):
    x = W.random_bf16((256, 1024), seed=23, scale_log2_range=(-60, 60))
    q1, s1 = oracle.quantize(x, fmt)
    y = f64_to_bf16_exact(oracle.dequantize(q1, s1, fmt, 1024))
    q2, s2 = oracle.quantize(y, fmt)
    assert np.array_equal(s1, s2)
    assert np.array_equal(q1, q2)


# ------------------------------------------------------------------ amax invariant

@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8, oracle.NVFP4],
                         ids=["mxfp4", "mxfp8", "nvfp4"])
def test_amax_element_lands_in_top_binade(fmt):
    bs = oracle.BLOCK[fmt]
    x = W.random_bf16((512, 2048), seed=24, scale_log2_range=(-30, 30))
    tsf = float(W.tensor_scale(x)) if fmt == oracle.NVFP4 else 1.0
    q, s = oracle.quantize(x, fmt, tsf)
    c = unpack(fmt, q).reshape(-1, bs)
    mag = np.abs(W.bf16_to_f32(x).astype(np.float64)).reshape(-1, bs)
    arg = mag.argmax(axis=1)
    cmag = magnitude_code(fmt, c)
    amax_code = cmag[np.arange(c.shape[0]), arg]
    assert np.array_equal(amax_code, cmag.max(axis=1))
    sc = s.reshape(-1)
    if fmt == oracle.NVFP4:
        normal = sc >= 8                                 # exponent field >= 1
        assert np.all(amax_code[normal] == 7)
        return
    X = sc.astype(np.int64) - 127
    scaled = mag.max(axis=1) * np.exp2(-X.astype(np.float64))
    if fmt == oracle.MXFP4:
        assert np.all((amax_code & 0x6) == 0x6)          # magnitude 4 or 6
        assert np.array_equal(amax_code == 7, scaled > 5)
    else:
        assert np.all((amax_code & 0x78) == 0x78)        # exponent field 15
        assert np.array_equal(amax_code == 0x7E, scaled >= 432)


# ------------------------------------------------------------------ error bounds

def _e2m1_half_ulp(v):
    return np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))


def _e4m3_half_ulp(v):
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
    return np.exp2(e - 3) / 2


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8], ids=["mxfp4", "mxfp8"])
def test_mx_dequant_error_bound(fmt):
    bs = 32
    x = W.random_bf16((512, 2048), seed=25, scale_log2_range=(-40, 40))
    q, s = oracle.quantize(x, fmt)
    deq = oracle.dequantize(q, s, fmt, 2048)
    xv = W.bf16_to_f32(x).astype(np.float64)
    u = np.repeat(np.exp2(s.astype(np.float64) - 127), bs, axis=1)
    v = np.abs(xv) / u
    err = np.abs(xv - deq)
    top = 6.0 if fmt == oracle.MXFP4 else 448.0
    half = _e2m1_half_ulp(v) if fmt == oracle.MXFP4 else _e4m3_half_ulp(v)
    sat = v > top
    assert np.all(err[~sat] <= half[~sat] * u[~sat])
    assert np.all(err[sat] < (2.0 if fmt == oracle.MXFP4 else 64.0) * u[sat])
    assert np.all(v < (8.0 if fmt == oracle.MXFP4 else 512.0))


def test_nvfp4_dequant_error_bound():
    bs = 16
    x = W.random_bf16((512, 2048), seed=26, scale_log2_range=(-4, 4))
    tsf = float(W.tensor_scale(x))
    q, s = oracle.quantize(x, oracle.NVFP4, tsf)
    deq = oracle.dequantize(q, s, oracle.NVFP4, 2048, tsf)
    xv = W.bf16_to_f32(x).astype(np.float64)
    d = np.repeat(np.array([[oracle.e4m3_decode(int(b)) for b in row] for row in s]) * tsf,
                  bs, axis=1)
    ok = d > 0
    v = np.abs(xv[ok]) / d[ok]
    # half an E2M1 ulp at v, plus the fp32 roundings of d, 1/d and x * inv
    bound = (_e2m1_half_ulp(v) + v * 2.0 ** -21) * d[ok]
    assert np.all(v <= 6.0 * (1 + 2.0 ** -20) + 0.5)    # no saturation with a fitting tsf
    assert np.all(np.abs(xv[ok] - deq[ok]) <= bound)


# ------------------------------------------------------------------ invariants

@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8, oracle.NVFP4],
                         ids=["mxfp4", "mxfp8", "nvfp4"])
def test_sign_monotone_and_scale_range(fmt):
    bs = oracle.BLOCK[fmt]
    x = W.random_bf16((256, 1024), seed=27, scale_log2_range=(-100, 100))
    tsf = 1.0
    q, s = oracle.quantize(x, fmt, tsf)
    c = unpack(fmt, q)
    assert np.array_equal(sign_of_code(fmt, c), (x >> 15).astype(np.uint8))
    mag = np.abs(W.bf16_to_f32(x).astype(np.float64)).reshape(-1, bs)
    cm = magnitude_code(fmt, c).reshape(-1, bs)
    order = np.argsort(mag, axis=1, kind="stable")
    assert np.all(np.diff(np.take_along_axis(cm, order, axis=1).astype(int), axis=1) >= 0)
    if fmt == oracle.MXFP4:
        assert s.max() <= 252
    elif fmt == oracle.MXFP8:
        assert s.max() <= 246


# ------------------------------------------------------------------ grouped form

def _random_grouping(rng, rows, G, pad=128, empty_frac=0.4):
    w = rng.random(G) * (rng.random(G) > empty_frac)
    if w.sum() == 0:
        w[0] = 1
    counts = rng.multinomial(rows, w / w.sum())
    ro, so = W.offsets_from_counts(counts, pad)
    return counts, ro, so


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8, oracle.NVFP4],
                         ids=["mxfp4", "mxfp8", "nvfp4"])
def test_grouped_one_group_equals_dense(fmt):
    x = W.random_bf16((97, 512), seed=28)
    tsf = np.float32(0.0123)
    qd, sd = oracle.quantize(x, fmt, tsf)
    qg, sg = oracle.grouped_quantize(x, fmt, [0, 97], [0, 97], [0], np.array([tsf]), 97, 97)
    assert np.array_equal(qd, qg) and np.array_equal(sd, sg)


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8, oracle.NVFP4],
                         ids=["mxfp4", "mxfp8", "nvfp4"])
@pytest.mark.parametrize("gather", [False, True], ids=["direct", "gather"])
def test_grouped_slices_equal_dense_on_gathered_rows(fmt, gather):
    rng = np.random.default_rng(29)
    S, K, G, E = 40, 256, 33, 50
    rows = 300 if gather else S
    x = W.random_bf16((S, K), seed=30)
    counts, ro, so = _random_grouping(rng, rows, G, pad=8)
    ids = rng.permutation(E)[:G].astype(np.int32)
    sf = (rng.random(E) * 0.05 + 1e-3).astype(np.float32)
    ri = rng.integers(0, S, rows).astype(np.int32) if gather else None
    bs = oracle.BLOCK[fmt]
    qs = np.full((rows + 5, oracle.code_width(fmt, K)), 0xA5, np.uint8)
    ss = np.full((int(so[-1]) + 3, K // bs), 0xA5, np.uint8)
    qg, sg = oracle.grouped_quantize(x, fmt, ro, so, ids, sf if fmt == oracle.NVFP4 else None,
                                     rows + 5, int(so[-1]) + 3, row_indices=ri,
                                     codes=qs, scales=ss)
    touched_q = np.zeros(qg.shape[0], bool)
    touched_s = np.zeros(sg.shape[0], bool)
    # mapping rows to groups with a library binary search (upper bound - 1)
    for r in range(int(ro[0]), int(ro[-1])):
        g = int(np.searchsorted(ro, r, side="right")) - 1
        src = ri[r] if gather else r
        qd, sd = oracle.quantize(x[src:src + 1], fmt, sf[ids[g]] if fmt == oracle.NVFP4 else 1.0)
        srow = int(so[g]) + r - int(ro[g])
        assert np.array_equal(qg[r], qd[0]) and np.array_equal(sg[srow], sd[0]), (r, g)
        touched_q[r] = True
        touched_s[srow] = True
    assert np.all(qg[~touched_q] == 0xA5)
    assert np.all(sg[~touched_s] == 0xA5)
    assert touched_s.sum() == counts.sum()


def test_grouped_validation_catches_bad_metadata():
    x = W.random_bf16((8, 64), seed=31)
    with pytest.raises(ValueError):   # decreasing row offsets
        oracle.grouped_quantize(x, oracle.MXFP4, [0, 5, 3], [0, 8, 16], [0, 1], None, 8, 16)
    with pytest.raises(ValueError):   # scale gap smaller than the group
        oracle.grouped_quantize(x, oracle.MXFP4, [0, 5, 8], [0, 4, 16], [0, 1], None, 8, 16)
    with pytest.raises(ValueError):   # gather index out of range
        oracle.grouped_quantize(x, oracle.MXFP4, [0, 5, 8], [0, 8, 16], [0, 1], None, 8, 16,
                                row_indices=np.array([0, 1, 2, 3, 4, 5, 6, 99], np.int32))
