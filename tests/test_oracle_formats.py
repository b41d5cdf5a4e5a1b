"""Pins of the oracle's format layer against things other than itself.

* Hand-worked examples (tests/golden/hand_examples.json), derived from the
  format definitions before any code existed.
* Library cross-checks: BF16, E4M3 and E8M0 decoding against torch's dtype
  view-casts; E4M3 round-to-nearest-even against torch's float -> float8_e4m3fn
  cast where torch does not saturate (|v| <= 464).
* The exact spec's fp32 emulation against numpy's IEEE float32 arithmetic.
* The C oracle's element encoders against the spec's brute-force search.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import spec

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


def _block_from_fixture(b):
    x = np.zeros((1, b["bs"]), np.uint16)
    for k, v in b["x"].items():
        x[0, int(k)] = int(v, 16)
    return x


# ---------------------------------------------------------------- golden

@pytest.mark.parametrize("v,code,why", GOLDEN["element_points"]["e2m1"])
def test_e2m1_points(v, code, why):
    assert oracle.e2m1_code(v) == code, why
    assert (spec.e2m1_code_of(abs(Fraction(v))) | (8 if math.copysign(1, v) < 0 else 0)) == code


@pytest.mark.parametrize("v,code,why", GOLDEN["element_points"]["e4m3"])
def test_e4m3_points(v, code, why):
    assert oracle.e4m3_code(v) == code, why
    assert (spec.e4m3_code_of(abs(Fraction(v))) | (0x80 if v < 0 else 0)) == code


@pytest.mark.parametrize("b,val", GOLDEN["element_points"]["e8m0"])
def test_e8m0_points(b, val):
    assert oracle.e8m0_decode(b) == val
    assert spec.e8m0_value(b) == Fraction(val)


@pytest.mark.parametrize("case", GOLDEN["blocks"], ids=[b["name"] for b in GOLDEN["blocks"]])
def test_hand_blocks(case):
    x = _block_from_fixture(case)
    fmt, tsf = case["fmt"], case["tsf"]
    q, s = oracle.quantize(x, fmt, tsf)
    assert s[0, 0] == int(case["scale"], 16), case["why"]
    assert q[0].tobytes().hex().upper() == case["codes"], case["why"]
    sq, ss = spec.quantize_rows([list(map(int, x[0]))], fmt, case["bs"], np.float32(tsf))
    assert ss[0][0] == int(case["scale"], 16)
    assert bytes(sq[0]).hex().upper() == case["codes"]


def test_e2m1_table_closed_form():
    # E2M1 magnitudes written out from the field definition (bias 1,
    # subnormal 0.5 * m): 0, 0.5, 1, 1.5, 2, 3, 4, 6
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [oracle.e2m1_decode(c) for c in range(8)] == table
    assert [oracle.e2m1_decode(c | 8) for c in range(8)] == [-t for t in table]
    assert [float(v) for v in spec.E2M1_VALUES] == table


# ---------------------------------------------------------------- library cross-checks

def test_bf16_decode_matches_torch_all_patterns():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).double().numpy()
    ours = np.array([oracle.bf16_decode(int(h)) for h in pats])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))


def test_e4m3_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    ours = np.array([oracle.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))
    spec_vals = [float(v) for v in spec.E4M3_VALUES]
    assert spec_vals == list(ref[:127])


def test_e8m0_decode_matches_torch_all_bytes():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).double().numpy()
    ours = np.array([oracle.e8m0_decode(i) for i in range(256)])
    assert np.isnan(ref[255]) and np.isnan(ours[255])
    assert np.array_equal(ref[:255], ours[:255])


def _e4m3_probe_values():
    """All BF16 magnitudes in [0, 464], the E4M3 midpoints and their fp32
    neighbours: every rounding decision below the saturation threshold."""
    h = np.arange(0, 0x7F80, dtype=np.uint32)
    f = (h << 16).view(np.float32)
    f = f[f <= 464]
    mags = np.array([float(v) for v in spec.E4M3_VALUES], np.float64)
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(0)), mids,
                           np.nextafter(mids, np.float32(1e9))])
    v = np.concatenate([f, near, np.float32([448, 456, 460, 463.99997])])
    return np.concatenate([v, -v]).astype(np.float32)


def test_e4m3_rne_matches_torch_below_saturation():
    v = _e4m3_probe_values()
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([oracle.e4m3_code(float(a)) for a in v], np.uint8)
    bad = np.nonzero(ref != ours)[0]
    assert bad.size == 0, [(float(v[i]), int(ref[i]), int(ours[i])) for i in bad[:10]]


def test_e4m3_saturation_closed_form():
    # above 464 torch's cast gives NaN; the reading saturates to +-448
    for a in [464.0, 464.00003, 479.9, 480.0, 1e6, 3.0e38, float("inf")]:
        assert oracle.e4m3_code(a) == 0x7E
        assert oracle.e4m3_code(-a) == 0xFE


# ---------------------------------------------------------------- spec's exact fp32 emulation

def _f32_frac(x):
    return Fraction(float(np.float32(x)))


def test_spec_round_fp32_matches_numpy_division_and_product():
    rng = np.random.default_rng(7)
    a = (rng.standard_normal(3000) * np.exp2(rng.integers(-140, 120, 3000))).astype(np.float32)
    b = (rng.standard_normal(3000) * np.exp2(rng.integers(-60, 60, 3000))).astype(np.float32)
    with np.errstate(all="ignore"):
        q = a / b
        p = a * b
    for i in range(a.size):
        if b[i] == 0:
            continue
        rq = spec.round_fp32(_f32_frac(a[i]) / _f32_frac(b[i]))
        rp = spec.round_fp32(_f32_frac(a[i]) * _f32_frac(b[i]))
        for r, ref in ((rq, q[i]), (rp, p[i])):
            if np.isinf(ref):
                assert r in (spec.INF, -spec.INF) and (r > 0) == (ref > 0)
            else:
                assert r == Fraction(float(ref)), (a[i], b[i])


def test_spec_round_fp32_subnormal_and_overflow_edges():
    tiny = Fraction(2) ** -149
    assert spec.round_fp32(tiny / 2) == 0                     # tie to even (0)
    assert spec.round_fp32(tiny * Fraction(3, 2)) == 2 * tiny  # tie 1/2 -> even 2
    assert spec.round_fp32(tiny * Fraction(3, 4)) == tiny
    big = Fraction(float(np.finfo(np.float32).max))
    half_ulp = Fraction(2) ** (127 - 24)
    assert spec.round_fp32(big + half_ulp - Fraction(1)) == big
    assert spec.round_fp32(big + half_ulp) == spec.INF        # tie goes to the even 2^128


def test_spec_floor_log2_matches_frexp():
    rng = np.random.default_rng(3)
    for v in np.concatenate([rng.random(500) * np.exp2(rng.integers(-140, 128, 500)),
                             np.exp2(np.arange(-149, 128)).astype(np.float64)]):
        if v == 0:
            continue
        assert spec.floor_log2(Fraction(float(v))) == math.frexp(float(v))[1] - 1


# ---------------------------------------------------------------- C encoders vs brute force

def test_e2m1_encoder_vs_brute_force_dense_grid():
    # every multiple of 1/64 up to 8 (all ties and both sides of each tie)
    for k in range(0, 8 * 64 + 1):
        a = Fraction(k, 64)
        assert oracle.e2m1_code(float(a)) == spec.e2m1_code_of(a), float(a)
        assert oracle.e2m1_code(-float(a)) == 8 | spec.e2m1_code_of(a)


def test_e4m3_encoder_vs_brute_force_all_bf16_magnitudes():
    for h in range(0, 0x7F80, 3):
        a = spec.bf16_magnitude(h)
        assert oracle.e4m3_code(float(a)) == spec.e4m3_code_of(a), hex(h)
