"""Exhaustive brute force: the C oracle against the exact spec on every BF16
bit pattern at every element position of a block.

Each sweep matrix is [bs * 65536, bs]: row p * 65536 + h carries pattern h at
position p over a background (zeros, or one anchor element at (p + 1) % bs,
or seeded N(0, 1) values).  The oracle quantizes the whole matrix; the spec
(exact rationals, brute-force nearest search) quantizes each distinct block
once and its result is rotated into place for every position.
"""
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import spec

N = 65536
MX_ANCHORS = {"one": 0x3F80, "2^100": 0x7180, "2^-120": 0x0380, "56=448/8": 0x4260}
NV_TSF = [1.0, 2.0 ** -10, float(np.float32(1.0) / np.float32(2688.0)), 3.0]


def _spec_chunk(args):
    fmt, bs, tsf, anchor, lo, hi = args
    scales = np.empty(hi - lo, np.uint8)
    codes = np.empty((hi - lo, bs), np.uint8)
    for i, h in enumerate(range(lo, hi)):
        blk = [h] + [0] * (bs - 1)
        if anchor is not None and bs > 1:
            blk[1] = anchor
        s, c = spec.quantize_block(blk, fmt, np.float32(tsf))
        scales[i] = s
        codes[i] = c
    return lo, scales, codes


def spec_canonical(fmt, bs, tsf, anchor):
    """Spec result for the canonical layout (pattern at 0, anchor at 1)."""
    scales = np.empty(N, np.uint8)
    codes = np.empty((N, bs), np.uint8)
    step = N // 8
    jobs = [(fmt, bs, tsf, anchor, lo, lo + step) for lo in range(0, N, step)]
    with ProcessPoolExecutor(8) as ex:
        for lo, s, c in ex.map(_spec_chunk, jobs):
            scales[lo:lo + step] = s
            codes[lo:lo + step] = c
    return scales, codes


def unpack(fmt, q, bs):
    if fmt == oracle.MXFP8:
        return q
    out = np.empty((q.shape[0], q.shape[1] * 2), np.uint8)
    out[:, 0::2] = q & 0xF
    out[:, 1::2] = q >> 4
    return out


def check_sweep(fmt, tsf, background, anchor):
    bs = oracle.BLOCK[fmt]
    x = W.sweep_matrix(bs, background, anchor or 0)
    q, s = oracle.quantize(x, fmt, tsf, nthreads=8)
    codes = unpack(fmt, q, bs).reshape(bs, N, bs)
    scales = s.reshape(bs, N)
    ref_s, ref_c = spec_canonical(fmt, bs, tsf, anchor)
    for p in range(bs):
        assert np.array_equal(scales[p], ref_s), (fmt, p)
        want = np.roll(ref_c, p, axis=1)
        bad = np.nonzero((codes[p] != want).any(axis=1))[0]
        assert bad.size == 0, (fmt, p, [hex(int(h)) for h in bad[:8]])


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8], ids=["mxfp4", "mxfp8"])
@pytest.mark.parametrize("anchor", [None] + list(MX_ANCHORS), ids=lambda a: f"bg_{a}")
def test_mx_exhaustive(fmt, anchor):
    check_sweep(fmt, 1.0, "zeros" if anchor is None else "anchor",
                None if anchor is None else MX_ANCHORS[anchor])


@pytest.mark.parametrize("tsf", NV_TSF, ids=["tsf1", "tsf2^-10", "tsf1/2688", "tsf3"])
@pytest.mark.parametrize("anchor", [None, "one", "2^100"], ids=lambda a: f"bg_{a}")
def test_nvfp4_exhaustive(tsf, anchor):
    check_sweep(oracle.NVFP4, tsf, "zeros" if anchor is None else "anchor",
                None if anchor is None else MX_ANCHORS[anchor])


@pytest.mark.parametrize("fmt,tsf", [(oracle.MXFP4, 1.0), (oracle.MXFP8, 1.0),
                                     (oracle.NVFP4, 1.0), (oracle.NVFP4, NV_TSF[2])],
                         ids=["mxfp4", "mxfp8", "nvfp4", "nvfp4_2688"])
def test_normal_background_sampled(fmt, tsf):
    """Seeded N(0, 1) background: every pattern at every position goes through
    the oracle; 2048 sampled rows are checked against the spec."""
    bs = oracle.BLOCK[fmt]
    x = W.sweep_matrix(bs, "normal", seed=11)
    q, s = oracle.quantize(x, fmt, tsf, nthreads=8)
    rows = np.random.default_rng(12).choice(x.shape[0], 2048, replace=False)
    sq, ss = spec.quantize_rows([list(map(int, x[r])) for r in rows], fmt, bs, np.float32(tsf))
    assert np.array_equal(s[rows], np.array(ss, np.uint8))
    assert np.array_equal(q[rows], np.array(sq, np.uint8))


def test_tiny_blocks_all_pairs():
    """Block sizes 1, 2 and 4 over all pairs from a reduced BF16 set (signs,
    zeros, subnormals, binade edges, ties, Inf, NaN): the oracle accepts any
    block size dividing K, and agrees with the spec on each."""
    base = [0x0000, 0x8000, 0x0001, 0x007F, 0x0080, 0x3E80, 0x3F40, 0x3F80, 0x3FA0, 0x3FC0,
            0x3FE0, 0x4020, 0x4060, 0x40A0, 0x40C0, 0x40E0, 0x4100, 0x43E0, 0x43E8, 0x7F7F,
            0x7F80, 0x7FC0, 0xBF80, 0xC0A0, 0xFF80, 0x3D4C, 0x3AAB]
    pairs = np.array([(a, b) for a in base for b in base], np.uint16)
    for fmt in (oracle.MXFP4, oracle.MXFP8, oracle.NVFP4):
        for bs in (1, 2, 4) if fmt == oracle.MXFP8 else (2, 4):
            if bs == 4:
                x = np.concatenate([pairs, pairs[::-1]], axis=1)
            elif bs == 2:
                x = pairs
            else:
                x = pairs.reshape(-1, 1)
            for tsf in ((1.0,) if fmt != oracle.NVFP4 else (1.0, 2.0 ** -10, 0.37)):
                q, s = oracle.quantize(np.ascontiguousarray(x), fmt, tsf, bs=bs)
                sq, ss = spec.quantize_rows([list(map(int, r)) for r in x], fmt, bs,
                                            np.float32(tsf))
                assert np.array_equal(s, np.array(ss, np.uint8)), (fmt, bs, tsf)
                assert np.array_equal(q, np.array(sq, np.uint8)), (fmt, bs, tsf)
