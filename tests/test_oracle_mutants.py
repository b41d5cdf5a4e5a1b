"""The pins catch plausible mistakes in the oracle.

Each case below plants one mistake in a copy of ``oracle/oracle.c`` (on the
CPU, in a temporary directory), builds it, and runs the pin battery against
it: the hand-worked blocks and element points, the exact spec on a random
matrix with special values, and the grouped-reduces-to-dense check.  Every
mutant must fail at least one pin; the unmutated source must pass them all.
"""
import ctypes
import json
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads as W
from decode_ref import numpy_dequantize, same_f64
from oracle import build as oracle_build
from oracle import spec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "hand_examples.json")))

# (name, original text, mutated text): each a mistake someone could make
MUTANTS = [
    ("ties_away_from_zero", "return (k % 2 == 0) ? k : k + 1;", "return k + 1;"),
    ("ties_down", "return (k % 2 == 0) ? k : k + 1;", "return k;"),
    ("nibble_order_swapped", "qrow[k / 2] = (uint8_t)((qrow[k / 2] & 0xF0) | tmp[i]);",
     "qrow[k / 2] = (uint8_t)((qrow[k / 2] & 0x0F) | (tmp[i] << 4));"),
    ("mx_exponent_ceil_like", "int X = (amax == 0.0) ? -127 : floor_log2(amax) - emax;",
     "int X = (amax == 0.0) ? -127 : floor_log2(amax) - emax + 1;"),
    ("mx_clamp_at_126", "if (X < -127) X = -127;", "if (X < -126) X = -126;"),
    ("mx_emax_fp8_wrong", "int emax = (fmt == O_MXFP4) ? 2 : 8;", "int emax = (fmt == O_MXFP4) ? 2 : 7;"),
    ("nvfp4_tsf_multiplied", "float t2 = t1 / tsf;", "float t2 = t1 * tsf;"),
    ("nvfp4_divides_by_4", "float t1 = amax_f / 6.0f;", "float t1 = amax_f / 4.0f;"),
    ("nvfp4_d_without_tsf", "float d = (float)E4M3_TAB[s] * tsf;", "float d = (float)E4M3_TAB[s];"),
    ("signed_zero_dropped", "return (uint8_t)((neg ? 8 : 0) | rne_sat_code(E2M1_TAB, 8, fabs(v)));",
     "return (uint8_t)(((neg && v != 0) ? 8 : 0) | rne_sat_code(E2M1_TAB, 8, fabs(v)));"),
    ("e4m3_no_saturation", "if (a >= vals[n - 1]) return n - 1;",
     "if (a > 464.0) return n; if (a >= vals[n - 1]) return n - 1;"),
    ("mx_nan_scale_wrong", "*scale = 0xFF;", "*scale = 0x7F;"),
    ("inf_not_special", "static int bf16_is_special(uint16_t h) { return ((h >> 7) & 0xFF) == 0xFF; }",
     "static int bf16_is_special(uint16_t h) { return ((h >> 7) & 0xFF) == 0xFF && (h & 0x7F); }"),
    ("amax_signed", "else if (bf16_magnitude(x[i]) > amax) amax = bf16_magnitude(x[i]);\n    }\n    if (special) {\n        *scale = 0xFF;",
     "else if (bf16_value(x[i]) > amax) amax = bf16_value(x[i]);\n    }\n    if (special) {\n        *scale = 0xFF;"),
    ("e4m3_subnormal_decode", "if (e == 0) return ldexp((double)m, -9);", "if (e == 0) return ldexp((double)m, -10);"),
    ("e2m1_subnormal_decode", "if (e == 0) return 0.5 * m;", "if (e == 0) return 0.25 * m;"),
    ("grouped_scale_row_unpadded",
     "int64_t srow = (int64_t)scales_offsets[g] + (r - (int64_t)row_offsets[g]);",
     "int64_t srow = r;"),
    ("grouped_sf_by_group", "tsf = sf[e];", "tsf = sf[g];"),
    ("grouped_gather_ignored",
     "int64_t src = row_indices ? (int64_t)row_indices[r] : r;\n        if (src < 0 || src >= num_src_rows) { bad = 1; continue; }",
     "int64_t src = r;\n        if (src < 0 || src >= num_src_rows) { bad = 1; continue; }"),
    # the tensor-scale producer
    ("tsf_divides_by_448", "float t = (float)amax / 2688.0f;", "float t = (float)amax / 448.0f;"),
    ("tsf_keeps_specials", "if (!bf16_is_special(x[k]) && bf16_magnitude(x[k]) > amax)",
     "if (bf16_magnitude(x[k]) > amax)"),
    ("tsf_zero_gives_zero", "if (amax == 0.0) return 1.0f;", "if (amax == 0.0) return 0.0f;"),
    ("tsf_no_high_clamp", "    if (t > ldexpf(1.0f, 100)) t = ldexpf(1.0f, 100);\n", ""),
    ("tsf_low_clamp_wrong", "if (t < ldexpf(1.0f, -117)) t = ldexpf(1.0f, -117);",
     "if (t < ldexpf(1.0f, -126)) t = ldexpf(1.0f, -126);"),
    ("grouped_tsf_by_group", "if (expert_ids[g] != e) continue;", "if (g != e) continue;"),
    # the consumer side: dequantize and the naive GEMM
    ("dequant_nvfp4_scale_sign_dropped", "if (fmt == O_NVFP4 && (sb & 0x80)) sc = -sc;", ""),
    ("dequant_fp4_nibbles_swapped", "c = (k % 2 == 0) ? (b & 0xF) : (b >> 4);",
     "c = (k % 2 == 0) ? (b >> 4) : (b & 0xF);"),
    ("gemm_operands_not_rounded", "for (int64_t i = 0; i < M * K; ++i) A[i] = (double)(float)A[i];",
     ""),
    ("gemm_b_tsf_from_a", "b_codes, N, K, ldb_q, b_scales, ldb_s, b_tsf, B);",
     "b_codes, N, K, ldb_q, b_scales, ldb_s, a_tsf, B);"),
    ("gemm_skips_last_k", "for (int64_t k = 0; k < K; ++k) sum +=",
     "for (int64_t k = 0; k + 1 < K; ++k) sum +="),
    # the MFMA scale layout
    ("mfma_lane_and_byte_swapped",
     "4 * ((r % 16) + 16 * (kb % 4)) + (kb % 16) / 4;",
     "4 * ((r % 16) + 16 * ((kb % 16) / 4)) + kb % 4;"),
    ("mfma_record_stride", "(kb / 16) * 256 +", "(kb / 16) * 128 +"),
    ("grouped_tsf_gather_ignored",
     "int64_t src = row_indices ? (int64_t)row_indices[r] : r;\n                if (src < 0",
     "int64_t src = r;\n                if (src < 0"),
]


LO, HI = np.float32(2.0 ** -117), np.float32(2.0 ** 100)


def numpy_tensor_scale(x_bits):
    """The tensor scale from numpy alone: max over the finite |x|, one fp32
    division by 2688, clamped; 1.0 when that max is 0."""
    f = W.bf16_to_f32(x_bits).astype(np.float64)
    f = np.abs(f[np.isfinite(f)])
    amax = f.max() if f.size else 0.0
    if amax == 0:
        return np.float32(1.0)
    return np.clip(np.float32(amax) / np.float32(2688.0), LO, HI)


def build_variant(tmp_path, text, name):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", *oracle_build.CFLAGS, str(src), "-o", str(lib), "-lm"], check=True)
    return str(lib)


@pytest.fixture(scope="module")
def references():
    """Expected results that do not come from any build of oracle.c."""
    x = W.random_bf16((24, 256), seed=91, scale_log2_range=(-30, 30), special_frac=0.02)
    x[0, :16] = 0x0000
    x[0, 1] = 0x8000                      # a block of signed zeros
    x[1, :32] = np.uint16(0x0003)         # a block of subnormals
    x[2, 40] = 0xFF80                     # -Inf alone in a block
    rows = [list(map(int, r)) for r in x]
    ref = {}
    for fmt, tsfs in ((0, (1.0,)), (1, (1.0,)), (2, (1.0, 0.0123, 2.0 ** -10))):
        for tsf in tsfs:
            q, s = spec.quantize_rows(rows, fmt, oracle.BLOCK[fmt], np.float32(tsf))
            ref[(fmt, tsf)] = (np.array(q, np.uint8), np.array(s, np.uint8))
    return x, ref


def run_battery(lib_path, references):
    """Returns the names of the pins that fail with the library at lib_path."""
    failed = []
    saved = oracle._lib
    oracle._lib = None
    real_path = oracle._LIB_PATH
    oracle._LIB_PATH = lib_path
    try:
        oracle._load()
        # hand-worked blocks and element points
        for b in GOLDEN["blocks"]:
            x = np.zeros((1, b["bs"]), np.uint16)
            for k, v in b["x"].items():
                x[0, int(k)] = int(v, 16)
            q, s = oracle.quantize(x, b["fmt"], b["tsf"])
            if s[0, 0] != int(b["scale"], 16) or q[0].tobytes().hex().upper() != b["codes"]:
                failed.append("hand:" + b["name"])
        for v, code, _ in GOLDEN["element_points"]["e2m1"]:
            if oracle.e2m1_code(v) != code:
                failed.append("e2m1_point")
                break
        for v, code, _ in GOLDEN["element_points"]["e4m3"]:
            if oracle.e4m3_code(v) != code:
                failed.append("e4m3_point")
                break
        if [oracle.e2m1_decode(c) for c in range(8)] != [0, 0.5, 1, 1.5, 2, 3, 4, 6]:
            failed.append("e2m1_table")
        # exact spec on random blocks with specials
        x, ref = references
        for (fmt, tsf), (rq, rs) in ref.items():
            q, s = oracle.quantize(x, fmt, tsf)
            if not (np.array_equal(q, rq) and np.array_equal(s, rs)):
                failed.append(f"spec:{fmt}:{tsf}")
        # grouped reduces to per-row dense runs
        rng = np.random.default_rng(5)
        xs = W.random_bf16((30, 128), seed=6)
        ro = np.array([0, 7, 7, 19, 26], np.uint32)
        so = np.array([0, 8, 8, 24, 32], np.uint32)
        ids = np.array([3, 0, 1, 2], np.int32)
        sf = np.array([0.01, 0.02, 0.005, 0.3], np.float32)
        ri = rng.integers(0, 30, 26).astype(np.int32)
        for fmt in (0, 1, 2):
            qg, sg = oracle.grouped_quantize(xs, fmt, ro, so, ids, sf if fmt == 2 else None, 26,
                                             32, row_indices=ri)
            for r in range(26):
                g = int(np.searchsorted(ro, r, side="right")) - 1
                qd, sd = oracle.quantize(xs[ri[r]:ri[r] + 1], fmt,
                                         sf[ids[g]] if fmt == 2 else 1.0)
                if not (np.array_equal(qg[r], qd[0]) and
                        np.array_equal(sg[so[g] + r - ro[g]], sd[0])):
                    failed.append(f"grouped:{fmt}")
                    break
        # tensor-scale producer against numpy
        with_inf = xs.copy()
        with_inf[3, 5], with_inf[7, 9] = 0x7F80, 0xFFC0   # Inf and NaN among moderate values
        for xt in (x, xs, with_inf, np.zeros((2, 32), np.uint16),
                   np.full((1, 16), 0x7F7F, np.uint16), np.full((1, 16), 0x0001, np.uint16)):
            if oracle.tensor_scale(xt) != numpy_tensor_scale(xt):
                failed.append("tsf:dense")
                break
        sf_e = oracle.grouped_tensor_scale(xs, ro, ids, 5, row_indices=ri)
        for e in range(5):
            rows = [ri[r] for g in range(4) if ids[g] == e for r in range(ro[g], ro[g + 1])]
            want = numpy_tensor_scale(xs[rows]) if rows else np.float32(1.0)
            if sf_e[e] != want:
                failed.append("tsf:grouped")
                break
        # consumer side: dequantize over every code and scale byte; GEMM vs numpy
        for fmt, tsf in ((0, 1.0), (1, 1.0), (2, 0.0123)):
            K = 256 if fmt == 1 else 512
            codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
            scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], K // oracle.BLOCK[fmt], 1)
            if not same_f64(oracle.dequantize(codes, scales, fmt, K, tsf),
                            numpy_dequantize(codes, scales, fmt, K, tsf)):
                failed.append(f"dequant:{fmt}")
        g = np.random.default_rng(17)
        K = 256
        a_c = g.integers(0, 256, (9, K // 2)).astype(np.uint8)
        b_c = g.integers(0, 256, (7, K // 2)).astype(np.uint8)
        a_s = g.integers(0x08, 0x7E, (9, K // 16)).astype(np.uint8)
        b_s = g.integers(0x08, 0x7E, (7, K // 16)).astype(np.uint8)
        got = oracle.block_scaled_matmul(a_c, a_s, b_c, b_s, 2, K, 0.0123, 3.5)
        A = numpy_dequantize(a_c, a_s, 2, K, 0.0123).astype(np.float32).astype(np.float64)
        B = numpy_dequantize(b_c, b_s, 2, K, 3.5).astype(np.float32).astype(np.float64)
        if not np.all(np.abs(got - A @ B.T) <= 2 * K * 2.0 ** -53 * (np.abs(A) @ np.abs(B).T)):
            failed.append("gemm")
        # MFMA scale layout, seen from the lanes: K step T, lane L holds (L % 16, 4T + L // 16)
        sc = g.integers(0, 256, (20, 40)).astype(np.uint8)
        lay = oracle.scales_to_mfma16(sc, fill=0xEE)
        ok = True
        for grp in range(lay.shape[0]):
            for rec in range(lay.shape[1] // 256):
                dw = lay[grp, rec * 256:(rec + 1) * 256].reshape(64, 4)
                for L in range(64):
                    for T in range(4):
                        r, kb = 16 * grp + L % 16, 16 * rec + 4 * T + L // 16
                        want = sc[r, kb] if r < 20 and kb < 40 else 0xEE
                        ok &= bool(dw[L, T] == want)
        if not ok:
            failed.append("mfma_layout")
    finally:
        oracle._lib = saved
        oracle._LIB_PATH = real_path
    return failed


def test_unmutated_source_passes_the_battery(tmp_path, references):
    assert run_battery(build_variant(tmp_path, SRC, "orig"), references) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_every_mutant_is_caught(tmp_path, references, name, old, new):
    assert SRC.count(old) == 1, f"mutation site for {name} not unique in oracle.c"
    failed = run_battery(build_variant(tmp_path, SRC.replace(old, new), name), references)
    assert failed, f"mutant {name} passed every pin"
