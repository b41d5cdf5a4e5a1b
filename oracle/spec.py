"""Exact executable specification of block-scaled quantization (S1).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  This module pins the
C oracle: it is written independently of ``oracle.c`` and uses a different
method everywhere --

* numbers are exact rationals (``fractions.Fraction``), never floats;
* every format's value set is enumerated from its field definition, and a
  value is encoded by brute-force search for the nearest member of that finite
  set (ties to the even code).  Saturation is then a consequence, not a rule:
  past the largest magnitude the nearest finite member *is* the largest;
* fp32 rounding, where the NVFP4 reading fixes it, is emulated exactly
  (round to nearest even at the fp32 quantum, subnormals, overflow to inf).

What is computed (formats and arguments) follows the Modular
"block_scaled_quantization" module page (three block-scaled formats NVFP4,
MXFP4, MXFP8), "quantize_dynamic_scaled_async_fp4_kernel" (scalar fp32
tensor_sf; SF_VECTOR_SIZE elements per scale) and
"grouped_quantize_dynamic_scaled_fp4_async_kernel" (row_offsets,
scales_offsets, expert_ids, per-expert sf, optional row_indices).  The pages
define no formula; the scale and rounding readings (OCP MX v1.0 for MX;
RNE(amax / 6 / tensor_sf) for NVFP4) and the zero / NaN / Inf rules are the
same readings the C oracle documents.
"""
from fractions import Fraction
from functools import lru_cache

MXFP4, MXFP8, NVFP4 = 0, 1, 2
INF = float("inf")


def pow2(k: int) -> Fraction:
    return Fraction(2) ** k


def floor_log2(a: Fraction) -> int:
    """Largest integer E with 2^E <= a, for rational a > 0 (exact)."""
    assert a > 0
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while pow2(e) > a:
        e -= 1
    while pow2(e + 1) <= a:
        e += 1
    return e


# ---------------------------------------------------------------- formats

def bf16_fields(h: int):
    return h >> 15, (h >> 7) & 0xFF, h & 0x7F


def bf16_is_special(h: int) -> bool:
    return bf16_fields(h)[1] == 0xFF


@lru_cache(maxsize=None)
def bf16_magnitude(h: int) -> Fraction:
    """|value| of a finite BF16 pattern: 8 exponent bits (bias 127), 7 stored
    mantissa bits, exponent field 0 subnormal."""
    _, e, m = bf16_fields(h)
    assert e != 0xFF
    if e == 0:
        return Fraction(m) * pow2(-126 - 7)
    return (1 + Fraction(m, 128)) * pow2(e - 127)


def _minifloat_values(ebits: int, mbits: int, bias: int, ncodes: int):
    """Magnitudes of a sign-magnitude minifloat, indexed by magnitude code."""
    vals = []
    for c in range(ncodes):
        e, m = c >> mbits, c & ((1 << mbits) - 1)
        if e == 0:
            vals.append(Fraction(m, 1 << mbits) * pow2(1 - bias))
        else:
            vals.append((1 + Fraction(m, 1 << mbits)) * pow2(e - bias))
    return tuple(vals)


# E2M1: 2 exponent bits, bias 1, 1 mantissa bit, no Inf/NaN: 8 magnitudes.
E2M1_VALUES = _minifloat_values(2, 1, 1, 8)
# E4M3 (FN): 4 exponent bits, bias 7, 3 mantissa bits; magnitude code 127 is
# NaN and there is no Inf: 127 finite magnitudes.
E4M3_VALUES = _minifloat_values(4, 3, 7, 127)


def e8m0_value(b: int):
    """E8M0 byte: 2^(b - 127); 255 is NaN (returned as None)."""
    return None if b == 255 else pow2(b - 127)


def nearest_code(values, a) -> int:
    """Brute force: the code of the member of ``values`` nearest to a >= 0
    (a may be INF).  Equidistant members: the even code."""
    if a == INF:
        return len(values) - 1
    best, best_d = None, None
    for c, v in enumerate(values):
        d = abs(a - v)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best


@lru_cache(maxsize=1 << 20)
def e2m1_code_of(a) -> int:
    return nearest_code(E2M1_VALUES, a)


@lru_cache(maxsize=1 << 20)
def e4m3_code_of(a) -> int:
    return nearest_code(E4M3_VALUES, a)


def round_fp32(q):
    """Exact value of the IEEE binary32 nearest to rational q (ties to even),
    with subnormals; magnitudes that round past the largest finite value give
    +-INF.  Returns a Fraction or +-INF."""
    if q == 0:
        return Fraction(0)
    neg = q < 0
    a = -q if neg else q
    e = floor_log2(a)
    quantum = pow2(max(e, -126) - 23)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= pow2(128):
        return -INF if neg else INF
    return -r if neg else r


# ---------------------------------------------------------------- blocks

def mx_block(bits, fmt):
    """MX block (OCP MX v1.0 reading): returns (E8M0 scale byte, codes).
    NaN/Inf anywhere -> (0xFF, all-zero codes).  Otherwise
    X = max(floor(log2 amax) - emax, -127) (X = -127 when amax = 0), scale byte
    X + 127, and each code is the nearest element-format value to x * 2^-X,
    signed by the sign bit of x."""
    assert fmt in (MXFP4, MXFP8)
    if any(bf16_is_special(h) for h in bits):
        return 0xFF, [0] * len(bits)
    values = E2M1_VALUES if fmt == MXFP4 else E4M3_VALUES
    emax = floor_log2(values[-1])  # 2 for E2M1 (6 = 1.5 * 2^2), 8 for E4M3 (448 = 1.75 * 2^8)
    sign_bit = 3 if fmt == MXFP4 else 7
    amax = max(bf16_magnitude(h) for h in bits)
    X = -127 if amax == 0 else max(floor_log2(amax) - emax, -127)
    enc = e2m1_code_of if fmt == MXFP4 else e4m3_code_of
    codes = [((h >> 15) << sign_bit) | enc(bf16_magnitude(h) * pow2(-X)) for h in bits]
    return X + 127, codes


def nvfp4_block(bits, tensor_sf):
    """NVFP4 block: returns (E4M3 scale byte, E2M1 codes).
    NaN/Inf anywhere -> (0x7F, zeros).  Otherwise, with exact fp32 rounding
    fl(): t1 = fl(amax / 6), t2 = fl(t1 / tsf), s = nearest E4M3 to t2,
    d = fl(s * tsf), inv = 0 if d == 0 else fl(1 / d), and each code is the
    nearest E2M1 value to |fl(x * inv)|, signed by the sign bit of x."""
    if any(bf16_is_special(h) for h in bits):
        return 0x7F, [0] * len(bits)
    tsf = Fraction(float(tensor_sf))  # exact value of the fp32 tensor scale
    amax = max(bf16_magnitude(h) for h in bits)
    t1 = round_fp32(amax / 6)
    t2 = round_fp32(t1 / tsf)
    s = e4m3_code_of(t2)
    d = round_fp32(E4M3_VALUES[s] * tsf)
    inv = Fraction(0) if d == 0 else round_fp32(1 / d)
    codes = [((h >> 15) << 3) | _nvfp4_element(bf16_magnitude(h), inv) for h in bits]
    return s, codes


@lru_cache(maxsize=1 << 20)
def _nvfp4_element(mag, inv) -> int:
    """Magnitude code of one NVFP4 element: nearest E2M1 value to fl(|x| * inv)."""
    return e2m1_code_of(round_fp32(mag * inv))


def quantize_block(bits, fmt, tensor_sf=1.0):
    if fmt == NVFP4:
        return nvfp4_block(bits, tensor_sf)
    return mx_block(bits, fmt)


def pack_fp4(codes):
    """Two 4-bit codes per byte, lower-indexed element in the low nibble."""
    return [codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(len(codes) // 2)]


def quantize_rows(rows, fmt, bs, tensor_sf=1.0):
    """Dense form over a list of rows of BF16 patterns: (packed code rows,
    scale rows)."""
    qrows, srows = [], []
    for row in rows:
        q, s = [], []
        for j in range(0, len(row), bs):
            sc, codes = quantize_block(row[j:j + bs], fmt, tensor_sf)
            s.append(sc)
            q.extend(codes)
        qrows.append(pack_fp4(q) if fmt != MXFP8 else q)
        srows.append(s)
    return qrows, srows


def group_of(row_offsets, r):
    """The group owning routed row r: the unique g with
    row_offsets[g] <= r < row_offsets[g + 1] (None if no group owns r)."""
    for g in range(len(row_offsets) - 1):
        if row_offsets[g] <= r < row_offsets[g + 1]:
            return g
    return None
