"""CPU oracle for dynamic block-scaled quantization (MXFP4, MXFP8, NVFP4).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the GPU library (``fp8_quantization_amd``) and neither imports the other.

Two independent implementations live here:

* ``liboracle.so`` (``oracle.c``): plain scalar C, the reference the GPU output
  is compared with byte for byte.  Wrapped below with numpy arrays.
* ``spec`` (``spec.py``): exact rational arithmetic (``fractions.Fraction``) and
  brute-force nearest-value search; it pins the C oracle on the CPU.

Formats follow the Modular "block_scaled_quantization" module page (three
formats: NVFP4, MXFP4, MXFP8) and the two kernel pages
("quantize_dynamic_scaled_async_fp4_kernel": scalar fp32 tensor_sf and
SF_VECTOR_SIZE; "grouped_quantize_dynamic_scaled_fp4_async_kernel": offsets,
expert ids, per-expert sf, optional row_indices).  Parity with the pages' own
kernels is unpinned (the pages print no values); the pins are the format
definitions, exhaustive brute force, invariants and error bounds.
"""
import ctypes
import os

import numpy as np

MXFP4, MXFP8, NVFP4 = 0, 1, 2
BLOCK = {MXFP4: 32, MXFP8: 32, NVFP4: 16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.oracle_quantize.argtypes = [i32, i32, p, i64, i64, i64, p, i64, p, i64, ctypes.c_float, i32]
    lib.oracle_quantize.restype = i32
    lib.oracle_grouped_quantize.argtypes = [i32, i32, p, i64, i64, i64, p, p, p, p, p, i64, i64,
                                            p, i64, p, i64, i32]
    lib.oracle_grouped_quantize.restype = i32
    lib.oracle_validate_grouped.argtypes = [p, p, p, p, i64, i64, i64, i64, i64]
    lib.oracle_validate_grouped.restype = i32
    lib.oracle_dequantize.argtypes = [i32, i32, p, i64, i64, i64, p, i64, ctypes.c_float, p]
    lib.oracle_dequantize.restype = i32
    lib.oracle_block_scaled_matmul.argtypes = [i32, i32, p, i64, p, i64, ctypes.c_float,
                                               p, i64, p, i64, ctypes.c_float, i64, i64, i64, p]
    lib.oracle_block_scaled_matmul.restype = i32
    lib.oracle_mfma16_scale_offset.argtypes = [i64, i64, i64]
    lib.oracle_mfma16_scale_offset.restype = i64
    lib.oracle_scales_to_mfma16.argtypes = [p, i64, i64, i64, p, i64]
    lib.oracle_scales_to_mfma16.restype = i32
    lib.oracle_tensor_scale.argtypes = [p, i64, i64, i64]
    lib.oracle_tensor_scale.restype = ctypes.c_float
    lib.oracle_grouped_tensor_scale.argtypes = [p, i64, i64, i64, p, p, p, i64, i64, p]
    lib.oracle_grouped_tensor_scale.restype = i32
    for name in ("oracle_e2m1_code", "oracle_e4m3_code"):
        getattr(lib, name).argtypes = [ctypes.c_double]
        getattr(lib, name).restype = i32
    for name in ("oracle_e2m1_decode", "oracle_e4m3_decode", "oracle_e8m0_decode",
                 "oracle_bf16_decode"):
        getattr(lib, name).argtypes = [i32]
        getattr(lib, name).restype = ctypes.c_double
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _ld(a, unit: int) -> int:
    """Row stride in elements of size ``unit``; a single-row view may report 0."""
    return a.strides[0] // unit if a.shape[0] > 1 else a.shape[1]


def code_width(fmt: int, K: int) -> int:
    """Bytes of packed codes per row: two FP4 codes per byte, one FP8 code per byte."""
    return K if fmt == MXFP8 else K // 2


def quantize(x_bits: np.ndarray, fmt: int, tensor_sf: float = 1.0, bs: int | None = None,
             nthreads: int = 1, codes: np.ndarray | None = None,
             scales: np.ndarray | None = None):
    """Dense form.  ``x_bits``: uint16 [M, K] BF16 bit patterns (row stride may
    exceed K).  Returns (codes uint8 [M, K/2 or K], scales uint8 [M, K/bs]).
    Pre-filled ``codes``/``scales`` may be passed (their bytes outside the
    written area are left alone)."""
    lib = _load()
    bs = BLOCK[fmt] if bs is None else bs
    assert x_bits.dtype == np.uint16 and x_bits.ndim == 2 and x_bits.strides[1] == 2
    M, K = x_bits.shape
    ldx = _ld(x_bits, 2)
    if codes is None:
        codes = np.zeros((M, code_width(fmt, K)), np.uint8)
    if scales is None:
        scales = np.zeros((M, K // bs), np.uint8)
    assert codes.dtype == np.uint8 and codes.strides[1] == 1 and codes.shape[0] >= M
    assert scales.dtype == np.uint8 and scales.strides[1] == 1 and scales.shape[0] >= M
    rc = lib.oracle_quantize(fmt, bs, _ptr(x_bits), M, K, ldx, _ptr(codes), _ld(codes, 1),
                             _ptr(scales), _ld(scales, 1), float(np.float32(tensor_sf)),
                             nthreads)
    if rc != 0:
        raise ValueError("oracle_quantize rejected its arguments")
    return codes, scales


def grouped_quantize(x_bits, fmt, row_offsets, scales_offsets, expert_ids, tensor_sf,
                     max_rows, num_scale_rows, row_indices=None, codes=None, scales=None,
                     bs=None, nthreads=1):
    """Grouped per-expert form.  Returns (codes [max_rows, ...], scales
    [num_scale_rows, K/bs]); rows no group owns keep their prior bytes (zero
    unless pre-filled buffers are passed)."""
    lib = _load()
    bs = BLOCK[fmt] if bs is None else bs
    assert x_bits.dtype == np.uint16 and x_bits.ndim == 2 and x_bits.strides[1] == 2
    S, K = x_bits.shape
    row_offsets = np.ascontiguousarray(row_offsets, np.uint32)
    scales_offsets = np.ascontiguousarray(scales_offsets, np.uint32)
    expert_ids = np.ascontiguousarray(expert_ids, np.int32)
    G = expert_ids.shape[0]
    assert row_offsets.shape[0] == G + 1 and scales_offsets.shape[0] == G + 1
    sf = None if tensor_sf is None else np.ascontiguousarray(tensor_sf, np.float32)
    E = 0 if sf is None else sf.shape[0]
    ri = None if row_indices is None else np.ascontiguousarray(row_indices, np.int32)
    if codes is None:
        codes = np.zeros((max_rows, code_width(fmt, K)), np.uint8)
    if scales is None:
        scales = np.zeros((num_scale_rows, K // bs), np.uint8)
    e_bound = E if sf is not None else 2**31 - 1  # MX formats read no per-expert scale
    bad = lib.oracle_validate_grouped(_ptr(row_offsets), _ptr(scales_offsets), _ptr(expert_ids),
                                      _ptr(ri), G, e_bound, max_rows, num_scale_rows, S)
    if bad:
        raise ValueError(f"grouped preconditions violated (check {bad})")
    rc = lib.oracle_grouped_quantize(fmt, bs, _ptr(x_bits), S, K, _ld(x_bits, 2),
                                     _ptr(ri), _ptr(row_offsets), _ptr(scales_offsets),
                                     _ptr(expert_ids), _ptr(sf), G, E, _ptr(codes),
                                     _ld(codes, 1), _ptr(scales), _ld(scales, 1), nthreads)
    if rc != 0:
        raise ValueError("oracle_grouped_quantize rejected its arguments")
    return codes, scales


def dequantize(codes, scales, fmt, K, tensor_sf=1.0, bs=None):
    """Decode codes and block scales into float64 [M, K] (exact products)."""
    lib = _load()
    bs = BLOCK[fmt] if bs is None else bs
    M = codes.shape[0]
    out = np.empty((M, K), np.float64)
    rc = lib.oracle_dequantize(fmt, bs, _ptr(codes), M, K, _ld(codes, 1), _ptr(scales),
                               _ld(scales, 1), float(np.float32(tensor_sf)), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_dequantize rejected its arguments")
    return out


def block_scaled_matmul(a_codes, a_scales, b_codes, b_scales, fmt, K, a_tsf=1.0, b_tsf=1.0,
                        bs=None):
    """c = A @ B.T in float64 [M, N], A and B the fp32-rounded dequantized
    operands ([M, K] and [N, K], blocks along K), summed in ascending k."""
    lib = _load()
    bs = BLOCK[fmt] if bs is None else bs
    M, N = a_codes.shape[0], b_codes.shape[0]
    c = np.empty((M, N), np.float64)
    rc = lib.oracle_block_scaled_matmul(
        fmt, bs, _ptr(a_codes), _ld(a_codes, 1), _ptr(a_scales), _ld(a_scales, 1),
        float(np.float32(a_tsf)), _ptr(b_codes), _ld(b_codes, 1), _ptr(b_scales),
        _ld(b_scales, 1), float(np.float32(b_tsf)), M, N, K, _ptr(c))
    if rc != 0:
        raise ValueError("oracle_block_scaled_matmul rejected its arguments")
    return c


def block_scaled_matmul_blas(a_codes, a_scales, b_codes, b_scales, fmt, K, a_tsf=1.0, b_tsf=1.0,
                             bs=None):
    """The same c = A @ B.T as ``block_scaled_matmul`` (fp32-rounded
    dequantized operands, products and sums in float64, a NaN anywhere in row
    m of A or row n of B making c[m, n] NaN), with numpy's float64 matrix
    product as the summation step instead of the C loop: the sums are taken
    in another order, so the two agree to within the float64 rounding of K
    additions (about K * 2^-53 of sum |a b|), far below any float32 error.
    For full-size checks, where the C loop would take minutes."""
    A = dequantize(a_codes, a_scales, fmt, K, a_tsf, bs).astype(np.float32).astype(np.float64)
    B = dequantize(b_codes, b_scales, fmt, K, b_tsf, bs).astype(np.float32).astype(np.float64)
    nan_a, nan_b = np.isnan(A).any(axis=1), np.isnan(B).any(axis=1)
    A[nan_a] = 0.0
    B[nan_b] = 0.0
    c = A @ B.T
    c[nan_a, :] = np.nan
    c[:, nan_b] = np.nan
    return c


def mfma16_scale_bytes(rows: int, nblk: int) -> int:
    """Row-group stride (bytes) of the packed MFMA scale layout: 256 bytes per
    16 rows x 512 elements record."""
    return ((nblk + 15) // 16) * 256


def mfma16_scale_offset(r: int, kb: int, lds: int) -> int:
    return _load().oracle_mfma16_scale_offset(r, kb, lds)


def scales_to_mfma16(scales_rm: np.ndarray, lds_out=None, fill=0) -> np.ndarray:
    """Row-major scales [rows, nblk] in the MFMA 16x16x128 layout: uint8
    [ceil(rows / 16), lds_out] (bytes no scale lands in hold ``fill``)."""
    lib = _load()
    rows, nblk = scales_rm.shape
    lds_out = mfma16_scale_bytes(rows, nblk) if lds_out is None else lds_out
    out = np.full(((rows + 15) // 16, lds_out), fill, np.uint8)
    src = np.ascontiguousarray(scales_rm)
    if lib.oracle_scales_to_mfma16(_ptr(src), rows, nblk, nblk, _ptr(out), lds_out) != 0:
        raise ValueError("oracle_scales_to_mfma16 rejected its arguments")
    return out


def tensor_scale(x_bits: np.ndarray) -> np.float32:
    """NVFP4 tensor scale of a BF16 matrix: fl32(amax / 2688) over the finite
    elements, 1.0 when that amax is 0, clamped to [2^-117, 2^100]."""
    lib = _load()
    assert x_bits.dtype == np.uint16 and x_bits.ndim == 2
    assert x_bits.shape[0] == 0 or x_bits.strides[1] == 2
    M, K = x_bits.shape
    return np.float32(lib.oracle_tensor_scale(_ptr(x_bits), M, K, _ld(x_bits, 2) if M else K))


def grouped_tensor_scale(x_bits, row_offsets, expert_ids, num_experts, row_indices=None):
    """Per-expert NVFP4 tensor scales over the routed rows of each expert's
    groups (float32 [num_experts]); experts without rows get 1.0."""
    lib = _load()
    S, K = x_bits.shape
    ro = np.ascontiguousarray(row_offsets, np.uint32)
    ids = np.ascontiguousarray(expert_ids, np.int32)
    ri = None if row_indices is None else np.ascontiguousarray(row_indices, np.int32)
    out = np.empty(num_experts, np.float32)
    rc = lib.oracle_grouped_tensor_scale(_ptr(x_bits), S, K, _ld(x_bits, 2) if S else K, _ptr(ri),
                                         _ptr(ro), _ptr(ids), ids.shape[0], num_experts, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_grouped_tensor_scale rejected its arguments")
    return out


def e2m1_code(v: float) -> int:
    return _load().oracle_e2m1_code(float(v))


def e4m3_code(v: float) -> int:
    return _load().oracle_e4m3_code(float(v))


def e2m1_decode(c: int) -> float:
    return _load().oracle_e2m1_decode(int(c))


def e4m3_decode(c: int) -> float:
    return _load().oracle_e4m3_decode(int(c))


def e8m0_decode(b: int) -> float:
    return _load().oracle_e8m0_decode(int(b))


def bf16_decode(h: int) -> float:
    return _load().oracle_bf16_decode(int(h))
