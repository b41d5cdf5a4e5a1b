"""Host-side checks of the C ABI that need no GPU.

The library loads, exports every function ``include/bsq.h`` declares, and
rejects bad arguments on the host before any HIP call (those paths return
without touching the runtime, so they run on a machine with no GPU).  The
pointers passed here are never dereferenced: every call below fails
validation or is a no-op.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsq.h")
LIB = os.path.join(ROOT, "fp8_quantization_amd", "libbsq.so")

OK, INVALID, UNSUPPORTED = 0, 1, 2
MXFP4, MXFP8, NVFP4 = 0, 1, 2
FAKE = 0x10000  # aligned, never dereferenced


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from fp8_quantization_amd import build

        build.build()
    lib = ctypes.CDLL(LIB)
    i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.quantize_block_scaled.argtypes = [i32, i32, i32, p, i64, i64, i64, p, i64, p, i64,
                                          ctypes.c_float, p]
    lib.grouped_quantize_block_scaled.argtypes = [i32, i32, i32, p, i64, i64, i64, p, p, p, p, p,
                                                  i64, i64, i64, i64, p, i64, p, i64, p]
    lib.tensor_scale_nvfp4.argtypes = [p, i64, i64, i64, p, p]
    lib.grouped_tensor_scale_nvfp4.argtypes = [p, i64, i64, i64, p, p, p, i64, i64, i64, p, p]
    lib.dequantize_block_scaled.argtypes = [i32, i32, i32, p, i64, i64, i64, p, i64,
                                            ctypes.c_float, p, i64, p]
    lib.block_scaled_matmul_naive.argtypes = [i32, i32, i32, p, i64, p, i64, ctypes.c_float, p,
                                              i64, p, i64, ctypes.c_float, i64, i64, i64, p, i64,
                                              p]
    lib.block_scaled_matmul_mfma.argtypes = [i32, i32, i32, p, i64, p, i64, p, i64, p, i64, i64,
                                             i64, i64, p, i64, p]
    lib.bsq_last_error.restype = ctypes.c_char_p
    lib.bsq_version.restype = ctypes.c_char_p
    return lib


def test_header_declares_the_abi():
    assert declared_functions() == sorted(["quantize_block_scaled",
                                           "grouped_quantize_block_scaled", "bsq_last_error",
                                           "bsq_version", "tensor_scale_nvfp4",
                                           "grouped_tensor_scale_nvfp4",
                                           "dequantize_block_scaled",
                                           "block_scaled_matmul_naive",
                                           "block_scaled_matmul_mfma",
                                           "grouped_block_scaled_matmul_mfma",
                                           "bsq_time_next_launch"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.bsq_version().decode().count(".") == 2


def test_ceiling_library_exports_its_header_and_rejects_bad_arguments():
    """libbsq_ceiling.so (the measurement streams) exports what
    include/bsq_ceiling.h declares, and refuses bad arguments before any HIP
    call (return 1), with M = 0 a no-op (0)."""
    header = os.path.join(ROOT, "include", "bsq_ceiling.h")
    assert declared_functions(header) == ["bsq_ceiling_expand", "bsq_ceiling_stream"]
    path = os.path.join(ROOT, "fp8_quantization_amd", "libbsq_ceiling.so")
    if not os.path.exists(path):
        from fp8_quantization_amd import build

        build.build()
    c = ctypes.CDLL(path)
    i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    c.bsq_ceiling_stream.argtypes = [i32, p, i64, i64, p, p, i32, p, p, p]
    c.bsq_ceiling_expand.argtypes = [i32, p, p, i64, i64, p, i32, p, p, p]
    assert c.bsq_ceiling_stream(0, FAKE, 4, 700, FAKE, FAKE, 1, None, None, None) == 1
    assert c.bsq_ceiling_stream(0, FAKE, 4, 512, FAKE, FAKE, 3, None, None, None) == 1
    assert c.bsq_ceiling_stream(3, FAKE, 4, 512, FAKE, FAKE, 1, None, None, None) == 1
    assert c.bsq_ceiling_stream(0, FAKE, 0, 512, FAKE, FAKE, 1, None, None, None) == 0
    assert c.bsq_ceiling_expand(0, FAKE, FAKE, 4, 700, FAKE, 1, None, None, None) == 1
    assert c.bsq_ceiling_expand(1, FAKE, FAKE, 4, 512, FAKE, 8, None, None, None) == 1
    assert c.bsq_ceiling_expand(2, FAKE, FAKE, 4, 512, FAKE + 4, 1, None, None, None) == 1
    assert c.bsq_ceiling_expand(2, FAKE, FAKE, 4, 512, FAKE, 1, FAKE, None, None) == 1
    assert c.bsq_ceiling_expand(2, FAKE, FAKE, 0, 512, FAKE, 1, None, None, None) == 0


def dense(lib, fmt=MXFP4, bs=32, layout=0, x=FAKE, M=4, K=64, ldx=64, codes=FAKE, ldq=None,
          scales=FAKE, lds=None, tsf=1.0):
    if ldq is None:
        ldq = K if fmt == MXFP8 else K // 2
    if lds is None:
        lds = K // bs if bs > 0 else 1
    return lib.quantize_block_scaled(fmt, bs, layout, x, M, K, ldx, codes, ldq, scales, lds, tsf,
                                     None)


@pytest.mark.parametrize("fmt,bs", [(MXFP4, 16), (MXFP8, 16), (NVFP4, 32), (3, 32), (-1, 32),
                                    (MXFP4, 0)])
def test_unsupported_pairs(lib, fmt, bs):
    assert dense(lib, fmt=fmt, bs=bs) == UNSUPPORTED
    assert lib.bsq_last_error()


def test_last_error_is_cleared_by_a_successful_call(lib):
    assert dense(lib, K=48) == INVALID                          # K % 32
    assert b"K=48" in lib.bsq_last_error()
    assert dense(lib, M=0, x=None, codes=None, scales=None) == OK   # no-op, returns BSQ_OK
    assert lib.bsq_last_error() == b""


def test_time_next_launch_needs_both_events_or_neither(lib):
    """Arming takes a start and a stop event; one alone is rejected (and
    disarms), none disarms.  No event is touched on the host."""
    lib.bsq_time_next_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    assert lib.bsq_time_next_launch(FAKE, None) == INVALID
    assert b"both" in lib.bsq_last_error()
    assert lib.bsq_time_next_launch(None, FAKE) == INVALID
    assert lib.bsq_time_next_launch(None, None) == OK
    assert lib.bsq_last_error() == b""
    # armed events are consumed by the next call, even one that fails validation
    assert lib.bsq_time_next_launch(FAKE, FAKE) == OK
    assert dense(lib, K=48) == INVALID
    assert dense(lib, M=0, x=None, codes=None, scales=None) == OK


def test_unsupported_layout(lib):
    assert dense(lib, layout=2) == UNSUPPORTED
    assert b"layout" in lib.bsq_last_error()
    assert dense(lib, fmt=NVFP4, bs=16, layout=1, tsf=0.5) == UNSUPPORTED   # MFMA layout: MX only
    assert b"MX only" in lib.bsq_last_error()


def test_mfma_layout_row_group_stride(lib):
    # K = 1024: two 256-byte records per 16-row group
    assert dense(lib, layout=1, K=1024, ldx=1024, lds=256) == INVALID
    assert b"lds" in lib.bsq_last_error()
    assert dense(lib, layout=1, K=1024, ldx=1024, lds=514) == INVALID    # not a multiple of 4
    assert dense(lib, fmt=MXFP8, layout=1, K=1024, ldx=1024, lds=511) == INVALID


@pytest.mark.parametrize("kw", [
    dict(M=-1), dict(K=-32), dict(K=48, ldx=48),                 # negative, K % bs
    dict(x=None), dict(codes=None), dict(scales=None),           # null pointers
    dict(x=FAKE + 8), dict(ldx=60), dict(ldx=32),                # x alignment, ldx
    dict(codes=FAKE + 2), dict(ldq=30), dict(ldq=34),            # FP4 codes
    dict(lds=1),                                                 # scale row too short
], ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_invalid_dense_args(lib, kw):
    assert dense(lib, **kw) == INVALID
    assert lib.bsq_last_error()


def test_fp8_code_alignment(lib):
    assert dense(lib, fmt=MXFP8, codes=FAKE + 4) == INVALID
    assert dense(lib, fmt=MXFP8, ldq=68) == INVALID


@pytest.mark.parametrize("tsf", [0.0, -1.0, float("inf"), float("nan"), 2.0 ** -118, 2.0 ** 101])
def test_nvfp4_tensor_scale_domain(lib, tsf):
    assert dense(lib, fmt=NVFP4, bs=16, tsf=tsf) == INVALID
    assert b"tensor_sf" in lib.bsq_last_error()


def test_noops_touch_nothing(lib):
    # M == 0 or K == 0 with null pointers: nothing to do, nothing launched
    assert dense(lib, M=0, x=None, codes=None, scales=None) == OK
    assert dense(lib, K=0, ldx=0, x=None, codes=None, scales=None, ldq=0, lds=0) == OK
    assert lib.bsq_last_error() == b""


def grouped(lib, fmt=MXFP4, bs=32, S=8, K=64, ri=None, ro=FAKE, so=FAKE, ids=FAKE, sf=None,
            G=2, E=0, max_rows=8, nsr=8, x=FAKE, codes=FAKE, scales=FAKE):
    ldq = K if fmt == MXFP8 else K // 2
    return lib.grouped_quantize_block_scaled(fmt, bs, 0, x, S, K, K, ri, ro, so, ids, sf, G, E,
                                             max_rows, nsr, codes, ldq, scales, K // bs, None)


def test_grouped_validation(lib):
    assert grouped(lib, G=-1) == INVALID
    assert grouped(lib, max_rows=-1) == INVALID
    assert grouped(lib, ro=None) == INVALID
    assert grouped(lib, so=None) == INVALID
    assert grouped(lib, max_rows=9) == INVALID                 # no gather: max_rows > S
    assert grouped(lib, fmt=NVFP4, bs=16) == INVALID           # NVFP4 without sf / experts
    assert grouped(lib, fmt=NVFP4, bs=16, sf=FAKE, E=0) == INVALID
    assert grouped(lib, fmt=NVFP4, bs=16, sf=FAKE, E=4, ids=None) == INVALID
    assert grouped(lib, max_rows=(1 << 32) + 1, ri=FAKE) == INVALID
    assert grouped(lib, bs=16) == UNSUPPORTED
    assert grouped(lib, G=0, ro=None, so=None) == OK           # no groups: no-op
    assert grouped(lib, max_rows=0) == OK


def test_tensor_scale_validation(lib):
    ts = lambda **kw: lib.tensor_scale_nvfp4(kw.get("x", FAKE), kw.get("M", 4), kw.get("K", 64),
                                             kw.get("ldx", 64), kw.get("out", FAKE), None)
    assert ts(M=-1) == INVALID
    assert ts(K=40, ldx=40) == INVALID                         # K % 16
    assert ts(out=None) == INVALID
    assert ts(out=FAKE + 2) == INVALID
    assert ts(x=None) == INVALID
    assert ts(x=FAKE + 8) == INVALID
    assert ts(ldx=60) == INVALID
    gts = lambda **kw: lib.grouped_tensor_scale_nvfp4(
        kw.get("x", FAKE), kw.get("S", 8), 64, 64, kw.get("ri", None), kw.get("ro", FAKE),
        kw.get("ids", FAKE), kw.get("G", 2), kw.get("E", 4), kw.get("max_rows", 8),
        kw.get("out", FAKE), None)
    assert gts(E=0) == INVALID
    assert gts(G=-1) == INVALID
    assert gts(ro=None) == INVALID
    assert gts(ids=None) == INVALID
    assert gts(max_rows=9) == INVALID                          # no gather: max_rows > S
    assert gts(out=None) == INVALID


def test_dequantize_validation(lib):
    def dq(fmt=MXFP4, bs=32, layout=0, codes=FAKE, M=4, K=64, ldq=None, scales=FAKE, lds=None,
           tsf=1.0, out=FAKE, ldo=64):
        ldq = (K if fmt == MXFP8 else K // 2) if ldq is None else ldq
        lds = K // max(bs, 1) if lds is None else lds
        return lib.dequantize_block_scaled(fmt, bs, layout, codes, M, K, ldq, scales, lds, tsf,
                                           out, ldo, None)
    assert dq(bs=16) == UNSUPPORTED
    assert dq(layout=2) == UNSUPPORTED
    assert dq(fmt=NVFP4, bs=16, layout=1) == UNSUPPORTED
    assert dq(layout=1, lds=255) == INVALID
    assert dq(M=-1) == INVALID
    assert dq(K=48, ldo=48) == INVALID                         # K % 32
    assert dq(codes=None) == INVALID
    assert dq(scales=None) == INVALID
    assert dq(codes=FAKE + 2) == INVALID                       # FP4 codes 4-byte aligned
    assert dq(fmt=MXFP8, codes=FAKE + 4) == INVALID            # FP8 codes 8-byte aligned
    assert dq(ldq=30) == INVALID
    assert dq(lds=1) == INVALID
    assert dq(out=None) == INVALID
    assert dq(out=FAKE + 8) == INVALID                         # 16-byte aligned
    assert dq(ldo=60) == INVALID                               # ldo < K
    assert dq(ldo=66) == INVALID                               # ldo % 4
    assert dq(fmt=NVFP4, bs=16, tsf=0.0) == INVALID
    assert dq(M=0, codes=None, scales=None, out=None) == OK
    assert dq(K=0, ldq=0, lds=0, codes=None, scales=None, out=None) == OK


def test_naive_matmul_validation(lib):
    def mm(fmt=MXFP4, bs=32, M=4, N=3, K=64, a=FAKE, b=FAKE, c=FAKE, ldc=3, ta=1.0, tb=1.0,
           ldq=None):
        ldq = (K if fmt == MXFP8 else K // 2) if ldq is None else ldq
        lds = K // max(bs, 1)
        return lib.block_scaled_matmul_naive(fmt, bs, 0, a, ldq, FAKE, lds, ta, b, ldq, FAKE,
                                             lds, tb, M, N, K, c, ldc, None)
    assert mm(bs=16) == UNSUPPORTED
    assert mm(N=-1) == INVALID
    assert mm(K=40) == INVALID
    assert mm(a=None) == INVALID
    assert mm(b=None) == INVALID
    assert mm(c=None) == INVALID
    assert mm(c=FAKE + 2) == INVALID
    assert mm(ldc=2) == INVALID
    assert mm(ldq=30) == INVALID
    assert mm(fmt=NVFP4, bs=16, ta=float("nan")) == INVALID
    assert mm(fmt=NVFP4, bs=16, tb=2.0 ** 101) == INVALID
    assert mm(M=1 << 20, N=1 << 19) == INVALID                 # M * N > 2^38
    assert mm(M=0, a=None, b=None, c=None) == OK
    assert mm(N=0, a=None, b=None, c=None) == OK


def test_mfma_matmul_validation(lib):
    def mm(fmt=MXFP4, bs=32, layout=1, M=32, N=16, K=512, a=FAKE, b=FAKE, sa=FAKE, c=FAKE, ldc=16,
           ldq=None, lds=256):
        ldq = (K if fmt == MXFP8 else K // 2) if ldq is None else ldq
        return lib.block_scaled_matmul_mfma(fmt, bs, layout, a, ldq, sa, lds, b, ldq, FAKE, lds, M,
                                            N, K, c, ldc, None)
    assert mm(fmt=NVFP4, bs=16) == UNSUPPORTED
    assert mm(layout=0) == UNSUPPORTED
    assert mm(K=96) == INVALID                                  # K % 128
    assert mm(a=FAKE + 8) == INVALID                            # code rows 16-byte aligned
    assert mm(ldq=264) == INVALID                               # ldq % 16 (FP4: >= 256)
    assert mm(sa=FAKE + 4) == INVALID                           # scales 16-byte aligned
    assert mm(lds=260) == INVALID                               # lds % 16
    assert mm(lds=128) == INVALID                               # one record per 512 of K
    assert mm(c=None) == INVALID
    assert mm(ldc=8) == INVALID
    assert mm(M=0, a=None, b=None, c=None) == OK


def test_grouped_mfma_matmul_validation(lib):
    i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    f = lib.grouped_block_scaled_matmul_mfma
    f.argtypes = [i32, i32, i32, p, i64, p, i64, p, p, p, i64, i64, i64, p, i64, p, i64, i64, i64,
                  i64, p, i64, p]

    def gm(fmt=MXFP4, bs=32, layout=1, G=2, max_rows=64, nsr=64, E=2, N=32, K=512, ro=FAKE,
           a=FAKE, c=FAKE, ldc=32, sb=FAKE, ldb_s=256):
        ldq = K if fmt == MXFP8 else K // 2
        return f(fmt, bs, layout, a, ldq, FAKE, 256, ro, FAKE, FAKE, G, max_rows, nsr, FAKE, ldq,
                 sb, ldb_s, E, N, K, c, ldc, None)
    assert gm(fmt=NVFP4, bs=16) == UNSUPPORTED
    assert gm(layout=0) == UNSUPPORTED
    assert gm(E=0) == INVALID
    assert gm(K=96) == INVALID
    assert gm(ro=None) == INVALID
    assert gm(a=FAKE + 8) == INVALID
    assert gm(sb=FAKE + 4) == INVALID                           # scales 16-byte aligned
    assert gm(ldb_s=260) == INVALID                             # lds % 16
    assert gm(c=None) == INVALID
    assert gm(ldc=16) == INVALID
    assert gm(max_rows=(1 << 32) + 1) == INVALID
    assert gm(G=0, ro=None, a=None, c=None) == OK
    assert gm(N=0, ro=None, a=None, c=None) == OK


def test_python_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    """The binding has no CPU fallback: with the library missing, import raises."""
    import importlib.util

    src = os.path.join(ROOT, "fp8_quantization_amd", "__init__.py")
    pkg = tmp_path / "fp8_quantization_amd"
    pkg.mkdir()
    (pkg / "__init__.py").write_text(open(src).read())
    spec = importlib.util.spec_from_file_location("bsq_nolib", pkg / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError):
        spec.loader.exec_module(mod)


def test_oracle_and_product_share_no_code():
    """Neither side imports, includes or links the other."""
    prod = os.path.join(ROOT, "fp8_quantization_amd")
    for dirpath, _, files in os.walk(prod):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                for bad in ("import oracle", "from oracle", "liboracle", "oracle.c", "spec.py"):
                    assert bad not in text, (f, bad)
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c", ".h")):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            for bad in ("import fp8_quantization_amd", "from fp8_quantization_amd", "bsq.h",
                        "libbsq", "bsq_internal"):
                assert bad not in text, (f, bad)


def test_grouped_num_groups_limit(lib):
    """At most 2^28 groups (the search addresses the offsets in 32 bits)."""
    def call(G):
        return lib.grouped_quantize_block_scaled(MXFP4, 32, 0, FAKE, 64, 64, 64, None, FAKE, FAKE,
                                                 FAKE, None, G, 1, 64, 64, FAKE, 32, FAKE, 2, None)
    assert call((1 << 28) + 1) == INVALID
    assert b"2^28" in lib.bsq_last_error()
