"""Python binding of libbsq: block-scaled quantization of BF16 activations to
MXFP4, MXFP8 and NVFP4 on AMD Instinct MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libbsq.so``; torch provides device memory (``torch.empty``),
pointers (``data_ptr``) and the current stream.  There is no CPU fallback:
if the library is not built, importing this package raises ``ImportError``.

The functions carry the names of the C ABI's entry points (``include/bsq.h``);
the quantizers are the MI355X counterparts of the launchers on the Modular
"block_scaled_quantization" module page, and the grouped arguments follow the
"grouped_quantize_dynamic_scaled_fp4_async_kernel" page (uint32 row_offsets
and scales_offsets, int32 expert_ids, fp32 per-expert scale, optional int32
row_indices).

The C ABI receives pointers and strides only, so the sizes of the tensors
behind them are checked here: every tensor a call reads or writes must hold
the window the kernels touch, or the call raises before anything runs
(``BsqError`` with BSQ_ERR_INVALID_ARG for a size, ``TypeError`` for a dtype,
device or layout).
"""
import ctypes
import os

import torch

MXFP4, MXFP8, NVFP4 = 0, 1, 2
BLOCK_SIZE = {MXFP4: 32, MXFP8: 32, NVFP4: 16}
SCALES_ROW_MAJOR, SCALES_MFMA16 = 0, 1
FORMAT_NAMES = {"mxfp4": MXFP4, "mxfp8": MXFP8, "nvfp4": NVFP4}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run fp8_quantization_amd/build.py "
                      "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)
_i64, _i32, _p, _f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float
_lib.quantize_block_scaled.argtypes = [_i32, _i32, _i32, _p, _i64, _i64, _i64, _p, _i64, _p, _i64,
                                       _f32, _p]
_lib.quantize_block_scaled.restype = _i32
_lib.grouped_quantize_block_scaled.argtypes = [_i32, _i32, _i32, _p, _i64, _i64, _i64, _p, _p, _p,
                                               _p, _p, _i64, _i64, _i64, _i64, _p, _i64, _p, _i64,
                                               _p]
_lib.grouped_quantize_block_scaled.restype = _i32
_lib.tensor_scale_nvfp4.argtypes = [_p, _i64, _i64, _i64, _p, _p]
_lib.tensor_scale_nvfp4.restype = _i32
_lib.grouped_tensor_scale_nvfp4.argtypes = [_p, _i64, _i64, _i64, _p, _p, _p, _i64, _i64, _i64, _p,
                                            _p]
_lib.grouped_tensor_scale_nvfp4.restype = _i32
_lib.dequantize_block_scaled.argtypes = [_i32, _i32, _i32, _p, _i64, _i64, _i64, _p, _i64, _f32,
                                         _p, _i64, _p]
_lib.dequantize_block_scaled.restype = _i32
_lib.block_scaled_matmul_naive.argtypes = [_i32, _i32, _i32, _p, _i64, _p, _i64, _f32, _p, _i64,
                                           _p, _i64, _f32, _i64, _i64, _i64, _p, _i64, _p]
_lib.block_scaled_matmul_naive.restype = _i32
_lib.block_scaled_matmul_mfma.argtypes = [_i32, _i32, _i32, _p, _i64, _p, _i64, _p, _i64, _p,
                                          _i64, _i64, _i64, _i64, _p, _i64, _p]
_lib.block_scaled_matmul_mfma.restype = _i32
_lib.grouped_block_scaled_matmul_mfma.argtypes = [_i32, _i32, _i32, _p, _i64, _p, _i64, _p, _p,
                                                  _p, _i64, _i64, _i64, _p, _i64, _p, _i64, _i64,
                                                  _i64, _i64, _p, _i64, _p]
_lib.grouped_block_scaled_matmul_mfma.restype = _i32
_lib.bsq_time_next_launch.argtypes = [_p, _p]
_lib.bsq_time_next_launch.restype = _i32
_lib.bsq_last_error.argtypes = []
_lib.bsq_last_error.restype = ctypes.c_char_p
_lib.bsq_version.argtypes = []
_lib.bsq_version.restype = ctypes.c_char_p

STATUS = {0: "BSQ_OK", 1: "BSQ_ERR_INVALID_ARG", 2: "BSQ_ERR_UNSUPPORTED", 3: "BSQ_ERR_HIP"}


class BsqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded ``libbsq.so`` (for callers that want the raw C ABI)."""
    return _lib


def version() -> str:
    return _lib.bsq_version().decode()


def time_next_launch(start, stop):
    """Arm this thread's next library call to launch its main kernel with the
    events ``start`` / ``stop`` (``torch.cuda.Event(enable_timing=True)``,
    already recorded once so that they exist) bound to the kernel's own
    dispatch: ``start.elapsed_time(stop)`` is then that kernel's execution
    time.  ``None, None`` disarms."""
    def handle(e):
        if e is None:
            return None
        if not e.cuda_event:
            raise ValueError("record the event once before arming it (torch creates it lazily)")
        return ctypes.c_void_p(e.cuda_event)
    _check(_lib.bsq_time_next_launch(handle(start), handle(stop)))


def _check(status: int):
    if status != 0:
        raise BsqError(status, _lib.bsq_last_error().decode())


def _fmt(fmt) -> int:
    return FORMAT_NAMES[fmt.lower()] if isinstance(fmt, str) else int(fmt)


def code_width(fmt, K: int) -> int:
    """Bytes of codes per row: K/2 (FP4, two per byte) or K (FP8)."""
    return K if _fmt(fmt) == MXFP8 else K // 2


def scale_shape(fmt, rows: int, K: int, scale_layout: int = SCALES_ROW_MAJOR):
    """Shape of a uint8 scales buffer for rows x K: [rows, K/block_size]
    row-major, or [ceil(rows/16), 256 * ceil(K/512)] in the MFMA layout (one
    256-byte record per 16 rows x 512 elements)."""
    f = _fmt(fmt)
    nblk = K // BLOCK_SIZE[f] if f in BLOCK_SIZE else 0
    if scale_layout == SCALES_MFMA16:
        return ((rows + 15) // 16, ((nblk + 15) // 16) * 256)
    return (rows, nblk)


def _stream_ptr(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ld(t: torch.Tensor) -> int:
    return t.stride(0) if t.dim() == 2 and t.shape[0] > 1 else t.shape[-1]


def _need(name, t, dtype, rows, cols):
    """A 2-D GPU tensor of ``dtype`` with unit column stride holding at least
    rows x cols (the window the kernels read or write)."""
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.dim() != 2 or not t.is_cuda \
            or (t.shape[1] > 1 and t.stride(1) != 1):
        raise TypeError(f"{name} must be a 2-D row-major {dtype} GPU tensor")
    if t.shape[0] < rows or t.shape[1] < cols:
        raise BsqError(1, f"{name} is {tuple(t.shape)}; it must be at least [{rows}, {cols}]")
    return t


def _need_vec(name, t, dtypes, n):
    """A contiguous 1-D GPU tensor of one of ``dtypes`` with at least n entries."""
    if not isinstance(t, torch.Tensor) or t.dtype not in dtypes or not t.is_cuda or \
            not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous GPU tensor of dtype {dtypes}")
    if t.numel() < n:
        raise BsqError(1, f"{name} has {t.numel()} entries; it needs at least {n}")
    return t


_OFFSETS = (torch.uint32, torch.int32)


def _as_bf16_matrix(x: torch.Tensor) -> torch.Tensor:
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"x must hold BF16 values (bfloat16/int16/uint16), got {x.dtype}")
    if x.dim() != 2 or x.stride(1) != 1:
        raise TypeError("x must be a 2-D row-major tensor with unit column stride")
    if not x.is_cuda:
        raise TypeError("x must be a GPU tensor")
    return x


def quantize_block_scaled(x: torch.Tensor, fmt, tensor_sf: float = 1.0, codes=None, scales=None,
                          stream=None, scale_layout: int = SCALES_ROW_MAJOR):
    """Dense form.  x: BF16 [M, K] on the GPU.  Returns (codes, scales):
    uint8 [M, K/2] (FP4) or [M, K] (FP8), and the scales in ``scale_layout``
    (``scale_shape``).  ``tensor_sf`` is the fp32 NVFP4 tensor scale (ignored
    for MX).  Output tensors may be passed in (any row stride the C ABI
    accepts)."""
    f = _fmt(fmt)
    x = _as_bf16_matrix(x)
    M, K = x.shape
    bs = BLOCK_SIZE.get(f, 0)
    if codes is None:
        codes = torch.empty((M, code_width(f, K) if bs else 0), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(scale_shape(f, M, K, scale_layout) if bs else (M, 0),
                             dtype=torch.uint8, device=x.device)
    if bs:
        _need("codes", codes, torch.uint8, M, code_width(f, K))
        _need("scales", scales, torch.uint8, *scale_shape(f, M, K, scale_layout))
    _check(_lib.quantize_block_scaled(f, bs, scale_layout, _ptr(x), M, K, _ld(x), _ptr(codes),
                                      _ld(codes), _ptr(scales), _ld(scales),
                                      float(tensor_sf), _stream_ptr(stream, x.device)))
    return codes, scales


def grouped_quantize_block_scaled(x: torch.Tensor, fmt, row_offsets: torch.Tensor,
                                  scales_offsets: torch.Tensor, expert_ids: torch.Tensor,
                                  tensor_sf: torch.Tensor | None, max_rows: int,
                                  num_scale_rows: int, row_indices: torch.Tensor | None = None,
                                  codes=None, scales=None, stream=None,
                                  scale_layout: int = SCALES_ROW_MAJOR):
    """Grouped per-expert form.  x: BF16 [num_src_rows, K]; row_offsets /
    scales_offsets: uint32 (or int32 bit-identical) [G+1]; expert_ids int32
    [G]; tensor_sf fp32 [num_experts] (NVFP4) or None; row_indices int32
    [max_rows] or None.  Returns (codes [max_rows, ...], scales
    [num_scale_rows, K/bs]); bytes no group owns are left as they were (new
    outputs are uninitialised there)."""
    f = _fmt(fmt)
    x = _as_bf16_matrix(x)
    S, K = x.shape
    bs = BLOCK_SIZE.get(f, 0)
    _need_vec("expert_ids", expert_ids, (torch.int32,), 0)
    G = expert_ids.shape[0]
    for name, t in (("row_offsets", row_offsets), ("scales_offsets", scales_offsets)):
        _need_vec(name, t, _OFFSETS, G + 1)
        if t.shape[0] != G + 1:
            raise ValueError("row_offsets and scales_offsets must have num_groups + 1 entries")
    E = 0
    if tensor_sf is not None:
        E = _need_vec("tensor_sf", tensor_sf, (torch.float32,), 0).shape[0]
    if row_indices is not None:
        _need_vec("row_indices", row_indices, (torch.int32,), max_rows)
    if codes is None:
        codes = torch.empty((max_rows, code_width(f, K) if bs else 0), dtype=torch.uint8,
                            device=x.device)
    if scales is None:
        scales = torch.empty(scale_shape(f, num_scale_rows, K, scale_layout) if bs else
                             (num_scale_rows, 0), dtype=torch.uint8, device=x.device)
    if bs:
        _need("codes", codes, torch.uint8, max_rows, code_width(f, K))
        _need("scales", scales, torch.uint8, *scale_shape(f, num_scale_rows, K, scale_layout))
    _check(_lib.grouped_quantize_block_scaled(
        f, bs, scale_layout, _ptr(x), S, K, _ld(x), _ptr(row_indices), _ptr(row_offsets),
        _ptr(scales_offsets), _ptr(expert_ids), _ptr(tensor_sf), G, E, max_rows, num_scale_rows,
        _ptr(codes), _ld(codes), _ptr(scales), _ld(scales), _stream_ptr(stream, x.device)))
    return codes, scales


def tensor_scale_nvfp4(x: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """NVFP4 tensor scale of a BF16 matrix on the GPU: fl32(amax / 2688) over
    the finite elements (1.0 when amax is 0), clamped to [2^-117, 2^100].
    Returns a float32 [1] GPU tensor (``out`` if given)."""
    x = _as_bf16_matrix(x)
    M, K = x.shape
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    _need_vec("out", out, (torch.float32,), 1)
    _check(_lib.tensor_scale_nvfp4(_ptr(x), M, K, _ld(x), _ptr(out),
                                   _stream_ptr(stream, x.device)))
    return out


def grouped_tensor_scale_nvfp4(x: torch.Tensor, row_offsets: torch.Tensor,
                               expert_ids: torch.Tensor, num_experts: int, max_rows: int,
                               row_indices: torch.Tensor | None = None,
                               out: torch.Tensor | None = None, stream=None):
    """Per-expert NVFP4 tensor scales over each expert's routed rows (float32
    [num_experts] GPU tensor; experts without rows get 1.0).  The result can be
    passed as ``tensor_sf`` to ``grouped_quantize_block_scaled``."""
    x = _as_bf16_matrix(x)
    S, K = x.shape
    G = _need_vec("expert_ids", expert_ids, (torch.int32,), 0).shape[0]
    if _need_vec("row_offsets", row_offsets, _OFFSETS, G + 1).shape[0] != G + 1:
        raise ValueError("row_offsets must have num_groups + 1 entries")
    if row_indices is not None:
        _need_vec("row_indices", row_indices, (torch.int32,), max_rows)
    if out is None:
        out = torch.empty(num_experts, dtype=torch.float32, device=x.device)
    _need_vec("out", out, (torch.float32,), num_experts)
    _check(_lib.grouped_tensor_scale_nvfp4(
        _ptr(x), S, K, _ld(x), _ptr(row_indices), _ptr(row_offsets), _ptr(expert_ids), G,
        num_experts, max_rows, _ptr(out), _stream_ptr(stream, x.device)))
    return out


def _as_code_matrix(name, t):
    if t.dtype != torch.uint8 or t.dim() != 2 or t.stride(1) != 1 or not t.is_cuda:
        raise TypeError(f"{name} must be a 2-D row-major uint8 GPU tensor")
    return t


def dequantize_block_scaled(codes: torch.Tensor, scales: torch.Tensor, fmt, K: int,
                            tensor_sf: float = 1.0, out=None, stream=None,
                            scale_layout: int = SCALES_ROW_MAJOR):
    """fp32 [M, K] values of a quantizer's codes ([M, K/2] FP4 or [M, K] FP8)
    and block scales ([M, K/block_size]); NVFP4 values include tensor_sf."""
    f = _fmt(fmt)
    codes, scales = _as_code_matrix("codes", codes), _as_code_matrix("scales", scales)
    M = codes.shape[0]
    if f in BLOCK_SIZE:
        _need("codes", codes, torch.uint8, M, code_width(f, K))
        _need("scales", scales, torch.uint8, *scale_shape(f, M, K, scale_layout))
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=codes.device)
    _need("out", out, torch.float32, M, K)
    _check(_lib.dequantize_block_scaled(f, BLOCK_SIZE.get(f, 0), scale_layout, _ptr(codes), M,
                                        K, _ld(codes), _ptr(scales), _ld(scales), float(tensor_sf),
                                        _ptr(out), _ld(out), _stream_ptr(stream, codes.device)))
    return out


def _check_operands(f, K, scale_layout, *operands):
    """Each GEMM operand (codes, scales, rows, name prefix) holds rows x K codes
    and the scales of those rows in ``scale_layout``."""
    if f not in BLOCK_SIZE:
        return
    for codes, scales, rows, pre in operands:
        _need(pre + "codes", codes, torch.uint8, rows, code_width(f, K))
        _need(pre + "scales", scales, torch.uint8, *scale_shape(f, rows, K, scale_layout))


def block_scaled_matmul_naive(a_codes, a_scales, b_codes, b_scales, fmt, K: int,
                              a_tsf: float = 1.0, b_tsf: float = 1.0, out=None, stream=None,
                              scale_layout: int = SCALES_ROW_MAJOR):
    """Reference GEMM c = A @ B.T (fp32 [M, N]) over two quantizer outputs of
    one format, both blocked along K; one thread per output, fp32 sums in
    ascending k.  Not a fast GEMM."""
    f = _fmt(fmt)
    a_codes, a_scales = _as_code_matrix("a_codes", a_codes), _as_code_matrix("a_scales", a_scales)
    b_codes, b_scales = _as_code_matrix("b_codes", b_codes), _as_code_matrix("b_scales", b_scales)
    M, N = a_codes.shape[0], b_codes.shape[0]
    _check_operands(f, K, scale_layout, (a_codes, a_scales, M, "a_"), (b_codes, b_scales, N, "b_"))
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a_codes.device)
    _need("out", out, torch.float32, M, N)
    _check(_lib.block_scaled_matmul_naive(
        f, BLOCK_SIZE.get(f, 0), scale_layout, _ptr(a_codes), _ld(a_codes), _ptr(a_scales),
        _ld(a_scales), float(a_tsf), _ptr(b_codes), _ld(b_codes), _ptr(b_scales), _ld(b_scales),
        float(b_tsf), M, N, K, _ptr(out), _ld(out), _stream_ptr(stream, a_codes.device)))
    return out


def block_scaled_matmul_mfma(a_codes, a_scales, b_codes, b_scales, fmt, K: int, out=None,
                             stream=None):
    """c = A @ B.T (fp32 [M, N]) on the matrix cores, over two MX quantizer
    outputs with scales in the MFMA layout (``scale_layout=SCALES_MFMA16``);
    K % 128 == 0."""
    f = _fmt(fmt)
    a_codes, a_scales = _as_code_matrix("a_codes", a_codes), _as_code_matrix("a_scales", a_scales)
    b_codes, b_scales = _as_code_matrix("b_codes", b_codes), _as_code_matrix("b_scales", b_scales)
    M, N = a_codes.shape[0], b_codes.shape[0]
    _check_operands(f, K, SCALES_MFMA16, (a_codes, a_scales, M, "a_"),
                    (b_codes, b_scales, N, "b_"))
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a_codes.device)
    _need("out", out, torch.float32, M, N)
    _check(_lib.block_scaled_matmul_mfma(
        f, BLOCK_SIZE.get(f, 0), SCALES_MFMA16, _ptr(a_codes), _ld(a_codes), _ptr(a_scales),
        _ld(a_scales), _ptr(b_codes), _ld(b_codes), _ptr(b_scales), _ld(b_scales), M, N, K,
        _ptr(out), _ld(out), _stream_ptr(stream, a_codes.device)))
    return out


def grouped_block_scaled_matmul_mfma(a_codes, a_scales, row_offsets, scales_offsets, expert_ids,
                                     max_rows: int, num_scale_rows: int, b_codes, b_scales,
                                     num_experts: int, fmt, K: int, out=None, stream=None):
    """Per-expert c[r] = A[r] @ B[expert_ids[g]].T for the routed rows r of each
    group g, on the matrix cores.  A: the grouped quantizer's MX output with
    MFMA-layout scales (scales_offsets multiples of 16); B: [num_experts * N,
    K/2 or K] codes and their MFMA-layout scales ([num_experts *
    ceil(N/16), ...]).  Returns fp32 [max_rows, N]; rows no group owns are
    left as they were (uninitialised in a new output)."""
    f = _fmt(fmt)
    a_codes, a_scales = _as_code_matrix("a_codes", a_codes), _as_code_matrix("a_scales", a_scales)
    b_codes, b_scales = _as_code_matrix("b_codes", b_codes), _as_code_matrix("b_scales", b_scales)
    if num_experts < 1 or b_codes.shape[0] % num_experts:
        raise BsqError(1, "b_codes must hold num_experts * N rows, num_experts >= 1")
    N = b_codes.shape[0] // num_experts
    G = _need_vec("expert_ids", expert_ids, (torch.int32,), 0).shape[0]
    for name, t in (("row_offsets", row_offsets), ("scales_offsets", scales_offsets)):
        if _need_vec(name, t, _OFFSETS, G + 1).shape[0] != G + 1:
            raise ValueError("row_offsets and scales_offsets must have num_groups + 1 entries")
    if f in BLOCK_SIZE:
        _need("a_codes", a_codes, torch.uint8, max_rows, code_width(f, K))
        _need("a_scales", a_scales, torch.uint8, *scale_shape(f, num_scale_rows, K, SCALES_MFMA16))
        groups_b, width_b = scale_shape(f, N, K, SCALES_MFMA16)
        _need("b_scales", b_scales, torch.uint8, num_experts * groups_b, width_b)
        _need("b_codes", b_codes, torch.uint8, num_experts * N, code_width(f, K))
    if out is None:
        out = torch.empty((max_rows, N), dtype=torch.float32, device=a_codes.device)
    _need("out", out, torch.float32, max_rows, N)
    _check(_lib.grouped_block_scaled_matmul_mfma(
        f, BLOCK_SIZE.get(f, 0), SCALES_MFMA16, _ptr(a_codes), _ld(a_codes), _ptr(a_scales),
        _ld(a_scales), _ptr(row_offsets), _ptr(scales_offsets), _ptr(expert_ids), G, max_rows,
        num_scale_rows, _ptr(b_codes), _ld(b_codes), _ptr(b_scales), _ld(b_scales), num_experts,
        N, K, _ptr(out), _ld(out), _stream_ptr(stream, a_codes.device)))
    return out


# ------------------------------------------------------------------ measurement aid

_ceiling_lib = None


def ceiling_stream(x: torch.Tensor, fmt, chunks_per_wave: int, codes=None, scales=None,
                   start=None, stop=None, stream=None):
    """The trivial stream of ``libbsq_ceiling.so`` (``include/bsq_ceiling.h``):
    the memory traffic of a dense quantizer launch on x (BF16 [M, K], K a
    multiple of 512) with ``chunks_per_wave`` chunks per wave, computing
    nothing of the method.  ``start`` / ``stop``: optional recorded
    ``torch.cuda.Event`` pair bound to the kernel's dispatch.  Returns the
    written (codes, scales)."""
    lib_c = _ceiling()
    f = _fmt(fmt)
    x = _as_bf16_matrix(x)
    if not x.is_contiguous():
        raise TypeError("x must be contiguous")
    M, K = x.shape
    if codes is None:
        codes = torch.empty((M, code_width(f, K)), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, K // BLOCK_SIZE[f]), dtype=torch.uint8, device=x.device)
    for name, t, cols in (("codes", codes, code_width(f, K)), ("scales", scales,
                                                               K // BLOCK_SIZE[f])):
        if not t.is_contiguous() or tuple(t.shape) != (M, cols) or t.dtype != torch.uint8:
            raise TypeError(f"{name} must be a contiguous uint8 [{M}, {cols}] tensor")
    ev = [None if e is None else ctypes.c_void_p(e.cuda_event) for e in (start, stop)]
    st = lib_c.bsq_ceiling_stream(f, _ptr(x), M, K, _ptr(codes), _ptr(scales), chunks_per_wave,
                                  ev[0], ev[1], _stream_ptr(stream, x.device))
    if st != 0:
        raise BsqError(st, "bsq_ceiling_stream rejected its arguments or failed to launch")
    return codes, scales


def ceiling_expand(codes: torch.Tensor, scales: torch.Tensor, fmt, K: int,
                   chunks_per_wave: int, out=None, start=None, stop=None, stream=None):
    """The dequantizer-mix trivial stream of ``libbsq_ceiling.so``
    (``include/bsq_ceiling.h``): reads dense codes [M, K/2 or K] and row-major
    scales [M, K/32 or K/16] and writes fp32 [M, K] with the dequantizer's
    tiles and instructions, decoding nothing.  Returns out."""
    lib_c = _ceiling()
    f = _fmt(fmt)
    M = codes.shape[0]
    for name, t, cols in (("codes", codes, code_width(f, K)),
                          ("scales", scales, K // BLOCK_SIZE[f])):
        if not t.is_contiguous() or tuple(t.shape) != (M, cols) or t.dtype != torch.uint8:
            raise TypeError(f"{name} must be a contiguous uint8 [{M}, {cols}] tensor")
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=codes.device)
    if not out.is_contiguous() or tuple(out.shape) != (M, K) or out.dtype != torch.float32:
        raise TypeError(f"out must be a contiguous float32 [{M}, {K}] tensor")
    ev = [None if e is None else ctypes.c_void_p(e.cuda_event) for e in (start, stop)]
    st = lib_c.bsq_ceiling_expand(f, _ptr(codes), _ptr(scales), M, K, _ptr(out), chunks_per_wave,
                                  ev[0], ev[1], _stream_ptr(stream, codes.device))
    if st != 0:
        raise BsqError(st, "bsq_ceiling_expand rejected its arguments or failed to launch")
    return out


def _ceiling():
    """libbsq_ceiling.so, loaded on first use."""
    global _ceiling_lib
    if _ceiling_lib is None:
        path = os.path.join(os.path.dirname(LIB_PATH), "libbsq_ceiling.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run fp8_quantization_amd/build.py")
        lib_c = ctypes.CDLL(path)
        lib_c.bsq_ceiling_stream.argtypes = [_i32, _p, _i64, _i64, _p, _p, _i32, _p, _p, _p]
        lib_c.bsq_ceiling_stream.restype = _i32
        lib_c.bsq_ceiling_expand.argtypes = [_i32, _p, _p, _i64, _i64, _p, _i32, _p, _p, _p]
        lib_c.bsq_ceiling_expand.restype = _i32
        _ceiling_lib = lib_c
    return _ceiling_lib
