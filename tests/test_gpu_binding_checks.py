"""The Python binding checks the tensors behind the C ABI's pointers: a
buffer smaller than the window a kernel would touch raises BsqError
(BSQ_ERR_INVALID_ARG), and a wrong dtype raises TypeError, before any
launch.  Nothing here runs a kernel on an undersized buffer."""
import pytest
import torch

pytestmark = pytest.mark.gpu
MXFP4, MXFP8, NVFP4 = 0, 1, 2


@pytest.fixture(scope="module")
def bsq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantization_amd as m
    return m


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8, device="cuda")


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16, device="cuda")


def i32(*vals):
    return torch.tensor(vals, dtype=torch.int32, device="cuda")


def test_quantize_outputs(bsq):
    x = bf16(20, 512)
    with pytest.raises(bsq.BsqError, match="codes"):
        bsq.quantize_block_scaled(x, MXFP8, codes=u8(19, 512))
    with pytest.raises(bsq.BsqError, match="codes"):
        bsq.quantize_block_scaled(x, MXFP4, codes=u8(20, 255))
    with pytest.raises(bsq.BsqError, match="scales"):
        bsq.quantize_block_scaled(x, MXFP8, scales=u8(20, 15))
    with pytest.raises(bsq.BsqError, match="scales"):          # MFMA layout: 2 row groups
        bsq.quantize_block_scaled(x, MXFP8, scales=u8(1, 256), scale_layout=bsq.SCALES_MFMA16)
    with pytest.raises(TypeError):
        bsq.quantize_block_scaled(x, MXFP8, codes=torch.zeros((20, 512), dtype=torch.int8,
                                                              device="cuda"))


def test_grouped_quantize(bsq):
    x = bf16(30, 256)
    ro, ids = i32(0, 10, 25), i32(0, 1)
    sf = torch.ones(2, dtype=torch.float32, device="cuda")
    with pytest.raises(bsq.BsqError, match="codes"):
        bsq.grouped_quantize_block_scaled(x, NVFP4, ro, ro.clone(), ids, sf, 25, 25,
                                          codes=u8(24, 128))
    with pytest.raises(bsq.BsqError, match="scales"):
        bsq.grouped_quantize_block_scaled(x, NVFP4, ro, ro.clone(), ids, sf, 25, 25,
                                          scales=u8(24, 16))
    with pytest.raises(bsq.BsqError, match="row_indices"):
        bsq.grouped_quantize_block_scaled(x, NVFP4, ro, ro.clone(), ids, sf, 25, 25,
                                          row_indices=i32(*range(24)))
    with pytest.raises(TypeError):
        bsq.grouped_quantize_block_scaled(x, NVFP4, ro.long(), ro.clone(), ids, sf, 25, 25)


def test_tensor_scale_outputs(bsq):
    x = bf16(8, 64)
    with pytest.raises(bsq.BsqError, match="out"):
        bsq.tensor_scale_nvfp4(x, out=torch.empty(0, dtype=torch.float32, device="cuda"))
    with pytest.raises(bsq.BsqError, match="out"):
        bsq.grouped_tensor_scale_nvfp4(x, i32(0, 4, 8), i32(0, 2), 3, 8,
                                       out=torch.empty(2, dtype=torch.float32, device="cuda"))


def test_dequantize(bsq):
    with pytest.raises(bsq.BsqError, match="codes"):
        bsq.dequantize_block_scaled(u8(4, 100), u8(4, 8), MXFP4, 256)
    with pytest.raises(bsq.BsqError, match="scales"):
        bsq.dequantize_block_scaled(u8(4, 256), u8(3, 8), MXFP8, 256)
    with pytest.raises(bsq.BsqError, match="out"):
        bsq.dequantize_block_scaled(u8(4, 256), u8(4, 8), MXFP8, 256,
                                    out=torch.empty((4, 255), dtype=torch.float32, device="cuda"))


def test_gemms(bsq):
    K = 512
    a, la = u8(40, K), u8(3, 256)
    b, lb = u8(20, K), u8(2, 256)
    with pytest.raises(bsq.BsqError, match="a_scales"):
        bsq.block_scaled_matmul_mfma(a, u8(2, 256), b, lb, MXFP8, K)
    with pytest.raises(bsq.BsqError, match="b_codes"):
        bsq.block_scaled_matmul_mfma(a, la, u8(20, K - 16), lb, MXFP8, K)
    with pytest.raises(bsq.BsqError, match="out"):
        bsq.block_scaled_matmul_mfma(a, la, b, lb, MXFP8, K,
                                     out=torch.empty((40, 19), dtype=torch.float32, device="cuda"))
    with pytest.raises(bsq.BsqError, match="a_scales"):
        bsq.block_scaled_matmul_naive(a, u8(40, 15), b, u8(20, 16), MXFP8, K)
    ro, ids = i32(0, 16, 40), i32(0, 1)
    with pytest.raises(bsq.BsqError, match="b_scales"):      # 2 experts x 2 row groups of N = 20
        bsq.grouped_block_scaled_matmul_mfma(a, la, ro, ro.clone(), ids, 40, 40, u8(40, K),
                                             u8(3, 256), 2, MXFP8, K)
    with pytest.raises(bsq.BsqError, match="num_experts"):
        bsq.grouped_block_scaled_matmul_mfma(a, la, ro, ro.clone(), ids, 40, 40, u8(40, K),
                                             u8(4, 256), 0, MXFP8, K)
