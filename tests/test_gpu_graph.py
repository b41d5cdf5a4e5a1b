"""The entry points launch kernels only on the caller's stream (no
allocation, synchronization or memset inside), so a sequence of them can be
captured in a HIP graph.  The graph below holds dense MXFP8 quantization,
the NVFP4 tensor scale feeding the grouped quantizer, and a matrix-core GEMM
of MX operands with MFMA-layout scales.  It is replayed several times, with
the outputs cleared and other eager work run between replays, and every
replay must equal the eager results bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
MXFP4, MXFP8, NVFP4 = 0, 1, 2


@pytest.fixture(scope="module")
def bsq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantization_amd as m
    return m


def dev(a, dt=np.int16):
    return torch.from_numpy(np.ascontiguousarray(a).view(dt)).cuda()


def test_captured_sequence_replays_match_eager(bsq):
    M, K = 300, 2048
    x = dev(W.random_bf16((M, K), seed=31, scale_log2_range=(-10, 10), special_frac=0.001))
    y = dev(W.random_bf16((M, K), seed=32, scale_log2_range=(-4, 4)))
    other = dev(W.random_bf16((64, 512), seed=33))
    ro = torch.tensor([0, 100, 100, 260], dtype=torch.int32, device="cuda")
    so = torch.tensor([0, 112, 112, 272], dtype=torch.int32, device="cuda")
    ids = torch.tensor([2, 0, 1], dtype=torch.int32, device="cuda")
    L = bsq.SCALES_MFMA16

    def run(outs):
        bsq.quantize_block_scaled(x, MXFP8, codes=outs["q8"], scales=outs["s8"])
        bsq.grouped_tensor_scale_nvfp4(x, ro, ids, 3, M, out=outs["tsf"])
        bsq.grouped_quantize_block_scaled(x, NVFP4, ro, so, ids, outs["tsf"], M, 272,
                                          codes=outs["q4"], scales=outs["s4"])
        bsq.quantize_block_scaled(y, MXFP4, codes=outs["qa"], scales=outs["la"], scale_layout=L)
        bsq.block_scaled_matmul_mfma(outs["qa"][:128], outs["la"][:8], outs["qa"][128:],
                                     outs["la"][8:], MXFP4, K, out=outs["c"])

    def fresh():
        return {"q8": torch.zeros((M, K), dtype=torch.uint8, device="cuda"),
                "s8": torch.zeros((M, K // 32), dtype=torch.uint8, device="cuda"),
                "tsf": torch.zeros(3, dtype=torch.float32, device="cuda"),
                "q4": torch.zeros((M, K // 2), dtype=torch.uint8, device="cuda"),
                "s4": torch.zeros((272, K // 16), dtype=torch.uint8, device="cuda"),
                "qa": torch.zeros((M, K // 2), dtype=torch.uint8, device="cuda"),
                "la": torch.zeros(bsq.scale_shape(MXFP4, M, K, L), dtype=torch.uint8,
                                  device="cuda"),
                "c": torch.zeros((128, 172), dtype=torch.float32, device="cuda")}

    eager = fresh()
    run(eager)                                     # (first calls cache the CU count on the host)
    torch.cuda.synchronize()

    outs = fresh()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):                      # captures on torch's capture stream
        run(outs)
    torch.cuda.synchronize()

    for rep in range(3):
        for t in outs.values():
            t.zero_()                              # eager work between replays
        bsq.quantize_block_scaled(other, MXFP4)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in outs.items():
            a, b = t.cpu(), eager[name].cpu()
            if t.dtype == torch.float32:
                a, b = a.view(torch.int32), b.view(torch.int32)
            assert torch.equal(a, b), (rep, name)
