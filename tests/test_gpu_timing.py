"""The measurement aids: kernel events bound to a launch's dispatch
(``bsq_time_next_launch``) and the same-byte-mix trivial streams of
``libbsq_ceiling.so`` (the quantizer's and the dequantizer's).

The events must time the kernel alone and leave its results unchanged; the
trivial streams must write exactly the bytes their header documents, so that
their times are those of streams moving the kernels' bytes."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantization_amd as m
    return m


def event_pair():
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    b.record()                      # torch creates its events on first record
    torch.cuda.synchronize()
    return a, b


def test_events_time_the_quantizer_alone(bsq):
    """An armed launch gives the same bytes as an unarmed one, and its kernel
    time lies inside the span of events recorded around the call."""
    x = W.random_bf16((2048, 7168), seed=31, scale_log2_range=(-6, 6))
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    q0, s0 = bsq.quantize_block_scaled(xd, oracle.MXFP8)
    k0, k1 = event_pair()
    o0, o1 = event_pair()
    o0.record()
    bsq.time_next_launch(k0, k1)
    q1, s1 = bsq.quantize_block_scaled(xd, oracle.MXFP8)
    o1.record()
    torch.cuda.synchronize()
    kernel, outer = k0.elapsed_time(k1), o0.elapsed_time(o1)
    print(f"kernel {kernel * 1e3:.2f} us inside {outer * 1e3:.2f} us")
    assert 0.0 < kernel <= outer
    assert torch.equal(q0, q1) and torch.equal(s0, s1)
    qh, sh = oracle.quantize(x[:64], oracle.MXFP8, 1.0)
    assert np.array_equal(q1[:64].cpu().numpy(), qh) and np.array_equal(s1[:64].cpu().numpy(), sh)


def test_events_are_consumed_once(bsq):
    """The armed pair is used by the next call only: a second call leaves it
    as it was."""
    x = torch.from_numpy(W.random_bf16((1024, 4096), seed=32).view(np.int16)).cuda()
    k0, k1 = event_pair()
    bsq.time_next_launch(k0, k1)
    bsq.quantize_block_scaled(x, oracle.MXFP4)
    torch.cuda.synchronize()
    first = k0.elapsed_time(k1)
    bsq.quantize_block_scaled(x, oracle.MXFP4)      # not armed: the events stay
    torch.cuda.synchronize()
    assert k0.elapsed_time(k1) == first > 0.0


def test_events_time_the_tensor_scale_amax_pass(bsq):
    x = W.random_bf16((4096, 7168), seed=33, scale_log2_range=(-4, 4))
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    k0, k1 = event_pair()
    o0, o1 = event_pair()
    o0.record()
    bsq.time_next_launch(k0, k1)
    out = bsq.tensor_scale_nvfp4(xd)
    o1.record()
    torch.cuda.synchronize()
    assert 0.0 < k0.elapsed_time(k1) <= o0.elapsed_time(o1)
    assert out.cpu().numpy()[0] == np.float32(oracle.tensor_scale(x))


def ceiling_expected(x16, fmt, u):
    """The bytes bsq_ceiling_stream documents, from the input's bits."""
    M, K = x16.shape
    x32 = np.ascontiguousarray(x16).view(np.uint32)          # word i of lane l, chunk c:
    if fmt == oracle.MXFP8:                                   # x32[r, 256 c + 4 l + i]
        w = x32.reshape(M, K // 4, 2)
        codes = (w[:, :, 0] ^ w[:, :, 1]).view(np.uint8).reshape(M, K)
    else:
        w = x32.reshape(M, K // 8, 4)
        codes = (w[:, :, 0] ^ w[:, :, 1] ^ w[:, :, 2] ^ w[:, :, 3]).view(np.uint8)
        codes = codes.reshape(M, K // 2)
    L = 2 if fmt == oracle.NVFP4 else 4
    bs = 8 * L
    scales = np.empty((M, K // bs), np.uint8)
    for kb in range(K // bs):
        c, b = divmod(kb * bs, 512)
        b //= bs
        j = c % min(u, L)
        scales[:, kb] = x16[:, 512 * c + 8 * (L * b + j)] & 0xFF
    return codes, scales


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8, oracle.NVFP4])
@pytest.mark.parametrize("u", [1, 2, 4])
@pytest.mark.parametrize("M,K", [(5, 7168), (3, 1536), (9, 512)])
def test_ceiling_stream_writes_the_documented_bytes(bsq, fmt, u, M, K):
    rng = np.random.default_rng(M * K + u + fmt)
    x16 = rng.integers(0, 1 << 16, (M, K), dtype=np.uint16)
    want_q, want_s = ceiling_expected(x16, fmt, u)
    xd = torch.from_numpy(x16.view(np.int16)).cuda()
    q, s = bsq.ceiling_stream(xd, fmt, u)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), want_q)
    assert np.array_equal(s.cpu().numpy(), want_s)


def test_ceiling_stream_rejects_bad_arguments(bsq):
    x = torch.zeros((4, 700), dtype=torch.int16, device="cuda")
    with pytest.raises(bsq.BsqError):
        bsq.ceiling_stream(x, oracle.MXFP8, 2)                 # K not a multiple of 512
    x = torch.zeros((4, 512), dtype=torch.int16, device="cuda")
    with pytest.raises(bsq.BsqError):
        bsq.ceiling_stream(x, oracle.MXFP8, 3)                 # 3 chunks per wave


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.MXFP8, oracle.NVFP4])
@pytest.mark.parametrize("u", [1, 2, 4])
@pytest.mark.parametrize("M,K", [(5, 7168), (3, 1536), (9, 512)])
def test_ceiling_expand_writes_the_documented_words(bsq, fmt, u, M, K):
    rng = np.random.default_rng(M * K + u + fmt + 99)
    width = K if fmt == oracle.MXFP8 else K // 2
    bs = 16 if fmt == oracle.NVFP4 else 32
    codes = rng.integers(0, 256, (M, width), dtype=np.uint8)
    scales = rng.integers(0, 256, (M, K // bs), dtype=np.uint8)
    lanes = K // 8                                              # lane-slots of 8 elements
    if fmt == oracle.MXFP8:
        w = codes.view(np.uint32).reshape(M, lanes, 2)
        q0, q1 = w[:, :, 0], w[:, :, 1]
    else:
        q0, q1 = codes.view(np.uint32).reshape(M, lanes), np.zeros((M, lanes), np.uint32)
    s = scales[:, (8 * np.arange(lanes)) // bs].astype(np.uint32)
    want = np.concatenate([np.repeat((q0 ^ s)[:, :, None], 4, 2),
                           np.repeat((q1 ^ s)[:, :, None], 4, 2)], axis=2).reshape(M, K)
    out = bsq.ceiling_expand(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                             fmt, K, u)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)


def test_ceiling_expand_rejects_bad_arguments(bsq):
    q = torch.zeros((4, 256), dtype=torch.uint8, device="cuda")
    s = torch.zeros((4, 16), dtype=torch.uint8, device="cuda")
    with pytest.raises(bsq.BsqError):
        bsq.ceiling_expand(q, s, oracle.MXFP4, 512, 3)            # 3 chunks per wave
    q = torch.zeros((4, 350), dtype=torch.uint8, device="cuda")
    s = torch.zeros((4, 21), dtype=torch.uint8, device="cuda")
    with pytest.raises(bsq.BsqError):
        bsq.ceiling_expand(q, s, oracle.MXFP4, 700, 1)            # K not a multiple of 512
