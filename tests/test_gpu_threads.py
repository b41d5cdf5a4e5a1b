"""Calls from several host threads at once, each on its own stream: every
thread's outputs must equal the oracle's, and the error message of one
thread's invalid calls must not show in another thread (the message is
thread-local; ctypes releases the GIL, so the threads are inside the
library together)."""
import threading

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


def test_threads_on_their_own_streams(bsq):
    fmts = [oracle.MXFP4, oracle.MXFP8, oracle.NVFP4, oracle.MXFP8]
    inputs = [W.random_bf16((64 + 17 * i, 1024), seed=400 + i, scale_log2_range=(-10, 10))
              for i in range(len(fmts))]
    tsfs = [float(oracle.tensor_scale(x)) if f == oracle.NVFP4 else 1.0
            for f, x in zip(fmts, inputs)]
    results, errors = [None] * len(fmts), []

    def work(i):
        try:
            stream = torch.cuda.Stream()
            x = torch.from_numpy(inputs[i].view(np.int16)).cuda()
            torch.cuda.current_stream().synchronize()   # x is on the device before `stream` reads it
            outs = []
            for rep in range(20):
                if i == 3:                          # this thread also makes invalid calls
                    try:
                        bsq.quantize_block_scaled(x[:, :40], oracle.MXFP8, stream=stream)
                        errors.append("invalid call accepted")
                    except bsq.BsqError as e:
                        if "K=40" not in str(e):
                            errors.append(f"wrong message: {e}")
                with torch.cuda.stream(stream):
                    q, s = bsq.quantize_block_scaled(x, fmts[i], tsfs[i], stream=stream)
                outs.append((q, s))
                # a successful call leaves no message behind on this thread
                if bsq.lib().bsq_last_error() != b"":
                    errors.append(f"thread {i}: stale message after a successful call")
            stream.synchronize()
            results[i] = [(q.cpu().numpy(), s.cpu().numpy()) for q, s in outs]
        except Exception as e:                     # reported on the main thread
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(fmts))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    for i, f in enumerate(fmts):
        qh, sh = oracle.quantize(inputs[i], f, tsfs[i])
        for q, s in results[i]:
            assert np.array_equal(q, qh) and np.array_equal(s, sh), i
