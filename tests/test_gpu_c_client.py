"""The C ABI from C alone: ``tests/c_abi/bsq_c_client`` (built by
``__graft_entry__.build()``) allocates its own device memory and stream with
the HIP runtime, quantizes a seeded BF16 matrix through include/bsq.h (for
NVFP4 with the tensor scale produced on the device), and writes the outputs,
which must equal the oracle's byte for byte.  Its invalid call must come back
as BSQ_ERR_INVALID_ARG with a message, before any launch."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu
CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "bsq_c_client")


@pytest.mark.parametrize("fmt,M,K,specials", [
    (oracle.MXFP8, 97, 1056, 0.001), (oracle.MXFP4, 3, 512, 0.001),
    (oracle.NVFP4, 130, 2064, 0.001),      # huge finite values: the tensor scale clamps at 2^100
    (oracle.NVFP4, 64, 512, 0.0)])         # an ordinary tensor scale
def test_c_client_matches_oracle(tmp_path, fmt, M, K, specials):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(CLIENT):
        pytest.fail(f"{CLIENT} is not built; run __graft_entry__.build()")
    x = W.random_bf16((M, K), seed=M + K + fmt, scale_log2_range=(-12, 12),
                      special_frac=specials)
    paths = {n: str(tmp_path / f"{n}.bin") for n in ("x", "q", "s", "tsf")}
    x.tofile(paths["x"])
    res = subprocess.run([CLIENT, str(fmt), str(M), str(K), paths["x"], paths["q"], paths["s"],
                          paths["tsf"]], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr)
    assert res.returncode == 0
    assert "invalid K: status 1, message: K=" in res.stdout
    tsf = np.fromfile(paths["tsf"], np.float32)[0]
    if fmt == oracle.NVFP4:
        assert tsf.view(np.uint32) == np.float32(oracle.tensor_scale(x)).view(np.uint32)
        assert (tsf == np.float32(2.0 ** 100)) == (specials > 0)
    qh, sh = oracle.quantize(x, fmt, tsf)
    assert np.array_equal(np.fromfile(paths["q"], np.uint8).reshape(qh.shape), qh)
    assert np.array_equal(np.fromfile(paths["s"], np.uint8).reshape(sh.shape), sh)


def routing(rng, S, G, E, rows, gather, first):
    """Random groups (some empty) over `rows` routed rows starting at row
    `first`, expert ids drawn with repeats, scale rows padded to 16 with some
    extra padding; with gather, routed rows read random source rows."""
    w = rng.random(G) * (rng.random(G) > 0.3)
    w[0] += 1e-3
    counts = rng.multinomial(rows, w / w.sum())
    ro = (first + np.concatenate([[0], np.cumsum(counts)])).astype(np.uint32)
    pads = -(-counts // 16) * 16 + 16 * rng.integers(0, 2, G)
    so = np.concatenate([[0], np.cumsum(pads)]).astype(np.uint32)
    ids = rng.integers(0, E, G).astype(np.int32)
    max_rows = int(ro[-1]) + 5
    ri = rng.integers(0, S, max_rows).astype(np.int32) if gather else None
    return ro, so, ids, max_rows, int(so[-1]) + 16, ri


@pytest.mark.parametrize("fmt,S,K,G,E,rows,gather,first", [
    (oracle.MXFP4, 64, 2048, 256, 256, 512, True, 0),       # decode gather shape
    (oracle.MXFP8, 40, 1056, 30, 7, 300, True, 3),          # ragged K, rows before the first group
    (oracle.NVFP4, 900, 1024, 9, 12, 880, False, 0),        # per-expert tensor scales on the device
    (oracle.NVFP4, 50, 512, 40, 16, 400, True, 2)])
def test_c_client_grouped_matches_oracle(tmp_path, fmt, S, K, G, E, rows, gather, first):
    """grouped_tensor_scale_nvfp4 then grouped_quantize_block_scaled from C:
    codes, scales (padding and rows no group owns included: they keep 0xA5)
    and the per-expert tensor scales all equal the oracle's."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(CLIENT):
        pytest.fail(f"{CLIENT} is not built; run __graft_entry__.build()")
    rng = np.random.default_rng(S + K + G + fmt)
    x = W.random_bf16((S, K), seed=S * K + fmt, scale_log2_range=(-10, 10), special_frac=0.001)
    ro, so, ids, max_rows, nsr, ri = routing(rng, S, G, E, rows, gather, first)
    if not gather:
        assert max_rows <= S
    for name, a in (("x", x), ("ro", ro), ("so", so), ("ids", ids), ("ri", ri)):
        if a is not None:
            a.tofile(str(tmp_path / f"{name}.bin"))
    res = subprocess.run([CLIENT, "grouped", str(fmt), str(S), str(K), str(G), str(E),
                          str(max_rows), str(nsr), "1" if gather else "0", str(tmp_path)],
                         capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr)
    assert res.returncode == 0
    assert "without tensor scales: status 1, message: NVFP4 needs" in res.stdout
    tsf = None
    if fmt == oracle.NVFP4:
        tsf = np.fromfile(str(tmp_path / "tsf.bin"), np.float32)
        want = oracle.grouped_tensor_scale(x, ro, ids, E, row_indices=ri)
        assert np.array_equal(tsf.view(np.uint32), np.asarray(want, np.float32).view(np.uint32))
    width = K if fmt == oracle.MXFP8 else K // 2
    bs = oracle.BLOCK[fmt]
    qh, sh = oracle.grouped_quantize(x, fmt, ro, so, ids, tsf, max_rows, nsr, row_indices=ri,
                                     codes=np.full((max_rows, width), 0xA5, np.uint8),
                                     scales=np.full((nsr, K // bs), 0xA5, np.uint8))
    assert np.array_equal(np.fromfile(str(tmp_path / "q.bin"), np.uint8).reshape(qh.shape), qh)
    assert np.array_equal(np.fromfile(str(tmp_path / "s.bin"), np.uint8).reshape(sh.shape), sh)
