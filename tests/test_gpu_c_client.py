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
