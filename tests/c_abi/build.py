"""Build the C client of libbsq (``bsq_c_client``) with gcc: host C only,
the HIP runtime API and ``include/bsq.h``.  It links libbsq.so from the
package directory (run-time path relative to the binary) and the HIP runtime
from /opt/rocm/lib.  Test infrastructure: ``tests/test_gpu_c_client.py``
runs it."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "bsq_c_client.c")
BIN = os.path.join(HERE, "bsq_c_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    tmp = BIN + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"), SRC,
           "-o", tmp, "-L" + os.path.join(ROOT, "fp8_quantization_amd"), "-lbsq",
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../fp8_quantization_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("gcc failed building the C client")
    if verbose and (res.stdout + res.stderr).strip():
        print(res.stdout + res.stderr)
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    build(verbose=True)
