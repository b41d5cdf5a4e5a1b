"""Build ``libbsq.so`` in-tree with hipcc for gfx950.

Flags that matter for bit-exact results:
  -ffp-contract=off                          no fused multiply-adds are formed
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE division (the NVFP4 scale)
  -fno-gpu-flush-denormals-to-zero           fp32 subnormals are kept
and, for this GPU pool, packed fp32 instructions are disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops; the host pass warns that
it does not know the feature, which is harmless).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbsq.so")
SOURCES = [os.path.join(CSRC, "bsq_api.cpp"), os.path.join(CSRC, "bsq_kernels.hip"),
           os.path.join(CSRC, "bsq_consume.hip")]
# the same-byte-mix streaming kernel the bench compares the quantizers with
CEILING_LIB = os.path.join(HERE, "libbsq_ceiling.so")
CEILING_SOURCES = [os.path.join(CSRC, "bsq_ceiling.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def build(verbose: bool = False, extra=()) -> str:
    """Build libbsq.so, then libbsq_ceiling.so; returns the path of the first."""
    _build_one(LIB, SOURCES, verbose, extra)
    _build_one(CEILING_LIB, CEILING_SOURCES, verbose, extra)
    return LIB


def _build_one(lib, sources, verbose, extra):
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(lib)}")
    noise = [ln for ln in (res.stdout + res.stderr).splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln]
    if verbose and noise:
        print("\n".join(noise))
    os.replace(tmp, lib)


if __name__ == "__main__":
    build(verbose=True)
