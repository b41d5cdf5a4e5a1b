"""build() on a fresh checkout: none of the libraries exist yet.

The package's __init__ refuses to load before libbsq.so is built, so build()
must reach the build scripts without importing the package first.  This copies
the sources (no built files) into a temporary directory and runs build() there
in a new interpreter.  CPU only: hipcc cross-compiles gfx950 without a GPU.
"""
import os
import shutil
import subprocess
import sys

from conftest import ROOT

SOURCES = ["__graft_entry__.py", "workloads.py", "include", "oracle", "fp8_quantization_amd",
           os.path.join("tests", "c_abi")]
BUILT = (".so", ".tmp", "bsq_c_client")


def _ignore(_dir, names):
    return [n for n in names if n.endswith(BUILT) or n == "__pycache__"]


def test_build_on_fresh_checkout(tmp_path):
    for rel in SOURCES:
        src, dst = os.path.join(ROOT, rel), tmp_path / rel
        if os.path.isdir(src):
            shutil.copytree(src, dst, ignore=_ignore)
        else:
            dst.parent.mkdir(parents=True, exist_ok=True)
            shutil.copy2(src, dst)
    assert not (tmp_path / "fp8_quantization_amd" / "libbsq.so").exists()
    env = {k: v for k, v in os.environ.items() if k != "PYTHONPATH"}
    res = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.build()"],
                         cwd=tmp_path, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    for lib in ("fp8_quantization_amd/libbsq.so", "oracle/liboracle.so",
                "tests/c_abi/bsq_c_client"):
        assert (tmp_path / lib).is_file(), lib
