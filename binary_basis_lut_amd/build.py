"""Compile libfluxbin.so for gfx950 with hipcc (in-tree, under binary_basis_lut_amd/_build/)."""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SRC = PKG / "csrc" / "fluxbin.hip"
DEPS = [SRC, PKG / "csrc" / "kernels.hpp", ROOT / "include" / "fluxbin.h"]
LIB = PKG / "_build" / "libfluxbin.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> Path:
    LIB.parent.mkdir(parents=True, exist_ok=True)
    tmp = LIB.with_name(LIB.name + ".tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", str(ROOT / "include"), "-o", str(tmp), str(SRC)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}) building {LIB.name}")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not LIB.exists():
        return True
    t = LIB.stat().st_mtime
    return any(p.stat().st_mtime > t for p in DEPS)


if __name__ == "__main__":
    print(build(verbose=True))
