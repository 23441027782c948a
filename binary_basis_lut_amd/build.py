"""Compile libfluxbin.so for gfx950 with hipcc (in-tree, under binary_basis_lut_amd/_build/).

Each translation unit (the host side with the auxiliary kernels, and one per
table width and row-scale format for the GEMV kernel instances) compiles to
an object in parallel; the objects link into one shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
SOURCES = [CSRC / "fluxbin.hip"] + [CSRC / f"gemv_g{g}_rs{rs}_t{t}.hip" for g in (4, 8) for rs in (0, 1)
                                   for t in (32, 16)] + [CSRC / "gemv_g8_banked.hip"]
HEADERS = [CSRC / "common.hpp", CSRC / "gemv_kernel.hpp", CSRC / "gemv_banked.hpp", CSRC / "aux_kernels.hpp",
           CSRC / "decomp_kernels.hpp", CSRC / "probes.hpp", ROOT / "include" / "fluxbin.h"]
DEPS = SOURCES + HEADERS
BUILD = PKG / "_build"
LIB = BUILD / "libfluxbin.so"
ARCH = "gfx950"

COMPILE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    return res.returncode, res.stdout + res.stderr


def build(verbose: bool = False, jobs: int | None = None) -> Path:
    BUILD.mkdir(parents=True, exist_ok=True)
    objs = [BUILD / (src.stem + ".o") for src in SOURCES]
    cmds = [[hipcc(), *COMPILE_FLAGS, "-I", str(ROOT / "include"), "-c", "-o", str(o), str(src)]
            for src, o in zip(SOURCES, objs)]
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, out), src in zip(results, SOURCES):
        if rc != 0:
            sys.stderr.write(out)
            raise RuntimeError(f"hipcc failed ({rc}) compiling {src.name}")
        if verbose and out:
            sys.stderr.write(out)
    tmp = LIB.with_name(LIB.name + ".tmp")
    rc, out = _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)])
    if rc != 0:
        sys.stderr.write(out)
        raise RuntimeError(f"hipcc failed ({rc}) linking {LIB.name}")
    for o in objs:
        o.unlink()
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not LIB.exists():
        return True
    t = LIB.stat().st_mtime
    return any(p.stat().st_mtime > t for p in DEPS)


if __name__ == "__main__":
    print(build(verbose=True))
