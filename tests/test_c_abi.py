"""The C ABI from plain C: tests/c_abi/consumer.c, compiled with gcc (C11, -pedantic, warnings
as errors) against include/fluxbin.h and linked to libfluxbin.so, runs its host-only checks
(version, a plan, a workspace size, the error path).  No GPU needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib_dir():
    from binary_basis_lut_amd import build as B
    if B.is_stale():
        B.build()
    return str(B.LIB.parent)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_plain_c_program_uses_the_abi(lib_dir, tmp_path):
    exe = tmp_path / "consumer"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    "-o", str(exe), os.path.join(ROOT, "tests", "c_abi", "consumer.c"), "-L", lib_dir, "-lfluxbin",
                    f"-Wl,-rpath,{lib_dir}"], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "FAIL" not in res.stdout
