"""include/msa.h from plain C: the header compiles as C99 and C11 with
pedantic warnings as errors, and a C program linked against libmsa.so runs
its host-only calls (status strings, plans, workspace sizes, rejection of
bad arguments) without a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
PKG = os.path.join(ROOT, "block_sparse_top_msa_amd")
GCC = shutil.which("gcc")

pytestmark = pytest.mark.skipif(GCC is None, reason="needs gcc")


@pytest.mark.parametrize("std", ["c99", "c11"])
def test_header_compiles_as_c(tmp_path, std):
    src = tmp_path / "h.c"
    src.write_text('#include "msa.h"\nint msa_header_only(void) { return (int)MSA_OK; }\n')
    r = subprocess.run([GCC, f"-std={std}", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", INC,
                        "-c", str(src), "-o", str(tmp_path / "h.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_program_uses_the_library(tmp_path):
    if not os.path.exists(os.path.join(PKG, "libmsa.so")):
        pytest.skip("libmsa.so is not built")
    exe = tmp_path / "abi_from_c"
    r = subprocess.run([GCC, "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", INC,
                        os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-L", PKG, "-lmsa",
                        f"-Wl,-rpath,{PKG}", "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "C ABI checks passed" in r.stdout
