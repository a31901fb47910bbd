"""The C ABI from C: ``include/cpattn.h`` compiles as C99 and as C++17 with
warnings as errors, and a plain C program (``tests/c/abi_client.c``) linked
against ``libcpattn.so`` gets the expected answers from the entry points that
need no device (version, order selection with its byte counts, workspace
size, argument errors).  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
PKG = os.path.join(ROOT, "context_attention_cpattn_amd")
SRC = os.path.join(ROOT, "tests", "c", "abi_client.c")


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


@pytest.mark.parametrize("cmd", [["gcc", "-std=c99"], ["g++", "-std=c++17", "-x", "c++"]], ids=["c99", "cxx17"])
def test_header_compiles(cmd, tmp_path):
    _need(cmd[0])
    r = subprocess.run(cmd + ["-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", f"-I{INC}", SRC],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_client_runs(tmp_path):
    _need("gcc")
    lib = os.path.join(PKG, "libcpattn.so")
    if not os.path.exists(lib):
        pytest.skip("libcpattn.so not built")
    exe = str(tmp_path / "abi_client")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", f"-I{INC}", SRC, "-o", exe,
                        f"-L{PKG}", "-lcpattn", f"-Wl,-rpath,{PKG}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi client ok" in r.stdout
