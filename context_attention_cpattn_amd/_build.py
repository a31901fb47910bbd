"""Build libcpattn.so (HIP kernels + C ABI) for gfx950 with hipcc.

Usage: ``python context_attention_cpattn_amd/_build.py`` (run as a script, so the
package -- which loads the library -- is not imported first) or ``build()``.
Objects go to ``_build/`` at the repository root; the shared library is
written next to this file, where the Python binding loads it from.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcpattn.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "partial_bf16.hip", "partial_f32.hip", "merge.hip", "decode.hip", "copy.hip", "scratch.hip"]

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 VALU ops stay off in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in arch VGPRs: the softmax reads S directly, and the
    # 32-row, two-waves-per-SIMD kernels fit in 256 registers without AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = os.path.join(rocm, "bin", "hipcc")
    if not os.path.exists(exe):
        exe = shutil.which("hipcc") or exe
    return exe


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in (r.stderr or "").splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = False) -> str:
    """Compile every source and link libcpattn.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD, src.rsplit(".", 1)[0] + ".o")
        cmd = [cc, *COMMON]
        if src.endswith(".cpp"):
            cmd += ["-x", "hip"]
        cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
        return obj

    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    _run(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
