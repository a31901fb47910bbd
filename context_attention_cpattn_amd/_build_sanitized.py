"""Host AddressSanitizer + UndefinedBehaviorSanitizer build of the C ABI layer.

Builds ``_build/sanitized/libcpattn_sanitized.so``: ``api.cpp`` (argument
checks, ring layout, drivers) with ASan and UBSan instrumentation of its host
code only, linked with the ordinary kernel objects.  The device code is built
exactly as in the product library.  Loaded by a process that preloads clang's
ASan runtime (see ``tests/test_sanitized_abi.py``), it lets the CPU ABI tests
run every validation path under the sanitizers.  No GPU is needed or used.

  python context_attention_cpattn_amd/_build_sanitized.py
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import _build  # noqa: E402

OUT_DIR = os.path.join(_build.BUILD, "sanitized")
LIB = os.path.join(OUT_DIR, "libcpattn_sanitized.so")
# every sanitizer flag is preceded by -Xarch_host: the host half of the compile is instrumented,
# the gfx950 half is not
HOST_SAN = "-Xarch_host -fsanitize=address,undefined -Xarch_host -fno-sanitize-recover=all".split()


def asan_runtime() -> str | None:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hits = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    cc = _build.hipcc()
    kernels = []
    for src in _build.SOURCES:
        if src.endswith(".cpp"):
            continue
        obj = os.path.join(OUT_DIR, src.rsplit(".", 1)[0] + ".o")
        _build._run([cc, *_build.COMMON, "-c", os.path.join(_build.CSRC, src), "-o", obj])
        kernels.append(obj)
    api = os.path.join(OUT_DIR, "api.o")
    _build._run([cc, *_build.COMMON, *HOST_SAN, "-g", "-fno-omit-frame-pointer", "-x", "hip", "-c",
                 os.path.join(_build.CSRC, "api.cpp"), "-o", api])
    _build._run([cc, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", *HOST_SAN, "-shared-libsan", "-o", LIB,
                 api, *kernels])
    return LIB


if __name__ == "__main__":
    print(build())
