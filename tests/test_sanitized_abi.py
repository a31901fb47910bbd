"""The CPU ABI tests again, against a build whose host code (argument checks, ring layout, drivers)
carries AddressSanitizer and UndefinedBehaviorSanitizer; any report fails the run.

The sanitized library is built by ``context_attention_cpattn_amd/_build_sanitized.py`` and loaded
through ``CPATTN_LIB`` into a child interpreter that preloads clang's ASan runtime.  No GPU is used.
"""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "context_attention_cpattn_amd"))


@pytest.mark.skipif(torch.cuda.is_available(), reason="the ABI validation probes run only without a GPU")
@pytest.mark.timeout(600)
def test_abi_under_host_sanitizers():
    sb = pytest.importorskip("_build_sanitized")
    rt = sb.asan_runtime()
    if rt is None:
        pytest.skip("clang's ASan runtime is not installed")
    lib = sb.build()
    env = dict(os.environ, LD_PRELOAD=rt, CPATTN_LIB=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-s",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=500)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out and " failed" not in out
