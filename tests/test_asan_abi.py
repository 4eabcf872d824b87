"""The host-side C++ of libgpt2.so (argument checks, configuration validation, the arena layout,
error paths of every entry point) under AddressSanitizer: the ABI tests run in a child process
against libgpt2_asan.so (host code instrumented, GPU code as usual) with the ASan runtime
preloaded. No GPU is needed; any heap or stack error aborts the child with an ASan report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_host_asan():
    from transformer_lm_pretraining_gpt_amd import build as B
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc is not available to build the instrumented library")
    lib = B.build(asan=True)  # incremental: recompiles only what changed
    rt = B.asan_runtime()
    if rt is None:
        pytest.skip("the compiler ships no host AddressSanitizer runtime")
    env = dict(os.environ, LD_PRELOAD=rt, GPT2_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
