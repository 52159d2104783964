"""The C ABI layer under host AddressSanitizer and UndefinedBehaviorSanitizer: builds
libbsa_sanitized.so (bsa_api.hip with -fsanitize=address,undefined on its host code) and runs
tests/test_abi.py against it in a child process with the sanitizer runtime preloaded.  Any
sanitizer report aborts the child (halt_on_error), so the run passes only if argument
validation, the launch plans and the workspace arithmetic are free of memory errors and
undefined behaviour on every case test_abi.py exercises.  CPU only: nothing is launched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_host_sanitizers():
    from long_context_attention_sparse_amd import build as bld

    try:
        bld.hipcc()
        runtime = bld.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(f"no sanitizer toolchain: {e}")
    lib = bld.build(sanitize=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, BSA_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-s",
                          "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
