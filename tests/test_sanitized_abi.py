"""The C-ABI tests against librz_san.so, the library built with its host
code instrumented by AddressSanitizer and UndefinedBehaviorSanitizer
(`python -m invariant_logprob_is_amd.build --sanitize`, part of the entry
build).  Every argument check, the workspace arithmetic and the no-device
path run under the sanitizers in a child process; any report fails it."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "invariant_logprob_is_amd", "librz_san.so")


@pytest.mark.skipif(not os.path.exists(SAN_LIB), reason="librz_san.so not built")
def test_abi_under_address_and_undefined_sanitizers():
    from invariant_logprob_is_amd import build
    rt = build.sanitizer_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ)
    # the sanitizer runtime must come first among the preloaded libraries
    env["LD_PRELOAD"] = " ".join(p for p in (rt, env.get("LD_PRELOAD", "")) if p)
    env["RZ_LIB_PATH"] = SAN_LIB
    # the interpreter itself is not instrumented: its leaks are not ours
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=87"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
