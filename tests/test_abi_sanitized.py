"""The C-ABI argument checks (tests/test_abi.py) run again against a build of the library whose
host code is compiled with AddressSanitizer and UndefinedBehaviorSanitizer: no argument
combination those tests try may read or write out of bounds, overflow a signed integer or
otherwise hit undefined behaviour in the host layer.  CPU only (no kernel is launched)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_checks_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from sparse_offset_causal_amd.build import build_sanitized, sanitizer_runtime

    lib = build_sanitized()
    rt = sanitizer_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ)
    env["SOC_ATTN_LIB"] = lib
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"  # the interpreter's own allocations are not ours
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert "passed" in r.stdout
