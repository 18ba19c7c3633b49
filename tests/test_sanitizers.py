"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): the library's packing step and C-ABI validation and the oracle, built
with both sanitizers (tests/native/build_sanitized.py), run the host-side test
files in a child Python process with clang's sanitizer runtime preloaded.  Any
out-of-bounds access, use after free or undefined behaviour aborts that
process and fails this test."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_host_code_clean_under_asan_and_ubsan(tmp_path):
    from tests.native.build_sanitized import build, runtime
    try:
        rt = runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib, oracle = build(str(tmp_path))
    env = dict(os.environ, LD_PRELOAD=rt, SVDQ_LIBRARY=lib, SVDQ_ORACLE_LIBRARY=oracle,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               PYTHONPATH=ROOT)
    files = ["tests/test_pack_host.py", "tests/test_abi.py", "tests/test_nf4_pack.py", "tests/test_binding_checks.py",
             "tests/test_oracle_quant.py", "tests/test_oracle_pack.py", "tests/test_oracle_linear.py",
             "tests/test_oracle_qkvnorm.py", "tests/test_oracle_awq.py", "tests/test_oracle_nf4.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu and not slow", "-p", "no:cacheprovider"]
                       + files, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
