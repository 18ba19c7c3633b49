"""The INT4 group scale of the library (one rule shared by the host packing
step and the activation kernel) equals fl32(absmax / 7), rounded upward below
the normal range, for every finite fp32 absmax >= 0.  Exhaustive: a small C++
program built against the library's own header runs all 2^31 - 2^23 values."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "w4a4_rank_corrected_quantize_amd", "csrc")


def test_int4_group_scale_exhaustive(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    exe = tmp_path / "scale_exhaustive"
    # fma contraction off, as for the library; only host code runs
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17", "-ffp-contract=off",
                    "-Xarch_host", "-mfma", "-pthread",
                    "-I", CSRC, os.path.join(HERE, "native", "scale_exhaustive.cpp"), "-o", str(exe)],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout
