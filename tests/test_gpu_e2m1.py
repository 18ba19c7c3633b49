"""The hardware E2M1 conversion (v_cvt_scalef32_pk_fp4_f32 at unit scale) that
the MXFP4 activation step and the fused requantizing epilogue use equals the
OCP Microscaling v1.0 element rule -- nearest E2M1 magnitude, ties to the even
index, saturation at 6, sign kept for zero -- for every fp32 |t| < 16, both
signs.  Those kernels convert t = v 2^-X, which is exact and below 16 by the
choice of X, so this sweep covers every input they can see.  The sweep is a
native program built in-tree (tests/native/build.py) and run as a child
process on the GPU."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SWEEP = os.path.join(HERE, "native", "e2m1_sweep")

pytestmark = pytest.mark.gpu


def test_hardware_e2m1_conversion_exhaustive():
    assert os.path.exists(SWEEP), "tests/native/e2m1_sweep is not built (run the build step first)"
    print("e2m1 sweep: all fp32 |t| < 16, both signs", file=sys.stderr, flush=True)
    r = subprocess.run([SWEEP], capture_output=True, text=True, timeout=120)
    print(r.stdout, file=sys.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checked 2197815296 values, mismatches 0" in r.stdout
