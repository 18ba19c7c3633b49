"""One layer through libsvdq's C ABI with no Python in the path: a native
program (tests/native/c_abi_layer.cpp, built in-tree by the build step) packs
the weights, allocates with plain hipMalloc, runs the activation step and the
linear, and checks codes, scales, h and Y against the fp64 oracle it links.
This pins that the boundary is usable as a C library on its own, with the
binding's marshalling out of the picture."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
PROG = os.path.join(HERE, "native", "c_abi_layer")

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("prec", ["int4", "mxfp4"])
def test_c_abi_layer(prec):
    assert os.path.exists(PROG), "tests/native/c_abi_layer is not built (run the build step first)"
    print(f"c abi layer {prec}", file=sys.stderr, flush=True)
    r = subprocess.run([PROG, prec], capture_output=True, text=True, timeout=120)
    print(r.stdout, file=sys.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi layer ok" in r.stdout
