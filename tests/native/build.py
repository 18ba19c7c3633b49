"""Build the native test programs (test infrastructure, not part of libsvdq):
e2m1_sweep, the exhaustive GPU check of the hardware E2M1 conversion, and
c_abi_layer, one layer through the C ABI alone checked against the oracle
(linked against the in-tree libsvdq.so and liboracle.so, so it is built after
them).  Built in-tree on the CPU (hipcc cross-compiles gfx950); the GPU tests
run them."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
E2M1_SWEEP = os.path.join(HERE, "e2m1_sweep")
C_ABI_LAYER = os.path.join(HERE, "c_abi_layer")
ROOT = os.path.dirname(os.path.dirname(HERE))


def build(verbose: bool = False) -> str:
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-fno-fast-math",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(HERE, "e2m1_sweep.hip"), "-o", E2M1_SWEEP + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for e2m1_sweep.hip:\n" + r.stdout + r.stderr)
    os.replace(E2M1_SWEEP + ".tmp", E2M1_SWEEP)
    # host code only; the libraries are found next to the tree ($ORIGIN), so the
    # program runs wherever the repository is copied
    cmd = [HIPCC, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "c_abi_layer.cpp"), "-o", C_ABI_LAYER + ".tmp",
           "-L", os.path.join(ROOT, "w4a4_rank_corrected_quantize_amd"), "-l:libsvdq.so",
           "-L", os.path.join(ROOT, "oracle"), "-l:liboracle.so",
           "-Wl,-rpath,$ORIGIN/../../w4a4_rank_corrected_quantize_amd:$ORIGIN/../../oracle"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for c_abi_layer.cpp:\n" + r.stdout + r.stderr)
    os.replace(C_ABI_LAYER + ".tmp", C_ABI_LAYER)
    return E2M1_SWEEP


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
