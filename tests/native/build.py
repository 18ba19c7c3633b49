"""Build the native test programs (test infrastructure, not part of libsvdq):
e2m1_sweep, the exhaustive GPU check of the hardware E2M1 conversion.  Built
in-tree on the CPU (hipcc cross-compiles gfx950); the GPU test runs it."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
E2M1_SWEEP = os.path.join(HERE, "e2m1_sweep")


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
    return E2M1_SWEEP


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
