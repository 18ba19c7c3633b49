"""Build address- and undefined-behaviour-sanitized copies of the host code
(CPU only): libsvdq with its host packing step and C-ABI layer instrumented
(the GPU kernels compile as usual), and the oracle.  The sanitizer runtime is
clang's; the tests preload it into a child Python process
(tests/test_sanitizers.py)."""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "w4a4_rank_corrected_quantize_amd")
CSRC = os.path.join(PKG, "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]
COMMON = ["--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-fno-fast-math", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def runtime() -> str:
    """clang's shared address-sanitizer runtime (it carries the undefined-behaviour checks too)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's address-sanitizer runtime is not installed")
    return hits[-1]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")


def build(out_dir: str, verbose: bool = False) -> tuple[str, str]:
    """Returns (sanitized libsvdq path, sanitized oracle path)."""
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        name = os.path.basename(src)
        obj = os.path.join(out_dir, name + ".o")
        flags = COMMON + ["-ffp-contract=off"] if name in ("pack_host.hip", "quant_act.hip") else list(COMMON)
        if name in ("pack_host.hip", "api.hip"):
            flags += SAN_HOST
        if name == "w4a4_gemm.hip":
            flags += ["-mllvm", "-amdgpu-mfma-vgpr-form"]
        _run([HIPCC] + flags + ["-c", src, "-o", obj], verbose)
        objs.append(obj)
    lib = os.path.join(out_dir, "libsvdq_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib] + objs + ["-lpthread"], verbose)
    oracle = os.path.join(out_dir, "liboracle_san.so")
    _run([CLANG, "-O1", "-g", "-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
          os.path.join(ROOT, "oracle", "svdq_oracle.c"), "-o", oracle, "-lm"], verbose)
    return lib, oracle


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else "/tmp/svdq_san", verbose=True))
