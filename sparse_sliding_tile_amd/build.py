"""Builds libsta.so (and the benchmark's libsta_calib.so) in-tree with hipcc
for gfx950.

Usage: python -m sparse_sliding_tile_amd.build  (or call build()).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsta.so")
SOURCES = ["api.hip", "reorder.hip", "f32_debug.hip", "fwd_bf16.hip", "bwd_bf16.hip", "mass.hip"]
# the matrix-core calibration loop the benchmark times: its own library, not
# part of libsta's interface
CALIB_SOURCES = ["calib.hip"]
CALIB_LIB = os.path.join(HERE, "libsta_calib.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # LLVM's iterative ILP scheduler: bit-identical code order for the
    # arithmetic, 1-1.5% faster backward passes, forward unchanged or faster
    "-mllvm", "-amdgpu-sched-strategy=iterative-ilp",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(sources, out, verbose, extra_flags):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra_flags, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose=False, extra_flags=()):
    """Compile every HIP source: libsta.so and libsta_calib.so, in-tree."""
    _compile(CALIB_SOURCES, CALIB_LIB, verbose, extra_flags)
    return _compile(SOURCES, LIB, verbose, extra_flags)


if __name__ == "__main__":
    print(build(verbose=True))
