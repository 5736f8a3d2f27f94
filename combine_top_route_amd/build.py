"""Build libubep.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Each source compiles to an object under _build/ (in parallel), then the
objects link into combine_top_route_amd/libubep.so.  Flags:
  -ffp-contract=off   no multiply-add fusion except explicit fmaf
  -packed-fp32-ops    target feature switched off: no packed fp32 instructions
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libubep.so")
SOURCES = ["api.hip", "gate.hip", "layout.hip", "layout_dispatch.hip", "dispatch.hip", "combine.hip",
           "chunked.hip", "sentinel.hip", "expert.hip", "aux.hip"]
ARCH = os.environ.get("UBEP_OFFLOAD_ARCH", "gfx950")

# -amdgpu-atomic-optimizer-strategy=None: every device atomic here is issued by
# one lane, and the optimizer's wave-level rewrite reads the result back right
# after the atomic, which stalls the wave for a full memory round trip where
# the code means to overlap it (ticket claims, done counts).
CFLAGS = ["-std=c++20", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
          "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
