"""Build libarchead.so (the C-ABI library with the gfx950 kernels) in-tree.

Run ``python compressed_output_head_amd/build.py`` (by path: importing the
package itself loads the library this script produces).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libarchead.so")
SOURCES = ["archead.hip", "prep.hip", "decode.hip", "decode_small.hip", "batch.hip", "batch_g4.hip", "batch_r8.hip", "tile.hip", "tile_stats.hip", "stats.hip",
           "quantize.hip", "topk.hip", "fit.hip", "logit_error.hip"]
# dense products and factorisations of the construction step
LINK_LIBS = ["-L/opt/rocm/lib", "-lrocblas", "-lrocsolver"]
ARCH = os.environ.get("ARCHEAD_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden", "-Wall", "-Wno-unused-result",
    f"--offload-arch={ARCH}",
    # keep fp32 denormals (fp16 scales can be subnormal) and never emit packed fp32 ops
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libarchead.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source to its own object in parallel, then link."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _run([hipcc(), *compile_flags, "-c", os.path.join(CSRC, so[0]), "-o", so[1]],
                                    verbose), zip(SOURCES, objs)))
    _run([hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, *LINK_LIBS, "-o", LIB + ".tmp"], verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
