"""Build the HIP libraries in-tree for gfx950.

  libnvfp4moe.so    the MoE layer (C-ABI in include/nvfp4_moe.h)
  libnvfp4synth.so  seeded synthetic weights (include/nvfp4_synth.h)

Every source is compiled with hipcc for gfx950 only, with packed fp32
instructions disabled (-packed-fp32-ops).  Objects go to _build/ (ignored by
git); the shared libraries are written next to this file.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]

LIBS = {
    "libnvfp4moe.so": ["quantize.hip", "moe_kernels.hip", "gemm_kernels.hip", "moe_api.cpp", "noalloc.hip"],
    "libnvfp4synth.so": ["synth_weights.hip"],
}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the GPU-only feature flag
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if err and verbose:
        print(err, flush=True)


def build(verbose: bool = False) -> dict:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for lib, srcs in LIBS.items():
        for src in srcs:
            obj = os.path.join(BUILD, src + ".o")
            jobs.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    out = {}
    for lib, srcs in LIBS.items():
        target = os.path.join(HERE, lib)
        tmp = target + ".tmp"
        objs = [os.path.join(BUILD, s + ".o") for s in srcs]
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
        os.replace(tmp, target)
        out[lib] = target
    return out


if __name__ == "__main__":
    for k, v in build(verbose="-v" in sys.argv).items():
        print(k, v)
