"""Build libawq.so (HIP for gfx950) in-tree.

    python -m post_weight_quantization_channel_amd.build

Each .hip source is compiled to an object in _build/ (in parallel), then linked into
post_weight_quantization_channel_amd/libawq.so. Arithmetic flags:
  -ffp-contract=off                     no silent a*b+c -> fma: the quantizer's fp32 steps are
                                        each rounded exactly as specified; wanted FMAs are
                                        written explicitly
  -fhip-fp32-correctly-rounded-divide-sqrt
                                        fp32 '/' is IEEE division
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                        no packed fp32 (v_pk_*_f32) instructions
Denormals are left enabled (no -fgpu-flush-denormals-to-zero), no fast-math.
Per-source additions (FILE_FLAGS):
  w4a16.hip: -mllvm -amdgpu-mfma-vgpr-form
                                        MFMA results in VGPRs: the tiled kernel scales every
                                        group's partial sums with vector instructions, which would
                                        otherwise first copy them out of AGPRs
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libawq.so")
ARCH = os.environ.get("AWQ_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]

FILE_FLAGS = {
    "w4a16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libawq")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature and says so; drop that line
    err = "\n".join(ln for ln in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link libawq.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
