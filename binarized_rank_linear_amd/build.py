"""Build liblittlebit.so (HIP, gfx950) in-tree.

    python -m binarized_rank_linear_amd.build

Every .hip under csrc/ is compiled with hipcc for gfx950 into _build/ and
linked into binarized_rank_linear_amd/liblittlebit.so.  Packed-fp32 VALU
instructions are disabled for the device code.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblittlebit.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

CFLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-result"]
# matrix-instruction accumulators stay in VGPRs (no copies through AGPRs) in
# the decode kernels; the GEMM kernels keep their 256 accumulators in AGPRs
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
AGPR_ACC = {"lb_gemm.hip"}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    extra = [] if os.path.basename(src) in AGPR_ACC else VGPR_FORM
    cmd = [HIPCC] + CFLAGS + extra + ["-c", src, "-o", obj]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless.
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, out))
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link the shared library; return its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed:\n" + p.stdout)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
