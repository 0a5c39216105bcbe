"""Build libssd.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m mamba_ssd_sequence_amd.build [--jobs N]

Objects go to mamba_ssd_sequence_amd/_build/, the library to
mamba_ssd_sequence_amd/libssd.so.  Every call recompiles.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libssd.so")

ARCH = "gfx950"
SOURCES = ["api.cpp", "prep.hip", "fwd_blocks.hip", "fwd_o1_scan.hip", "fwd_o2_prep.hip", "fwd_o2_state.hip", "decode.hip",
           "bwd.hip"]

# Packed fp32 VALU ops are disabled for all device code: the kernels use plain
# fp32 arithmetic only.  hipcc's host pass warns that it does not know the
# feature; that warning is expected.  MFMA accumulators are kept in the
# architectural VGPRs (-amdgpu-mfma-vgpr-form): otherwise the compiler places
# some of them in AGPRs, and every VALU use of such a result (decays, splits,
# the output arithmetic) costs an extra v_accvgpr_read/write.
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", INCLUDE, "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libssd.so)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *CFLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in r.stderr.splitlines() if noise not in l).strip()
    if warn:
        print(f"[build] {src}:\n{warn}", file=sys.stderr)
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    a = ap.parse_args(argv)
    print(build(a.jobs))


if __name__ == "__main__":
    main()
