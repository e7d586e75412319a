"""Build the HIP library of the drafting step for gfx950 (in-tree).

``python -m block_diffusion_drafter_feature_amd.build`` compiles
``csrc/dflash_api.hip`` (and the headers it includes) into
``block_diffusion_drafter_feature_amd/libdflash.so`` with hipcc.  The library is
written to a temporary name and renamed, so a half-written file is never loaded.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdflash.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32) on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in VGPRs: keeps GEMM accumulators in place across the K loop
    # (the AGPR form made the register allocator rotate them with copies every slab)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the drafting-step library)")


def build(verbose: bool = False, timeout: int = 1200) -> str:
    """Compile the library; returns its path.  Raises on failure."""
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), *FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp, os.path.join(CSRC, "dflash_api.hip")]
    t0 = time.time()
    p = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (p.stderr or "").splitlines() if noise not in l)
    if p.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({p.returncode}):\n{' '.join(cmd)}\n{err}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f} s", flush=True)
        if err.strip():
            print(err)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
