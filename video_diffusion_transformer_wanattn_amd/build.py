"""Build the native pieces in-tree:

* ``libwanattn.so`` -- the HIP kernels and the C ABI (hipcc, gfx950 only).
* ``seeded/libseeded.so`` -- the seeded input generator (host C).

Run ``python -m video_diffusion_transformer_wanattn_amd.build``.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libwanattn.so")
SEEDED_SRC = os.path.join(PKG, "seeded", "seeded.c")
SEEDED_LIB = os.path.join(PKG, "seeded", "libseeded.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in arch VGPRs: the scores are read by VALU right after the
    # product, and the AGPR form made the compiler copy them back and forth
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # no NaN operands reach the kernels' arithmetic (masks use -inf, LDS is
    # zeroed); this lets row maxima map to v_max3 without NaN canonicalisation
    "-fno-honor-nans",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build_hip() -> str:
    tmp = LIB + ".tmp"
    # the q/k/v projections of the prologue are plain GEMMs in hipBLASLt
    _run([HIPCC, *HIP_FLAGS, "-o", tmp, os.path.join(CSRC, "wanattn_api.hip"), "-lhipblaslt"])
    os.replace(tmp, LIB)
    return LIB


def build_seeded() -> str:
    tmp = SEEDED_LIB + ".tmp"
    _run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", tmp, SEEDED_SRC, "-lm"])
    os.replace(tmp, SEEDED_LIB)
    return SEEDED_LIB


def build_all() -> None:
    build_seeded()
    build_hip()


if __name__ == "__main__":
    build_all()
    print(LIB)
