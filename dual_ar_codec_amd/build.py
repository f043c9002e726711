"""Build the HIP library (gfx950) and the seeded-input generator in-tree."""
from __future__ import annotations

import os
import subprocess

from . import synth

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libs2ar.so")
SOURCES = ["engine.hip", "kernels.hip", "prefill.hip", "batch.hip", "measure.hip"]

HIPCC_FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off (hipcc's host pass warns that it does not know the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-Wno-unused-value",
]


def build_hip(out: str = LIB) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build_all() -> None:
    synth.build_lib(force=True)
    build_hip()


if __name__ == "__main__":
    build_all()
