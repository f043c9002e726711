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


def build_hip(out: str = LIB, defines=()) -> str:
    """Compile the sources in parallel (one hipcc per file) and link libs2ar.so."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    tag = "".join("_" + d for d in defines)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", tag + ".o"))
        cmd = [hipcc, *[f for f in HIPCC_FLAGS if f != "-shared"], "-c", *[f"-D{d}" for d in defines],
               "-I", os.path.join(ROOT, "include"), "-o", obj, os.path.join(CSRC, src)]
        procs.append(subprocess.Popen(cmd))
        objs.append(obj)
    if any(p.wait() for p in procs):
        raise RuntimeError("hipcc failed")
    tmp = out + ".tmp"
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


def build_all() -> None:
    synth.build_lib(force=True)
    build_hip()


if __name__ == "__main__":
    build_all()
