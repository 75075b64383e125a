"""Builds libla_gdn.so (HIP kernels for gfx950 plus the C-ABI layer) in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libla_gdn.so")
SOURCES = [os.path.join(CSRC, "la_gdn_kernels.hip"), os.path.join(CSRC, "la_gdn_api.cpp"),
           os.path.join(CSRC, "la_gdn_noalloc.hip")]

# -packed-fp32-ops: keep the compiler from forming packed fp32 instructions
# (the host pass warns that it does not know the feature; that is harmless).
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build la_gdn")


def build(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *SOURCES]
    res = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    os.replace(tmp, LIB_PATH)
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
