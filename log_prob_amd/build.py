"""Build libflce.so (HIP, gfx950 only) in-tree with hipcc.

    python -m log_prob_amd.build            # -> log_prob_amd/libflce.so
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["flce_kernels.hip", "flce_api.cpp"]
LIB = os.path.join(HERE, "libflce.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 arithmetic is disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory() as tmp:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc, *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"),
                   "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            objs.append(obj)
        out_tmp = out + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out_tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
