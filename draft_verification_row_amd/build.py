"""Build the HIP library libspecverify.so for gfx950, in-tree.

    python -m draft_verification_row_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "spec_verify.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libspecverify.so")

# Packed fp32 instructions are disabled for every HIP translation unit: the
# library's float code is written for scalar v_*_f32 forms.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def build_library(out: str = LIB, extra_flags=()) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I" + INCLUDE, "-o", tmp, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library())
