"""Builds the HIP library (gfx950) into dsa_sparse_attention_amd/lib/libdsa_mi355x.so."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "lib", "libdsa_mi355x.so")
SOURCES = ["api.hip", "compress.hip", "score_topk.hip", "attention.hip", "frontend.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU ops are kept off: the compiler must not form v_pk_* fp32 math.  MFMA results are
# allocated in ordinary VGPRs where they fit (instead of accumulation registers with copies around
# every VALU use): the multi-query sliding-window kernel then fits its 4 queries' state without spills.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    cmd = [HIPCC, *FLAGS, *extra, *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"HIP build failed:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
