"""Build step: compile ``libattnvar.so`` for gfx950 with hipcc, in-tree.

Usage: ``python -m attention_variants_amd.build`` (also called by
``__graft_entry__.build()``).  Always recompiles.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["attnvar_api.cpp", "attn_fwd.hip", "attn_decode.hip", "attn_bwd.hip", "diff_attn_fwd.hip", "evoformer.hip",
           "evo_fused.hip", "doc_order.hip"]
OUT = os.path.join(HERE, "libattnvar.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
BUILD_DIR = os.path.join(ROOT, "_build")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]
# Kernel sources never produce or consume NaN on purpose (masked scores are
# -inf, which stays honoured); without NaN semantics fmaxf needs no quieting
# of its MFMA-produced inputs.  The host-side ABI keeps full IEEE semantics
# because it rejects NaN parameters.
KERNEL_FLAGS = ["-fno-honor-nans"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in (r.stderr or "").splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        extra = KERNEL_FLAGS if src.endswith(".hip") else []
        _run([HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = OUT + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
