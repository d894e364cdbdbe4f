"""Build libattn.so in-tree for gfx950 with hipcc.

Usage: python -m memory_efficient_tiled_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("attn_fwd.hip", "attn_bwd.hip")]
OUT = os.path.join(PKG, "libattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from emitting packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
]


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = [HIPCC, *FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; harmless
    err = "\n".join(ln for ln in r.stderr.splitlines()
                    if "not a recognized feature for this target" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
