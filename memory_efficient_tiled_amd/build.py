"""Build libattn.so in-tree for gfx950 with hipcc.

Each source is compiled to an object file in parallel (the forward kernels
of every head dimension are a translation unit of their own), then linked.

Usage: python -m memory_efficient_tiled_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in (
    "attn_fwd.hip", "attn_fwd_d64.hip", "attn_fwd_d80.hip", "attn_fwd_d96.hip",
    "attn_fwd_d128.hip", "attn_fwd_d256.hip", "attn_fwd_d192v128.hip", "attn_fwd_fp8.hip",
    "attn_bwd.hip", "ffn_chunked.hip")]
OUT = os.path.join(PKG, "libattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from emitting packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _filter(stderr: str) -> str:
    # the host pass does not know the packed-fp32 feature and says so; harmless
    return "\n".join(ln for ln in stderr.splitlines()
                     if "not a recognized feature for this target" not in ln)


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    return r.returncode, _filter(r.stderr)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1))
    with tempfile.TemporaryDirectory(prefix="attn_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in SOURCES]
        cmds = [[HIPCC, *FLAGS, "-c", s, "-o", o] for s, o in zip(SOURCES, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, err), src in zip(results, SOURCES):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{err}")
            if err.strip() and verbose:
                print(err, file=sys.stderr)
        tmp_out = OUT + ".tmp"
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_out,
                "-L/opt/rocm/lib", "-lhipblaslt"]
        if verbose:
            print(" ".join(link), flush=True)
        rc, err = _run(link)
        if rc != 0:
            raise RuntimeError(f"hipcc link failed ({rc}):\n{err}")
        os.replace(tmp_out, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
