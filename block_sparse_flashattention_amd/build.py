"""Compile libbsfa.so for gfx950 in-tree with hipcc (runs on a CPU-only host too).

Usage: python -m block_sparse_flashattention_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f)
           for f in ("bsfa_host.cpp", "bsfa_fwd.hip", "bsfa_decode.hip", "bsfa_calib.hip")]
OUTPUT = os.path.join(HERE, "libbsfa.so")

# Packed fp32 VALU forms are disabled for all device code (-packed-fp32-ops); the host
# compile pass prints a harmless "not a recognized feature" warning for it.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    tmp = OUTPUT + ".tmp"
    cmd = [hipcc(), *FLAGS, "-o", tmp, *SOURCES]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError(f"hipcc failed ({proc.returncode}): {' '.join(cmd)}")
    if verbose:
        noise = "not a recognized feature"
        msg = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l)
        if msg.strip():
            print(msg)
    os.replace(tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    print(build(verbose=True))
