"""Build libqsa.so in-tree with hipcc for gfx950.

    python -m block_sparse_decode_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["qsa_api.hip", "qsa_index.hip", "qsa_select.hip", "qsa_decode.hip", "qsa_store.hip", "qsa_rollback.hip", "qsa_static.hip"]
OUT = os.path.join(HERE, "libqsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-ffp-contract=fast",
]


def command(out: str = OUT):
    return [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", out,
            *[os.path.join(CSRC, s) for s in SOURCES]]


def build(verbose: bool = False) -> str:
    cmd = command()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err and verbose:
        print(err, file=sys.stderr)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
