"""Build libspecverify.so for gfx950 with hipcc (in-tree, next to the binding)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("sv_stats.hip", "sv_kernels.hip", "sv_tree.hip", "sv_filter.hip", "sv_api.hip", "sv_noalloc.hip")]
HEADERS = [os.path.join(HERE, "csrc", h) for h in ("sv_internal.h", "sv_stream.h", "sv_draw.h")] + \
    [os.path.join(ROOT, "include", "spec_verify.h")]
OUT = os.path.join(HERE, "libspecverify.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # the HIP runtime torch ships (ROCm 7.0) loads code objects v5 reliably
    "-mcode-object-version=5",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    cmd = [HIPCC, *FLAGS, *SOURCES, "-o", OUT + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
