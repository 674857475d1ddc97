"""Build the HIP library ``libapsp.so`` in-tree for gfx950 (hipcc)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "apsp.hip")
SOURCES = [SRC] + [os.path.join(PKG, "csrc", f) for f in ("batched.hip", "ceiling.hip", "johnson.hip", "gemm.hip", "host.hip", "paths.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libapsp.so")
ARCH = "gfx950"

# Packed fp32 VALU instructions are switched off (-packed-fp32-ops); the
# kernels only use scalar 32-bit adds and mins anyway.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def build_library(out: str = LIB_PATH, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compile the csrc/ sources into ``out`` (always recompiles)."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", *(extra or []), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out
