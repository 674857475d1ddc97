"""Build the HIP library ``libapsp.so`` in-tree for gfx950 (hipcc)."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "apsp.hip")
SOURCES = [SRC] + [os.path.join(PKG, "csrc", f) for f in ("batched.hip", "ceiling.hip", "johnson.hip", "gemm.hip", "host.hip", "paths.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libapsp.so")
ARCH = "gfx950"

# Packed fp32 VALU instructions are switched off (-packed-fp32-ops); the
# kernels only use scalar 32-bit adds and mins anyway.
COMPILE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
HIPCC_FLAGS = COMPILE_FLAGS + ["-shared"]  # one-command form (compile and link)


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def build_library(out: str = LIB_PATH, extra: list[str] | None = None, verbose: bool = False,
                  jobs: int | None = None) -> str:
    """Compile the csrc/ sources into ``out`` (always recompiles): each source
    to an object in parallel (no device code crosses files), then one link."""
    jobs = jobs or min(len(SOURCES), int(os.environ.get("MAX_JOBS", "0")) or os.cpu_count() or 1)
    work = tempfile.mkdtemp(prefix="apsp_build_")
    try:
        def compile_one(src: str) -> str:
            obj = os.path.join(work, os.path.splitext(os.path.basename(src))[0] + ".o")
            cmd = [hipcc(), *COMPILE_FLAGS, f"-I{INCLUDE}", *(extra or []), "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            return obj
        with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        tmp = out + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    finally:
        shutil.rmtree(work, ignore_errors=True)
    return out
