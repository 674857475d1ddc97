"""Python binding of the gfx950 blocked Floyd-Warshall library (libapsp.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/apsp.h.  PyTorch is used for
device memory and streams; nothing here computes distances, and there is no
CPU fallback -- a missing library raises.

Raw entry points (same names and arguments as the C ABI; pointers and
streams are integers):
    apsp_fw_i32(d_ptr, n, ld, inf, stream) -> status
    apsp_fw_f32(d_ptr, n, ld, inf, stream) -> status
    apsp_fw_rounds_i32(d_ptr, n, ld, inf, r0, r1, stream) -> status
    apsp_fw_rounds_f32(d_ptr, n, ld, inf, r0, r1, stream) -> status
    apsp_fw_signed_i32 / _f32(d_ptr, n, ld, inf, stream) -> status
    apsp_fw_timed_i32(d_ptr, n, ld, inf, stream) -> (status, ms[4], launches[4], arith)
    apsp_fw_timed_f32(d_ptr, n, ld, inf, stream) -> (status, ms[4], launches[4], arith)
    apsp_fw_batched_i32 / _f32(d_ptr, batch, n, ld, stride, inf, stream) -> status
    apsp_johnson_i32(row_ptr, col, w, n, nnz, d_ptr, ld, inf, h_ptr, delta, stream) -> status
    apsp_johnson_timed_i32(...same...) -> (status, ms[4], counts[4])
    apsp_trace_begin(max_launches), apsp_trace_end() -> (status, ms[4], launches[4], dropped)
    apsp_set_int32_arith(mode), apsp_get_int32_arith(), apsp_minplus_ceiling(arith)
    apsp_pivot_block(n), apsp_status_string(s), apsp_last_hip_error(), apsp_version()

Tensor convenience:
    fw(t, inf=None)              in-place APSP of a 2-D int32/float32 CUDA tensor
    fw_rounds(t, r0, r1, inf=None)
    fw_signed(t, inf=None)       in-place APSP with negative weights, synchronous
    fw_timed(t, inf=None)        -> (phase_ms, launches, arith), synchronised
    fw_batched(t, inf=None)      in-place APSP of every graph of a 3-D tensor
    johnson(row_ptr, col, w, out=None, inf=None, h=None, delta=-1)
                                 Johnson's APSP of a CSR graph into a dense
                                 (n, >= n) int32 tensor, synchronised
"""
from __future__ import annotations

import atexit
import ctypes
import os

from ._build import LIB_PATH

APSP_OK = 0
APSP_ERR_INVALID_VALUE = 1
APSP_ERR_NO_DEVICE = 2
APSP_ERR_LAUNCH = 3
APSP_ERR_NEGATIVE_CYCLE = 4
APSP_ERR_RANGE = 5

APSP_ARITH_AUTO = 0
APSP_ARITH_F32_WHEN_EXACT = 1
APSP_ARITH_INT32 = 2

INF_I32 = 0x3FFFFFFF

# Every symbol that include/apsp.h declares.
EXPORTS = (
    "apsp_fw_i32", "apsp_fw_f32", "apsp_fw_rounds_i32", "apsp_fw_rounds_f32",
    "apsp_fw_timed_i32", "apsp_fw_timed_f32", "apsp_set_int32_arith",
    "apsp_get_int32_arith", "apsp_minplus_ceiling", "apsp_minplus_ceiling_waves",
    "apsp_pivot_block",
    "apsp_status_string", "apsp_last_hip_error", "apsp_version",
    "apsp_fw_batched_i32", "apsp_fw_batched_f32", "apsp_johnson_i32",
    "apsp_johnson_timed_i32", "apsp_fw_signed_i32", "apsp_fw_signed_f32",
    "apsp_trace_begin", "apsp_trace_end", "apsp_minplus_gemm_i32", "apsp_minplus_gemm_f32",
    "apsp_fw_host_i32", "apsp_fw_host_f32", "apsp_fw_host_plan", "apsp_successors_i32",
    "apsp_successors_f32", "apsp_fw_paths_i32", "apsp_fw_paths_f32", "apsp_fw_paths_last_form",
    "apsp_path",
    "apsp_fw_i32_noalloc", "apsp_release_events",
)

_lib = None


class APSPError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = f"{what}: {apsp_status_string(status)}"
        if status == APSP_ERR_LAUNCH:
            msg += f" (hipError {apsp_last_hip_error()})"
        super().__init__(msg)


class NegativeCycleError(APSPError):
    """The graph has a cycle of negative total weight."""


def _raise(status: int, what: str):
    if status == APSP_ERR_NEGATIVE_CYCLE:
        raise NegativeCycleError(status, what)
    raise APSPError(status, what)


def lib_path() -> str:
    return LIB_PATH


def load(path: str | None = None):
    """Load libapsp.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    # torch ships its own HIP runtime whose SONAME matches the one libapsp.so
    # links against; importing torch first makes the dynamic linker bind
    # libapsp.so to that already-loaded runtime, so device pointers and
    # streams from torch are valid inside the library (one runtime only).
    import torch  # noqa: F401
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950); there is no fallback")
    lib = ctypes.CDLL(p)
    i64, i32, vp, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float
    dp, lp = ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)
    ip = ctypes.POINTER(ctypes.c_int)
    sig = {
        "apsp_fw_i32": ([vp, i64, i64, i32, vp], ctypes.c_int),
        "apsp_fw_f32": ([vp, i64, i64, f32, vp], ctypes.c_int),
        "apsp_fw_i32_noalloc": ([vp, i64, i64, i32, vp], ctypes.c_int),
        "apsp_fw_rounds_i32": ([vp, i64, i64, i32, i64, i64, vp], ctypes.c_int),
        "apsp_fw_rounds_f32": ([vp, i64, i64, f32, i64, i64, vp], ctypes.c_int),
        "apsp_fw_timed_i32": ([vp, i64, i64, i32, vp, dp, lp, ip], ctypes.c_int),
        "apsp_fw_timed_f32": ([vp, i64, i64, f32, vp, dp, lp, ip], ctypes.c_int),
        "apsp_fw_batched_i32": ([vp, i64, i64, i64, i64, i32, vp], ctypes.c_int),
        "apsp_fw_batched_f32": ([vp, i64, i64, i64, i64, f32, vp], ctypes.c_int),
        "apsp_minplus_gemm_i32": ([vp, i64, vp, i64, vp, i64, i64, i64, i64, i32, vp], ctypes.c_int),
        "apsp_minplus_gemm_f32": ([vp, i64, vp, i64, vp, i64, i64, i64, i64, f32, vp], ctypes.c_int),
        "apsp_fw_host_i32": ([vp, i64, i64, i32, i64, vp, lp], ctypes.c_int),
        "apsp_fw_host_f32": ([vp, i64, i64, f32, i64, vp, lp], ctypes.c_int),
        "apsp_fw_host_plan": ([i64, i64, i64, lp, ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
        "apsp_successors_i32": ([vp, i64, vp, i64, vp, i64, i64, i32, vp], ctypes.c_int),
        "apsp_successors_f32": ([vp, i64, vp, i64, vp, i64, i64, f32, vp], ctypes.c_int),
        "apsp_fw_paths_i32": ([vp, i64, vp, i64, i64, i32, vp], ctypes.c_int),
        "apsp_fw_paths_f32": ([vp, i64, vp, i64, i64, f32, vp], ctypes.c_int),
        "apsp_fw_paths_last_form": ([], ctypes.c_int),
        "apsp_path": ([vp, i64, i64, i64, i64, vp, i64], i64),
        "apsp_trace_begin": ([i64], ctypes.c_int),
        "apsp_trace_end": ([dp, lp, lp], ctypes.c_int),
        "apsp_fw_signed_i32": ([vp, i64, i64, i32, vp], ctypes.c_int),
        "apsp_fw_signed_f32": ([vp, i64, i64, f32, vp], ctypes.c_int),
        "apsp_johnson_i32": ([vp, vp, vp, i64, i64, vp, i64, i32, vp, i32, vp], ctypes.c_int),
        "apsp_johnson_timed_i32": ([vp, vp, vp, i64, i64, vp, i64, i32, vp, i32, vp, dp, lp],
                                   ctypes.c_int),
        "apsp_set_int32_arith": ([ctypes.c_int], ctypes.c_int),
        "apsp_release_events": ([], ctypes.c_int),
        "apsp_get_int32_arith": ([], ctypes.c_int),
        "apsp_minplus_ceiling": ([ctypes.c_int, dp], ctypes.c_int),
        "apsp_minplus_ceiling_waves": ([ctypes.c_int, ctypes.c_int, dp], ctypes.c_int),
        "apsp_pivot_block": ([i64], i64),
        "apsp_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "apsp_last_hip_error": ([], ctypes.c_int),
        "apsp_version": ([], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    if path is None:
        _lib = lib
        # Pooled timing events go back before interpreter shutdown, while the
        # HIP runtime is whole (Python exit handlers run before the static
        # destructors of the runtime and of torch).
        atexit.register(_release_at_exit, lib)
    return lib


def _release_at_exit(lib) -> None:
    try:
        lib.apsp_release_events()
    except Exception:  # noqa: BLE001 - nothing to report at exit
        pass


# ---- raw C-ABI mirrors ------------------------------------------------------

def apsp_fw_i32(d_ptr: int, n: int, ld: int, inf: int, stream: int = 0) -> int:
    return load().apsp_fw_i32(d_ptr or None, n, ld, inf, stream or None)


def apsp_fw_i32_noalloc(d_ptr: int, n: int, ld: int, inf: int, stream: int = 0) -> int:
    return load().apsp_fw_i32_noalloc(d_ptr or None, n, ld, inf, stream or None)


def apsp_fw_f32(d_ptr: int, n: int, ld: int, inf: float, stream: int = 0) -> int:
    return load().apsp_fw_f32(d_ptr or None, n, ld, inf, stream or None)


def apsp_fw_rounds_i32(d_ptr, n, ld, inf, r0, r1, stream=0) -> int:
    return load().apsp_fw_rounds_i32(d_ptr or None, n, ld, inf, r0, r1, stream or None)


def apsp_fw_rounds_f32(d_ptr, n, ld, inf, r0, r1, stream=0) -> int:
    return load().apsp_fw_rounds_f32(d_ptr or None, n, ld, inf, r0, r1, stream or None)


def apsp_fw_batched_i32(d_ptr, batch, n, ld, stride, inf, stream=0) -> int:
    return load().apsp_fw_batched_i32(d_ptr, batch, n, ld, stride, inf, stream)


def apsp_fw_batched_f32(d_ptr, batch, n, ld, stride, inf, stream=0) -> int:
    return load().apsp_fw_batched_f32(d_ptr, batch, n, ld, stride, inf, stream)


def apsp_minplus_gemm_i32(c, ldc, a, lda, b, ldb, m, n, k, inf, stream=0) -> int:
    return load().apsp_minplus_gemm_i32(c or None, ldc, a or None, lda, b or None, ldb, m, n, k,
                                        inf, stream or None)


def apsp_minplus_gemm_f32(c, ldc, a, lda, b, ldb, m, n, k, inf, stream=0) -> int:
    return load().apsp_minplus_gemm_f32(c or None, ldc, a or None, lda, b or None, ldb, m, n, k,
                                        inf, stream or None)


def apsp_fw_host_i32(h_ptr, n, ld, inf, device_bytes=0, stream=0):
    """(status, outer block S used)."""
    blk = ctypes.c_int64(0)
    st = load().apsp_fw_host_i32(h_ptr or None, n, ld, inf, device_bytes, stream or None,
                                 ctypes.byref(blk))
    return int(st), int(blk.value)


def apsp_fw_host_f32(h_ptr, n, ld, inf, device_bytes=0, stream=0):
    blk = ctypes.c_int64(0)
    st = load().apsp_fw_host_f32(h_ptr or None, n, ld, inf, device_bytes, stream or None,
                                 ctypes.byref(blk))
    return int(st), int(blk.value)


def apsp_fw_host_plan(n, elem_bytes, device_bytes):
    """(status, outer block S, panel sets: 0 in-core, 1 or 2)."""
    blk = ctypes.c_int64(0)
    sets = ctypes.c_int32(0)
    st = load().apsp_fw_host_plan(n, elem_bytes, device_bytes, ctypes.byref(blk),
                                  ctypes.byref(sets))
    return int(st), int(blk.value), int(sets.value)


def apsp_successors_i32(w, ldw, d, ldd, nxt, ldn, n, inf, stream=0) -> int:
    return load().apsp_successors_i32(w or None, ldw, d or None, ldd, nxt or None, ldn, n, inf,
                                      stream or None)


def apsp_successors_f32(w, ldw, d, ldd, nxt, ldn, n, inf, stream=0) -> int:
    return load().apsp_successors_f32(w or None, ldw, d or None, ldd, nxt or None, ldn, n, inf,
                                      stream or None)


def apsp_fw_paths_i32(d, ld, nxt, ldn, n, inf, stream=0) -> int:
    return load().apsp_fw_paths_i32(d or None, ld, nxt or None, ldn, n, inf, stream or None)


def apsp_fw_paths_f32(d, ld, nxt, ldn, n, inf, stream=0) -> int:
    return load().apsp_fw_paths_f32(d or None, ld, nxt or None, ldn, n, inf, stream or None)


def apsp_fw_paths_last_form() -> int:
    return int(load().apsp_fw_paths_last_form())


def apsp_path(nxt_host_ptr, ldn, n, i, j, path_ptr=0, cap=0) -> int:
    return int(load().apsp_path(nxt_host_ptr or None, ldn, n, i, j, path_ptr or None, cap))


def apsp_trace_begin(max_launches: int) -> int:
    return int(load().apsp_trace_begin(max_launches))


def apsp_trace_end():
    """(status, ms per kind [4], launches per kind [4], dropped launches)."""
    ms = (ctypes.c_double * 4)()
    cnt = (ctypes.c_int64 * 4)()
    dropped = ctypes.c_int64(0)
    st = load().apsp_trace_end(ms, cnt, ctypes.byref(dropped))
    return int(st), list(ms), list(cnt), int(dropped.value)


def apsp_fw_signed_i32(d_ptr, n, ld, inf, stream=0) -> int:
    return load().apsp_fw_signed_i32(d_ptr or None, n, ld, inf, stream or None)


def apsp_fw_signed_f32(d_ptr, n, ld, inf, stream=0) -> int:
    return load().apsp_fw_signed_f32(d_ptr or None, n, ld, inf, stream or None)


def apsp_johnson_i32(row_ptr, col, w, n, nnz, d_ptr, ld, inf, h_ptr=0, delta=-1, stream=0) -> int:
    return load().apsp_johnson_i32(row_ptr or None, col or None, w or None, n, nnz, d_ptr or None,
                                   ld, inf, h_ptr or None, delta, stream or None)


def apsp_johnson_timed_i32(row_ptr, col, w, n, nnz, d_ptr, ld, inf, h_ptr=0, delta=-1, stream=0):
    """(status, phase ms [validate, Bellman-Ford, reweight, searches],
    counts [Bellman-Ford rounds, search steps, vertices removed, edge
    relaxations])."""
    ms = (ctypes.c_double * 4)()
    counts = (ctypes.c_int64 * 4)()
    st = load().apsp_johnson_timed_i32(row_ptr or None, col or None, w or None, n, nnz,
                                       d_ptr or None, ld, inf, h_ptr or None, delta,
                                       stream or None, ms, counts)
    return st, list(ms), list(counts)


def _timed(fn, d_ptr, n, ld, inf, stream):
    ms = (ctypes.c_double * 4)()
    cnt = (ctypes.c_int64 * 4)()
    arith = ctypes.c_int(-1)
    st = fn(d_ptr or None, n, ld, inf, stream or None, ms, cnt, ctypes.byref(arith))
    return st, list(ms), list(cnt), int(arith.value)


def apsp_fw_timed_i32(d_ptr, n, ld, inf, stream=0):
    return _timed(load().apsp_fw_timed_i32, d_ptr, n, ld, inf, stream)


def apsp_fw_timed_f32(d_ptr, n, ld, inf, stream=0):
    return _timed(load().apsp_fw_timed_f32, d_ptr, n, ld, inf, stream)


def apsp_release_events() -> int:
    return int(load().apsp_release_events())


def apsp_set_int32_arith(mode: int) -> int:
    return int(load().apsp_set_int32_arith(mode))


def apsp_get_int32_arith() -> int:
    return int(load().apsp_get_int32_arith())


class int32_arith:
    """Context manager: run int32 calls under an arithmetic policy."""

    def __init__(self, mode: int):
        self.mode = mode

    def __enter__(self):
        self.prev = apsp_get_int32_arith()
        if apsp_set_int32_arith(self.mode) != APSP_OK:
            raise ValueError(f"bad arithmetic policy {self.mode}")
        return self

    def __exit__(self, *exc):
        apsp_set_int32_arith(self.prev)
        return False


def apsp_minplus_ceiling(arith: int):
    """(status, relaxations/s) of the register-only min-plus core."""
    r = ctypes.c_double(0.0)
    st = load().apsp_minplus_ceiling(arith, ctypes.byref(r))
    return int(st), float(r.value)


def apsp_minplus_ceiling_waves(arith: int, waves_per_simd: int):
    """(status, relaxations/s) of the register-only min-plus core at exactly
    waves_per_simd waves per SIMD (1 to 4)."""
    r = ctypes.c_double(0.0)
    st = load().apsp_minplus_ceiling_waves(arith, waves_per_simd, ctypes.byref(r))
    return int(st), float(r.value)


def apsp_pivot_block(n: int = 0) -> int:
    return int(load().apsp_pivot_block(n))


def apsp_status_string(status: int) -> str:
    return load().apsp_status_string(status).decode()


def apsp_last_hip_error() -> int:
    return int(load().apsp_last_hip_error())


def apsp_version() -> int:
    return int(load().apsp_version())


# ---- tensor convenience -----------------------------------------------------

def _tensor_args(t, inf):
    import torch
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    n = t.shape[0]
    if t.shape[1] < n:
        raise ValueError("expected at least n columns")
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError("tensor rows must be contiguous (stride(1) == 1)")
    ld = max(t.stride(0), t.shape[1], 1) if n <= 1 else t.stride(0)
    if t.dtype == torch.int32:
        kind = "i32"
        inf = INF_I32 if inf is None else int(inf)
    elif t.dtype == torch.float32:
        kind = "f32"
        inf = float("inf") if inf is None else float(inf)
    else:
        raise ValueError("dtype must be int32 or float32")
    stream = torch.cuda.current_stream(t.device).cuda_stream
    return kind, t.data_ptr(), n, ld, inf, stream


def fw(t, inf=None):
    """In-place APSP of t[:n, :n] (n = t.shape[0]) on the current stream."""
    import torch
    kind, p, n, ld, inf, s = _tensor_args(t, inf)
    with torch.cuda.device(t.device):
        st = (apsp_fw_i32 if kind == "i32" else apsp_fw_f32)(p, n, ld, inf, s)
    if st != APSP_OK:
        raise APSPError(st, "apsp_fw_" + kind)
    return t


def fw_signed(t, inf=None):
    """In-place APSP of t[:n, :n] with negative weights allowed (synchronous).
    Raises NegativeCycleError on a negative cycle."""
    import torch
    kind, p, n, ld, inf, s = _tensor_args(t, inf)
    with torch.cuda.device(t.device):
        st = (apsp_fw_signed_i32 if kind == "i32" else apsp_fw_signed_f32)(p, n, ld, inf, s)
    if st != APSP_OK:
        _raise(st, "apsp_fw_signed_" + kind)
    return t


def fw_rounds(t, r0, r1, inf=None):
    import torch
    kind, p, n, ld, inf, s = _tensor_args(t, inf)
    with torch.cuda.device(t.device):
        st = (apsp_fw_rounds_i32 if kind == "i32" else apsp_fw_rounds_f32)(p, n, ld, inf, r0, r1, s)
    if st != APSP_OK:
        raise APSPError(st, "apsp_fw_rounds_" + kind)
    return t


def fw_timed(t, inf=None):
    """Like fw, synchronised; returns (ms per kind, launches per kind, arith)
    with kinds [Phase 1, Phase 2, Phase 3, int32 scan and conversion] and arith 1 when the
    call computed in binary32."""
    import torch
    kind, p, n, ld, inf, s = _tensor_args(t, inf)
    with torch.cuda.device(t.device):
        st, ms, cnt, arith = (apsp_fw_timed_i32 if kind == "i32" else apsp_fw_timed_f32)(p, n, ld, inf, s)
    if st != APSP_OK:
        raise APSPError(st, "apsp_fw_timed_" + kind)
    return ms, cnt, arith


def fw_batched(t, inf=None):
    """In-place APSP of every graph of a 3-D tensor t[g, :n, :n]
    (n = t.shape[1] <= 128, rows contiguous) on the current stream."""
    import torch
    if t.dim() != 3:
        raise ValueError("expected a 3-D tensor (batch, n, >= n columns)")
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    batch, n = t.shape[0], t.shape[1]
    if t.shape[2] < n:
        raise ValueError("expected at least n columns")
    if t.stride(2) != 1 and t.shape[2] > 1:
        raise ValueError("tensor rows must be contiguous (stride(2) == 1)")
    ld = t.stride(1) if n > 1 else max(t.shape[2], 1)
    stride = t.stride(0) if batch > 1 else max((n - 1) * ld + n, 1)
    if t.dtype == torch.int32:
        fn, inf = apsp_fw_batched_i32, (INF_I32 if inf is None else int(inf))
    elif t.dtype == torch.float32:
        fn, inf = apsp_fw_batched_f32, (float("inf") if inf is None else float(inf))
    else:
        raise ValueError("dtype must be int32 or float32")
    with torch.cuda.device(t.device):
        st = fn(t.data_ptr(), batch, n, ld, stride, inf,
                torch.cuda.current_stream(t.device).cuda_stream)
    if st != APSP_OK:
        raise APSPError(st, "apsp_fw_batched")
    return t


def johnson(row_ptr, col, w, out=None, inf=None, h=None, delta=-1, timed=False):
    """Johnson's APSP of a CSR graph (device tensors: row_ptr int64 [n+1],
    col int32 [nnz], w int32 [nnz]) into out[:n, :n] (int32, rows contiguous;
    allocated as (n, n) when None).  h: optional int32 [n] output of the
    potentials.  Synchronous.  Returns out, or (out, phase_ms, counts) with
    timed=True (see apsp_johnson_timed_i32).  Raises NegativeCycleError on a negative cycle."""
    import torch
    for name, t, dt in (("row_ptr", row_ptr, torch.int64), ("col", col, torch.int32),
                        ("w", w, torch.int32)):
        if not t.is_cuda or t.dtype != dt or t.dim() != 1 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 1-D {dt} CUDA tensor")
    n = row_ptr.shape[0] - 1
    nnz = col.shape[0]
    if n < 0 or w.shape[0] != nnz:
        raise ValueError("row_ptr needs n + 1 entries and w one weight per column index")
    if out is None:
        out = torch.empty((n, n), dtype=torch.int32, device=row_ptr.device)
    if out.dtype != torch.int32 or out.dim() != 2 or out.shape[0] != n or out.shape[1] < n:
        raise ValueError("out must be an int32 (n, >= n) tensor")
    if n > 1 and out.stride(1) != 1:
        raise ValueError("out rows must be contiguous")
    ld = out.stride(0) if n > 1 else max(out.shape[1], 1)
    if h is not None and (h.dtype != torch.int32 or h.numel() != n or not h.is_contiguous()):
        raise ValueError("h must be a contiguous int32 tensor of n entries")
    inf = INF_I32 if inf is None else int(inf)
    hp = h.data_ptr() if h is not None else 0
    with torch.cuda.device(row_ptr.device):
        s = torch.cuda.current_stream(row_ptr.device).cuda_stream
        args = (row_ptr.data_ptr(), col.data_ptr() if nnz else 0, w.data_ptr() if nnz else 0,
                n, nnz, out.data_ptr() if n else 0, ld, inf, hp, int(delta), s)
        if timed:
            st, ms, counts = apsp_johnson_timed_i32(*args)
        else:
            st, ms, counts = apsp_johnson_i32(*args), None, None
    if st != APSP_OK:
        _raise(st, "apsp_johnson_i32")
    return (out, ms, counts) if timed else out


def minplus_gemm(c, a, b, inf=None):
    """c <- min(c, a (x) b) for 2-D CUDA tensors (rows contiguous, same dtype
    int32 or float32), on the current stream."""
    import torch
    for t in (c, a, b):
        if not t.is_cuda or t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
            raise ValueError("operands must be 2-D CUDA tensors with contiguous rows")
    if not (c.dtype == a.dtype == b.dtype) or c.dtype not in (torch.int32, torch.float32):
        raise ValueError("operands must share dtype int32 or float32")
    m, n, k = c.shape[0], c.shape[1], a.shape[1]
    if a.shape[0] != m or b.shape[0] != k or b.shape[1] != n:
        raise ValueError("shapes must be c (m, n), a (m, k), b (k, n)")
    ld = lambda t: max(t.stride(0), t.shape[1], 1)
    is_int = c.dtype == torch.int32
    inf = (INF_I32 if is_int else float("inf")) if inf is None else inf
    fn = apsp_minplus_gemm_i32 if is_int else apsp_minplus_gemm_f32
    with torch.cuda.device(c.device):
        st = fn(c.data_ptr(), ld(c), a.data_ptr(), ld(a), b.data_ptr(), ld(b), m, n, k, inf,
                torch.cuda.current_stream(c.device).cuda_stream)
    if st != APSP_OK:
        _raise(st, "apsp_minplus_gemm")
    return c


def fw_host(t, inf=None, device_bytes=0):
    """In-place APSP of a 2-D int32/float32 CPU tensor (pin it for speed),
    streamed through the GPU in outer blocks; returns the outer block used."""
    import torch
    if t.is_cuda or t.dim() != 2 or t.shape[1] < t.shape[0]:
        raise ValueError("expected a 2-D host tensor with at least n columns")
    n = t.shape[0]
    if n > 1 and t.stride(1) != 1:
        raise ValueError("rows must be contiguous")
    ld = t.stride(0) if n > 1 else max(t.shape[1], 1)
    if t.dtype == torch.int32:
        fn, inf = apsp_fw_host_i32, (INF_I32 if inf is None else int(inf))
    elif t.dtype == torch.float32:
        fn, inf = apsp_fw_host_f32, (float("inf") if inf is None else float(inf))
    else:
        raise ValueError("dtype must be int32 or float32")
    st, blk = fn(t.data_ptr(), n, ld, inf, device_bytes,
                 torch.cuda.current_stream().cuda_stream)
    if st != APSP_OK:
        _raise(st, "apsp_fw_host")
    return blk


def fw_paths(t, nxt=None, inf=None):
    """In-place APSP of t[:n, :n] plus the successor matrix (int32 (n, n)
    CUDA tensor, allocated when None); returns nxt.  Dense int32 inputs in
    range take one pass of the rounds on successor keys (the call then
    synchronises its stream once); apsp_fw_paths_last_form() tells which
    form ran."""
    import torch
    kind, p, n, ld, inf, s = _tensor_args(t, inf)
    if nxt is None:
        nxt = torch.empty((n, n), dtype=torch.int32, device=t.device)
    if nxt.dtype != torch.int32 or nxt.dim() != 2 or nxt.shape[0] != n or nxt.shape[1] < n:
        raise ValueError("nxt must be an int32 (n, >= n) tensor")
    ldn = nxt.stride(0) if n > 1 else max(nxt.shape[1], 1)
    with torch.cuda.device(t.device):
        st = (apsp_fw_paths_i32 if kind == "i32" else apsp_fw_paths_f32)(p, ld, nxt.data_ptr(),
                                                                         ldn, n, inf, s)
    if st != APSP_OK:
        _raise(st, "apsp_fw_paths_" + kind)
    return nxt


def path(nxt_host, i, j):
    """Vertices of the path i -> j from a successor matrix in host memory (a
    contiguous int32 numpy array): a list, [] when unreachable.  Raises on a
    successor cycle."""
    import numpy as np
    a = np.ascontiguousarray(nxt_host, dtype=np.int32)
    n, ldn = a.shape[0], a.shape[1]
    buf = np.empty(n + 1, dtype=np.int32)
    r = apsp_path(a.ctypes.data, ldn, n, i, j, buf.ctypes.data, len(buf))
    if r == -1:
        return []
    if r < 0:
        raise ValueError(f"apsp_path failed ({r})")
    return buf[:r].tolist()
