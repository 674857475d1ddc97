"""ctypes wrapper for the CPU oracle (``oracle/oracle.c``) -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the bench's CPU-baseline leg may
import this module.  The product path (``graph_all_pairs_amd``) never does.

Functions mirror the C library:
  * ``fw_i32(m, k_end=None)`` / ``fw_f64(m, k_end=None)``: plain Floyd-Warshall
    on a copy of the matrix (pivots 0 .. k_end-1), returned as a new array;
  * ``fw_in_steps(m, step, progress)``: the same recurrence run as
    consecutive pivot ranges, reporting after each (long full-size runs);
  * ``sssp_rows_i32(w, inf, srcs)`` / ``sssp_rows_f64(w, inf, srcs)``:
    Dijkstra from each listed source, one output row per source;
  * ``fw_guarded(m, inf)``: Floyd-Warshall with negative weights allowed
    (candidates through the sentinel are never formed) and a negative-cycle
    flag;
  * ``bf_rows_csr(row_ptr, col, w, n, srcs, inf)``: Bellman-Ford from each
    listed source over a CSR graph (negative weights allowed);
  * ``johnson_potentials(row_ptr, col, w, n)``: Johnson's h from an added
    vertex with 0-weight edges to every vertex (Bellman-Ford);
  * ``minplus(c, a, b, inf)``: the min-plus product min(c, a (x) b);
  * ``successors(w, d, inf)``: the first-hop matrix of weights w and
    distances d; ``successors_rows(w, d, inf, rows)`` the listed rows of it;
  * ``apsp(m, inf)``: the full distance matrix of an int32 or float32 input
    (float32 is widened exactly to binary64 and the result stays binary64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(out: str = LIB, src: str = SRC, extra: tuple = ()) -> str:
    """Compile the oracle with gcc (OpenMP, -O2, no fast-math, no FMA)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-ffp-contract=off", "-fno-fast-math", *extra, src, "-o", out]
    subprocess.run(cmd, check=True)
    return out


def load(path: str = LIB):
    global _lib
    if path == LIB and _lib is not None:
        return _lib
    if not os.path.exists(path):
        build(path)
    lib = ctypes.CDLL(path)
    i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.oracle_fw_i32.argtypes = [p, i64, i64, i64]
    lib.oracle_fw_i32.restype = None
    lib.oracle_fw_f64.argtypes = [p, i64, i64, i64]
    lib.oracle_fw_f64.restype = None
    lib.oracle_fw_range_i32.argtypes = [p, i64, i64, i64, i64]
    lib.oracle_fw_range_i32.restype = None
    lib.oracle_fw_range_f64.argtypes = [p, i64, i64, i64, i64]
    lib.oracle_fw_range_f64.restype = None
    lib.oracle_fw_batched_i32.argtypes = [p, i64, i64, i64, i64]
    lib.oracle_fw_batched_i32.restype = None
    lib.oracle_fw_batched_f64.argtypes = [p, i64, i64, i64, i64]
    lib.oracle_fw_batched_f64.restype = None
    lib.oracle_fw_guarded_i64.argtypes = [p, i64, i64, i64]
    lib.oracle_fw_guarded_i64.restype = ctypes.c_int
    lib.oracle_sssp_bf_csr_i64.argtypes = [p, p, p, i64, i64, p]
    lib.oracle_sssp_bf_csr_i64.restype = ctypes.c_int
    lib.oracle_sssp_bf_rows_i64.argtypes = [p, p, p, i64, p, i64, p, i64, p]
    lib.oracle_sssp_bf_rows_i64.restype = ctypes.c_int
    lib.oracle_minplus_i64.argtypes = [p, i64, p, i64, p, i64, i64, i64, i64, i64]
    lib.oracle_minplus_i64.restype = None
    lib.oracle_minplus_f64.argtypes = [p, i64, p, i64, p, i64, i64, i64, i64]
    lib.oracle_minplus_f64.restype = None
    lib.oracle_successors_i64.argtypes = [p, p, p, i64, i64, i64]
    lib.oracle_successors_i64.restype = None
    lib.oracle_successors_rows_i64.argtypes = [p, p, p, i64, p, i64, i64]
    lib.oracle_successors_rows_i64.restype = None
    lib.oracle_sssp_i32.argtypes = [p, i64, i64, i32, i64, p]
    lib.oracle_sssp_i32.restype = ctypes.c_int
    lib.oracle_sssp_f64.argtypes = [p, i64, i64, ctypes.c_double, i64, p]
    lib.oracle_sssp_f64.restype = ctypes.c_int
    lib.oracle_sssp_rows_i32.argtypes = [p, i64, i64, i32, p, i64, p, i64]
    lib.oracle_sssp_rows_i32.restype = ctypes.c_int
    lib.oracle_sssp_rows_f64.argtypes = [p, i64, i64, ctypes.c_double, p, i64, p, i64]
    lib.oracle_sssp_rows_f64.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    if path == LIB:
        _lib = lib
    return lib


class Oracle:
    """Bound view of one oracle build (the default one, or a test's variant)."""

    def __init__(self, path: str = LIB):
        self.lib = load(path)

    def set_threads(self, t: int) -> None:
        self.lib.oracle_set_threads(int(t))

    def threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def fw_i32(self, m: np.ndarray, k_end: int | None = None) -> np.ndarray:
        a = np.array(m, dtype=np.int32, order="C", copy=True)
        n = a.shape[0]
        ld = a.shape[1] if a.ndim == 2 and n else max(n, 1)
        self.lib.oracle_fw_i32(a.ctypes.data, n, ld, n if k_end is None else int(k_end))
        return a

    def fw_f64(self, m: np.ndarray, k_end: int | None = None) -> np.ndarray:
        a = np.array(m, dtype=np.float64, order="C", copy=True)
        n = a.shape[0]
        ld = a.shape[1] if a.ndim == 2 and n else max(n, 1)
        self.lib.oracle_fw_f64(a.ctypes.data, n, ld, n if k_end is None else int(k_end))
        return a

    def fw_in_steps(self, m: np.ndarray, step: int, progress=None) -> np.ndarray:
        """The whole recurrence (int32 stays int32; floats in binary64) on a
        copy, run as consecutive pivot ranges of `step` pivots.  After each
        range, progress(k_done, n) is called; the result is the same as one
        fw_i32 / fw_f64 call, since the ranges take the pivots in order."""
        is_int = np.asarray(m).dtype == np.int32
        a = np.array(m, dtype=np.int32 if is_int else np.float64, order="C", copy=True)
        n = a.shape[0]
        ld = a.shape[1] if a.ndim == 2 and n else max(n, 1)
        fn = self.lib.oracle_fw_range_i32 if is_int else self.lib.oracle_fw_range_f64
        step = max(1, int(step))
        for k0 in range(0, n, step):
            k1 = min(n, k0 + step)
            fn(a.ctypes.data, n, ld, k0, k1)
            if progress is not None:
                progress(k1, n)
        return a

    def fw_batched_i32(self, m: np.ndarray) -> np.ndarray:
        """Every graph of a (batch, n, ld) int32 array, closed independently."""
        a = np.array(m, dtype=np.int32, order="C", copy=True)
        b, n, ld = a.shape
        if b and n:
            self.lib.oracle_fw_batched_i32(a.ctypes.data, b, n, ld, n * ld)
        return a

    def fw_batched_f64(self, m: np.ndarray) -> np.ndarray:
        """Every graph of a (batch, n, ld) array in binary64 (float32 inputs
        are widened exactly)."""
        a = np.array(m, dtype=np.float64, order="C", copy=True)
        b, n, ld = a.shape
        if b and n:
            self.lib.oracle_fw_batched_f64(a.ctypes.data, b, n, ld, n * ld)
        return a

    def fw_guarded(self, m: np.ndarray, inf: int):
        """Shortest distances with negative weights allowed: returns
        (distances as int64, has_negative_cycle).  Entries equal to inf are
        "no edge"; candidates through inf are never formed."""
        a = np.array(m, dtype=np.int64, order="C", copy=True)
        n = a.shape[0]
        ld = a.shape[1] if a.ndim == 2 and n else max(n, 1)
        neg = self.lib.oracle_fw_guarded_i64(a.ctypes.data, n, ld, int(inf)) if n else 0
        return a, bool(neg)

    def sssp_rows_i32(self, w: np.ndarray, inf: int, srcs) -> np.ndarray:
        a = np.ascontiguousarray(w, dtype=np.int32)
        n, ld = a.shape[0], a.shape[1]
        s = np.ascontiguousarray(np.asarray(srcs, dtype=np.int64))
        out = np.empty((len(s), max(n, 1)), dtype=np.int32)
        if len(s):
            rc = self.lib.oracle_sssp_rows_i32(a.ctypes.data, n, ld, int(inf),
                                               s.ctypes.data, len(s), out.ctypes.data,
                                               out.shape[1])
            if rc != 0:
                raise ValueError("oracle_sssp_rows_i32 rejected its arguments")
        return out[:, :n]

    def sssp_rows_f64(self, w: np.ndarray, inf: float, srcs) -> np.ndarray:
        a = np.ascontiguousarray(w, dtype=np.float64)
        n, ld = a.shape[0], a.shape[1]
        s = np.ascontiguousarray(np.asarray(srcs, dtype=np.int64))
        out = np.empty((len(s), max(n, 1)), dtype=np.float64)
        if len(s):
            rc = self.lib.oracle_sssp_rows_f64(a.ctypes.data, n, ld, float(inf),
                                               s.ctypes.data, len(s), out.ctypes.data,
                                               out.shape[1])
            if rc != 0:
                raise ValueError("oracle_sssp_rows_f64 rejected its arguments")
        return out[:, :n]

    def bf_rows_csr(self, row_ptr, col, w, n: int, srcs, inf: int):
        """Bellman-Ford from each listed source over a CSR graph (weights may
        be negative).  Returns (rows as int64 with `inf` for unreached
        vertices, per-source negative-cycle flags)."""
        rp = np.ascontiguousarray(row_ptr, dtype=np.int64)
        c = np.ascontiguousarray(col, dtype=np.int32)
        wt = np.ascontiguousarray(w, dtype=np.int64)
        s = np.ascontiguousarray(np.asarray(srcs, dtype=np.int64))
        out = np.empty((len(s), max(n, 1)), dtype=np.int64)
        neg = np.zeros(len(s), dtype=np.int32)
        if len(s):
            rc = self.lib.oracle_sssp_bf_rows_i64(rp.ctypes.data, c.ctypes.data, wt.ctypes.data,
                                                  n, s.ctypes.data, len(s), out.ctypes.data,
                                                  out.shape[1], neg.ctypes.data)
            if rc != 0:
                raise ValueError("oracle_sssp_bf_rows_i64 rejected its arguments")
        out = out[:, :n]
        out[out == np.iinfo(np.int64).max] = inf
        return out, neg.astype(bool)

    def johnson_potentials(self, row_ptr, col, w, n: int):
        """The potentials h of Johnson's algorithm as the page builds them:
        extendGraph adds vertex n with a 0-weight edge to every vertex, and
        Bellman-Ford from it gives h(v), the shortest distance from the added
        vertex.  Returns (h as int64 [n], has_negative_cycle)."""
        rp = np.asarray(row_ptr, dtype=np.int64)
        ext_rp = np.concatenate([rp, [rp[-1] + n]])
        ext_col = np.concatenate([np.asarray(col, dtype=np.int32), np.arange(n, dtype=np.int32)])
        ext_w = np.concatenate([np.asarray(w, dtype=np.int64), np.zeros(n, dtype=np.int64)])
        rows, neg = self.bf_rows_csr(ext_rp, ext_col, ext_w, n + 1, [n], inf=0)
        return rows[0, :n].copy(), bool(neg[0])

    def minplus(self, c, a, b, inf=None):
        """min(c, a (x) b) as a new array.  Integer inputs: int64 arithmetic,
        entries equal to inf are "no path" (never summed).  Float inputs:
        binary64 (+inf sums to +inf by itself)."""
        if np.issubdtype(np.asarray(c).dtype, np.integer):
            cc = np.array(c, dtype=np.int64, order="C", copy=True)
            aa = np.ascontiguousarray(a, dtype=np.int64)
            bb = np.ascontiguousarray(b, dtype=np.int64)
            m, n = cc.shape
            k = aa.shape[1]
            if m and n and k:
                self.lib.oracle_minplus_i64(cc.ctypes.data, n, aa.ctypes.data, k, bb.ctypes.data,
                                            n, m, n, k, int(inf))
            return cc
        cc = np.array(c, dtype=np.float64, order="C", copy=True)
        aa = np.ascontiguousarray(a, dtype=np.float64)
        bb = np.ascontiguousarray(b, dtype=np.float64)
        m, n = cc.shape
        k = aa.shape[1]
        if m and n and k:
            self.lib.oracle_minplus_f64(cc.ctypes.data, n, aa.ctypes.data, k, bb.ctypes.data, n,
                                        m, n, k)
        return cc

    def successors(self, w, d, inf):
        """First-hop matrix (int32) of weights w and distances d (both n x n
        integer arrays): smallest u != i minimising w[i][u] + d[u][j] over
        the candidates below inf; -1 when there is none (j unreachable, as a
        distance that is not below inf is), i on the diagonal."""
        ww = np.ascontiguousarray(w, dtype=np.int64)
        dd = np.ascontiguousarray(d, dtype=np.int64)
        n = ww.shape[0]
        nxt = np.empty((n, n), dtype=np.int32)
        if n:
            self.lib.oracle_successors_i64(ww.ctypes.data, dd.ctypes.data, nxt.ctypes.data, n, n,
                                           int(inf))
        return nxt

    def successors_rows(self, w, d, inf, rows):
        """Rows `rows` of successors(w, d, inf), without the others (for spot
        checks of large matrices): an int32 (len(rows), n) array."""
        dd = np.ascontiguousarray(d, dtype=np.int64)
        n = dd.shape[0]
        rr = np.ascontiguousarray(rows, dtype=np.int64)
        wr = np.ascontiguousarray(np.asarray(w)[rr, :n], dtype=np.int64)
        out = np.empty((len(rr), n), dtype=np.int32)
        if len(rr) and n:
            self.lib.oracle_successors_rows_i64(wr.ctypes.data, dd.ctypes.data, rr.ctypes.data,
                                                len(rr), out.ctypes.data, n, int(inf))
        return out

    def apsp(self, m: np.ndarray) -> np.ndarray:
        """Full distance matrix: int32 stays int32, float32 becomes float64."""
        if m.dtype == np.int32:
            return self.fw_i32(m)
        return self.fw_f64(m.astype(np.float64))


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def fw_i32(m, k_end=None):
    return default().fw_i32(m, k_end)


def fw_f64(m, k_end=None):
    return default().fw_f64(m, k_end)


def sssp_rows_i32(w, inf, srcs):
    return default().sssp_rows_i32(w, inf, srcs)


def sssp_rows_f64(w, inf, srcs):
    return default().sssp_rows_f64(w, inf, srcs)


def apsp(m):
    return default().apsp(m)
