"""Seeded synthetic inputs for all-pairs shortest paths (APSP).

This module builds the dense distance/weight matrices that both the HIP path
and the CPU oracle consume.  It holds no shortest-path arithmetic at all: it
only decides which edges exist and what their weights are, and lays the
result out as a row-major matrix with a leading dimension ``ld >= n``.

Matrix convention (the one every consumer assumes):
  * ``W[i, j]`` is the weight of the directed edge i -> j,
  * ``W[i, i] = 0``,
  * ``W[i, j] = inf`` (the caller's sentinel) when there is no edge,
  * columns ``n .. ld-1`` of every row are padding, filled with ``canary``.

Randomness is counter based, so every entry can be produced independently
and in any order: ``u64(seed, stream, counter)`` is the SplitMix64 output
function (Steele, Lea & Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014) applied to a key derived from (seed, stream) plus
``(counter + 1)`` times the golden-ratio increment.  Integer uniforms on
[lo, hi] use Lemire's multiply-shift reduction of the top 32 bits.

Graph families follow the workloads on the pages:
  * directed Erdos-Renyi G(n, p): each ordered pair i != j is an edge with
    probability p, independently (no self loops);
  * complete digraph: every ordered pair i != j is an edge;
  * Barabasi-Albert preferential attachment (the scale-free generator used
    for the betweenness-centrality page's inputs, "Study of Betweenness
    Centrality Algorithms in GPU", experimental setup): beta undirected edges
    per new vertex, each stored as two directed edges with one shared weight;
  * small structured graphs (rings, paths, grids, disjoint rings) whose
    shortest distances have closed forms;
  * graphs with negative weights but no negative cycle (for Johnson's
    algorithm): non-negative weights w0 shifted by vertex potentials,
    w(u, v) = w0(u, v) + p(u) - p(v), so every cycle keeps its w0 length;
  * batches of many small independent graphs (the "many small graphs" case of
    the page "Loops into zones"): graph g of a batch draws the same families
    with counters offset by g * n * n, laid out as a (batch, n, ld) array.
"""
from __future__ import annotations

import hashlib

import numpy as np

__all__ = [
    "INF_I32", "GAMMA", "mix64", "u64", "u64_array",
    "erdos_renyi", "complete", "complete_f32", "barabasi_albert",
    "ring", "undirected_path", "grid", "complete_equal", "edgeless",
    "two_rings", "WORKLOADS", "make_workload", "sha256_matrix", "pad_ld",
    "erdos_renyi_batch", "complete_f32_batch", "BATCH_WORKLOADS", "make_batch_workload",
    "erdos_renyi_potential", "csr_from_dense", "JOHNSON_WORKLOADS", "make_johnson_workload",
    "regular_out_csr",
]

INF_I32 = 0x3FFFFFFF          # the int32 "no edge" sentinel of the workloads
GAMMA = 0x9E3779B97F4A7C15    # SplitMix64 increment (odd, ~2^64 / phi)
_M64 = (1 << 64) - 1

# Streams: one independent counter space per purpose.
_S_EDGE, _S_WEIGHT, _S_BA_PICK, _S_BA_WEIGHT, _S_POTENTIAL = 1, 2, 3, 4, 5


def mix64(z: int) -> int:
    """SplitMix64 output mix of one 64-bit word (Python int)."""
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def _key(seed: int, stream: int) -> int:
    return mix64(((seed & _M64) * GAMMA + (stream & 0xFFFFFFFF)) & _M64)


def u64(seed: int, stream: int, counter: int) -> int:
    """One 64-bit random word for (seed, stream, counter)."""
    return mix64((_key(seed, stream) + ((counter + 1) * GAMMA)) & _M64)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = z.copy()
    z ^= z >> np.uint64(30)
    z *= np.uint64(0xBF58476D1CE4E5B9)
    z ^= z >> np.uint64(27)
    z *= np.uint64(0x94D049BB133111EB)
    z ^= z >> np.uint64(31)
    return z


def u64_array(seed: int, stream: int, counters: np.ndarray) -> np.ndarray:
    """Vectorised ``u64``: same values as the scalar function, elementwise."""
    c = np.asarray(counters, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(_key(seed, stream)) + (c + np.uint64(1)) * np.uint64(GAMMA)
        return _mix64_np(z)


def _uniform_int(u: np.ndarray, lo: int, hi: int) -> np.ndarray:
    """Lemire multiply-shift: top 32 bits of u scaled onto [lo, hi]."""
    span = np.uint64(hi - lo + 1)
    return (np.int64(lo) + ((u >> np.uint64(32)) * span >> np.uint64(32)).astype(np.int64))


def _uniform01(u: np.ndarray) -> np.ndarray:
    """Top 53 bits as a double in [0, 1)."""
    return (u >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def pad_ld(n: int, multiple: int = 1) -> int:
    """Smallest ld >= max(n, 1) that is a multiple of ``multiple``."""
    m = max(int(multiple), 1)
    return max(((max(n, 1) + m - 1) // m) * m, 1)


def _alloc(n: int, ld: int | None, dtype, inf, canary):
    ld = n if ld is None else int(ld)
    if ld < max(n, 1):
        raise ValueError("ld must be >= max(n, 1)")
    m = np.full((n, ld), inf, dtype=dtype)
    if ld > n:
        m[:, n:] = canary
    return m


def _rows_chunks(n: int, chunk_elems: int = 1 << 23):
    step = max(1, chunk_elems // max(n, 1))
    for r0 in range(0, n, step):
        yield r0, min(n, r0 + step)


def erdos_renyi(n: int, p: float, wlo: int, whi: int, seed: int,
                inf: int = INF_I32, ld: int | None = None,
                canary: int = -7) -> np.ndarray:
    """Directed G(n, p) with integer weights uniform on [wlo, whi] (int32)."""
    m = _alloc(n, ld, np.int32, inf, canary)
    j = np.arange(n, dtype=np.uint64)
    for r0, r1 in _rows_chunks(n):
        i = np.arange(r0, r1, dtype=np.uint64)[:, None]
        idx = i * np.uint64(n) + j[None, :]
        edge = _uniform01(u64_array(seed, _S_EDGE, idx)) < p
        w = _uniform_int(u64_array(seed, _S_WEIGHT, idx), wlo, whi)
        blk = np.where(edge, w, inf).astype(np.int32)
        ii = np.arange(r0, r1)
        blk[ii - r0, ii] = 0
        m[r0:r1, :n] = blk
    return m


def complete(n: int, wlo: int, whi: int, seed: int, inf: int = INF_I32,
             ld: int | None = None, canary: int = -7, out: np.ndarray | None = None) -> np.ndarray:
    """Complete digraph with integer weights uniform on [wlo, whi] (int32).
    With ``out`` (an int32 array of shape (n, >= n), e.g. a view of pinned
    host memory) the matrix is written there in row chunks."""
    if out is not None:
        if out.dtype != np.int32 or out.ndim != 2 or out.shape[0] != n or out.shape[1] < n:
            raise ValueError("out must be an int32 (n, >= n) array")
        m = out
    else:
        m = _alloc(n, ld, np.int32, inf, canary)
    j = np.arange(n, dtype=np.uint64)
    for r0, r1 in _rows_chunks(n):
        i = np.arange(r0, r1, dtype=np.uint64)[:, None]
        idx = i * np.uint64(n) + j[None, :]
        blk = _uniform_int(u64_array(seed, _S_WEIGHT, idx), wlo, whi).astype(np.int32)
        ii = np.arange(r0, r1)
        blk[ii - r0, ii] = 0
        m[r0:r1, :n] = blk
    return m


def complete_f32(n: int, seed: int, wlo: float = 0.01, whi: float = 1.0,
                 ld: int | None = None, canary: float = -7.0,
                 inf: float = float("inf")) -> np.ndarray:
    """Complete digraph with float32 weights wlo + (whi - wlo) * u, u in [0, 1)
    drawn with 24 random bits (so the open upper end is never hit)."""
    m = _alloc(n, ld, np.float32, inf, canary)
    j = np.arange(n, dtype=np.uint64)
    for r0, r1 in _rows_chunks(n):
        i = np.arange(r0, r1, dtype=np.uint64)[:, None]
        idx = i * np.uint64(n) + j[None, :]
        u24 = (u64_array(seed, _S_WEIGHT, idx) >> np.uint64(40)).astype(np.float64)
        blk = (wlo + (whi - wlo) * (u24 * (1.0 / 16777216.0))).astype(np.float32)
        ii = np.arange(r0, r1)
        blk[ii - r0, ii] = 0.0
        m[r0:r1, :n] = blk
    return m


def barabasi_albert_edges(n: int, beta: int, seed: int) -> np.ndarray:
    """Undirected edge list (m x 2) of a Barabasi-Albert graph.

    Start from ``beta`` isolated seed vertices.  Vertex ``beta`` links to all
    of them; every later vertex v links to ``beta`` distinct earlier vertices,
    each drawn with probability proportional to its current degree (uniform
    pick from the list of all edge endpoints so far, redrawn on a repeat).
    """
    if n <= beta:
        return np.zeros((0, 2), dtype=np.int64)
    m = beta * (n - beta)
    endpoints = np.empty(2 * m, dtype=np.int64)
    edges = np.empty((m, 2), dtype=np.int64)
    ne = 0
    # Random words are consumed strictly in counter order; they are produced
    # in batches only to keep the Python loop cheap.
    batch = 1 << 14
    buf = u64_array(seed, _S_BA_PICK, np.arange(batch, dtype=np.uint64)) >> np.uint64(32)
    buf = buf.tolist()
    counter = 0
    for v in range(beta, n):
        if v == beta:
            targets = list(range(beta))
        else:
            chosen: set[int] = set()
            targets = []
            total = 2 * ne
            while len(targets) < beta:
                k = counter % batch
                if k == 0 and counter:
                    buf = (u64_array(seed, _S_BA_PICK,
                                     np.arange(counter, counter + batch, dtype=np.uint64))
                           >> np.uint64(32)).tolist()
                r = buf[k]
                counter += 1
                t = int(endpoints[(r * total) >> 32])
                if t not in chosen:
                    chosen.add(t)
                    targets.append(t)
        for t in targets:
            edges[ne, 0] = v
            edges[ne, 1] = t
            endpoints[2 * ne] = v
            endpoints[2 * ne + 1] = t
            ne += 1
    return edges[:ne]


def barabasi_albert(n: int, beta: int, wlo: int, whi: int, seed: int,
                    inf: int = INF_I32, ld: int | None = None,
                    canary: int = -7) -> np.ndarray:
    """Symmetric int32 matrix of a BA graph: one weight per undirected edge,
    uniform on [wlo, whi], stored in both directions."""
    m = _alloc(n, ld, np.int32, inf, canary)
    e = barabasi_albert_edges(n, beta, seed)
    if len(e):
        w = _uniform_int(u64_array(seed, _S_BA_WEIGHT, np.arange(len(e))), wlo, whi).astype(np.int32)
        m[e[:, 0], e[:, 1]] = w
        m[e[:, 1], e[:, 0]] = w
    ii = np.arange(n)
    m[ii, ii] = 0
    return m


# ---- structured graphs with closed-form distances ------------------------

def _blank(n, ld, dtype, inf, canary):
    m = _alloc(n, ld, dtype, inf, canary)
    ii = np.arange(n)
    m[ii, ii] = 0
    return m


def ring(n: int, w=1, directed: bool = True, dtype=np.int32, inf=INF_I32,
         ld: int | None = None, canary=-7, reverse: bool = False) -> np.ndarray:
    """Ring i -> i+1 (mod n) of weight w (or i -> i-1 when ``reverse``);
    both directions when not ``directed``."""
    m = _blank(n, ld, dtype, inf, canary)
    if n >= 2:
        i = np.arange(n)
        nxt = (i - 1) % n if reverse else (i + 1) % n
        m[i, nxt] = w
        if not directed:
            m[nxt, i] = w
    return m


def undirected_path(n: int, w=1, dtype=np.int32, inf=INF_I32,
                    ld: int | None = None, canary=-7) -> np.ndarray:
    """Path 0 - 1 - ... - (n-1), both directions, weight w."""
    m = _blank(n, ld, dtype, inf, canary)
    if n >= 2:
        i = np.arange(n - 1)
        m[i, i + 1] = w
        m[i + 1, i] = w
    return m


def grid(rows: int, cols: int, w=1, dtype=np.int32, inf=INF_I32,
         ld: int | None = None, canary=-7) -> np.ndarray:
    """rows x cols 4-neighbour grid, both directions, weight w; vertex
    (r, c) has index r * cols + c."""
    n = rows * cols
    m = _blank(n, ld, dtype, inf, canary)
    for r in range(rows):
        for c in range(cols):
            v = r * cols + c
            if c + 1 < cols:
                m[v, v + 1] = w
                m[v + 1, v] = w
            if r + 1 < rows:
                m[v, v + cols] = w
                m[v + cols, v] = w
    return m


def complete_equal(n: int, w=1, dtype=np.int32, inf=INF_I32,
                   ld: int | None = None, canary=-7) -> np.ndarray:
    m = _alloc(n, ld, dtype, inf, canary)
    m[:, :n] = w
    ii = np.arange(n)
    m[ii, ii] = 0
    return m


def edgeless(n: int, dtype=np.int32, inf=INF_I32, ld: int | None = None,
             canary=-7) -> np.ndarray:
    return _blank(n, ld, dtype, inf, canary)


def two_rings(n1: int, n2: int, w=1, dtype=np.int32, inf=INF_I32,
              ld: int | None = None, canary=-7) -> np.ndarray:
    """Directed ring on vertices [0, n1) and another on [n1, n1+n2)."""
    n = n1 + n2
    m = _blank(n, ld, dtype, inf, canary)
    for base, k in ((0, n1), (n1, n2)):
        if k >= 2:
            i = np.arange(k)
            m[base + i, base + (i + 1) % k] = w
    return m


def _alloc_batch(batch: int, n: int, ld: int | None, dtype, inf, canary):
    ld = n if ld is None else int(ld)
    if ld < max(n, 1):
        raise ValueError("ld must be >= max(n, 1)")
    m = np.full((batch, n, ld), inf, dtype=dtype)
    if ld > n:
        m[:, :, n:] = canary
    return m


def _batch_chunks(batch: int, n: int, chunk_elems: int = 1 << 23):
    step = max(1, chunk_elems // max(n * n, 1))
    for g0 in range(0, batch, step):
        yield g0, min(batch, g0 + step)


def erdos_renyi_batch(batch: int, n: int, p: float, wlo: int, whi: int, seed: int,
                      inf: int = INF_I32, ld: int | None = None,
                      canary: int = -7) -> np.ndarray:
    """``batch`` independent directed G(n, p) graphs with integer weights
    uniform on [wlo, whi]; shape (batch, n, ld), int32."""
    m = _alloc_batch(batch, n, ld, np.int32, inf, canary)
    ij = np.arange(n * n, dtype=np.uint64).reshape(n, n)
    for g0, g1 in _batch_chunks(batch, n):
        g = np.arange(g0, g1, dtype=np.uint64)[:, None, None]
        idx = g * np.uint64(n * n) + ij[None]
        edge = _uniform01(u64_array(seed, _S_EDGE, idx)) < p
        w = _uniform_int(u64_array(seed, _S_WEIGHT, idx), wlo, whi)
        blk = np.where(edge, w, inf).astype(np.int32)
        d = np.arange(n)
        blk[:, d, d] = 0
        m[g0:g1, :, :n] = blk
    return m


def complete_f32_batch(batch: int, n: int, seed: int, wlo: float = 0.01, whi: float = 1.0,
                       ld: int | None = None, canary: float = -7.0,
                       inf: float = float("inf")) -> np.ndarray:
    """``batch`` independent complete digraphs with float32 weights as in
    ``complete_f32``; shape (batch, n, ld)."""
    m = _alloc_batch(batch, n, ld, np.float32, inf, canary)
    ij = np.arange(n * n, dtype=np.uint64).reshape(n, n)
    for g0, g1 in _batch_chunks(batch, n):
        g = np.arange(g0, g1, dtype=np.uint64)[:, None, None]
        idx = g * np.uint64(n * n) + ij[None]
        u24 = (u64_array(seed, _S_WEIGHT, idx) >> np.uint64(40)).astype(np.float64)
        blk = (wlo + (whi - wlo) * (u24 * (1.0 / 16777216.0))).astype(np.float32)
        d = np.arange(n)
        blk[:, d, d] = 0.0
        m[g0:g1, :, :n] = blk
    return m


def erdos_renyi_potential(n: int, p: float, wlo: int, whi: int, plo: int, phi: int,
                          seed: int, inf: int = INF_I32, ld: int | None = None,
                          canary: int = -7) -> np.ndarray:
    """Directed G(n, p) whose weights may be negative but whose cycles are
    not: w(u, v) = w0(u, v) + pot(u) - pot(v) with w0 uniform on [wlo, whi]
    (wlo >= 0) and vertex potentials pot uniform on [plo, phi] (int32)."""
    m = erdos_renyi(n, p, wlo, whi, seed, inf=inf, ld=ld, canary=canary)
    pot = _uniform_int(u64_array(seed, _S_POTENTIAL, np.arange(n, dtype=np.uint64)), plo, phi)
    blk = m[:, :n].astype(np.int64)
    edge = (blk != inf) & ~np.eye(n, dtype=bool)
    blk = np.where(edge, blk + pot[:, None] - pot[None, :], blk)
    m[:, :n] = blk.astype(np.int32)
    return m


def regular_out_csr(n: int, deg: int, wlo: int, whi: int, seed: int, plo: int = 0,
                    phi: int = 0):
    """A sparse digraph built straight in CSR form (no dense matrix), for
    vertex counts whose n x n matrix would not fit the host: every vertex u
    has ``deg`` out-edges to targets u + 1 + (r mod (n - 1)) (mod n), r drawn
    per edge, so never u itself (parallel edges may occur).  Weights w0 are
    uniform on [wlo, whi]; with phi > plo every edge is shifted by vertex
    potentials p uniform on [plo, phi]: w = w0 + p(u) - p(v), which leaves
    every cycle's weight unchanged (no negative cycle when w0 >= 0).
    Returns (row_ptr int64 [n+1], col int32 [n*deg], w int32 [n*deg])."""
    if n < 2:
        raise ValueError("needs n >= 2")
    m = n * deg
    e = np.arange(m, dtype=np.uint64)
    u = (np.arange(m, dtype=np.int64) // deg)
    r = (u64_array(seed, _S_EDGE, e) >> np.uint64(1)) % np.uint64(n - 1)
    col = ((u + 1 + r.astype(np.int64)) % n).astype(np.int32)
    w = _uniform_int(u64_array(seed, _S_WEIGHT, e), wlo, whi)
    if phi > plo:
        pot = _uniform_int(u64_array(seed, _S_POTENTIAL, np.arange(n, dtype=np.uint64)), plo, phi)
        w = w + pot[u] - pot[col]
    row_ptr = np.arange(n + 1, dtype=np.int64) * deg
    return row_ptr, col, w.astype(np.int32)


def csr_from_dense(m: np.ndarray, inf, n: int | None = None):
    """Compressed sparse rows of the edges of a dense matrix: every (u, v)
    with u != v and m[u, v] != inf.  Returns (row_ptr int64 [n+1],
    col int32 [nnz], weight [nnz] in m's dtype), rows in order, columns
    ascending within a row."""
    n = m.shape[0] if n is None else n
    blk = m[:n, :n]
    mask = blk != inf
    np.fill_diagonal(mask, False)
    counts = mask.sum(axis=1)
    row_ptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    rows, cols = np.nonzero(mask)
    return row_ptr, cols.astype(np.int32), blk[rows, cols]


# ---- the named workloads --------------------------------------------------

WORKLOADS = {
    # name: (builder, description)
    "er-256-p0.1-i32": dict(kind="er", n=256, p=0.1, wlo=1, whi=100, seed=1, dtype="i32"),
    "er-2048-p0.05-i32": dict(kind="er", n=2048, p=0.05, wlo=1, whi=1000, seed=2, dtype="i32"),
    "complete-8192-i32": dict(kind="complete", n=8192, wlo=1, whi=10000, seed=3, dtype="i32"),
    "ba-16000-b8-i32": dict(kind="ba", n=16000, beta=8, wlo=1, whi=255, seed=4, dtype="i32"),
    "complete-12288-f32": dict(kind="complete_f32", n=12288, seed=5, dtype="f32"),
}

# Host-resident matrices for the out-of-core path: the matrix stays in
# (pinned) host memory and streams through a device budget smaller than it.
HOST_WORKLOADS = {
    # a 4 GiB matrix in pinned host memory, 3 GiB of device memory to run in
    "host-complete-32768-i32": dict(kind="complete", n=32768, wlo=1, whi=10000, seed=6,
                                    device_budget=3 << 30),
}


def make_workload(name: str, ld: int | None = None) -> np.ndarray:
    """Build one of the named workloads (row-major, leading dimension ld)."""
    w = WORKLOADS[name]
    k = w["kind"]
    if k == "er":
        return erdos_renyi(w["n"], w["p"], w["wlo"], w["whi"], w["seed"], ld=ld)
    if k == "complete":
        return complete(w["n"], w["wlo"], w["whi"], w["seed"], ld=ld)
    if k == "ba":
        return barabasi_albert(w["n"], w["beta"], w["wlo"], w["whi"], w["seed"], ld=ld)
    if k == "complete_f32":
        return complete_f32(w["n"], w["seed"], ld=ld)
    raise KeyError(name)


# Batches of many small graphs: (batch, n, ld) arrays, one graph per
# workgroup on the GPU.
BATCH_WORKLOADS = {
    "batch-er-8192x128-p0.1-i32": dict(kind="er", batch=8192, n=128, p=0.1, wlo=1, whi=100,
                                       seed=11, dtype="i32"),
    "batch-er-131072x32-p0.2-i32": dict(kind="er", batch=131072, n=32, p=0.2, wlo=1, whi=100,
                                        seed=12, dtype="i32"),
    "batch-complete-8192x100-f32": dict(kind="complete_f32", batch=8192, n=100, seed=13,
                                        dtype="f32"),
}


# Sparse graphs for Johnson's algorithm (CSR on the device, dense n x n
# distances out).  The two sparse configurations of the dense workloads, and
# a graph with negative weights.
JOHNSON_WORKLOADS = {
    "johnson-ba-16000-b8-i32": dict(dense="ba-16000-b8-i32"),
    "johnson-er-2048-p0.05-i32": dict(dense="er-2048-p0.05-i32"),
    "johnson-er-8192-p0.002-neg-i32": dict(kind="er_potential", n=8192, p=0.002, wlo=0,
                                           whi=1000, plo=-500, phi=500, seed=21),
}


def make_johnson_workload(name: str) -> np.ndarray:
    """Dense matrix of one of the Johnson workloads (row-major, ld = n)."""
    w = JOHNSON_WORKLOADS[name]
    if "dense" in w:
        return make_workload(w["dense"])
    return erdos_renyi_potential(w["n"], w["p"], w["wlo"], w["whi"], w["plo"], w["phi"], w["seed"])


def make_batch_workload(name: str, ld: int | None = None) -> np.ndarray:
    """Build one of the named batch workloads, shape (batch, n, ld)."""
    w = BATCH_WORKLOADS[name]
    if w["kind"] == "er":
        return erdos_renyi_batch(w["batch"], w["n"], w["p"], w["wlo"], w["whi"], w["seed"], ld=ld)
    if w["kind"] == "complete_f32":
        return complete_f32_batch(w["batch"], w["n"], w["seed"], ld=ld)
    raise KeyError(name)


def sha256_matrix(m: np.ndarray, n: int | None = None) -> str:
    """SHA-256 of the logical n x n block, row-major, native byte order."""
    n = m.shape[0] if n is None else n
    return hashlib.sha256(np.ascontiguousarray(m[:n, :n]).tobytes()).hexdigest()
