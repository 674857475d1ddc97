"""Helpers used by the tests only (golden parsing, brute force, checks)."""
from __future__ import annotations

import itertools
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name: str, inf) -> dict:
    """Parse a golden text fixture into {section: matrix}."""
    sections: dict[str, list[list]] = {}
    cur = None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("["):
                cur = line.strip("[]")
                sections[cur] = []
                continue
            sections[cur].append([inf if t == "inf" else int(t) for t in line.split()])
    return {k: np.array(v) for k, v in sections.items()}


def brute_force_apsp(w: np.ndarray, inf):
    """Minimum over every simple path (exhaustive DFS); n <= 8 only.

    With non-negative weights some shortest walk is a simple path, so this is
    the definition of the shortest-path distance, evaluated literally.
    Sums are Python ints / floats in path order.
    """
    n = w.shape[0]
    assert n <= 8
    best = [[inf] * n for _ in range(n)]
    adj = [[(v, w[u, v]) for v in range(n) if v != u and w[u, v] != inf] for u in range(n)]

    for s in range(n):
        best[s][s] = 0 if not isinstance(inf, float) else 0.0
        stack = [(s, 0 if not isinstance(inf, float) else 0.0, 1 << s)]
        while stack:
            u, dist, seen = stack.pop()
            for v, wt in adj[u]:
                if seen >> v & 1:
                    continue
                nd = dist + (int(wt) if not isinstance(inf, float) else float(wt))
                if nd < best[s][v]:
                    best[s][v] = nd
                stack.append((v, nd, seen | (1 << v)))
    return np.array(best, dtype=object)


def reachability(w: np.ndarray, inf) -> np.ndarray:
    """Boolean reach[i, j]: j reachable from i (BFS over the edge set)."""
    n = w.shape[0]
    adj = [np.nonzero((w[u, :n] != inf) & (np.arange(n) != u))[0] for u in range(n)]
    reach = np.zeros((n, n), dtype=bool)
    for s in range(n):
        seen = np.zeros(n, dtype=bool)
        seen[s] = True
        frontier = [s]
        while frontier:
            nxt = []
            for u in frontier:
                for v in adj[u]:
                    if not seen[v]:
                        seen[v] = True
                        nxt.append(v)
            frontier = nxt
        reach[s] = seen
    return reach


def triangle_ok(d: np.ndarray, ks=None) -> bool:
    """d[i, j] <= d[i, k] + d[k, j] for the given pivots (all when None)."""
    n = d.shape[0]
    dd = d.astype(np.float64) if d.dtype.kind == "f" else d.astype(np.int64)
    ks = range(n) if ks is None else ks
    for k in ks:
        if np.any(dd > dd[:, k:k + 1] + dd[k:k + 1, :]):
            return False
    return True


def bellman_rows_ok(w: np.ndarray, d: np.ndarray, rows, inf) -> bool:
    """Bellman optimality on the given rows, for strictly positive weights:
    d[i, j] = min over k != i with an edge (i, k) of w[i, k] + d[k, j],
    for every j != i (inf when no such k gives a finite value)."""
    n = d.shape[0]
    big = np.int64(inf) if w.dtype.kind != "f" else np.float64(inf)
    for i in rows:
        nb = np.nonzero((w[i, :n] != inf) & (np.arange(n) != i))[0]
        if len(nb) == 0:
            want = np.full(n, big)
        else:
            want = (w[i, nb].astype(np.int64 if w.dtype.kind != "f" else np.float64)[:, None]
                    + d[nb, :n].astype(np.int64 if w.dtype.kind != "f" else np.float64)).min(axis=0)
            want = np.minimum(want, big)
        want[i] = 0
        if not np.array_equal(want, d[i, :n].astype(want.dtype)):
            return False
    return True


def random_small_graph(rng: np.random.Generator, n: int, p: float, wmax: int, inf, floats=False):
    w = np.full((n, n), inf, dtype=np.float64 if floats else np.int32)
    mask = rng.random((n, n)) < p
    if floats:
        vals = np.round(rng.random((n, n)) * wmax, 3)
    else:
        vals = rng.integers(0, wmax + 1, size=(n, n))
    w[mask] = vals[mask]
    np.fill_diagonal(w, 0)
    return w
