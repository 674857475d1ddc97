"""The oracle's pins must be strong enough to catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (a dropped
term, a wrong sign, a transposed operand, a wrong index, a skipped pivot, a
wrong extraction order), builds the copy on the CPU, and runs a compact
battery of the same pins used in test_oracle_pins.py against it.  The battery
must fail for every mutant and pass for the unmodified source.
"""
import numpy as np
import pytest
import scipy.sparse.csgraph as csg

import graphgen as gg
import oracle
from _helpers import brute_force_apsp, random_small_graph, read_golden

INF = gg.INF_I32

MUTANTS = {
    # Floyd-Warshall, int32
    "fw_transposed_dik": ("int64_t d_ik = row_i[k];", "int64_t d_ik = d[k * ld + i];"),
    "fw_wrong_index_dkj": ("int64_t cand = d_ik + (int64_t)row_k[j];",
                           "int64_t cand = d_ik + (int64_t)row_k[i];"),
    "fw_dropped_term": ("int64_t cand = d_ik + (int64_t)row_k[j];",
                        "int64_t cand = (int64_t)row_k[j];"),
    "fw_row_i_for_row_k": ("int64_t cand = d_ik + (int64_t)row_k[j];",
                           "int64_t cand = d_ik + (int64_t)row_i[j];"),
    "fw_max_not_min": ("if (cand < row_i[j]) row_i[j] = (int32_t)cand;",
                       "if (cand > row_i[j]) row_i[j] = (int32_t)cand;"),
    "fw_skips_first_pivot": ("for (int64_t k = k_begin; k < k_end; ++k) {\n    const int32_t",
                             "for (int64_t k = k_begin + 1; k < k_end; ++k) {\n    const int32_t"),
    "fw_skips_last_pivot": ("int64_t k_begin, int64_t k_end) {\n  if (k_begin < 0) k_begin = 0;\n  if (k_end > n) k_end = n;\n  int nt = oracle_max_threads();\n  for (int64_t k = k_begin; k < k_end; ++k) {\n    const int32_t",
                            "int64_t k_begin, int64_t k_end) {\n  if (k_begin < 0) k_begin = 0;\n  if (k_end > n - 1) k_end = n - 1;\n  int nt = oracle_max_threads();\n  for (int64_t k = k_begin; k < k_end; ++k) {\n    const int32_t"),
    "fw_diagonal_only_rows": ("for (int64_t i = 0; i < n; ++i) {\n      int32_t *row_i",
                              "for (int64_t i = 0; i < n; i += 2) {\n      int32_t *row_i"),
    # Floyd-Warshall, binary64
    "fw64_max_not_min": ("if (cand < row_i[j]) row_i[j] = cand;",
                         "if (cand > row_i[j]) row_i[j] = cand;"),
    "fw64_transposed_dik": ("double d_ik = row_i[k];", "double d_ik = d[k * ld + i];"),
    "fw64_skips_first_pivot": ("for (int64_t k = k_begin; k < k_end; ++k) {\n    const double",
                               "for (int64_t k = k_begin + 1; k < k_end; ++k) {\n    const double"),
    "fw64_wrong_index_dkj": ("double cand = d_ik + row_k[j];", "double cand = d_ik + row_k[i];"),
    # Dijkstra, int32
    "sssp_extracts_max": ("(u < 0 || dist[v] < dist[u])) u = v;\n    if (u < 0) break;\n    settled[u] = 1;\n    const int32_t",
                          "(u < 0 || dist[v] > dist[u])) u = v;\n    if (u < 0) break;\n    settled[u] = 1;\n    const int32_t"),
    "sssp_transposed_edge": ("const int32_t *wu = w + u * ld;\n    for (int64_t v = 0; v < n; ++v) { /* RelaxEdge(u, v) */\n      if (v == u || wu[v] == inf) continue;\n      int64_t cand = dist[u] + (int64_t)wu[v];",
                             "const int32_t *wu = w + u * ld;\n    for (int64_t v = 0; v < n; ++v) { /* RelaxEdge(u, v) */\n      if (v == u || w[v * ld + u] == inf) continue;\n      int64_t cand = dist[u] + (int64_t)w[v * ld + u];"),
    "sssp_dropped_dist_u": ("int64_t cand = dist[u] + (int64_t)wu[v];", "int64_t cand = (int64_t)wu[v];"),
    # Floyd-Warshall with negative weights (INF-guarded), negative-cycle flag
    "guard_dropped_ik": ("      if (d_ik == inf) continue;\n", ""),
    "guard_dropped_kj": ("        if (row_k[j] == inf) continue;\n", ""),
    "guard_cycle_le": ("if (d[i * ld + i] < 0) return 1;", "if (d[i * ld + i] <= 0) return 1;"),
    "guard_cycle_never": ("if (d[i * ld + i] < 0) return 1;", "if (d[i * ld + i] < 0) return 0;"),
    "guard_skips_last_pivot": ("int oracle_fw_guarded_i64(int64_t *d, int64_t n, int64_t ld, int64_t inf) {\n  int nt = oracle_max_threads();\n  for (int64_t k = 0; k < n; ++k) {",
                               "int oracle_fw_guarded_i64(int64_t *d, int64_t n, int64_t ld, int64_t inf) {\n  int nt = oracle_max_threads();\n  for (int64_t k = 0; k < n - 1; ++k) {"),
    # Bellman-Ford from one source (CSR), negative-cycle result
    "bf_dropped_dist_u": ("const int64_t cand = dist[u] + w[e];", "const int64_t cand = w[e];"),
    "bf_max_not_min": ("if (cand < dist[v]) { dist[v] = cand; changed = 1; }",
                       "if (cand > dist[v] && dist[v] != INT64_MAX) { dist[v] = cand; changed = 1; }"),
    "bf_one_round_short": ("for (int64_t round = 0; round < n; ++round) {",
                           "for (int64_t round = 0; round < n - 1; ++round) {"),
    "bf_cycle_never": ("    if (!changed) return 0;\n  }\n  return 1;",
                       "    if (!changed) return 0;\n  }\n  return 0;"),
    "bf_edge_target_is_source": ("const int64_t v = col[e];", "const int64_t v = u;"),
    # successors
    "succ_largest_tie": ("if (arg < 0 || cand < best) { best = cand; arg = u; }",
                         "if (arg < 0 || cand <= best) { best = cand; arg = u; }"),
    "succ_self_allowed": ("if (u == i || w[i * ld + u] == inf || d[u * ld + j] == inf) continue;",
                          "if (w[i * ld + u] == inf || d[u * ld + j] == inf) continue;"),
    "succ_sentinel_sum_accepted": ("        if (cand >= inf) continue;", ""),
    # min-plus product
    "mp_transposed_b": ("const int64_t btj = b[t * ldb + j];", "const int64_t btj = b[j * ldb + t];"),
    "mp_ignores_c": ("        if (cand < c[i * ldc + j]) c[i * ldc + j] = cand;\n      }\n    }\n}\n\nvoid oracle_minplus_f64",
                     "        if (cand < c[i * ldc + j] || t == 0) c[i * ldc + j] = cand;\n      }\n    }\n}\n\nvoid oracle_minplus_f64"),
    "mp_last_t_skipped": ("    for (int64_t t = 0; t < k; ++t) {\n      const int64_t ait",
                          "    for (int64_t t = 0; t < k - 1; ++t) {\n      const int64_t ait"),
    "mp64_transposed_b": ("const double cand = ait + b[t * ldb + j];",
                          "const double cand = ait + b[j * ldb + t];"),
    "mp64_last_t_skipped": ("    for (int64_t t = 0; t < k; ++t) {\n      const double ait",
                            "    for (int64_t t = 0; t < k - 1; ++t) {\n      const double ait"),
    "mp64_max_not_min": ("if (cand < c[i * ldc + j]) c[i * ldc + j] = cand;\n      }\n    }\n}\n\n/*",
                         "if (cand > c[i * ldc + j]) c[i * ldc + j] = cand;\n      }\n    }\n}\n\n/*"),
    "mp_guard_dropped": ("      if (ait == inf) continue;\n      for (int64_t j = 0; j < n; ++j) {\n        const int64_t btj",
                         "      for (int64_t j = 0; j < n; ++j) {\n        const int64_t btj"),
}


def _battery(o: oracle.Oracle) -> None:
    g = read_golden("hand4_fw.txt", INF)
    w4 = g["input"].astype(np.int32)
    for k_end, key in [(1, "after_k 1"), (2, "after_k 2"), (3, "after_k 3"), (4, "final")]:
        assert np.array_equal(o.fw_i32(w4, k_end=k_end), g[key])
    assert np.array_equal(o.sssp_rows_i32(w4, INF, range(4)), g["final"])
    gf = read_golden("hand4_fw.txt", np.inf)
    assert np.array_equal(o.fw_f64(gf["input"].astype(np.float64)), gf["final"].astype(np.float64))
    for seed in range(40):
        rng = np.random.default_rng(77 + seed)
        n = int(rng.integers(2, 8))
        w = random_small_graph(rng, n, 0.4, 9, INF)
        want = brute_force_apsp(w, INF).astype(np.int64)
        assert np.array_equal(o.fw_i32(w).astype(np.int64), want)
        assert np.array_equal(o.sssp_rows_i32(w, INF, range(n)).astype(np.int64), want)
        wf = random_small_graph(rng, n, 0.4, 4, np.inf, floats=True)
        wantf = brute_force_apsp(wf, np.inf).astype(np.float64)
        gotf = o.fw_f64(wf)
        assert np.array_equal(np.isinf(gotf), np.isinf(wantf))
        fin = np.isfinite(wantf)
        assert np.allclose(gotf[fin], wantf[fin], rtol=1e-12)
    n = 33
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    assert np.array_equal(o.fw_i32(gg.ring(n, 3)), 3 * ((j - i) % n))
    w = gg.erdos_renyi(60, 0.08, 1, 20, 3)
    ref = csg.shortest_path(csg.csgraph_from_dense(w.astype(np.float64), null_value=float(INF)),
                            method="D")
    ref = np.where(np.isinf(ref), INF, ref).astype(np.int64)
    assert np.array_equal(o.fw_i32(w).astype(np.int64), ref)
    assert np.array_equal(o.sssp_rows_i32(w, INF, range(60)).astype(np.int64), ref)


def _battery_guarded(o: oracle.Oracle) -> None:
    w = np.array([[0, INF, INF], [INF, 0, -5], [INF, INF, 0]], dtype=np.int64)
    got, neg = o.fw_guarded(w, INF)
    assert not neg and got[0, 2] == INF and got[1, 2] == -5
    assert o.fw_guarded(np.array([[0, 3], [-4, 0]], dtype=np.int64), INF)[1]
    for seed in range(30):
        rng = np.random.default_rng(300 + seed)
        n = int(rng.integers(2, 8))
        w0 = random_small_graph(rng, n, 0.5, 9, INF).astype(np.int64)
        pot = rng.integers(-6, 7, size=n)
        edge = (w0 != INF) & ~np.eye(n, dtype=bool)
        w = np.where(edge, w0 + pot[:, None] - pot[None, :], w0)
        got, neg = o.fw_guarded(w, INF)
        assert not neg
        assert np.array_equal(got, brute_force_apsp(w, INF).astype(np.int64))
        u, v = 0, n - 1
        w2 = w.copy()
        w2[u, v], w2[v, u] = 3, -4   # cycle of weight -1
        assert o.fw_guarded(w2, INF)[1]


def _battery_bellman_ford(o: oracle.Oracle) -> None:
    # chain with negative weights: closed form
    rp = np.array([0, 1, 2, 3, 3], dtype=np.int64)
    col = np.array([1, 2, 3], dtype=np.int32)
    wt = np.array([-1, -2, -3], dtype=np.int64)
    h, neg = o.johnson_potentials(rp, col, wt, 4)
    assert not neg and h.tolist() == [0, -1, -3, -6]
    # two-vertex negative cycle
    rp2, col2 = np.array([0, 1, 2], dtype=np.int64), np.array([1, 0], dtype=np.int32)
    assert o.bf_rows_csr(rp2, col2, np.array([3, -4], dtype=np.int64), 2, [0], INF)[1][0]
    # a ring whose shortest paths need n - 1 edges (the longest chain of rounds)
    n = 9
    rp3 = np.arange(n + 1, dtype=np.int64)
    col3 = ((np.arange(n) + 1) % n).astype(np.int32)
    got, neg = o.bf_rows_csr(rp3, col3, np.full(n, 2, dtype=np.int64), n, [0], INF)
    assert not neg[0] and got[0].tolist() == [2 * j for j in range(n)]
    for seed in range(30):
        rng = np.random.default_rng(500 + seed)
        n = int(rng.integers(2, 8))
        w0 = random_small_graph(rng, n, 0.5, 9, INF).astype(np.int64)
        pot = rng.integers(-6, 7, size=n)
        edge = (w0 != INF) & ~np.eye(n, dtype=bool)
        w = np.where(edge, w0 + pot[:, None] - pot[None, :], w0)
        r, c, wv = gg.csr_from_dense(w, INF)
        got, neg = o.bf_rows_csr(r, c, wv, n, range(n), INF)
        assert not neg.any()
        assert np.array_equal(got, brute_force_apsp(w, INF).astype(np.int64))


def _battery_minplus(o: oracle.Oracle) -> None:
    a = np.array([[0, 4, INF], [2, INF, 1]], dtype=np.int64)
    b = np.array([[5, INF], [0, 3], [7, 1]], dtype=np.int64)
    c = np.array([[3, 2], [INF, INF]], dtype=np.int64)
    assert o.minplus(c, a, b, INF).tolist() == [[3, 2], [7, 2]]
    # a "no path" operand is never summed, even next to a negative entry
    neg = o.minplus(np.array([[INF]], dtype=np.int64), np.array([[INF]], dtype=np.int64),
                    np.array([[-5]], dtype=np.int64), INF)
    assert neg.tolist() == [[INF]]
    rng = np.random.default_rng(11)
    for _ in range(4):
        n = int(rng.integers(3, 40))
        w = random_small_graph(rng, n, 0.15, 30, INF)
        d = w.astype(np.int64)
        for _ in range(int(np.ceil(np.log2(n - 1))) if n > 2 else 1):
            d = o.minplus(d, d, d.copy(), INF)
        assert np.array_equal(d, o.fw_i32(w).astype(np.int64))
    # binary64: the hand-worked float product and squaring to the closure
    fa = np.array([[0.5, 0.25, np.inf], [1.5, np.inf, 0.125]])
    fb = np.array([[0.75, np.inf], [0.5, 2.0], [4.0, 0.375]])
    fc = np.array([[1.0, 2.5], [np.inf, np.inf]])
    assert o.minplus(fc, fa, fb).tolist() == [[0.75, 2.25], [2.25, 0.5]]
    for _ in range(3):
        n = int(rng.integers(3, 40))
        w = np.where(rng.random((n, n)) < 0.2, rng.integers(1, 64, (n, n)) / 8.0, np.inf)
        np.fill_diagonal(w, 0.0)
        d = w.copy()
        for _ in range(int(np.ceil(np.log2(n - 1))) if n > 2 else 1):
            d = o.minplus(d, d, d.copy())
        assert np.array_equal(d, o.fw_f64(w))


def _battery_successors(o: oracle.Oracle) -> None:
    g = read_golden("hand4_fw.txt", INF)
    assert np.array_equal(o.successors(g["input"], g["final"], INF), g["successors"])
    w = gg.grid(4, 5)
    nxt = o.successors(w, o.fw_i32(w), INF)
    assert nxt[19, 0] == 14 and nxt[0, 19] == 1 and nxt[7, 7] == 7
    w3 = np.array([[0, 6, 10], [10, 0, 6], [10, 10, 0]], dtype=np.int32)
    assert o.successors(w3, o.fw_i32(w3), 10)[0, 2] == -1


def _build_variant(tmp_path, name, edit):
    src = open(oracle.SRC).read()
    if edit is not None:
        old, new = edit
        assert src.count(old) >= 1, f"mutant {name}: anchor text not found"
        src = src.replace(old, new, 1)
    p = tmp_path / f"{name}.c"
    p.write_text(src)
    out = tmp_path / f"lib{name}.so"
    oracle.build(str(out), str(p))
    return oracle.Oracle(str(out))


def test_battery_passes_on_unmodified_oracle(tmp_path):
    o = _build_variant(tmp_path, "pristine", None)
    _battery(o)
    _battery_guarded(o)
    _battery_bellman_ford(o)
    _battery_minplus(o)
    _battery_successors(o)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_battery_catches_mutant(tmp_path, name):
    o = _build_variant(tmp_path, name, MUTANTS[name])
    with pytest.raises(AssertionError):
        _battery(o)
        _battery_guarded(o)
        _battery_bellman_ford(o)
        _battery_minplus(o)
        _battery_successors(o)
