"""Pins for the CPU oracle: checks that do not rest on the oracle itself.

Each test ties the oracle to something fixed from outside it:
  * a hand-worked example (tests/golden/hand4_fw.txt), step by step;
  * the literal definition (minimum over all simple paths) on tiny graphs;
  * library routines (scipy's Dijkstra and Johnson implementations);
  * closed forms (rings, paths, grids, complete graphs, disjoint rings);
  * invariants (zero diagonal, triangle inequality, d <= W, symmetry on
    undirected inputs, inf exactly on unreachable pairs, Bellman optimality);
  * serial == multi-threaded bit for bit.
"""
import numpy as np
import pytest
import scipy.sparse.csgraph as csg

import graphgen as gg
from _helpers import (bellman_rows_ok, brute_force_apsp, random_small_graph,
                      reachability, read_golden, triangle_ok)

INF = gg.INF_I32


# ---- hand-worked example -------------------------------------------------

def test_hand_example_every_pivot(orc):
    g = read_golden("hand4_fw.txt", INF)
    w = g["input"].astype(np.int32)
    for k_end, key in [(0, "input"), (1, "after_k 1"), (2, "after_k 2"),
                       (3, "after_k 3"), (4, "final")]:
        got = orc.fw_i32(w, k_end=k_end)
        assert np.array_equal(got, g[key]), key


def test_hand_example_f64_with_ieee_inf(orc):
    g = read_golden("hand4_fw.txt", np.inf)
    got = orc.fw_f64(g["input"].astype(np.float64))
    assert np.array_equal(got, g["final"].astype(np.float64))


def test_hand_example_dijkstra_rows(orc):
    g = read_golden("hand4_fw.txt", INF)
    w = g["input"].astype(np.int32)
    assert np.array_equal(orc.sssp_rows_i32(w, INF, range(4)), g["final"])


# ---- the definition, evaluated literally ---------------------------------

@pytest.mark.parametrize("seed", range(240))
def test_brute_force_small_int(orc, seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(1, 8))
    p = [0.15, 0.35, 0.6, 0.9][seed % 4]
    w = random_small_graph(rng, n, p, wmax=9, inf=INF)  # zero weights allowed
    want = brute_force_apsp(w, INF).astype(np.int64)
    assert np.array_equal(orc.fw_i32(w).astype(np.int64), want)
    assert np.array_equal(orc.sssp_rows_i32(w, INF, range(n)).astype(np.int64), want)


@pytest.mark.parametrize("seed", range(60))
def test_brute_force_small_float(orc, seed):
    rng = np.random.default_rng(5000 + seed)
    n = int(rng.integers(2, 8))
    w = random_small_graph(rng, n, 0.5, wmax=4, inf=np.inf, floats=True)
    want = brute_force_apsp(w, np.inf).astype(np.float64)
    got = orc.fw_f64(w)
    # path sums associate differently in FW and in the enumeration
    assert np.array_equal(np.isinf(got), np.isinf(want))
    fin = np.isfinite(want)
    assert np.allclose(got[fin], want[fin], rtol=1e-12, atol=0)
    got_d = orc.sssp_rows_f64(w, np.inf, range(n))
    assert np.array_equal(np.isinf(got_d), np.isinf(want))
    assert np.allclose(got_d[fin], want[fin], rtol=1e-12, atol=0)


# ---- library routines ----------------------------------------------------

def _scipy_apsp(w, inf, method):
    g = csg.csgraph_from_dense(w.astype(np.float64), null_value=float(inf))
    # csgraph_from_dense drops diagonal zeros only; explicit zero-weight
    # off-diagonal edges are kept because null_value is the sentinel.
    return csg.shortest_path(g, method=method, directed=True)


@pytest.mark.parametrize("n,p,seed", [(50, 0.1, 1), (200, 0.03, 2), (333, 0.02, 3), (257, 0.5, 4)])
def test_matches_scipy_dijkstra_and_johnson(orc, n, p, seed):
    w = gg.erdos_renyi(n, p, 0, 50, seed)  # includes zero-weight edges
    d = orc.fw_i32(w)
    for method in ("D", "J"):
        ref = _scipy_apsp(w, INF, method)
        ref = np.where(np.isinf(ref), INF, ref).astype(np.int64)
        assert np.array_equal(d.astype(np.int64), ref), method
    rows = orc.sssp_rows_i32(w, INF, range(n))
    assert np.array_equal(rows, d)


def test_float_matches_scipy(orc):
    w = gg.complete_f32(300, seed=9).astype(np.float64)
    d = orc.fw_f64(w)
    ref = _scipy_apsp(w, np.inf, "D")
    assert np.allclose(d, ref, rtol=1e-13, atol=0)


def test_zero_weight_edges_are_edges(orc):
    # 0 -> 1 (weight 0) -> 2 (weight 0): d(0,2) must be 0, and scipy agrees
    w = np.full((3, 3), INF, dtype=np.int32)
    np.fill_diagonal(w, 0)
    w[0, 1] = 0
    w[1, 2] = 0
    d = orc.fw_i32(w)
    assert d[0, 2] == 0 and d[2, 0] == INF
    ref = _scipy_apsp(w, INF, "D")
    assert ref[0, 2] == 0 and np.isinf(ref[2, 0])


# ---- closed forms ----------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 3, 17, 64, 65, 130])
def test_directed_ring(orc, n):
    w = 3
    d = orc.fw_i32(gg.ring(n, w))
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    assert np.array_equal(d, w * ((j - i) % n))
    dr = orc.fw_i32(gg.ring(n, w, reverse=True))
    assert np.array_equal(dr, w * ((i - j) % n))


def test_undirected_ring(orc):
    n = 41
    d = orc.fw_i32(gg.ring(n, 2, directed=False))
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    k = (j - i) % n
    assert np.array_equal(d, 2 * np.minimum(k, n - k))


def test_path_grid_complete_edgeless(orc):
    n = 37
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    assert np.array_equal(orc.fw_i32(gg.undirected_path(n, 5)), 5 * np.abs(i - j))
    r, c = 6, 9
    d = orc.fw_i32(gg.grid(r, c))
    v = np.arange(r * c)
    man = np.abs(v[:, None] // c - v[None, :] // c) + np.abs(v[:, None] % c - v[None, :] % c)
    assert np.array_equal(d, man)
    ce = orc.fw_i32(gg.complete_equal(n, 7))
    assert np.array_equal(ce, np.where(i == j, 0, 7))
    e = gg.edgeless(n)
    assert np.array_equal(orc.fw_i32(e), e)


def test_two_rings_keep_inf_between_components(orc):
    n1, n2 = 13, 20
    d = orc.fw_i32(gg.two_rings(n1, n2, 4))
    assert np.all(d[:n1, n1:] == INF) and np.all(d[n1:, :n1] == INF)
    i, j = np.meshgrid(np.arange(n2), np.arange(n2), indexing="ij")
    assert np.array_equal(d[n1:, n1:], 4 * ((j - i) % n2))


def test_float_closed_forms_are_exact(orc):
    n = 50
    d = orc.fw_f64(gg.ring(n, 0.5, dtype=np.float64, inf=np.inf))
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    assert np.array_equal(d, 0.5 * ((j - i) % n))
    d2 = orc.fw_f64(gg.two_rings(7, 9, 0.25, dtype=np.float64, inf=np.inf))
    assert np.all(np.isinf(d2[:7, 7:]))


# ---- invariants ------------------------------------------------------------

@pytest.mark.parametrize("n,p,seed", [(120, 0.03, 11), (97, 0.2, 12), (160, 0.01, 13)])
def test_invariants_random(orc, n, p, seed):
    w = gg.erdos_renyi(n, p, 1, 30, seed)
    d = orc.fw_i32(w)
    assert np.all(np.diag(d) == 0)
    assert np.all(d <= w)
    assert triangle_ok(d)
    reach = reachability(w, INF)
    assert np.array_equal(d == INF, ~reach)
    assert bellman_rows_ok(w, d, range(n), INF)


def test_undirected_input_gives_symmetric_output(orc):
    w = gg.barabasi_albert(300, 3, 1, 255, seed=21)
    d = orc.fw_i32(w)
    assert np.array_equal(d, d.T)
    assert triangle_ok(d)


def test_padding_columns_untouched(orc):
    n, ld = 45, 64
    w = gg.erdos_renyi(n, 0.1, 1, 9, 5, ld=ld, canary=-7)
    d = orc.fw_i32(w)
    assert np.all(d[:, n:] == -7)
    assert np.array_equal(d[:, :n], orc.fw_i32(np.ascontiguousarray(w[:, :n])))


# ---- threading -------------------------------------------------------------

def test_serial_equals_parallel(orc):
    w = gg.erdos_renyi(300, 0.05, 1, 100, 31)
    wf = gg.complete_f32(300, 32).astype(np.float64)
    orc.set_threads(1)
    try:
        a, af = orc.fw_i32(w), orc.fw_f64(wf)
    finally:
        orc.set_threads(0)
    orc.set_threads(8)
    try:
        b, bf = orc.fw_i32(w), orc.fw_f64(wf)
    finally:
        orc.set_threads(0)
    assert np.array_equal(a, b)
    assert np.array_equal(af.view(np.int64), bf.view(np.int64))


def test_dijkstra_rows_match_fw_on_workload_shapes(orc):
    # the two oracle routes agree on the workload families at reduced size
    for w in (gg.erdos_renyi(512, 0.05, 1, 1000, 2), gg.complete(384, 1, 10000, 3),
              gg.barabasi_albert(600, 8, 1, 255, 4)):
        d = orc.fw_i32(w)
        src = np.arange(0, w.shape[0], 7)
        assert np.array_equal(orc.sssp_rows_i32(w, INF, src), d[src])


# ---- many small graphs ------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_batched_oracle_is_the_definition_per_graph(orc, seed):
    """Every graph of a batch, closed by the batched entry, equals the literal
    minimum over simple paths of that graph (and nothing leaks between
    graphs: each graph's answer depends on its own weights only)."""
    rng = np.random.default_rng(9000 + seed)
    n = int(rng.integers(1, 8))
    batch = 25
    ld = n + int(rng.integers(0, 3))
    w = np.full((batch, n, ld), -7, dtype=np.int32)
    for g in range(batch):
        w[g, :, :n] = random_small_graph(rng, n, [0.2, 0.5, 0.8][g % 3], wmax=9, inf=INF)
    got = orc.fw_batched_i32(w)
    for g in range(batch):
        assert np.array_equal(got[g, :, :n].astype(np.int64),
                              brute_force_apsp(w[g, :, :n], INF).astype(np.int64))
    assert np.all(got[:, :, n:] == -7)


def test_batched_oracle_float_per_graph(orc):
    rng = np.random.default_rng(77)
    batch, n = 12, 6
    w = np.stack([random_small_graph(rng, n, 0.6, wmax=4, inf=np.inf, floats=True)
                  for _ in range(batch)])
    got = orc.fw_batched_f64(w)
    for g in range(batch):
        want = brute_force_apsp(w[g], np.inf).astype(np.float64)
        assert np.array_equal(np.isinf(got[g]), np.isinf(want))
        fin = np.isfinite(want)
        assert np.allclose(got[g][fin], want[fin], rtol=1e-12, atol=0)


# ---- negative weights (Johnson's setting) -----------------------------------

def _potential_graph(rng, n, p):
    """Random graph with negative weights and no negative cycle: w0 >= 0
    shifted by vertex potentials."""
    w0 = random_small_graph(rng, n, p, wmax=9, inf=INF).astype(np.int64)
    pot = rng.integers(-6, 7, size=n)
    edge = (w0 != INF) & ~np.eye(n, dtype=bool)
    return np.where(edge, w0 + pot[:, None] - pot[None, :], w0)


@pytest.mark.parametrize("seed", range(120))
def test_guarded_fw_negative_weights_brute_force(orc, seed):
    rng = np.random.default_rng(20000 + seed)
    n = int(rng.integers(1, 8))
    w = _potential_graph(rng, n, [0.2, 0.5, 0.8][seed % 3])
    got, neg = orc.fw_guarded(w, INF)
    assert not neg
    assert np.array_equal(got, brute_force_apsp(w, INF).astype(np.int64))


def test_guarded_fw_matches_scipy_johnson_and_detects_cycles(orc):
    sp = pytest.importorskip("scipy.sparse")
    csg = pytest.importorskip("scipy.sparse.csgraph")
    rng = np.random.default_rng(31)
    for trial in range(30):
        n = int(rng.integers(5, 40))
        w = _potential_graph(rng, n, 0.15)
        got, neg = orc.fw_guarded(w, INF)
        assert not neg
        mask = (w != INF) & ~np.eye(n, dtype=bool)
        r, c = np.nonzero(mask)
        # scipy treats explicit zeros as edges only when stored explicitly
        g = sp.csr_matrix((w[r, c].astype(np.float64), (r, c)), shape=(n, n))
        want = csg.johnson(g, directed=True)
        want = np.where(np.isinf(want), INF, want).astype(np.int64)
        assert np.array_equal(got, want)
        # plant a negative cycle: u -> v -> u with total weight -1
        u, v = rng.choice(n, size=2, replace=False)
        w2 = w.copy()
        w2[u, v], w2[v, u] = 3, -4
        _, neg2 = orc.fw_guarded(w2, INF)
        assert neg2
        r2, c2 = np.nonzero((w2 != INF) & ~np.eye(n, dtype=bool))
        g2 = sp.csr_matrix((w2[r2, c2].astype(np.float64), (r2, c2)), shape=(n, n))
        with pytest.raises(csg.NegativeCycleError):
            csg.johnson(g2, directed=True)


def test_guarded_fw_never_uses_the_sentinel_as_a_number(orc):
    # vertex 1 is unreachable from 0; its edge 1 -> 2 has weight -5, so an
    # unguarded sum inf + (-5) would wrongly beat inf at (0, 2)
    w = np.array([[0, INF, INF], [INF, 0, -5], [INF, INF, 0]], dtype=np.int64)
    got, neg = orc.fw_guarded(w, INF)
    assert not neg and got[0, 2] == INF and got[1, 2] == -5


def test_guarded_fw_equals_plain_fw_without_negative_weights(orc):
    w = gg.erdos_renyi(200, 0.03, 0, 50, 4)
    got, neg = orc.fw_guarded(w, INF)
    assert not neg and np.array_equal(got, orc.fw_i32(w).astype(np.int64))


# ---- Bellman-Ford from one source and Johnson's potentials ------------------

def _csr(w):
    return gg.csr_from_dense(w, INF)


@pytest.mark.parametrize("seed", range(80))
def test_bellman_ford_rows_brute_force(orc, seed):
    rng = np.random.default_rng(40000 + seed)
    n = int(rng.integers(1, 8))
    w = _potential_graph(rng, n, [0.2, 0.5, 0.8][seed % 3])
    rp, c, wt = _csr(w)
    got, neg = orc.bf_rows_csr(rp, c, wt, n, range(n), INF)
    assert not neg.any()
    assert np.array_equal(got, brute_force_apsp(w, INF).astype(np.int64))


def test_bellman_ford_matches_scipy_and_flags_reachable_cycles_only(orc):
    sp = pytest.importorskip("scipy.sparse")
    rng = np.random.default_rng(41)
    for trial in range(20):
        n = int(rng.integers(5, 60))
        w = _potential_graph(rng, n, 0.1)
        rp, c, wt = _csr(w)
        got, neg = orc.bf_rows_csr(rp, c, wt, n, range(n), INF)
        assert not neg.any()
        r, cc = np.nonzero((w != INF) & ~np.eye(n, dtype=bool))
        g = sp.csr_matrix((w[r, cc].astype(np.float64), (r, cc)), shape=(n, n))
        want = csg.bellman_ford(g, directed=True)
        assert np.array_equal(got, np.where(np.isinf(want), INF, want).astype(np.int64))
    # vertices 0 -> 1 -> 2 -> 1 with cycle 1 <-> 2 of weight -1, vertex 3 alone
    w = np.full((4, 4), INF, dtype=np.int64)
    np.fill_diagonal(w, 0)
    w[0, 1], w[1, 2], w[2, 1] = 5, 2, -3
    rp, c, wt = _csr(w)
    _, neg = orc.bf_rows_csr(rp, c, wt, 4, range(4), INF)
    assert list(neg) == [True, True, True, False]


def test_bellman_ford_self_loop_and_duplicate_edges(orc):
    # CSR may hold self loops and parallel edges: a negative self loop is a
    # negative cycle, a non-negative one changes nothing, the lighter of two
    # parallel edges counts
    rp = np.array([0, 3, 4, 4], dtype=np.int64)
    col = np.array([1, 1, 0, 1], dtype=np.int32)
    w = np.array([7, 4, 2, 0], dtype=np.int64)
    got, neg = orc.bf_rows_csr(rp, col, w, 3, [0, 1, 2], INF)
    assert not neg.any()
    assert got.tolist() == [[0, 4, INF], [INF, 0, INF], [INF, INF, 0]]
    w2 = w.copy()
    w2[3] = -1
    _, neg2 = orc.bf_rows_csr(rp, col, w2, 3, [0, 1, 2], INF)
    assert list(neg2) == [True, True, False]


def test_johnson_potentials_closed_form_chain(orc):
    # 0 -> 1 -> 2 -> 3 with weights -1, -2, -3: h(v) is the prefix sum, and
    # a vertex reached by nothing negative keeps h = 0
    rp = np.array([0, 1, 2, 3, 3, 3], dtype=np.int64)
    col = np.array([1, 2, 3], dtype=np.int32)
    w = np.array([-1, -2, -3], dtype=np.int64)
    h, neg = orc.johnson_potentials(rp, col, w, 5)
    assert not neg and h.tolist() == [0, -1, -3, -6, 0]


@pytest.mark.parametrize("seed", range(40))
def test_johnson_potentials_are_column_minima_and_reweight_non_negative(orc, seed):
    # h(v) = distance from an added vertex joined to all by 0-weight edges =
    # min over u of delta(u, v) (delta(v, v) = 0 gives h <= 0); with it every
    # reweighted edge w + h(u) - h(v) is >= 0 (the page's property 2)
    rng = np.random.default_rng(42000 + seed)
    n = int(rng.integers(1, 8)) if seed < 30 else int(rng.integers(20, 80))
    w = _potential_graph(rng, n, [0.2, 0.5, 0.8][seed % 3])
    rp, c, wt = _csr(w)
    h, neg = orc.johnson_potentials(rp, c, wt, n)
    assert not neg
    delta = brute_force_apsp(w, INF).astype(np.int64) if n <= 7 else orc.fw_guarded(w, INF)[0]
    assert np.array_equal(h, delta.min(axis=0))
    u = np.repeat(np.arange(n), np.diff(rp))
    assert (wt + h[u] - h[c] >= 0).all()


def test_johnson_potentials_flag_any_negative_cycle(orc):
    # the added vertex reaches every vertex, so every negative cycle counts
    w = np.full((5, 5), INF, dtype=np.int64)
    np.fill_diagonal(w, 0)
    w[3, 4], w[4, 3] = 1, -2
    rp, c, wt = _csr(w)
    assert orc.johnson_potentials(rp, c, wt, 5)[1]


@pytest.mark.parametrize("seed", range(40))
def test_float_fw_with_ieee_inf_handles_negative_weights(orc, seed):
    # with +infinity as "no edge", inf + (negative) stays inf, so the plain
    # binary64 recurrence is already guarded: it must equal brute force
    rng = np.random.default_rng(45000 + seed)
    n = int(rng.integers(1, 8))
    w0 = random_small_graph(rng, n, [0.3, 0.6][seed % 2], 4, np.inf, floats=True)
    pot = rng.uniform(-2.0, 2.0, size=n)
    edge = np.isfinite(w0) & ~np.eye(n, dtype=bool)
    w = np.where(edge, w0 + pot[:, None] - pot[None, :], w0)
    want = brute_force_apsp(w, np.inf).astype(np.float64)
    got = orc.fw_f64(w)
    assert np.array_equal(np.isinf(got), np.isinf(want))
    fin = np.isfinite(want)
    assert np.allclose(got[fin], want[fin], rtol=1e-12, atol=1e-12)


# ---- the min-plus product ---------------------------------------------------

def test_minplus_hand_example(orc):
    # worked by hand: a 2 x 3 by 3 x 2 product, one "no path" entry, C keeps
    # an entry the product cannot beat
    a = np.array([[0, 4, INF], [2, INF, 1]], dtype=np.int64)
    b = np.array([[5, INF], [0, 3], [7, 1]], dtype=np.int64)
    c = np.array([[3, 2], [INF, INF]], dtype=np.int64)
    got = orc.minplus(c, a, b, INF)
    # (0,0): min(3, 0+5, 4+0) = 3; (0,1): min(2, 4+3) = 2
    # (1,0): min(2+5, 1+7) = 7;    (1,1): min(1+1) = 2
    assert got.tolist() == [[3, 2], [7, 2]]
    # a "no path" operand is never summed, even next to a negative entry:
    # inf + (-5) must not beat inf
    one = lambda v: np.array([[v]], dtype=np.int64)
    assert orc.minplus(one(INF), one(INF), one(-5), INF).tolist() == [[INF]]
    assert orc.minplus(one(INF), one(-5), one(INF), INF).tolist() == [[INF]]
    assert orc.minplus(one(INF), one(-5), one(2), INF).tolist() == [[-3]]


def test_minplus_identity_and_associativity(orc):
    rng = np.random.default_rng(7)
    n = 30
    ident = np.full((n, n), INF, dtype=np.int64)
    np.fill_diagonal(ident, 0)
    empty = np.full((n, n), INF, dtype=np.int64)
    for trial in range(10):
        a = random_small_graph(rng, n, 0.3, 50, INF).astype(np.int64)
        b = random_small_graph(rng, n, 0.3, 50, INF).astype(np.int64)
        d = random_small_graph(rng, n, 0.3, 50, INF).astype(np.int64)
        assert np.array_equal(orc.minplus(empty, a, ident, INF), a)
        assert np.array_equal(orc.minplus(empty, ident, a, INF), a)
        ab = orc.minplus(empty, a, b, INF)
        bd = orc.minplus(empty, b, d, INF)
        assert np.array_equal(orc.minplus(empty, ab, d, INF), orc.minplus(empty, a, bd, INF))


@pytest.mark.parametrize("seed", range(8))
def test_minplus_squaring_reaches_the_floyd_warshall_closure(orc, seed):
    # W with a zero diagonal: W^(2^r) covers paths of up to 2^r edges, so
    # ceil(log2(n - 1)) squarings give delta, which the pinned plain
    # recurrence computes by another route
    rng = np.random.default_rng(900 + seed)
    n = int(rng.integers(2, 70))
    w = random_small_graph(rng, n, [0.05, 0.2][seed % 2], 30, INF)
    d = w.astype(np.int64)
    for _ in range(max(1, int(np.ceil(np.log2(max(n - 1, 2)))))):
        d = orc.minplus(d, d, d.copy(), INF)
    assert np.array_equal(d, orc.fw_i32(w).astype(np.int64))


def test_minplus_float_hand_example(orc):
    # worked by hand with binary fractions (every sum exact in binary64), a
    # "no path" +inf on each side, and C keeping nothing but its own +inf
    a = np.array([[0.5, 0.25, np.inf], [1.5, np.inf, 0.125]])
    b = np.array([[0.75, np.inf], [0.5, 2.0], [4.0, 0.375]])
    c = np.array([[1.0, 2.5], [np.inf, np.inf]])
    got = orc.minplus(c, a, b)
    # (0,0): min(1.0, 0.5+0.75, 0.25+0.5) = 0.75    (0,1): min(2.5, 0.25+2.0) = 2.25
    # (1,0): min(1.5+0.75, 0.125+4.0) = 2.25        (1,1): min(0.125+0.375) = 0.5
    assert got.tolist() == [[0.75, 2.25], [2.25, 0.5]]
    # C is kept where the product cannot beat it
    assert orc.minplus(np.array([[0.5]]), np.array([[0.25]]), np.array([[0.5]])).tolist() == [[0.5]]


@pytest.mark.parametrize("seed", range(6))
def test_minplus_float_squaring_reaches_the_floyd_warshall_closure(orc, seed):
    # binary64 weights that are multiples of 1/8 below 8: every path sum is
    # exact, so ceil(log2(n - 1)) squarings equal the pinned plain recurrence
    # bit for bit
    rng = np.random.default_rng(950 + seed)
    n = int(rng.integers(2, 60))
    w = np.where(rng.random((n, n)) < [0.08, 0.3][seed % 2],
                 rng.integers(1, 64, (n, n)) / 8.0, np.inf)
    np.fill_diagonal(w, 0.0)
    d = w.copy()
    for _ in range(max(1, int(np.ceil(np.log2(max(n - 1, 2)))))):
        d = orc.minplus(d, d, d.copy())
    assert np.array_equal(d, orc.fw_f64(w))


def test_minplus_float_with_ieee_inf(orc):
    rng = np.random.default_rng(8)
    m, n, k = 20, 25, 30
    a = np.where(rng.random((m, k)) < 0.5, rng.uniform(0.01, 1.0, (m, k)), np.inf)
    b = np.where(rng.random((k, n)) < 0.5, rng.uniform(0.01, 1.0, (k, n)), np.inf)
    c = np.full((m, n), np.inf)
    got = orc.minplus(c, a, b)
    want = np.min(a[:, :, None] + b[None, :, :], axis=1)   # every candidate at once
    assert np.array_equal(got, want)


# ---- successors (path reconstruction) ---------------------------------------

def test_successors_hand_example(orc):
    g = read_golden("hand4_fw.txt", INF)
    got = orc.successors(g["input"], g["final"], INF)
    assert np.array_equal(got, g["successors"])


def test_successors_sum_reaching_the_sentinel_is_unreachable(orc):
    # inf = 10: 0 -> 1 -> 2 weighs 12, so d(0, 2) stays at the sentinel and
    # 2 is unreachable from 0 in the sentinel's sense; no first hop either
    inf = 10
    w = np.array([[0, 6, inf], [inf, 0, 6], [inf, inf, 0]], dtype=np.int32)
    d = orc.fw_i32(w)
    assert d[0, 2] == inf and d[0, 1] == 6 and d[1, 2] == 6
    nxt = orc.successors(w, d, inf)
    assert nxt.tolist() == [[0, 1, -1], [-1, 1, 2], [-1, -1, 2]]


def all_shortest_first_hops(w, inf):
    """Brute force: the set of first vertices over every shortest simple
    path i -> j (n <= 7)."""
    n = w.shape[0]
    best = brute_force_apsp(w, inf)
    hops = [[set() for _ in range(n)] for _ in range(n)]
    for s in range(n):
        stack = [(s, 0, 1 << s, -1)]
        while stack:
            u, dist, seen, first = stack.pop()
            for v in range(n):
                if v == u or w[u, v] == inf or seen >> v & 1:
                    continue
                nd = dist + int(w[u, v])
                f = v if first < 0 else first
                if nd == best[s][v]:
                    hops[s][v].add(f)
                stack.append((v, nd, seen | (1 << v), f))
    return best, hops


@pytest.mark.parametrize("seed", range(60))
def test_successors_are_the_smallest_shortest_first_hop(orc, seed):
    # positive weights with many ties (weights in 1..3)
    rng = np.random.default_rng(60000 + seed)
    n = int(rng.integers(2, 8))
    w = random_small_graph(rng, n, [0.3, 0.6][seed % 2], 3, INF)
    w = np.where((w == 0) & ~np.eye(n, dtype=bool), 1, w)   # strictly positive weights
    best, hops = all_shortest_first_hops(w, INF)
    d = orc.fw_i32(w)
    nxt = orc.successors(w, d, INF)
    for i in range(n):
        for j in range(n):
            if i == j:
                assert nxt[i, j] == i
            elif best[i][j] == INF:
                assert nxt[i, j] == -1
            else:
                assert nxt[i, j] == min(hops[i][j])


@pytest.mark.parametrize("seed", range(8))
def test_successor_rows_are_the_listed_rows(orc, seed):
    # the row-restricted form takes the same definition for the listed rows,
    # in any order and with repeats; checked against brute force on tiny
    # graphs and against the full matrix on larger ones
    rng = np.random.default_rng(61000 + seed)
    n = int(rng.integers(2, 8))
    w = random_small_graph(rng, n, 0.5, 3, INF)
    w = np.where((w == 0) & ~np.eye(n, dtype=bool), 1, w)
    best, hops = all_shortest_first_hops(w, INF)
    d = orc.fw_i32(w)
    rows = rng.integers(0, n, size=5)
    got = orc.successors_rows(w, d, INF, rows)
    for k, i in enumerate(rows):
        for j in range(n):
            want = i if i == j else (-1 if best[i][j] == INF else min(hops[i][j]))
            assert got[k, j] == want
    w = gg.erdos_renyi(90, 0.2, 0, 4, 500 + seed)
    np.fill_diagonal(w, 0)
    d = orc.fw_i32(w)
    rows = rng.integers(0, 90, size=7)
    assert np.array_equal(orc.successors_rows(w, d, INF, rows), orc.successors(w, d, INF)[rows])


def test_successors_on_a_grid_closed_form(orc):
    # unit grid, vertex r*C + c: the smallest neighbour index that moves closer
    # is up (r - 1) if the target row is above, else left, else right, else down
    R, C = 6, 7
    w = gg.grid(R, C)
    d = orc.fw_i32(w)
    nxt = orc.successors(w, d, INF)
    for a in range(R * C):
        ra, ca = divmod(a, C)
        for b in range(R * C):
            rb, cb = divmod(b, C)
            if a == b:
                want = a
            elif rb < ra:
                want = a - C
            elif cb < ca:
                want = a - 1
            elif cb > ca:
                want = a + 1
            else:
                want = a + C
            assert nxt[a, b] == want, (a, b)


def test_fw_in_steps_takes_the_pivots_in_order(orc):
    """Consecutive pivot ranges are the recurrence itself: the hand-worked
    example's states after each pivot, and the one-call result on random
    graphs, for every range length."""
    g = read_golden("hand4_fw.txt", INF)
    w4 = g["input"].astype(np.int32)
    seen = []
    got = orc.fw_in_steps(w4, 1, lambda k, n: seen.append(k))
    assert seen == [1, 2, 3, 4]
    assert np.array_equal(got, g["final"])
    for k_end, key in [(1, "after_k 1"), (2, "after_k 2"), (3, "after_k 3")]:
        part = orc.fw_i32(w4, k_end=k_end)
        assert np.array_equal(part, g[key])
    rng = np.random.default_rng(5)
    for step in (1, 2, 3, 7, 50):
        w = random_small_graph(rng, 7, 0.4, 30, INF)
        assert np.array_equal(orc.fw_in_steps(w, step).astype(np.int64),
                              brute_force_apsp(w, INF).astype(np.int64))
        w = random_small_graph(rng, 61, 0.1, 30, INF)
        assert np.array_equal(orc.fw_in_steps(w, step), orc.fw_i32(w))
        wf = random_small_graph(rng, 7, 0.5, 4, np.inf, floats=True)
        want = brute_force_apsp(wf, np.inf).astype(np.float64)
        gotf = orc.fw_in_steps(wf, step)
        fin = np.isfinite(want)
        assert np.array_equal(np.isinf(gotf), ~fin)
        assert np.allclose(gotf[fin], want[fin], rtol=1e-12)
