"""Seeded input generator: determinism, shapes, distributions, padding."""
import numpy as np
import pytest

import graphgen as gg
import oracle


def test_counter_rng_scalar_matches_vector():
    c = np.arange(0, 1000, 37, dtype=np.uint64)
    v = gg.u64_array(42, 3, c)
    assert [gg.u64(42, 3, int(x)) for x in c] == [int(x) for x in v]


def test_splitmix64_reference_values():
    # SplitMix64 with state 0: the first outputs of the published generator
    # (state += 0x9E3779B97F4A7C15, then the output mix).
    z, out = 0, []
    for _ in range(3):
        z = (z + gg.GAMMA) & ((1 << 64) - 1)
        out.append(gg.mix64(z))
    assert out == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_same_seed_same_matrix_different_seed_differs():
    a = gg.erdos_renyi(300, 0.1, 1, 100, 1)
    b = gg.erdos_renyi(300, 0.1, 1, 100, 1)
    c = gg.erdos_renyi(300, 0.1, 1, 100, 2)
    assert gg.sha256_matrix(a) == gg.sha256_matrix(b) != gg.sha256_matrix(c)


def test_er_density_and_weights():
    n, p = 1000, 0.05
    m = gg.erdos_renyi(n, p, 1, 1000, 2)
    assert np.all(np.diag(m) == 0)
    off = m[~np.eye(n, dtype=bool)]
    edges = off[off != gg.INF_I32]
    exp = p * n * (n - 1)
    sd = np.sqrt(n * (n - 1) * p * (1 - p))
    assert abs(len(edges) - exp) < 5 * sd
    assert edges.min() >= 1 and edges.max() <= 1000
    # roughly uniform: each decile holds ~10 %
    h, _ = np.histogram(edges, bins=10, range=(0.5, 1000.5))
    assert np.all(np.abs(h / len(edges) - 0.1) < 0.01)


def test_complete_and_float():
    m = gg.complete(200, 1, 10000, 3)
    assert np.all(np.diag(m) == 0)
    off = m[~np.eye(200, dtype=bool)]
    assert off.min() >= 1 and off.max() <= 10000
    f = gg.complete_f32(200, 5)
    assert f.dtype == np.float32 and np.all(np.diag(f) == 0)
    offf = f[~np.eye(200, dtype=bool)]
    assert offf.min() >= np.float32(0.01) and offf.max() < 1.0


def test_barabasi_albert_shape():
    n, beta = 2000, 8
    e = gg.barabasi_albert_edges(n, beta, 4)
    assert len(e) == beta * (n - beta)
    assert np.all(e[:, 0] > e[:, 1])                  # new vertex -> older vertex
    for v in (beta + 1, 500, n - 1):                  # distinct targets
        t = e[e[:, 0] == v, 1]
        assert len(t) == beta and len(set(t.tolist())) == beta
    m = gg.barabasi_albert(n, beta, 1, 255, 4)
    assert np.array_equal(m, m.T)
    assert (m != gg.INF_I32).sum() - n == 2 * beta * (n - beta)
    deg = np.bincount(e.ravel(), minlength=n)
    assert deg.max() > 10 * beta                       # heavy-tailed hubs


@pytest.mark.parametrize("ld", [None, 64, 100])
def test_padding_and_canary(ld):
    m = gg.erdos_renyi(50, 0.2, 1, 9, 7, ld=ld, canary=-5)
    assert m.shape == (50, ld or 50)
    if ld:
        assert np.all(m[:, 50:] == -5)
    ref = gg.erdos_renyi(50, 0.2, 1, 9, 7)
    assert np.array_equal(m[:, :50], ref)


def test_workload_table_names():
    assert set(gg.WORKLOADS) == {"er-256-p0.1-i32", "er-2048-p0.05-i32", "complete-8192-i32",
                                 "ba-16000-b8-i32", "complete-12288-f32"}
    m = gg.make_workload("er-256-p0.1-i32")
    assert m.shape == (256, 256) and m.dtype == np.int32


def test_zero_size():
    m = gg.erdos_renyi(0, 0.5, 1, 9, 1, ld=4)
    assert m.shape == (0, 4)


def test_batch_generators():
    b = gg.erdos_renyi_batch(6, 9, 0.3, 1, 50, 21, ld=12)
    assert b.shape == (6, 9, 12) and b.dtype == np.int32
    # graph 0 is the single-graph generator with the same seed; graph g uses
    # the next n*n counters, so graphs differ
    assert np.array_equal(b[0], gg.erdos_renyi(9, 0.3, 1, 50, 21, ld=12))
    assert not np.array_equal(b[1], b[0])
    assert np.all(b[:, :, 9:] == -7)
    assert np.all(b[:, np.arange(9), np.arange(9)] == 0)
    assert np.array_equal(b, gg.erdos_renyi_batch(6, 9, 0.3, 1, 50, 21, ld=12))
    f = gg.complete_f32_batch(4, 5, 8)
    assert f.shape == (4, 5, 5) and f.dtype == np.float32
    assert np.array_equal(f[0], gg.complete_f32(5, 8))
    off = ~np.eye(5, dtype=bool)
    assert np.all((f[:, off] >= 0.01) & (f[:, off] < 1.0))


def test_batch_workload_table():
    for name, w in gg.BATCH_WORKLOADS.items():
        assert name.startswith("batch-") and w["n"] <= 128 and w["batch"] >= 1
        assert w["dtype"] in name


def test_regular_out_csr_structure():
    n, deg = 1000, 5
    rp, col, w = gg.regular_out_csr(n, deg, 3, 9, 17)
    assert rp.dtype == np.int64 and col.dtype == np.int32 and w.dtype == np.int32
    assert np.array_equal(rp, np.arange(n + 1) * deg)
    u = np.repeat(np.arange(n), deg)
    assert (col != u).all() and col.min() >= 0 and col.max() < n
    assert w.min() >= 3 and w.max() <= 9
    # deterministic, and a different seed gives a different graph
    rp2, col2, w2 = gg.regular_out_csr(n, deg, 3, 9, 17)
    assert np.array_equal(col, col2) and np.array_equal(w, w2)
    assert not np.array_equal(col, gg.regular_out_csr(n, deg, 3, 9, 18)[1])


def test_regular_out_csr_potentials_keep_cycle_weights():
    # w = w0 + p(u) - p(v): the shift telescopes around any cycle, so the
    # shifted graph's distances are the unshifted ones plus p(s) - p(t)
    n, deg = 300, 4
    rp, col, w0 = gg.regular_out_csr(n, deg, 0, 50, 5)
    _, col1, w = gg.regular_out_csr(n, deg, 0, 50, 5, -40, 40)
    assert np.array_equal(col, col1) and (w < 0).any()
    o = oracle.default()
    src = [0, 7, 299]
    d0, neg0 = o.bf_rows_csr(rp, col, w0, n, src, gg.INF_I32)
    d1, neg1 = o.bf_rows_csr(rp, col, w, n, src, gg.INF_I32)
    assert not neg0.any() and not neg1.any()
    shift = (w.astype(np.int64) - w0)                      # p(u) - p(v) per edge
    p = np.zeros(n, dtype=np.int64)                        # recover p up to a constant along BFS
    seen = np.zeros(n, dtype=bool)
    seen[0] = True
    stack = [0]
    while stack:
        u = stack.pop()
        for e in range(rp[u], rp[u + 1]):
            v = col[e]
            if not seen[v]:
                p[v] = p[u] - shift[e]
                seen[v] = True
                stack.append(v)
    reach = d0 < gg.INF_I32
    for k, s in enumerate(src):
        both = reach[k] & seen
        assert np.array_equal((d1[k] - d0[k])[both], (p[s] - p)[both])
