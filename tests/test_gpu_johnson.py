"""GPU parity of Johnson's all-pairs shortest paths on sparse graphs
(apsp_johnson_i32: CSR in, dense distances out, negative weights allowed)
against the CPU oracle.

The oracle side is the plain definition: the INF-guarded Floyd-Warshall
(negative weights, negative-cycle flag) for whole matrices, Bellman-Ford from
one source for sampled rows of large graphs, Dijkstra rows for non-negative
graphs, and Johnson's potentials from an added vertex by Bellman-Ford.  All
comparisons are bit-exact (int32).  Bytes outside the n x n output block are
never written (a canary fills them).
"""
import numpy as np
import torch  # noqa: F401
import pytest

import graph_all_pairs_amd as ga
import graphgen as gg
import oracle

pytestmark = pytest.mark.gpu

INF = gg.INF_I32
CANARY = -7


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(dev, rp, col, wt):
    return (torch.from_numpy(np.ascontiguousarray(rp, dtype=np.int64)).to(dev),
            torch.from_numpy(np.ascontiguousarray(col, dtype=np.int32)).to(dev),
            torch.from_numpy(np.ascontiguousarray(wt, dtype=np.int32)).to(dev))


def run(dev, csr, n, delta=-1, ld=None, want_h=False, inf=INF, timed=False):
    """Johnson on the GPU; returns (n x n result, h or None[, ms, rounds])
    after checking the canary outside the n x n block."""
    rp, col, wt = to_dev(dev, *csr)
    ld = n if ld is None else ld
    out = torch.full((n, ld), CANARY, dtype=torch.int32, device=dev)
    h = torch.full((n,), 12345, dtype=torch.int32, device=dev) if want_h else None
    r = ga.johnson(rp, col, wt, out=out, inf=inf, h=h, delta=delta, timed=timed)
    res = out.cpu().numpy()
    assert (res[:, n:] == CANARY).all(), "wrote outside the n x n block"
    hh = h.cpu().numpy() if want_h else None
    if timed:
        return res[:, :n], hh, r[1], r[2]
    return res[:, :n], hh


def guarded(orc, w):
    d, neg = orc.fw_guarded(w, INF)
    assert not neg
    return d


def neg_graph(n, p, seed, wlo=0, whi=50, plo=-40, phi=40):
    return gg.erdos_renyi_potential(n, p, wlo, whi, plo, phi, seed)


SIZES = [1, 2, 3, 5, 17, 31, 64, 100, 257, 600, 1031]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("p", [0.05, 0.3])
def test_negative_weights_match_oracle(dev, orc, n, p):
    print(f"case johnson negative ER n={n} p={p}", flush=True)
    w = neg_graph(n, p, seed=1000 + n)
    csr = gg.csr_from_dense(w, INF)
    got, h = run(dev, csr, n, want_h=True)
    assert np.array_equal(got.astype(np.int64), guarded(orc, w))
    want_h, neg = orc.johnson_potentials(*csr, n)
    assert not neg and np.array_equal(h.astype(np.int64), want_h)


@pytest.mark.parametrize("n,p", [(200, 0.02), (777, 0.01), (1500, 0.004)])
def test_non_negative_matches_oracle_and_fw(dev, orc, n, p):
    print(f"case johnson non-negative ER n={n} p={p}", flush=True)
    w = gg.erdos_renyi(n, p, 1, 100, 50 + n)
    got, h = run(dev, gg.csr_from_dense(w, INF), n, want_h=True)
    assert np.array_equal(got, orc.fw_i32(w))
    assert (h == 0).all()
    t = torch.from_numpy(w).to(dev)
    ga.fw(t, INF)
    assert np.array_equal(got, t.cpu().numpy())


@pytest.mark.parametrize("delta", [0, 1, 5, 37, 1000, 10 ** 7, -1])
def test_delta_does_not_change_the_result(dev, orc, delta):
    print(f"case johnson delta={delta}", flush=True)
    n = 700
    w = neg_graph(n, 0.02, seed=77)
    got, _ = run(dev, gg.csr_from_dense(w, INF), n, delta=delta)
    assert np.array_equal(got.astype(np.int64), guarded(orc, w))


@pytest.mark.parametrize("deg", [3, 12, 24, 48, 160])
def test_every_lane_group_width(dev, orc, deg):
    # average degree picks 8-, 16-, 32- or 64-lane groups per vertex
    print(f"case johnson average degree {deg}", flush=True)
    n = 640
    w = neg_graph(n, deg / n, seed=300 + deg)
    got, _ = run(dev, gg.csr_from_dense(w, INF), n)
    assert np.array_equal(got.astype(np.int64), guarded(orc, w))


def test_hub_vertex_and_queue_overflow(dev, orc):
    # a hub with an edge to and from every vertex (one adjacency of n - 1
    # edges shared by all waves), then a dense graph searched with a huge
    # delta so that one step removes more vertices than the queue holds
    print("case johnson hub and queue overflow", flush=True)
    n = 5000
    w = np.full((n, n), INF, dtype=np.int32)
    np.fill_diagonal(w, 0)
    rng = np.random.default_rng(5)
    w[0, 1:] = rng.integers(1, 1000, n - 1)
    w[1:, 0] = rng.integers(1, 1000, n - 1)
    got, _ = run(dev, gg.csr_from_dense(w, INF), n)
    # closed form: every path between two leaves goes through the hub
    want = w[1:, 0][:, None].astype(np.int64) + w[0, 1:][None, :]
    np.fill_diagonal(want, 0)
    assert np.array_equal(got[1:, 1:], want)
    assert np.array_equal(got[0], w[0]) and np.array_equal(got[:, 0], w[:, 0])
    assert np.array_equal(got[[0, 7, 4999]], orc.sssp_rows_i32(w, INF, [0, 7, 4999]))

    n2 = 3000
    w2 = gg.erdos_renyi(n2, 0.9, 1, 100, 9)
    csr2 = gg.csr_from_dense(w2, INF)
    srcs = np.array([0, 1, 1499, 2999])
    for delta in (10 ** 6, 0):
        got2, _ = run(dev, csr2, n2, delta=delta)
        assert np.array_equal(got2[srcs], orc.sssp_rows_i32(w2, INF, srcs))


def test_disconnected_components_and_isolated_vertices(dev, orc):
    print("case johnson disconnected", flush=True)
    n = 300
    w = np.full((n, n), INF, dtype=np.int32)
    np.fill_diagonal(w, 0)
    a = neg_graph(120, 0.05, seed=3)
    b = neg_graph(150, 0.05, seed=4)
    w[:120, :120] = a
    w[130:280, 130:280] = b          # vertices 120..129 and 280..299 are isolated
    got, _ = run(dev, gg.csr_from_dense(w, INF), n)
    want = guarded(orc, w)
    assert np.array_equal(got.astype(np.int64), want)
    assert (got[:120, 130:] == INF).all() and (got[120:130, :120] == INF).all()


def test_self_loops_and_parallel_edges(dev):
    print("case johnson self loops and parallel edges", flush=True)
    # 0 -> 1 twice (7 and 4), 0 -> 0 (self loop 2), 1 -> 2 (-3), 2 -> 2 (0)
    rp = np.array([0, 3, 4, 5], dtype=np.int64)
    col = np.array([1, 1, 0, 2, 2], dtype=np.int32)
    wt = np.array([7, 4, 2, -3, 0], dtype=np.int32)
    got, h = run(dev, (rp, col, wt), 3, want_h=True)
    assert got.tolist() == [[0, 4, 1], [INF, 0, -3], [INF, INF, 0]]
    assert h.tolist() == [0, 0, -3]


def test_negative_cycle_is_reported_and_nothing_is_written(dev):
    print("case johnson negative cycle", flush=True)
    n = 400
    w = neg_graph(n, 0.02, seed=8)
    w[10, 20], w[20, 30], w[30, 10] = 5, 5, -11      # cycle of weight -1
    rp, col, wt = to_dev(dev, *gg.csr_from_dense(w, INF))
    out = torch.full((n, n), CANARY, dtype=torch.int32, device=dev)
    h = torch.full((n,), 12345, dtype=torch.int32, device=dev)
    with pytest.raises(ga.NegativeCycleError):
        ga.johnson(rp, col, wt, out=out, h=h)
    assert (out == CANARY).all() and (h == 12345).all()
    # a negative self loop is a negative cycle too
    rp2 = torch.tensor([0, 1, 1], dtype=torch.int64, device=dev)
    col2 = torch.tensor([0], dtype=torch.int32, device=dev)
    w2 = torch.tensor([-1], dtype=torch.int32, device=dev)
    with pytest.raises(ga.NegativeCycleError):
        ga.johnson(rp2, col2, w2)


@pytest.mark.parametrize("case", ["col_high", "col_negative", "row_ptr_decreasing",
                                  "row_ptr_end", "row_ptr_start", "weight_inf",
                                  "weight_minus_inf"])
def test_malformed_graph_is_rejected_before_writing(dev, case):
    print(f"case johnson malformed {case}", flush=True)
    rp = np.array([0, 2, 3, 4], dtype=np.int64)
    col = np.array([1, 2, 2, 0], dtype=np.int32)
    wt = np.array([1, 2, 3, 4], dtype=np.int32)
    if case == "col_high":
        col[2] = 3
    elif case == "col_negative":
        col[0] = -1
    elif case == "row_ptr_decreasing":
        rp[1] = 4
    elif case == "row_ptr_end":
        rp[3] = 3
    elif case == "row_ptr_start":
        rp[0] = 1
    elif case == "weight_inf":
        wt[1] = INF
    else:
        wt[1] = -INF
    t = to_dev(dev, rp, col, wt)
    out = torch.full((3, 3), CANARY, dtype=torch.int32, device=dev)
    with pytest.raises(ga.APSPError) as e:
        ga.johnson(*t, out=out)
    assert e.value.status == ga.APSP_ERR_INVALID_VALUE
    assert (out == CANARY).all()


def test_unrepresentable_distance_is_a_range_error(dev):
    print("case johnson range", flush=True)
    # chain 0 -> 1 -> 2 with weights just under inf: d(0, 2) >= inf
    big = INF - 1
    rp = np.array([0, 1, 2, 2], dtype=np.int64)
    col = np.array([1, 2], dtype=np.int32)
    wt = np.array([big, big], dtype=np.int32)
    t = to_dev(dev, rp, col, wt)
    with pytest.raises(ga.APSPError) as e:
        ga.johnson(*t)
    assert e.value.status == ga.APSP_ERR_RANGE
    # a sentinel below some finite distance is a range error too
    wt2 = np.array([60, 50], dtype=np.int32)
    t2 = to_dev(dev, rp, col, wt2)
    with pytest.raises(ga.APSPError) as e2:
        ga.johnson(*t2, inf=100)
    assert e2.value.status == ga.APSP_ERR_RANGE
    got = ga.johnson(*t2, inf=111).cpu().numpy()
    assert got.tolist() == [[0, 60, 110], [111, 0, 50], [111, 111, 0]]


def test_row_beyond_lds_edgeless(dev):
    # n = 45000: a 180 KB row does not fit one workgroup's LDS, so the
    # searches keep their distances in the output rows in global memory
    print("case johnson n beyond the LDS row, edgeless", flush=True)
    n = 45000
    rp = torch.zeros(n + 1, dtype=torch.int64, device=dev)
    e = torch.zeros(0, dtype=torch.int32, device=dev)
    out = torch.full((n, n), CANARY, dtype=torch.int32, device=dev)
    ga.johnson(rp, e, e, out=out)
    rows = [0, 1, 22500, n - 1]
    got = out[rows].cpu().numpy()
    for k, r in enumerate(rows):
        want = np.full(n, INF, dtype=np.int32)
        want[r] = 0
        assert np.array_equal(got[k], want)
    assert bool((out.diagonal() == 0).all())
    del out


@pytest.mark.parametrize("neg", [False, True])
def test_rows_beyond_lds_match_oracle(dev, orc, neg):
    # 45000 vertices, 6 out-edges each, built straight as CSR; with neg the
    # weights are shifted by vertex potentials (negative edges, no negative
    # cycle) so Bellman-Ford and the reweighting run too
    print(f"case johnson n=45000 beyond the LDS row neg={neg}", flush=True)
    n = 45000
    rp, col, w = gg.regular_out_csr(n, 6, 0 if neg else 1, 100, 71, *((-50, 50) if neg else (0, 0)))
    assert bool((w < 0).any()) == neg
    t = to_dev(dev, rp, col, w)
    out = torch.full((n, n), CANARY, dtype=torch.int32, device=dev)
    ga.johnson(*t, out=out)
    src = np.array([0, 1, 12345, 22500, n - 1])
    want, negc = orc.bf_rows_csr(rp, col, w, n, src, INF)
    assert not negc.any()
    got = out[torch.from_numpy(src).to(dev)].cpu().numpy().astype(np.int64)
    assert np.array_equal(got, want)
    del out


def test_padded_output_repeat_calls_and_timed_variant(dev, orc):
    print("case johnson ld > n, repeat, timed", flush=True)
    n = 333
    w = neg_graph(n, 0.03, seed=12)
    csr = gg.csr_from_dense(w, INF)
    want = guarded(orc, w)
    for ld in (n + 1, n + 64):
        got, _ = run(dev, csr, n, ld=ld)
        assert np.array_equal(got.astype(np.int64), want)
    got, _, ms, counts = run(dev, csr, n, timed=True)
    assert np.array_equal(got.astype(np.int64), want)
    assert counts[0] >= 1 and all(x >= 0 for x in ms) and ms[3] > 0
    # every source removes at least the vertices it reaches and relaxes at
    # least every edge out of them, once
    reach = (want != INF)
    assert counts[2] >= reach.sum() and counts[1] >= n
    u = np.repeat(np.arange(n), np.diff(csr[0]))
    assert counts[3] >= int(reach[:, u].sum())
    wpos = gg.erdos_renyi(n, 0.03, 1, 9, 13)
    _, _, ms2, counts2 = run(dev, gg.csr_from_dense(wpos, INF), n, timed=True)
    assert counts2[0] == 0 and ms2[1] < ms[1]  # no Bellman-Ford rounds, only h = 0


def test_edgeless_and_single_vertex(dev):
    print("case johnson edgeless", flush=True)
    n = 70
    rp = np.zeros(n + 1, dtype=np.int64)
    e = np.zeros(0, dtype=np.int32)
    got, h = run(dev, (rp, e, e), n, want_h=True)
    want = np.full((n, n), INF, dtype=np.int32)
    np.fill_diagonal(want, 0)
    assert np.array_equal(got, want) and (h == 0).all()
    got1, _ = run(dev, (np.zeros(2, dtype=np.int64), e, e), 1)
    assert got1.tolist() == [[0]]


# ---- the named sparse workloads, as the bench runs them ---------------------

def sample_sources(n, k, seed):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(n, size=min(k, n), replace=False).tolist()) | {0, n - 1, n // 2}
    return np.array(sorted(s))


def test_workload_er_2048_full_oracle(dev, orc):
    print("case workload johnson-er-2048-p0.05-i32", flush=True)
    w = gg.make_johnson_workload("johnson-er-2048-p0.05-i32")
    n = w.shape[0]
    got, _ = run(dev, gg.csr_from_dense(w, INF), n)
    assert np.array_equal(got, orc.fw_i32(w))


def test_workload_ba_16000_sampled_and_against_fw(dev, orc):
    print("case workload johnson-ba-16000-b8-i32", flush=True)
    w = gg.make_johnson_workload("johnson-ba-16000-b8-i32")
    n = w.shape[0]
    rp, col, wt = to_dev(dev, *gg.csr_from_dense(w, INF))
    got = ga.johnson(rp, col, wt)
    src = sample_sources(n, 24, 5)
    rows = got[torch.from_numpy(src).to(dev)].cpu().numpy()
    assert np.array_equal(rows, orc.sssp_rows_i32(w, INF, src))
    assert torch.equal(got, got.t())                  # undirected input
    assert bool((torch.diagonal(got) == 0).all())
    t = torch.from_numpy(w).to(dev)                  # the blocked Floyd-Warshall
    ga.fw(t, INF)
    assert torch.equal(got, t)


def test_workload_er_8192_negative_sampled(dev, orc):
    print("case workload johnson-er-8192-p0.002-neg-i32", flush=True)
    w = gg.make_johnson_workload("johnson-er-8192-p0.002-neg-i32")
    n = w.shape[0]
    csr = gg.csr_from_dense(w, INF)
    assert (csr[2] < 0).any()
    rp, col, wt = to_dev(dev, *csr)
    h = torch.empty(n, dtype=torch.int32, device=dev)
    got = ga.johnson(rp, col, wt, h=h)
    src = sample_sources(n, 16, 6)
    rows = got[torch.from_numpy(src).to(dev)].cpu().numpy().astype(np.int64)
    want, neg = orc.bf_rows_csr(*csr, n, src, INF)
    assert not neg.any() and np.array_equal(rows, want)
    want_h, negh = orc.johnson_potentials(*csr, n)
    assert not negh and np.array_equal(h.cpu().numpy().astype(np.int64), want_h)
    assert bool((torch.diagonal(got) == 0).all())
