"""GPU parity of the dense Floyd-Warshall with negative weights
(apsp_fw_signed_i32 / apsp_fw_signed_f32) against the CPU oracle.

int32: bit-exact against the oracle's INF-guarded Floyd-Warshall, in both
arithmetics (binary32 with +infinity for "no edge", and int32 with the
sentinel as a large number plus a final clamp).  float32: within 1e-5 of the
oracle's binary64 recurrence with +infinity for "no edge" (IEEE infinity is
its own guard).  Negative cycles, malformed inputs and out-of-range weights
are reported without touching the matrix where the contract says so.
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
F32_RTOL = 1e-5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_i32(dev, w, inf=INF, ld=None, offset=0):
    n = w.shape[0]
    ld = n if ld is None else ld
    buf = torch.full((n * ld + offset + 4,), CANARY, dtype=torch.int32, device=dev)
    view = buf[offset:offset + n * ld].view(n, ld)
    view[:, :n] = torch.from_numpy(np.ascontiguousarray(w[:, :n], dtype=np.int32)).to(dev)
    st = ga.apsp_fw_signed_i32(view.data_ptr(), n, ld, inf, torch.cuda.current_stream().cuda_stream)
    host = buf.cpu().numpy()
    out = host[offset:offset + n * ld].reshape(n, ld)
    assert (out[:, n:] == CANARY).all() and (host[:offset] == CANARY).all()
    assert (host[offset + n * ld:] == CANARY).all()
    return st, out[:, :n]


def want_guarded(w):
    d, neg = oracle.default().fw_guarded(w.astype(np.int64), INF)
    assert not neg
    return d


POLICIES = [ga.APSP_ARITH_AUTO, ga.APSP_ARITH_F32_WHEN_EXACT, ga.APSP_ARITH_INT32]
SIZES = [1, 2, 3, 5, 31, 64, 65, 127, 128, 129, 257, 383, 1000, 1031]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("policy", POLICIES)
def test_negative_weights_match_oracle(dev, n, policy):
    print(f"case signed i32 n={n} policy={policy}", flush=True)
    w = gg.erdos_renyi_potential(n, 0.05 if n > 64 else 0.3, 0, 50, -40, 40, 600 + n)
    with ga.int32_arith(policy):
        st, got = run_i32(dev, w)
    assert st == ga.APSP_OK, ga.apsp_status_string(st)
    assert np.array_equal(got.astype(np.int64), want_guarded(w))


@pytest.mark.parametrize("policy", POLICIES)
def test_complete_graph_with_negative_weights(dev, policy):
    # no "no edge" entry at all: the int32 form needs no clamp
    print(f"case signed i32 complete policy={policy}", flush=True)
    n = 300
    rng = np.random.default_rng(3)
    w0 = rng.integers(0, 100, size=(n, n)).astype(np.int64)
    pot = rng.integers(-50, 50, size=n)
    w = (w0 + pot[:, None] - pot[None, :]).astype(np.int32)
    np.fill_diagonal(w, 0)
    with ga.int32_arith(policy):
        st, got = run_i32(dev, w)
    assert st == ga.APSP_OK
    assert np.array_equal(got.astype(np.int64), want_guarded(w))


def test_large_weights_take_int32_and_stay_exact(dev):
    # (n - 1) * W > 2^24 rules out binary32; (2n - 3) * W < inf keeps int32 exact
    print("case signed i32 large weights", flush=True)
    n = 300
    w = gg.erdos_renyi_potential(n, 0.05, 0, 100000, -100000, 100000, 17)
    assert (n - 1) * np.abs(w[(w != INF) & ~np.eye(n, dtype=bool)]).max() > 2 ** 24
    st, got = run_i32(dev, w)
    assert st == ga.APSP_OK
    assert np.array_equal(got.astype(np.int64), want_guarded(w))


def test_unreachable_pairs_never_use_the_sentinel(dev):
    # vertex 1 is unreachable from 0 and has a -5 edge: inf + (-5) must not count
    print("case signed i32 sentinel guard", flush=True)
    w = np.array([[0, INF, INF], [INF, 0, -5], [INF, INF, 0]], dtype=np.int32)
    for policy in POLICIES:
        with ga.int32_arith(policy):
            st, got = run_i32(dev, w)
        assert st == ga.APSP_OK and got.tolist() == [[0, INF, INF], [INF, 0, -5], [INF, INF, 0]]


@pytest.mark.parametrize("policy", POLICIES)
def test_negative_cycle_is_reported(dev, policy):
    print(f"case signed i32 negative cycle policy={policy}", flush=True)
    n = 260
    w = gg.erdos_renyi_potential(n, 0.05, 0, 50, -40, 40, 5)
    w[3, 200], w[200, 140], w[140, 3] = 5, 5, -11
    with ga.int32_arith(policy):
        st, _ = run_i32(dev, w)
    assert st == ga.APSP_ERR_NEGATIVE_CYCLE


@pytest.mark.parametrize("case", ["diag", "above_inf", "minus_inf"])
def test_malformed_matrix_is_rejected_untouched(dev, case):
    print(f"case signed i32 malformed {case}", flush=True)
    n = 40
    w = gg.erdos_renyi_potential(n, 0.2, 0, 50, -40, 40, 9)
    if case == "diag":
        w[7, 7] = -1
    elif case == "above_inf":
        w[1, 2] = INF + 1
    else:
        w[1, 2] = -INF
    st, got = run_i32(dev, w)
    assert st == ga.APSP_ERR_INVALID_VALUE and np.array_equal(got, w)


def test_out_of_range_weights_are_rejected_untouched(dev):
    print("case signed i32 range", flush=True)
    n = 2000
    w = gg.erdos_renyi_potential(n, 0.002, 0, 10 ** 6, -10 ** 6, 10 ** 6, 11)
    st, got = run_i32(dev, w)
    assert st == ga.APSP_ERR_RANGE and np.array_equal(got, w)
    # forced int32 cannot use the binary32 form either
    w2 = gg.erdos_renyi_potential(200, 0.05, 0, 50, -40, 40, 12, inf=300)
    with ga.int32_arith(ga.APSP_ARITH_INT32):
        st2, got2 = run_i32(dev, w2, inf=300)
    assert st2 == ga.APSP_ERR_RANGE and np.array_equal(got2, w2)


def test_small_sentinel_uses_binary32(dev):
    # inf = 3000: (2n - 3) * W >= inf rules out the int32 form, binary32 is exact
    print("case signed i32 small sentinel", flush=True)
    n = 100
    w = gg.erdos_renyi_potential(n, 0.05, 0, 20, -10, 10, 13, inf=3000)
    st, got = run_i32(dev, w, inf=3000)
    assert st == ga.APSP_OK
    want, neg = oracle.default().fw_guarded(w.astype(np.int64), 3000)
    assert not neg and np.array_equal(got.astype(np.int64), want)


def test_padding_and_unaligned_pointer(dev):
    print("case signed i32 ld and offset", flush=True)
    n = 301
    w = gg.erdos_renyi_potential(n, 0.03, 0, 50, -40, 40, 14)
    want = want_guarded(w)
    for ld, offset in ((n + 3, 0), (n + 64, 1), (n, 3)):
        for policy in (ga.APSP_ARITH_F32_WHEN_EXACT, ga.APSP_ARITH_INT32):
            with ga.int32_arith(policy):
                st, got = run_i32(dev, w, ld=ld, offset=offset)
            assert st == ga.APSP_OK and np.array_equal(got.astype(np.int64), want)


def test_matches_johnson_on_the_negative_workload(dev):
    # two GPU paths, one answer: the dense rounds and the sparse searches;
    # sampled rows against the oracle's Bellman-Ford
    print("case signed i32 vs johnson, johnson-er-8192-p0.002-neg-i32", flush=True)
    w = gg.make_johnson_workload("johnson-er-8192-p0.002-neg-i32")
    n = w.shape[0]
    t = torch.from_numpy(w).to(dev)
    ga.fw_signed(t)
    csr = gg.csr_from_dense(w, INF)
    rp, col, wt = (torch.from_numpy(np.ascontiguousarray(x, dtype=dt)).to(dev)
                   for x, dt in zip(csr, (np.int64, np.int32, np.int32)))
    j = ga.johnson(rp, col, wt)
    assert torch.equal(t, j)
    src = np.array([0, 1, 4095, 8191])
    rows, neg = oracle.default().bf_rows_csr(*csr, n, src, INF)
    assert not neg.any()
    assert np.array_equal(t[torch.from_numpy(src).to(dev)].cpu().numpy().astype(np.int64), rows)


def f32_graph(n, p, seed):
    rng = np.random.default_rng(seed)
    w0 = np.where(rng.random((n, n)) < p, rng.uniform(0.01, 1.0, (n, n)), np.inf)
    pot = rng.uniform(-0.5, 0.5, n)
    w = w0 + pot[:, None] - pot[None, :]
    np.fill_diagonal(w, 0.0)
    return w.astype(np.float32)


@pytest.mark.parametrize("n", [1, 5, 64, 129, 257, 1000])
@pytest.mark.parametrize("finite_inf", [False, True])
def test_f32_negative_weights(dev, n, finite_inf):
    print(f"case signed f32 n={n} finite_inf={finite_inf}", flush=True)
    w = f32_graph(n, 0.05 if n > 64 else 0.4, 700 + n)
    inf = 1e30 if finite_inf else float("inf")
    if finite_inf:
        w = np.where(np.isinf(w), np.float32(inf), w)
    t = torch.from_numpy(w).to(dev)
    ga.fw_signed(t, inf)
    got = t.cpu().numpy().astype(np.float64)
    want = oracle.fw_f64(np.where(w == np.float32(inf), np.inf, w).astype(np.float64))
    unreach = np.isinf(want)
    assert (got[unreach] == np.float32(inf)).all()
    fin = ~unreach
    err = np.abs(got[fin] - want[fin])
    # each rounding is relative to a partial sum of edge weights (magnitude
    # ~1 here), not to the final distance, which cancellation can bring near
    # zero: 1e-5 relative to max(|d|, 1)
    assert (err <= F32_RTOL * np.maximum(np.abs(want[fin]), 1.0)).all(), err.max()


def test_f32_negative_cycle(dev):
    print("case signed f32 negative cycle", flush=True)
    w = f32_graph(200, 0.05, 3)
    w[5, 6], w[6, 5] = 0.25, -0.5
    t = torch.from_numpy(w).to(dev)
    with pytest.raises(ga.NegativeCycleError):
        ga.fw_signed(t)
