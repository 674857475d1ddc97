"""GPU parity on the five named workloads, in the configuration the bench
times (full call, ld = n, one stream).

The two small workloads are compared element by element with the oracle's
full Floyd-Warshall.  The three large ones are compared on sampled rows
computed one source at a time by the oracle's Dijkstra, plus properties that
hold at any size (zero diagonal, d <= W, symmetry on undirected input).
"""
import numpy as np
import torch  # noqa: F401  (imported at collection, before any test timer starts)
import pytest

import graph_all_pairs_amd as ga
import graphgen as gg
import oracle

pytestmark = pytest.mark.gpu
INF = gg.INF_I32


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def run(torch_dev, w, inf):
    torch, dev = torch_dev
    t = torch.from_numpy(w).to(dev)
    ga.fw(t, inf)
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("name", ["er-256-p0.1-i32", "er-2048-p0.05-i32"])
@pytest.mark.parametrize("arith", [ga.APSP_ARITH_AUTO, ga.APSP_ARITH_F32_WHEN_EXACT])
def test_small_workloads_full_oracle(torch_dev, name, arith):
    print(f"case workload {name} arith policy {arith}", flush=True)
    w = gg.make_workload(name)
    with ga.int32_arith(arith):
        got = run(torch_dev, w, INF)
    assert np.array_equal(got, oracle.fw_i32(w))


def sample_sources(n, k, seed):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(n, size=min(k, n), replace=False).tolist())
    s |= {0, n - 1, n // 2, 127, 128}            # block edges and the ragged tail
    return np.array(sorted(x for x in s if x < n))


@pytest.mark.parametrize("name", ["complete-8192-i32", "ba-16000-b8-i32"])
def test_large_int_workloads_sampled(torch_dev, name):
    print(f"case workload {name}", flush=True)
    w = gg.make_workload(name)
    n = w.shape[0]
    d = run(torch_dev, w, INF)
    src = sample_sources(n, 24, 11)
    want = oracle.sssp_rows_i32(w, INF, src)
    assert np.array_equal(d[src], want)
    assert np.all(np.diag(d) == 0)
    assert np.all(d <= w)
    if name.startswith("ba"):
        assert np.array_equal(d, d.T)
        assert np.all(d < INF)           # the BA graph is connected
    # column samples too: d[:, j] for sampled j via the transposed graph
    wt = np.ascontiguousarray(w.T)
    cols = sample_sources(n, 8, 12)
    want_c = oracle.sssp_rows_i32(wt, INF, cols)
    assert np.array_equal(d[:, cols].T, want_c)


def test_large_float_workload_sampled(torch_dev):
    print("case workload complete-12288-f32", flush=True)
    w = gg.make_workload("complete-12288-f32")
    n = w.shape[0]
    d = run(torch_dev, w, np.inf).astype(np.float64)
    src = sample_sources(n, 16, 13)
    want = oracle.sssp_rows_f64(w.astype(np.float64), np.inf, src)
    got = d[src]
    assert np.all(np.isfinite(got))
    rel = np.abs(got - want) / np.maximum(want, np.finfo(np.float64).tiny)
    off = ~np.eye(n, dtype=bool)[src]
    assert float(rel[off].max()) <= 1e-5, float(rel[off].max())
    assert np.all(got[~off] == 0)
    assert np.all(d <= w.astype(np.float64))
