"""GPU parity on the five named workloads, in the configuration the bench
times (full call, ld = n, one stream).

Every workload is compared element by element with the oracle's full
Floyd-Warshall ("Katz and Kider" page, section 4.6: the blocked rounds reach
the distances of the plain recurrence; "Loops into zones", section "What it
does not change": the tiled version gives the serial version's values):
  * int32 matrices bit for bit, under the default arithmetic policy (the one
    the bench runs) and with int32 and binary32 arithmetic forced;
  * the float32 matrix within 1e-5 relative of the binary64 recurrence, with
    zeros exact, and bit-identical from one GPU run to the next.

The oracle needs minutes at n = 12288 and n = 16000 on the host, so each
large result is computed once per module, as consecutive pivot ranges that
report their progress.  A sampled check (Dijkstra rows and columns plus
properties that hold at any size) runs first, so a wrong result shows early.
"""
import time

import numpy as np
import torch  # noqa: F401  (imported at collection, before any test timer starts)
import pytest

import graph_all_pairs_amd as ga
import graphgen as gg
import oracle

pytestmark = pytest.mark.gpu
INF = gg.INF_I32
POLICIES = {"auto": ga.APSP_ARITH_AUTO, "int32": ga.APSP_ARITH_INT32,
            "f32": ga.APSP_ARITH_F32_WHEN_EXACT}


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


@pytest.fixture(scope="module")
def say(request):
    """Print at once, past pytest's output capture (progress of long steps)."""
    capman = request.config.pluginmanager.getplugin("capturemanager")

    def _say(msg):
        if capman is not None:
            with capman.global_and_fixture_disabled():
                print(msg, flush=True)
        else:
            print(msg, flush=True)
    return _say


class _Cache:
    """Workload matrices and full oracle results, built once per module."""

    def __init__(self, say):
        self.say = say
        self.inputs = {}
        self.results = {}

    def input(self, name):
        if name not in self.inputs:
            self.inputs[name] = gg.make_workload(name)
        return self.inputs[name]

    def oracle(self, name):
        if name not in self.results:
            w = self.input(name)
            n = w.shape[0]
            t0 = time.perf_counter()
            self.say(f"  oracle {name}: full Floyd-Warshall on {oracle.default().threads()} "
                     f"host threads")

            def progress(k, total):
                self.say(f"  oracle {name}: {k}/{total} pivots, "
                         f"{time.perf_counter() - t0:.0f} s")
            self.results[name] = oracle.default().fw_in_steps(w, max(512, n // 8), progress)
        return self.results[name]


@pytest.fixture(scope="module")
def cache(say):
    c = _Cache(say)
    yield c
    c.inputs.clear()
    c.results.clear()


def run(torch_dev, w, inf):
    torch, dev = torch_dev
    t = torch.from_numpy(w).to(dev)
    ga.fw(t, inf)
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("name", ["er-256-p0.1-i32", "er-2048-p0.05-i32"])
@pytest.mark.parametrize("arith", sorted(POLICIES))
def test_small_workloads_full_oracle(torch_dev, name, arith):
    print(f"case workload {name} arith policy {arith}", flush=True)
    w = gg.make_workload(name)
    with ga.int32_arith(POLICIES[arith]):
        got = run(torch_dev, w, INF)
    assert np.array_equal(got, oracle.fw_i32(w))


def sample_sources(n, k, seed):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(n, size=min(k, n), replace=False).tolist())
    s |= {0, n - 1, n // 2, 127, 128}            # block edges and the ragged tail
    return np.array(sorted(x for x in s if x < n))


@pytest.mark.parametrize("name", ["complete-8192-i32", "ba-16000-b8-i32"])
def test_large_int_workloads_sampled(torch_dev, cache, name):
    """Early check: sampled rows and columns against Dijkstra."""
    print(f"case workload {name} (sampled)", flush=True)
    w = cache.input(name)
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


def test_large_float_workload_sampled(torch_dev, cache):
    """Early check: sampled rows against binary64 Dijkstra."""
    print("case workload complete-12288-f32 (sampled)", flush=True)
    w = cache.input("complete-12288-f32")
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


def _first_mismatches(got, want, k=5):
    bad = np.argwhere(got != want)
    return [(int(i), int(j), int(got[i, j]), int(want[i, j])) for i, j in bad[:k]], len(bad)


@pytest.mark.parametrize("name,arith", [
    ("complete-8192-i32", "auto"), ("complete-8192-i32", "int32"), ("complete-8192-i32", "f32"),
    ("ba-16000-b8-i32", "auto"), ("ba-16000-b8-i32", "int32")])
def test_large_int_workloads_full_oracle(torch_dev, cache, say, name, arith):
    """Every element, bit for bit, against the oracle's full recurrence."""
    print(f"case workload {name} arith policy {arith} (full oracle)", flush=True)
    w = cache.input(name)
    with ga.int32_arith(POLICIES[arith]):
        got = run(torch_dev, w, INF)
    want = cache.oracle(name)
    first, count = _first_mismatches(got, want)
    say(f"  {name} [{arith}]: {count} of {got.size} elements differ from the oracle")
    assert count == 0, f"{count} elements differ; first (i, j, gpu, oracle): {first}"


def test_large_float_workload_full_oracle(torch_dev, cache, say):
    """Every element within 1e-5 relative of the binary64 recurrence; zeros
    exact; a second GPU run identical bit for bit."""
    name = "complete-12288-f32"
    print(f"case workload {name} (full oracle)", flush=True)
    w = cache.input(name)
    got = run(torch_dev, w, np.inf)
    again = run(torch_dev, w, np.inf)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))
    want = cache.oracle(name)
    g = got.astype(np.float64)
    assert np.array_equal(g == 0, want == 0)
    assert np.array_equal(np.isinf(g), np.isinf(want))
    fin = np.isfinite(want) & (want != 0)
    rel = np.abs(g[fin] - want[fin]) / want[fin]
    worst = float(rel.max())
    say(f"  {name}: largest relative difference from the binary64 oracle {worst:.3e}")
    assert worst <= 1e-5, worst
