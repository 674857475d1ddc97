"""GPU parity of the batched small-graph entry points (many independent
graphs of n <= 128, one workgroup each) against the CPU oracle.

int32: bit-exact per graph.  float32: within 1e-5 relative of the oracle's
binary64 distances, and bit-identical to the single-graph entry point on the
same graph (both close the graph pivot by pivot in order).  Bytes outside
each graph's n x n block (row padding, gaps between graphs) are never
touched.
"""
import numpy as np
import torch  # noqa: F401
import pytest

import graph_all_pairs_amd as ga
import graphgen as gg
import oracle

pytestmark = pytest.mark.gpu

INF = gg.INF_I32
F32_RTOL = 1e-5
# every size class (n rounded up to a multiple of 8, at least 16) at its edge
# and one past it, plus a few sizes inside classes
SIZES = [1, 2, 3, 5, 8, 9, 16, 17, 24, 25, 31, 32, 33, 40, 41, 47, 48, 49, 56, 57, 63, 64, 65,
         72, 73, 80, 81, 88, 89, 96, 97, 100, 104, 105, 112, 113, 120, 121, 127, 128]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_batched(dev, graphs, inf, ld=None, stride=None, offset=0, canary=-7):
    """Place graphs (batch, n, n) at base + g*stride with leading dimension
    ld, run the C-ABI batched entry, return (results (batch, n, n), flat
    buffer, layout) so callers can check the bytes around the graphs."""
    batch, n = graphs.shape[0], graphs.shape[1]
    ld = n if ld is None else ld
    span = (n - 1) * ld + n if n else 0
    stride = span if stride is None else stride
    total = offset + (batch - 1) * stride + span if batch else offset
    host = np.full(total + 8, canary, dtype=graphs.dtype)
    for g in range(batch):
        for i in range(n):
            a = offset + g * stride + i * ld
            host[a:a + n] = graphs[g, i]
    buf = torch.from_numpy(host.copy()).to(dev)
    ptr = buf.data_ptr() + offset * graphs.dtype.itemsize
    fn = ga.apsp_fw_batched_i32 if graphs.dtype == np.int32 else ga.apsp_fw_batched_f32
    st = fn(ptr, batch, n, ld, stride, inf, torch.cuda.current_stream().cuda_stream)
    assert st == ga.APSP_OK, ga.apsp_status_string(st)
    torch.cuda.synchronize()
    out = buf.cpu().numpy()
    res = np.empty_like(graphs)
    touched = np.zeros(out.shape[0], dtype=bool)
    for g in range(batch):
        for i in range(n):
            a = offset + g * stride + i * ld
            res[g, i] = out[a:a + n]
            touched[a:a + n] = True
    assert np.all(out[~touched] == canary), "bytes outside the graphs changed"
    return res


def assert_f32_close(got, want):
    got = got.astype(np.float64)
    assert np.array_equal(np.isinf(got), np.isinf(want))
    fin = np.isfinite(want)
    g, o = got[fin], want[fin]
    assert np.all((o == 0) == (g == 0))
    rel = np.abs(g - o) / np.maximum(np.abs(o), np.finfo(np.float64).tiny)
    assert float(rel.max(initial=0.0)) <= F32_RTOL, float(rel.max())


@pytest.mark.parametrize("n", SIZES)
def test_batched_i32_er_exact(dev, n):
    print(f"batched i32 ER n={n}", flush=True)
    w = gg.erdos_renyi_batch(37, n, 0.15, 1, 100, 100 + n)
    got = run_batched(dev, w, INF)
    assert np.array_equal(got, oracle.default().fw_batched_i32(w))


@pytest.mark.parametrize("n", [4, 32, 45, 48, 64, 65, 72, 80, 96, 99, 101, 112, 126, 128])
def test_batched_i32_complete_padded_layout(dev, n):
    # ld > n and a gap between graphs; the smallest legal stride too
    print(f"batched i32 complete n={n}", flush=True)
    w = gg.erdos_renyi_batch(19, n, 1.0, 1, 10000, 200 + n)
    want = oracle.default().fw_batched_i32(w)
    assert np.array_equal(run_batched(dev, w, INF, ld=n + 4, stride=(n + 4) * n + 12), want)
    assert np.array_equal(run_batched(dev, w, INF, ld=n + 3), want)   # stride = (n-1)*ld + n


@pytest.mark.parametrize("n", [8, 48, 64, 70, 77, 90, 128])
def test_batched_i32_unaligned_scalar_path(dev, n):
    print(f"batched i32 unaligned n={n}", flush=True)
    w = gg.erdos_renyi_batch(11, n, 0.3, 1, 50, 300 + n)
    got = run_batched(dev, w, INF, ld=n + 4, stride=(n + 4) * n, offset=1)
    assert np.array_equal(got, oracle.default().fw_batched_i32(w))


def test_batched_i32_rings_closed_form(dev):
    # directed ring of n vertices, weight 1: d(i, j) = (j - i) mod n
    print("batched rings", flush=True)
    for n in (5, 32, 100, 128):
        ring = gg.ring(n)
        w = np.stack([ring] * 9)
        got = run_batched(dev, w, INF)
        i = np.arange(n)
        want = ((i[None, :] - i[:, None]) % n).astype(np.int32)
        assert all(np.array_equal(got[g], want) for g in range(9))


@pytest.mark.parametrize("n", [5, 32, 40, 45, 64, 67, 72, 99, 100, 126, 128])
def test_batched_f32_matches_oracle_and_single_entry(dev, n):
    print(f"batched f32 n={n}", flush=True)
    w = gg.complete_f32_batch(13, n, 400 + n)
    got = run_batched(dev, w, float("inf"))
    want = oracle.default().fw_batched_f64(w)
    for g in range(13):
        assert_f32_close(got[g], want[g])
    # the single-graph entry closes an n <= 128 graph the same way
    for g in (0, 12):
        t = torch.from_numpy(w[g].copy()).to(dev)
        ga.fw(t)
        assert np.array_equal(t.cpu().numpy().view(np.int32), got[g].view(np.int32))


def test_batched_f32_finite_sentinel(dev):
    print("batched f32 finite sentinel", flush=True)
    n = 40
    big = np.float32(1e30)
    w = gg.erdos_renyi_batch(8, n, 0.03, 1, 9, 77).astype(np.float32)
    w[w == INF] = big
    got = run_batched(dev, w, float(big))
    want = oracle.default().fw_batched_f64(w.astype(np.float64))
    assert np.any(want == float(big))  # some pairs stay unreachable
    assert np.array_equal(got == big, want == float(big))
    fin = want < float(big)
    assert np.array_equal(got[fin].astype(np.float64), want[fin])  # small integers: exact


def test_batched_many_graphs_grid_stride(dev):
    # more graphs than workgroups in one launch (2^20): the kernel loops
    print("batched many graphs", flush=True)
    batch, n = (1 << 20) + 77, 3
    w = gg.erdos_renyi_batch(batch, n, 0.5, 1, 20, 500)
    t = torch.from_numpy(w).to(dev)
    ga.fw_batched(t)
    torch.cuda.synchronize()
    assert np.array_equal(t.cpu().numpy(), oracle.default().fw_batched_i32(w))


@pytest.mark.parametrize("n", [65, 73])
def test_batched_many_graphs_grid_stride_one_wave_classes(dev, n):
    # 2^20 + 77 graphs of the one-wave size classes: 64 distinct graphs
    # repeated on the device, every graph compared with the oracle's
    print(f"batched many graphs n={n}", flush=True)
    batch, distinct = (1 << 20) + 77, 64
    w = gg.erdos_renyi_batch(distinct, n, 0.3, 1, 50, 600 + n)
    want = torch.from_numpy(oracle.default().fw_batched_i32(w)).to(dev)
    t = torch.from_numpy(w).to(dev).repeat(batch // distinct + 1, 1, 1)[:batch].contiguous()
    ga.fw_batched(t)
    torch.cuda.synchronize()
    idx = torch.arange(batch, device=dev) % distinct
    for c0 in range(0, batch, 1 << 16):
        c1 = min(batch, c0 + (1 << 16))
        assert torch.equal(t[c0:c1], want[idx[c0:c1]]), f"graphs {c0}..{c1}"
    del t


def test_batched_empty_and_wrapper_errors(dev):
    t = torch.zeros((0, 5, 5), dtype=torch.int32, device=dev)
    ga.fw_batched(t)
    with pytest.raises(ga.APSPError):
        ga.fw_batched(torch.zeros((2, 129, 129), dtype=torch.int32, device=dev))
    with pytest.raises(ValueError):
        ga.fw_batched(torch.zeros((5, 5), dtype=torch.int32, device=dev))
