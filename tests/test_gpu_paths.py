"""GPU parity of path reconstruction: the successor (first-hop) matrix
(apsp_successors_*, apsp_fw_paths_*) against the oracle's definition --
for i != j the smallest u != i minimising w[i][u] + d[u][j] -- bit-exact for
int32, on graphs with many equal-length paths (small integer weights, unit
grids).  float32 successors are checked for validity: the path they give
has the shortest distance's weight.
"""
import numpy as np
import torch
import pytest

import graph_all_pairs_amd as ga
import graphgen as gg
import oracle

pytestmark = pytest.mark.gpu

INF = gg.INF_I32


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def gpu_successors(dev, w, d, ldn=None, offset=0, inf=None):
    n = w.shape[0]
    ldn = n if ldn is None else ldn
    tw = torch.from_numpy(np.ascontiguousarray(w)).to(dev)
    td = torch.from_numpy(np.ascontiguousarray(d)).to(dev)
    buf = torch.full((n * ldn + offset + 4,), -9, dtype=torch.int32, device=dev)
    out = buf[offset:offset + n * ldn].view(n, ldn)
    s = torch.cuda.current_stream().cuda_stream
    fn = ga.apsp_successors_i32 if w.dtype == np.int32 else ga.apsp_successors_f32
    if inf is None:
        inf = INF if w.dtype == np.int32 else float("inf")
    st = fn(tw.data_ptr(), n, td.data_ptr(), n, out.data_ptr(), ldn, n, inf, s)
    assert st == ga.APSP_OK, ga.apsp_status_string(st)
    host = buf.cpu().numpy()
    full = host[offset:offset + n * ldn].reshape(n, ldn)
    assert (full[:, n:] == -9).all() and (host[:offset] == -9).all()
    assert (host[offset + n * ldn:] == -9).all()
    return full[:, :n].copy()


def tie_graph(n, p, seed):
    w = gg.erdos_renyi(n, p, 1, 3, seed)        # weights 1..3: many equal-length paths
    return w


@pytest.mark.parametrize("n", [1, 2, 5, 64, 127, 128, 129, 300, 1000, 1031])
def test_int32_successors_match_oracle(dev, orc, n):
    print(f"case successors i32 n={n}", flush=True)
    w = tie_graph(n, 0.05 if n > 64 else 0.3, 500 + n)
    d = orc.fw_i32(w)
    got = gpu_successors(dev, w, d)
    assert np.array_equal(got, orc.successors(w, d, INF))


# The call picks one of two kernels from the number of finite off-diagonal
# weights: a neighbour-list kernel up to n^2 / 16, the dense product above.
# Both compute the same matrix; these cases sit on either side.

@pytest.mark.parametrize("n", [129, 1000])
def test_int32_successors_dense_side(dev, orc, n):
    print(f"case successors i32 dense side n={n}", flush=True)
    w = tie_graph(n, 0.12, 900 + n)
    assert ((w < INF).sum() - n) > n * n // 16
    d = orc.fw_i32(w)
    assert np.array_equal(gpu_successors(dev, w, d), orc.successors(w, d, INF))


# Dense int32 matrices take packed keys ((w + d) << shift | u in 32 bits)
# when every finite weight and distance is >= 0 and the largest finite
# weight plus the largest finite distance is below inf and 2^(31 - shift),
# shift = ceil(log2 n); otherwise the (value, index) kernel.  n = 300 gives
# shift 9 and a bound of 2^22: near-tied weights around 2^20 stay below it,
# around 2^21 they cross it.  Both sides match the oracle bit for bit.

@pytest.mark.parametrize("base", [1 << 20, 1 << 21])
def test_int32_successors_dense_around_the_packed_bound(dev, orc, base):
    print(f"case successors i32 dense weights base={base}", flush=True)
    n = 300
    rng = np.random.default_rng(base % 1000 + 7)
    w = (base + rng.integers(0, 4, size=(n, n))).astype(np.int32)
    w[rng.random((n, n)) < 0.5] = INF
    np.fill_diagonal(w, 0)
    d = orc.fw_i32(w)
    fin = d[d < INF]
    packed = int(w[(w < INF)].max()) + int(fin.max()) < (1 << 22)
    assert packed == (base == 1 << 20)
    assert np.array_equal(gpu_successors(dev, w, d), orc.successors(w, d, INF))


def test_int32_successors_hub_rows_take_several_gathers(dev, orc):
    # rows with more neighbours than one gather holds (2048), in a sparse matrix
    print("case successors i32 hub rows n=2500", flush=True)
    n = 2500
    w = tie_graph(n, 0.004, 31)
    rng = np.random.default_rng(5)
    for r in (0, 1, 1234, n - 1):
        w[r, :] = rng.integers(1, 4, size=n)
        w[r, r] = 0
    assert ((w < INF).sum() - n) <= n * n // 16
    d = orc.fw_i32(w)
    assert np.array_equal(gpu_successors(dev, w, d), orc.successors(w, d, INF))


@pytest.mark.parametrize("p", [0.02, 0.2])
def test_float32_successors_exact_on_integer_weights(dev, orc, p):
    # small integer weights are exact in binary32, so both kernels must give
    # the oracle's int32 matrix
    print(f"case successors f32 integer weights p={p}", flush=True)
    n = 500
    w = tie_graph(n, p, 77)
    d = orc.fw_i32(w)
    wf = np.where(w == INF, np.inf, w).astype(np.float32)
    df = np.where(d == INF, np.inf, d).astype(np.float32)
    assert np.array_equal(gpu_successors(dev, wf, df), orc.successors(w, d, INF))


@pytest.mark.parametrize("n,p", [(64, 0.02), (64, 0.5)])
def test_int32_successors_small_sentinel(dev, orc, n, p):
    # inf = 10 with weights 4..6: two-hop sums already reach the sentinel, and
    # a pair whose every path sum is >= inf has no first hop (as its distance
    # is inf); sparse (p = 0.02) and dense (p = 0.5) kernels
    print(f"case successors small sentinel n={n} p={p}", flush=True)
    inf = 10
    w = gg.erdos_renyi(n, p, 4, 6, 40 + int(p * 100), inf=inf)
    d = orc.fw_i32(w)
    want = orc.successors(w, d, inf)
    assert (want == -1).any() and (d == inf).any()
    assert np.array_equal(gpu_successors(dev, w, d, inf=inf), want)


def test_grid_successors_and_paths(dev, orc):
    print("case successors grid", flush=True)
    w = gg.grid(24, 30)
    d = orc.fw_i32(w)
    got = gpu_successors(dev, w, d, ldn=w.shape[0] + 5, offset=1)
    assert np.array_equal(got, orc.successors(w, d, INF))
    # walking the successors gives a path of the shortest length
    n = w.shape[0]
    rng = np.random.default_rng(1)
    for i, j in rng.integers(0, n, size=(50, 2)):
        p = ga.path(got, int(i), int(j))
        assert p[0] == i and p[-1] == j
        assert sum(int(w[a, b]) for a, b in zip(p, p[1:])) == d[i, j]


def test_fw_paths_combined(dev, orc):
    print("case fw_paths i32 and f32", flush=True)
    n = 700
    w = tie_graph(n, 0.01, 77)
    t = torch.from_numpy(w).to(dev)
    nxt = ga.fw_paths(t, inf=INF)
    d = orc.fw_i32(w)
    assert np.array_equal(t.cpu().numpy(), d)
    assert np.array_equal(nxt.cpu().numpy(), orc.successors(w, d, INF))
    # unreachable pairs give -1
    wf = gg.complete_f32(300, 9)
    wf[:150, 150:] = np.inf                        # no edge from the first half to the second
    tf = torch.from_numpy(wf).to(dev)
    nf = ga.fw_paths(tf).cpu().numpy()
    df = tf.cpu().numpy()
    assert (nf[:150, 150:] == -1).all()
    rng = np.random.default_rng(2)
    for i, j in rng.integers(0, 300, size=(200, 2)):
        p = ga.path(nf, int(i), int(j))
        if not np.isfinite(df[i, j]):
            assert p == []
            continue
        length = sum(float(wf[a, b]) for a, b in zip(p, p[1:]))
        assert abs(length - float(df[i, j])) <= 1e-5 * max(abs(float(df[i, j])), 1.0)


def test_successors_on_the_complete_workload_shape(dev, orc):
    print("case successors complete n=2048", flush=True)
    w = gg.complete(2048, 1, 20, 3)               # narrow weights: ties everywhere
    d = orc.fw_i32(w)
    got = gpu_successors(dev, w, d)
    assert np.array_equal(got, orc.successors(w, d, INF))


# ---- zero-weight cycles ------------------------------------------------------
# Weights may be 0, so two vertices joined by 0-weight edges both ways can tie
# as first hops towards the same target.  The successor matrix is still the
# defined one (smallest minimising u, equal to the oracle's), but following it
# may loop: apsp_path then returns -3.  Without a cycle of total weight 0 every
# walk reaches its target.

def walk_expected(nxt, i, j):
    """What the host walker must return for (i, j): the vertex count of the
    walk, -1 when j is unreachable, -3 when the walk does not reach j within
    n hops (it entered a successor cycle)."""
    n = nxt.shape[0]
    if nxt[i, j] < 0:
        return -1
    v, count = i, 1
    for _ in range(n):
        if v == j:
            return count
        v = int(nxt[v, j])
        count += 1
    return count if v == j else -3


def zero_cycle_graph(n, p, seed, a, b):
    """Sparse or dense integer weights 1..9 with a 0-weight 2-cycle a <-> b,
    a < every other vertex: a's only out-edge goes to b.  For every j that
    b reaches, a's first hop is b (its one candidate) and b's is a (0 +
    d(a, j) = d(b, j), and a is the smallest index), so the two name each
    other."""
    w = gg.erdos_renyi(n, p, 1, 9, seed)
    w[a, :] = INF
    w[a, a] = w[b, b] = 0
    w[a, b] = w[b, a] = 0
    return w


# (n, p, scale): dense packed keys, the neighbour lists (p = 0.02), and with
# weights scaled by 2^21 the dense (value, index) kernel (the keys no longer
# fit 32 bits at n = 300).
@pytest.mark.parametrize("n,p,scale", [(6, 0.9, 1), (64, 0.3, 1), (200, 0.02, 1), (300, 0.5, 1),
                                       (300, 0.5, 1 << 21)])
def test_zero_weight_two_cycle(dev, orc, n, p, scale):
    print(f"case successors with a zero-weight 2-cycle n={n} p={p} scale={scale}", flush=True)
    a, b = 0, n - 2
    w = zero_cycle_graph(n, p, 700 + n, a, b)
    w = np.where(w == INF, INF, w.astype(np.int64) * scale).astype(np.int32)
    d = orc.fw_i32(w)
    want = orc.successors(w, d, INF)
    got = gpu_successors(dev, w, d)
    assert np.array_equal(got, want)
    # the 2-cycle is real: some target has a and b naming each other
    loops = [j for j in range(n) if j not in (a, b) and want[a, j] == b and want[b, j] == a]
    assert loops, "the graph does not exercise the zero-weight cycle"
    buf = np.empty(n + 1, dtype=np.int32)
    g = np.ascontiguousarray(got)
    for i in range(n):
        for j in range(n):
            r = ga.apsp_path(g.ctypes.data, n, n, i, j, buf.ctypes.data, len(buf))
            assert r == walk_expected(want, i, j), (i, j, r)
            if r > 0:   # a finished walk has the shortest distance's weight
                hops = buf[:r]
                assert hops[0] == i and hops[-1] == j
                assert int(sum(int(w[x, y]) for x, y in zip(hops[:-1], hops[1:]))) == int(d[i, j])
    for j in loops:
        assert ga.apsp_path(g.ctypes.data, n, n, a, j, buf.ctypes.data, len(buf)) == -3
    # float32 takes the same definition (weights are small integers, exact)
    wf = np.where(w == INF, np.float32(np.inf), w.astype(np.float32)).astype(np.float32)
    df = np.where(d == INF, np.float32(np.inf), d.astype(np.float32)).astype(np.float32)
    assert np.array_equal(gpu_successors(dev, wf, df), want)


# ---- one pass of the rounds on successor keys (apsp_fw_paths_i32) ----------
# Dense int32 weights >= 0 with a zero diagonal and a bounded range take the
# key form (value << s | first hop); everything else takes the rounds and
# then the successor pass.  Both must give the oracle's distances and its
# successor matrix bit for bit; apsp_fw_paths_last_form says which ran.

def gpu_fw_paths(dev, w, inf=INF, ld=None, ldn=None, doff=0, noff=0):
    """apsp_fw_paths_i32 through the C ABI on w placed with leading dimension
    ld at element offset doff (nxt: ldn, noff); checks that no byte outside
    the two n x n blocks changed and returns (d, nxt, form)."""
    n = w.shape[0]
    ld = n if ld is None else ld
    ldn = n if ldn is None else ldn
    dbuf = torch.full((doff + n * ld + 4,), -7, dtype=torch.int32, device=dev)
    dv = dbuf[doff:doff + n * ld].view(n, ld)
    dv[:, :n] = torch.from_numpy(np.ascontiguousarray(w)).to(dev)
    nbuf = torch.full((noff + n * ldn + 4,), -9, dtype=torch.int32, device=dev)
    nv = nbuf[noff:noff + n * ldn].view(n, ldn)
    s = torch.cuda.current_stream().cuda_stream
    st = ga.apsp_fw_paths_i32(dv.data_ptr(), ld, nv.data_ptr(), ldn, n, inf, s)
    assert st == ga.APSP_OK, ga.apsp_status_string(st)
    form = ga.apsp_fw_paths_last_form()
    hd, hn = dbuf.cpu().numpy(), nbuf.cpu().numpy()
    d = hd[doff:doff + n * ld].reshape(n, ld)
    nx = hn[noff:noff + n * ldn].reshape(n, ldn)
    assert (hd[:doff] == -7).all() and (hd[doff + n * ld:] == -7).all() and (d[:, n:] == -7).all()
    assert (hn[:noff] == -9).all() and (hn[noff + n * ldn:] == -9).all() and (nx[:, n:] == -9).all()
    return d[:, :n].copy(), nx[:, :n].copy(), form


def check_fw_paths(dev, orc, w, form, inf=INF, **layout):
    d, nxt, got_form = gpu_fw_paths(dev, w, inf=inf, **layout)
    assert got_form == form
    want_d = orc.fw_i32(w)
    assert np.array_equal(d, want_d)
    assert np.array_equal(nxt, orc.successors(w, want_d, inf))
    return d, nxt


@pytest.mark.parametrize("n", [1, 2, 3, 5, 63, 64, 65, 127, 128, 129, 255, 256, 257, 500, 1031,
                               2049, 4100])
def test_fw_paths_keys_complete_with_ties(dev, orc, n):
    # weights 1..3 on every pair: many shortest paths per pair, so the
    # smallest-first-hop rule decides most entries
    print(f"case fw_paths keys complete n={n}", flush=True)
    w = gg.complete(n, 1, 3, 900 + n)
    check_fw_paths(dev, orc, w, 1 if n >= 2 else 0)


def test_fw_paths_keys_layouts(dev, orc):
    # padded leading dimensions, unaligned pointers (scalar loads) and
    # 16-byte-aligned ones with gaps
    print("case fw_paths keys layouts", flush=True)
    w = gg.complete(200, 1, 4, 77)
    check_fw_paths(dev, orc, w, 1, ld=203, ldn=201, doff=1, noff=3)
    check_fw_paths(dev, orc, w, 1, ld=204, ldn=208, doff=4, noff=8)
    check_fw_paths(dev, orc, w, 1, ld=200, ldn=203, doff=0, noff=1)


@pytest.mark.parametrize("n", [6, 130, 300])
def test_fw_paths_keys_zero_weights(dev, orc, n):
    # weights 0..2 on a complete graph: zero-weight cycles everywhere; the
    # matrix is still the defined one
    print(f"case fw_paths keys zero weights n={n}", flush=True)
    w = gg.complete(n, 0, 2, 40 + n)
    np.fill_diagonal(w, 0)
    check_fw_paths(dev, orc, w, 1)
    # and the dense 2-cycle graph (some off-diagonal entries inf)
    w = zero_cycle_graph(n, 0.9, 800 + n, 0, n - 2)
    check_fw_paths(dev, orc, w, 1)


@pytest.mark.parametrize("hi,form", [(3, 1), (10000, 0)])
def test_fw_paths_dense_with_missing_edges(dev, orc, hi, form):
    # p = 0.5 at n = 300: dense, with inf entries, so the bound is (n - 1)
    # times the largest weight against 2^(30 - 9) - 1: 897 takes the keys,
    # 2 990 000 the successor pass
    print(f"case fw_paths dense p=0.5 weights 1..{hi}", flush=True)
    w = gg.erdos_renyi(300, 0.5, 1, hi, 61)
    assert (w == INF).any()
    check_fw_paths(dev, orc, w, form)


def test_fw_paths_keys_range_bound(dev, orc):
    # n = 100: s = 7, keys exact while every stored value is below
    # 2^23 - 1 = 8388607; on a complete graph that is the largest weight
    print("case fw_paths keys range bound", flush=True)
    lim = (1 << 23) - 1
    w = gg.complete(100, lim - 1000, lim - 1, 5)
    w[3, 7] = lim - 1
    check_fw_paths(dev, orc, w, 1)
    w[3, 7] = lim
    check_fw_paths(dev, orc, w, 0)


def test_fw_paths_keys_small_sentinel(dev, orc):
    # inf = 60 with weights 20..40 at p = 0.1 (1409 edges, dense): two hops
    # already weigh 40 or more, and pairs whose every path weighs 60 or more
    # are unreachable (distance inf, no first hop)
    print("case fw_paths keys small sentinel", flush=True)
    inf = 60
    w = gg.erdos_renyi(120, 0.1, 20, 40, 19, inf=inf)
    d, nxt = check_fw_paths(dev, orc, w, 1, inf=inf)
    assert (d == inf).any() and (nxt == -1).any()


def test_fw_paths_other_inputs_take_the_successor_pass(dev, orc):
    print("case fw_paths fallbacks", flush=True)
    # sparse weights (at most n^2/16 finite): the neighbour-list pass is cheaper
    check_fw_paths(dev, orc, gg.erdos_renyi(400, 0.05, 1, 3, 8), 0)
    # a weight above the range of a complete graph of this size
    w = gg.complete(3000, 1, 3, 9)
    w[5, 9] = 1 << 18        # s = 12: the bound is 2^18 - 1
    check_fw_paths(dev, orc, w, 0)


def test_fw_paths_keys_complete_8192(dev, orc):
    # the complete-8192 workload (weights 1..10000): the key form at full
    # size, every distance against the oracle and sampled successor rows
    print("case fw_paths keys complete-8192", flush=True)
    w = gg.make_workload("complete-8192-i32")
    n = w.shape[0]
    d, nxt, form = gpu_fw_paths(dev, w)
    assert form == 1
    want_d = orc.fw_i32(w)
    assert np.array_equal(d, want_d)
    rows = np.array([0, 1, 127, 128, 4095, 4096, 8063, 8064, 8190, 8191]
                    + list(np.random.default_rng(3).integers(0, n, size=6)))
    assert np.array_equal(nxt[rows], orc.successors_rows(w, want_d, INF, rows))
