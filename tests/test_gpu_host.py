"""GPU parity of the min-plus product (apsp_minplus_gemm_*) and of the
host-resident blocked Floyd-Warshall (apsp_fw_host_*) against the CPU oracle.

The product is compared with the oracle's definition of min(C, A (x) B):
bit-exact for int32, within 1e-6 relative for float32 (each candidate is one
rounded sum).  The host-resident path is compared with the oracle's plain
Floyd-Warshall: bit-exact for int32 under every arithmetic policy and outer
block size, within 1e-5 relative for float32; bytes outside the n x n block
of the host matrix are never touched.
"""
import numpy as np
import torch
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


def rand_op(rng, rows, cols, p, wmax, dtype):
    if dtype == np.int32:
        v = rng.integers(0, wmax + 1, size=(rows, cols))
        return np.where(rng.random((rows, cols)) < p, v, INF).astype(np.int32)
    v = rng.uniform(-0.5 if wmax < 0 else 0.01, 1.0, size=(rows, cols))
    return np.where(rng.random((rows, cols)) < p, v, np.inf).astype(np.float32)


def gpu_gemm(dev, c, a, b, pad=0, offset=0):
    """Place each operand in a padded device buffer (leading dimension cols +
    pad, start offset elements in) and run the C-ABI product; check that the
    canary around C survives."""
    def place(x):
        rows, cols = x.shape
        ld = cols + pad
        dt = torch.int32 if x.dtype == np.int32 else torch.float32
        buf = torch.full((rows * ld + offset + 8,), CANARY, dtype=dt, device=dev)
        view = buf[offset:offset + rows * ld].view(rows, ld)[:, :cols]
        view.copy_(torch.from_numpy(x))
        return buf, view, ld
    cb, cv, ldc = place(c)
    _, av, lda = place(a)
    _, bv, ldb = place(b)
    m, n, k = c.shape[0], c.shape[1], a.shape[1]
    s = torch.cuda.current_stream().cuda_stream
    if c.dtype == np.int32:
        st = ga.apsp_minplus_gemm_i32(cv.data_ptr(), ldc, av.data_ptr(), lda, bv.data_ptr(), ldb,
                                      m, n, k, INF, s)
    else:
        st = ga.apsp_minplus_gemm_f32(cv.data_ptr(), ldc, av.data_ptr(), lda, bv.data_ptr(), ldb,
                                      m, n, k, float("inf"), s)
    assert st == ga.APSP_OK, ga.apsp_status_string(st)
    host = cb.cpu().numpy()
    full = host[offset:offset + m * ldc].reshape(m, ldc)
    assert (full[:, n:] == CANARY).all() and (host[:offset] == CANARY).all()
    assert (host[offset + m * ldc:] == CANARY).all()
    return full[:, :n].copy()


SHAPES = [(1, 1, 1), (5, 7, 3), (128, 128, 128), (129, 127, 130), (300, 260, 17),
          (257, 384, 1000), (1000, 513, 64), (64, 2000, 2048)]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_gemm_int32_matches_oracle(dev, m, n, k):
    print(f"case gemm i32 {m}x{n}x{k}", flush=True)
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    a = rand_op(rng, m, k, 0.6, 1000, np.int32)
    b = rand_op(rng, k, n, 0.6, 1000, np.int32)
    c = rand_op(rng, m, n, 0.3, 3000, np.int32)
    got = gpu_gemm(dev, c, a, b)
    assert np.array_equal(got.astype(np.int64), oracle.default().minplus(c, a, b, INF))


@pytest.fixture(scope="module")
def share_ops():
    """One GPU's share of round 32 when complete-8192-i32 is split into 8
    block rows (GPU 4's slab): C the 1024 x 8192 slab, A its pivot columns,
    B the round's 128 x 8192 pivot-row panel, and the oracle's product."""
    w = gg.make_workload("complete-8192-i32")
    rows, n, B, K, p = 1024, 8192, 128, 32, 4
    c = np.ascontiguousarray(w[p * rows:(p + 1) * rows, :n])
    a = np.ascontiguousarray(c[:, K * B:(K + 1) * B])
    b = np.ascontiguousarray(w[K * B:(K + 1) * B, :n])
    return c, a, b, oracle.default().minplus(c, a, b, INF)


@pytest.mark.parametrize("f32", [False, True])
def test_gemm_one_gpu_share_of_a_round(dev, share_ops, f32):
    """The multi-GPU design's per-GPU Phase-3 step at its real shape
    (bench.py --workload shard-complete-8192-i32-p8 times it).  Bit-exact
    against the oracle in int32 and in binary32 (integer weights, so every
    candidate is exact)."""
    print(f"case one GPU's share, f32={f32}", flush=True)
    c, a, b, want = share_ops
    if f32:
        tf = lambda x: np.where(x == INF, np.float32(np.inf), x.astype(np.float32))
        got = gpu_gemm(dev, tf(c), tf(a), tf(b))
        got = np.where(np.isinf(got), INF, got).astype(np.int64)
    else:
        got = gpu_gemm(dev, c, a, b).astype(np.int64)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("m,n,k", [(129, 127, 130), (300, 260, 17), (256, 256, 4096)])
@pytest.mark.parametrize("neg", [False, True])
def test_gemm_float32_matches_oracle(dev, m, n, k, neg):
    print(f"case gemm f32 {m}x{n}x{k} neg={neg}", flush=True)
    rng = np.random.default_rng(m + n + k)
    wmax = -1 if neg else 1
    a = rand_op(rng, m, k, 0.6, wmax, np.float32)
    b = rand_op(rng, k, n, 0.6, wmax, np.float32)
    c = rand_op(rng, m, n, 0.3, wmax, np.float32)
    got = gpu_gemm(dev, c, a, b)
    want = oracle.default().minplus(c.astype(np.float64), a.astype(np.float64), b.astype(np.float64))
    assert np.array_equal(np.isinf(got), np.isinf(want))
    fin = np.isfinite(want)
    err = np.abs(got[fin].astype(np.float64) - want[fin])
    assert (err <= 1e-6 * np.maximum(np.abs(want[fin]), 1.0)).all(), err.max()


def test_gemm_padding_and_scalar_path(dev):
    print("case gemm padded, unaligned", flush=True)
    rng = np.random.default_rng(3)
    m, n, k = 200, 300, 150
    a = rand_op(rng, m, k, 0.5, 100, np.int32)
    b = rand_op(rng, k, n, 0.5, 100, np.int32)
    c = rand_op(rng, m, n, 0.2, 300, np.int32)
    want = oracle.default().minplus(c, a, b, INF)
    for pad, offset in ((4, 0), (3, 1), (0, 2)):
        got = gpu_gemm(dev, c, a, b, pad=pad, offset=offset)
        assert np.array_equal(got.astype(np.int64), want)


def test_gemm_squaring_reaches_the_closure(dev):
    # repeated min-plus squaring of a zero-diagonal weight matrix is APSP
    print("case gemm squaring", flush=True)
    n = 700
    w = gg.erdos_renyi(n, 0.01, 1, 100, 21)
    d = torch.from_numpy(w).to(dev)
    for _ in range(int(np.ceil(np.log2(n - 1)))):
        ga.minplus_gemm(d, d.clone(), d.clone())
    assert np.array_equal(d.cpu().numpy(), oracle.fw_i32(w))


# ---- host-resident blocked Floyd-Warshall -----------------------------------

def run_host(w, inf, device_bytes, ld=None):
    n = w.shape[0]
    ld = n if ld is None else ld
    dt = torch.int32 if w.dtype == np.int32 else torch.float32
    h = torch.empty((n, ld), dtype=dt, pin_memory=True)
    h.fill_(CANARY)
    h[:, :n] = torch.from_numpy(w[:, :n])
    blk = ga.fw_host(h, inf, device_bytes)
    out = h.numpy()
    assert (out[:, n:] == CANARY).all(), "wrote outside the n x n block"
    return out[:, :n].copy(), blk


def budget_for(n, S, sets=1, itemsize=4):
    """The device bytes the host-resident call needs at outer block S with
    one or two panel sets."""
    ldr = (n + 3) // 4 * 4
    return itemsize * (sets * (S * ldr + n * S) + 4 * S * S)


# (n, budget, the plan the library must pick: outer block, panel sets).
# Sets 0: the matrix fits and runs in-core; 1: one panel set reloaded every
# outer round; 2: the next round's panels computed in place.
HOST_CASES = [
    (1, budget_for(1, 128), 128, 0),
    (100, budget_for(100, 128), 128, 0),
    (300, budget_for(300, 128), 384, 0),
    (1000, budget_for(1000, 256), 256, 1),             # 4 rounds, ragged
    (2000, budget_for(2000, 256), 256, 1),             # 8 rounds, ragged
    (2000, budget_for(2000, 384, 2), 512, 1),          # 4 rounds, ragged
    (1000, budget_for(1000, 128, 2), 128, 2),          # 8 rounds, ragged
    (1031, budget_for(1031, 128, 2), 128, 2),          # 9 rounds, 7-wide tail
]


@pytest.mark.parametrize("n,budget,S,sets", HOST_CASES)
@pytest.mark.parametrize("policy", [ga.APSP_ARITH_AUTO, ga.APSP_ARITH_INT32,
                                    ga.APSP_ARITH_F32_WHEN_EXACT])
def test_host_int32_matches_oracle(dev, n, budget, S, sets, policy):
    print(f"case host i32 n={n} budget={budget} policy={policy}", flush=True)
    assert ga.apsp_fw_host_plan(n, 4, budget) == (ga.APSP_OK, S, sets)
    w = gg.erdos_renyi(n, 0.02 if n > 100 else 0.2, 1, 100, 100 + n)
    with ga.int32_arith(policy):
        got, blk = run_host(w, INF, budget)
    assert blk == S
    assert np.array_equal(got, oracle.fw_i32(w))


@pytest.mark.parametrize("sets", [1, 2])
def test_host_int32_large_weights_and_padding(dev, sets):
    # weights above 2^24: int32 arithmetic throughout; ld > n with a canary
    print(f"case host i32 large weights, ld > n, sets={sets}", flush=True)
    n = 900
    budget = budget_for(n, 256 if sets == 1 else 128, sets)
    S = ga.apsp_fw_host_plan(n, 4, budget)[1]
    assert ga.apsp_fw_host_plan(n, 4, budget) == (ga.APSP_OK, S, sets)
    w = gg.erdos_renyi(n, 0.01, 1, 50_000_000, 7)
    got, blk = run_host(w, INF, budget, ld=n + 13)
    assert blk == S and np.array_equal(got, oracle.fw_i32(w))


@pytest.fixture(scope="module")
def complete_20481():
    # n = 5 * 4096 + 1, a 1.6 GiB matrix (about 16 s to generate), with its
    # in-core distances from apsp_fw_i32 in HBM
    print("generating complete n=20481 and its in-core distances", flush=True)
    n = 20481
    w = gg.complete(n, 1, 10000, 5)
    t = torch.from_numpy(w).to("cuda:0")
    ga.fw(t, INF)
    d = t.cpu().numpy()
    del t
    return w, d


@pytest.mark.parametrize("policy", [ga.APSP_ARITH_AUTO, ga.APSP_ARITH_INT32])
def test_host_two_sets_at_scale_equals_in_core(dev, complete_20481, policy):
    # just over the budget: two panel sets at S = 4096, balanced to 6 rounds
    # of 3456 (the last 3201 wide); against the in-core result and the
    # oracle's single-source rows
    print(f"case host complete n=20481 two sets policy={policy}", flush=True)
    w, want = complete_20481
    n = w.shape[0]
    budget = budget_for(n, 4096, 2)
    assert ga.apsp_fw_host_plan(n, 4, budget) == (ga.APSP_OK, 3456, 2)
    with ga.int32_arith(policy):
        got, blk = run_host(w, INF, budget)
    assert blk == 3456
    assert np.array_equal(got, want)
    rows = np.array([0, 1, 3455, 3456, 17280, 20480])
    assert np.array_equal(got[rows], oracle.sssp_rows_i32(w, INF, rows))


@pytest.mark.parametrize("n,budget,S,sets", [
    (500, budget_for(500, 128), 128, 1),
    (1000, budget_for(1000, 256), 256, 1),
    (1000, budget_for(1000, 128, 2), 128, 2),
    (600, 4 * 600 * 600, 640, 0),
])
def test_host_float32_matches_oracle(dev, n, budget, S, sets):
    print(f"case host f32 n={n} S={S} sets={sets}", flush=True)
    assert ga.apsp_fw_host_plan(n, 4, budget) == (ga.APSP_OK, S, sets)
    w = gg.complete_f32(n, 40 + n)
    got, blk = run_host(w, float("inf"), budget)
    want = oracle.fw_f64(w.astype(np.float64))
    rel = np.abs(got.astype(np.float64) - want) / np.maximum(np.abs(want), 1e-30)
    assert blk == S and float(rel.max()) <= 1e-5


@pytest.mark.parametrize("sets", [1, 2])
@pytest.mark.parametrize("late", ["weight-above-2^24", "inf-with-heavy-weight"])
def test_host_binary32_speculation_falls_back_to_int32(dev, sets, late):
    # Round 0's panels (row and column block 0) are exact in binary32, the
    # rest of the matrix is not: the call starts round 0 in binary32 while it
    # scans the rest, then must start over in int32 with the host untouched.
    print(f"case host speculation fallback sets={sets} late={late}", flush=True)
    n = 1000
    budget = budget_for(n, 256) if sets == 1 else budget_for(n, 128, 2)
    S = ga.apsp_fw_host_plan(n, 4, budget)[1]
    assert ga.apsp_fw_host_plan(n, 4, budget) == (ga.APSP_OK, S, sets)
    w = gg.erdos_renyi(n, 1.0, 1, 100, 41)
    if late == "weight-above-2^24":
        w[900, 950] = 50_000_000
    else:
        w[850, 860] = INF            # an inf entry, and (n - 1) * 20000 > 2^24
        w[870, 880] = 20000
    assert (w[:S] < 100_000).all() and (w[:, :S] < 100_000).all()
    got, blk = run_host(w, INF, budget)
    assert blk == S and np.array_equal(got, oracle.fw_i32(w))


def test_host_budget_too_small_is_a_range_error(dev):
    print("case host budget too small", flush=True)
    w = gg.erdos_renyi(500, 0.05, 1, 10, 3)
    h = torch.from_numpy(w.copy())
    with pytest.raises(ga.APSPError) as e:
        ga.fw_host(h, INF, device_bytes=1000)
    assert e.value.status == ga.APSP_ERR_RANGE
    assert np.array_equal(h.numpy(), w)


def test_host_pageable_memory_works(dev):
    print("case host pageable", flush=True)
    n = 1000
    w = gg.erdos_renyi(n, 0.02, 1, 100, 9)
    h = torch.from_numpy(w.copy())           # not pinned
    assert ga.fw_host(h, INF, budget_for(n, 128, 2)) == 128
    assert np.array_equal(h.numpy(), oracle.fw_i32(w))
