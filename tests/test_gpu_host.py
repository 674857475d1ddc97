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


def budget_for(n, S, itemsize=4):
    ldr = (n + 3) // 4 * 4
    return itemsize * (S * ldr + n * S + 4 * S * S)


@pytest.mark.parametrize("n,S", [(1, 128), (100, 128), (300, 128), (1000, 256), (1000, 384),
                                 (1031, 512), (2000, 2048)])
@pytest.mark.parametrize("policy", [ga.APSP_ARITH_AUTO, ga.APSP_ARITH_INT32,
                                    ga.APSP_ARITH_F32_WHEN_EXACT])
def test_host_int32_matches_oracle(dev, n, S, policy):
    print(f"case host i32 n={n} S={S} policy={policy}", flush=True)
    w = gg.erdos_renyi(n, 0.02 if n > 100 else 0.2, 1, 100, 100 + n)
    with ga.int32_arith(policy):
        got, blk = run_host(w, INF, budget_for(n, S))
    assert blk == min(S, (n + 127) // 128 * 128)
    assert np.array_equal(got, oracle.fw_i32(w))


def test_host_int32_large_weights_and_padding(dev):
    # weights above 2^24: int32 arithmetic throughout; ld > n with a canary
    print("case host i32 large weights, ld > n", flush=True)
    n = 900
    w = gg.erdos_renyi(n, 0.01, 1, 50_000_000, 7)
    got, blk = run_host(w, INF, budget_for(n, 256), ld=n + 13)
    assert blk == 256 and np.array_equal(got, oracle.fw_i32(w))


def test_host_complete_graph_equals_in_core(dev):
    print("case host complete n=3000 against apsp_fw_i32", flush=True)
    n = 3000
    w = gg.complete(n, 1, 10000, 5)
    got, blk = run_host(w, INF, budget_for(n, 1024))
    assert blk == 1024
    t = torch.from_numpy(w).to(dev)
    ga.fw(t, INF)
    assert np.array_equal(got, t.cpu().numpy())
    rows = np.array([0, 1, 1499, 2999])
    assert np.array_equal(got[rows], oracle.sssp_rows_i32(w, INF, rows))


@pytest.mark.parametrize("n,S", [(257, 128), (1000, 256)])
def test_host_float32_matches_oracle(dev, n, S):
    print(f"case host f32 n={n} S={S}", flush=True)
    w = gg.complete_f32(n, 40 + n)
    got, blk = run_host(w, float("inf"), budget_for(n, S))
    want = oracle.fw_f64(w.astype(np.float64))
    rel = np.abs(got.astype(np.float64) - want) / np.maximum(np.abs(want), 1e-30)
    assert blk == S and float(rel.max()) <= 1e-5


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
    n = 600
    w = gg.erdos_renyi(n, 0.02, 1, 100, 9)
    h = torch.from_numpy(w.copy())           # not pinned
    ga.fw_host(h, INF, budget_for(n, 256))
    assert np.array_equal(h.numpy(), oracle.fw_i32(w))
