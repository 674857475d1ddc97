"""The no-allocation int32 entry point, apsp_fw_i32_noalloc, through the C
ABI: its output must equal apsp_fw_i32's (and the oracle's) bit for bit, on
two calls in a row, the second with a smaller matrix, so that the shared
static scratch is shown to start each call afresh."""
import numpy as np
import pytest
import torch

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


def call(fn, w, dev, stream=None):
    """One call of `fn` (a raw entry point) on a device copy of w (n x ld)."""
    n = w.shape[0]
    t = torch.from_numpy(w).to(dev)
    s = stream if stream is not None else torch.cuda.current_stream()
    with torch.cuda.stream(s):
        st = fn(t.data_ptr(), n, t.stride(0), INF, s.cuda_stream)
    assert st == ga.APSP_OK, ga.apsp_status_string(st)
    s.synchronize()
    return t.cpu().numpy()


def big_weight(w, seed):
    """A copy of w with one finite off-diagonal weight above 2^24, which
    rules binary32 out for the whole matrix (the call computes in int32)."""
    out = w.copy()
    rng = np.random.default_rng(seed)
    n = w.shape[0]
    while True:
        i, j = (int(x) for x in rng.integers(0, n, size=2))
        if i != j and out[i, j] != INF:
            out[i, j] = (1 << 24) + 1000
            return out


@pytest.mark.parametrize("policy", [ga.APSP_ARITH_AUTO, ga.APSP_ARITH_F32_WHEN_EXACT])
def test_two_calls_second_smaller_binary32_then_int32(dev, policy):
    print(f"case noalloc: policy {policy}, n 3000 (exact) then n 1031 (weight > 2^24)",
          flush=True)
    first = gg.complete(3000, 1, 10000, 41)       # exact in binary32; 529 Phase-3 tiles
    second = big_weight(gg.erdos_renyi(1031, 0.05, 1, 1000, 42), 43)
    with ga.int32_arith(policy):
        got1 = call(ga.apsp_fw_i32_noalloc, first, dev)
        got2 = call(ga.apsp_fw_i32_noalloc, second, dev)
        ref1 = call(ga.apsp_fw_i32, first, dev)
        ref2 = call(ga.apsp_fw_i32, second, dev)
    assert np.array_equal(got1, ref1)
    assert np.array_equal(got2, ref2)
    assert np.array_equal(got2, oracle.fw_i32(second))
    assert np.array_equal(got1[:400], oracle.sssp_rows_i32(first, INF, range(400)))


def test_two_calls_second_smaller_int32_then_binary32(dev):
    print("case noalloc: binary32 forced, n 1000 (weight > 2^24) then n 300 (exact, ld > n)",
          flush=True)
    first = big_weight(gg.erdos_renyi(1000, 0.05, 1, 1000, 44), 45)
    second = gg.erdos_renyi(300, 0.05, 1, 100, 46, ld=308)   # padding carries a canary
    with ga.int32_arith(ga.APSP_ARITH_F32_WHEN_EXACT):
        got1 = call(ga.apsp_fw_i32_noalloc, first, dev)
        got2 = call(ga.apsp_fw_i32_noalloc, second, dev)
        ref1 = call(ga.apsp_fw_i32, first, dev)
        ref2 = call(ga.apsp_fw_i32, second, dev)
    assert np.array_equal(got1, ref1)
    assert np.array_equal(got2, ref2)
    assert np.array_equal(got1, oracle.fw_i32(first))
    assert np.array_equal(got2[:, :300], oracle.fw_i32(second[:, :300]))
    assert np.array_equal(got2[:, 300:], second[:, 300:])      # padding untouched


def test_calls_on_a_side_stream_and_argument_errors(dev):
    print("case noalloc: side stream, repeated calls, argument errors", flush=True)
    side = torch.cuda.Stream()
    w = gg.ring(777, 3)
    i, j = np.meshgrid(np.arange(777), np.arange(777), indexing="ij")
    with ga.int32_arith(ga.APSP_ARITH_F32_WHEN_EXACT):
        for _ in range(3):
            assert np.array_equal(call(ga.apsp_fw_i32_noalloc, w, dev, side), 3 * ((j - i) % 777))
    assert ga.apsp_fw_i32_noalloc(0, 4, 4, 100, 0) == ga.APSP_ERR_INVALID_VALUE
    assert ga.apsp_fw_i32_noalloc(0, 0, 1, 100, 0) == ga.APSP_OK
