"""int32 matrices computed in binary32: the result at the top of the exact
range.  A distance of exactly 2^24 must come back as 2^24 even when the
sentinel is 2^24 + 1, which rounds to 2^24 in binary32 (so the way back
compares with the sentinel as an integer).  Expected values are closed
forms, so no oracle run is needed:
  * complete graphs with every weight in [2^24 - 1000, 2^24]: every
    two-edge path is longer than any edge, so the distances are the
    weights themselves;
  * a directed chain of 256 edges of weight 2^16 (n = 257): d(i, j) =
    (j - i) 2^16 for i <= j, at most 2^24 = (n - 1) times the largest
    weight, the edge of the exactness condition when inf entries exist.
Every entry point that takes the binary32 path for int32 matrices is run:
apsp_fw_i32 (forced and automatic), the host-resident call and the signed
call; the batched call (int32 arithmetic) on the same inputs as a check of
the top of the range.
"""
import numpy as np
import torch
import pytest

import graph_all_pairs_amd as ga
import graphgen as gg

pytestmark = pytest.mark.gpu

TOP = 1 << 24
INF = TOP + 1


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def near_top_complete(n, seed):
    w = gg.erdos_renyi(n, 1.0, TOP - 1000, TOP, seed, inf=INF)
    assert (w == TOP).sum() > 0
    return w


def chain(n, step):
    w = np.full((n, n), INF, dtype=np.int32)
    np.fill_diagonal(w, 0)
    i = np.arange(n - 1)
    w[i, i + 1] = step
    return w


def chain_distances(n, step):
    i = np.arange(n)
    d = (i[None, :] - i[:, None]).astype(np.int64) * step
    return np.where(d >= 0, d, INF).astype(np.int32)


@pytest.mark.parametrize("n,policy", [(1000, ga.APSP_ARITH_F32_WHEN_EXACT),
                                      (1000, ga.APSP_ARITH_INT32),
                                      (3200, ga.APSP_ARITH_AUTO)])
def test_fw_complete_near_top(dev, n, policy):
    print(f"boundary fw complete n={n} policy={policy}", flush=True)
    w = near_top_complete(n, 31 + n)
    t = torch.from_numpy(w).to(dev)
    with ga.int32_arith(policy):
        ga.fw(t, INF)
    assert np.array_equal(t.cpu().numpy(), w)


def test_fw_chain_to_the_top(dev):
    print("boundary fw chain n=257", flush=True)
    n = 257
    t = torch.from_numpy(chain(n, 1 << 16)).to(dev)
    with ga.int32_arith(ga.APSP_ARITH_F32_WHEN_EXACT):
        ga.fw(t, INF)
    got = t.cpu().numpy()
    assert got[0, n - 1] == TOP
    assert np.array_equal(got, chain_distances(n, 1 << 16))


def test_fw_host_complete_near_top(dev):
    print("boundary fw_host complete n=1000", flush=True)
    n = 1000
    w = near_top_complete(n, 77)
    budget = 4 * (2 * 256 * n + 4 * 256 * 256)
    assert ga.apsp_fw_host_plan(n, 4, budget)[2] == 1
    h = torch.from_numpy(w.copy())
    ga.fw_host(h, INF, budget)
    assert np.array_equal(h.numpy(), w)


def test_fw_signed_chain_to_the_top(dev):
    print("boundary fw_signed chain n=257", flush=True)
    n = 257
    t = torch.from_numpy(chain(n, 1 << 16)).to(dev)
    with ga.int32_arith(ga.APSP_ARITH_F32_WHEN_EXACT):
        ga.fw_signed(t, INF)
    assert np.array_equal(t.cpu().numpy(), chain_distances(n, 1 << 16))


def test_batched_near_top(dev):
    print("boundary batched", flush=True)
    w = np.stack([near_top_complete(128, 90 + g) for g in range(6)])
    t = torch.from_numpy(w.copy()).to(dev)
    ga.fw_batched(t, INF)
    assert np.array_equal(t.cpu().numpy(), w)
    # n = 65: 64 edges of 2^18 reach 2^24 with inf entries present
    c = np.stack([chain(65, 1 << 18)] * 5)
    t = torch.from_numpy(c).to(dev)
    ga.fw_batched(t, INF)
    got = t.cpu().numpy()
    assert all(np.array_equal(got[g], chain_distances(65, 1 << 18)) for g in range(5))
