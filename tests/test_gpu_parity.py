"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

int32 results must be bit-exact; float32 results must be within 1e-5
relative of the oracle's binary64 distances (exact where the distance is 0
or unreachable) and bit-identical from run to run.
"""
import numpy as np
import torch  # noqa: F401  (imported at collection, before any test timer starts)
import pytest

import graph_all_pairs_amd as ga
import graphgen as gg
import oracle

pytestmark = pytest.mark.gpu

INF = gg.INF_I32
F32_RTOL = 1e-5


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def gpu_apsp(torch_dev, w, inf, ld=None, offset=0):
    """Copy w (n x ld_w) to the device, run the C-ABI entry point, return the
    full device buffer (n x ld) as numpy."""
    torch, dev = torch_dev
    n = w.shape[0]
    ld = w.shape[1] if ld is None else ld
    assert ld >= w.shape[1]
    host = np.zeros((n, ld + offset), dtype=w.dtype)
    canary = np.array(-7, dtype=w.dtype)
    host[:, :] = canary
    host[:, offset:offset + w.shape[1]] = w
    buf = torch.from_numpy(host.reshape(-1)).to(dev)
    ptr = buf.data_ptr() + offset * w.dtype.itemsize
    s = torch.cuda.current_stream().cuda_stream
    fn = ga.apsp_fw_i32 if w.dtype == np.int32 else ga.apsp_fw_f32
    st = fn(ptr, n, ld + offset if offset else ld, inf, s)
    assert st == ga.APSP_OK, ga.apsp_status_string(st)
    torch.cuda.synchronize()
    out = buf.cpu().numpy().reshape(n, ld + offset)
    return out[:, offset:] if offset else out


def assert_f32_close(got, want):
    got = got.astype(np.float64)
    assert np.array_equal(np.isinf(got), np.isinf(want))
    fin = np.isfinite(want)
    g, o = got[fin], want[fin]
    assert np.all((o == 0) == (g == 0))
    rel = np.abs(g - o) / np.maximum(np.abs(o), np.finfo(np.float64).tiny)
    assert float(rel.max(initial=0.0)) <= F32_RTOL, float(rel.max())


SIZES = [1, 2, 3, 5, 31, 63, 64, 65, 127, 128, 129, 255, 256, 257, 383, 997, 1000, 1024, 1031]


def family(name, n, seed):
    if name == "er":
        p = min(1.0, 4.0 / max(n, 1))      # sparse: some pairs stay unreachable
        return gg.erdos_renyi(n, p, 1, 100, seed)
    if name == "er_dense":
        return gg.erdos_renyi(n, 0.3, 1, 1000, seed)
    if name == "complete":
        return gg.complete(n, 1, 10000, seed)
    if name == "ring":
        return gg.ring(n, 3)
    if name == "two_rings":
        return gg.two_rings(n // 2, n - n // 2, 2)
    raise KeyError(name)


ARITH = {"auto": ga.APSP_ARITH_AUTO, "f32": ga.APSP_ARITH_F32_WHEN_EXACT,
         "i32": ga.APSP_ARITH_INT32}


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("fam", ["er", "complete", "ring", "two_rings"])
@pytest.mark.parametrize("arith", ["auto", "f32"])
def test_int32_sweep(torch_dev, n, fam, arith):
    print(f"case int32 {fam} n={n} arith={arith}", flush=True)
    w = family(fam, n, 100 + n)
    with ga.int32_arith(ARITH[arith]):
        got = gpu_apsp(torch_dev, w, INF)
    assert np.array_equal(got, oracle.fw_i32(w))


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("fam", ["er_dense", "complete_f32", "ring_half"])
def test_float32_sweep(torch_dev, n, fam):
    print(f"case float32 {fam} n={n}", flush=True)
    if fam == "complete_f32":
        w = gg.complete_f32(n, 200 + n)
    elif fam == "ring_half":
        w = gg.ring(n, 0.5, dtype=np.float32, inf=np.inf)
    else:
        wi = gg.erdos_renyi(n, min(1.0, 6.0 / max(n, 1)), 1, 1000, 300 + n)
        w = np.where(wi == INF, np.inf, wi.astype(np.float64) * 0.013).astype(np.float32)
    got = gpu_apsp(torch_dev, w, np.inf)
    want = oracle.fw_f64(w.astype(np.float64))
    assert_f32_close(got, want)
    if fam == "ring_half":   # exact in binary32: whole multiples of 0.5
        assert np.array_equal(got.astype(np.float64), want)


def test_hand_example(torch_dev):
    from _helpers import read_golden
    g = read_golden("hand4_fw.txt", INF)
    got = gpu_apsp(torch_dev, g["input"].astype(np.int32), INF)
    assert np.array_equal(got, g["final"])


@pytest.mark.parametrize("n,ld", [(45, 64), (300, 313), (257, 260), (1000, 1024), (129, 131)])
def test_leading_dimension_and_canary(torch_dev, n, ld):
    print(f"case ld n={n} ld={ld}", flush=True)
    w = gg.erdos_renyi(n, 0.05, 1, 50, n, ld=ld, canary=-7)
    got = gpu_apsp(torch_dev, w, INF)
    assert np.all(got[:, n:] == -7), "padding columns were written"
    assert np.array_equal(got[:, :n], oracle.fw_i32(w)[:, :n])


@pytest.mark.parametrize("n", [130, 300])
def test_unaligned_pointer_uses_scalar_path(torch_dev, n):
    # pointer 4 bytes past a 16-byte boundary, ld not a multiple of 4
    w = gg.erdos_renyi(n, 0.05, 1, 50, 7 + n)
    got = gpu_apsp(torch_dev, w, INF, offset=1)
    assert np.array_equal(got[:, :n], oracle.fw_i32(w))


def test_inf_preserved_between_components(torch_dev):
    w = gg.two_rings(200, 171, 5)
    got = gpu_apsp(torch_dev, w, INF)
    assert np.all(got[:200, 200:] == INF) and np.all(got[200:, :200] == INF)
    wf = gg.two_rings(200, 171, 0.25, dtype=np.float32, inf=np.inf)
    gotf = gpu_apsp(torch_dev, wf, np.inf)
    assert np.all(np.isinf(gotf[:200, 200:]))
    # a finite float sentinel behaves the same way
    wf2 = np.where(np.isinf(wf), np.float32(1e30), wf)
    gotf2 = gpu_apsp(torch_dev, wf2, 1e30)
    assert np.all(gotf2[:200, 200:] == np.float32(1e30))


def test_rounds_resume_matches_partial_oracle(torch_dev):
    torch, dev = torch_dev
    n = 300
    B = ga.apsp_pivot_block(n)
    w = gg.erdos_renyi(n, 0.02, 1, 100, 17)
    t = torch.from_numpy(w).to(dev)
    rounds = (n + B - 1) // B
    for r in range(rounds):
        ga.fw_rounds(t, r, r + 1, INF)
        torch.cuda.synchronize()
        want = oracle.fw_i32(w, k_end=min((r + 1) * B, n))
        assert np.array_equal(t.cpu().numpy(), want), f"after round {r}"


def test_repeat_runs_bit_identical_float(torch_dev):
    w = gg.complete_f32(1031, 99)
    a = gpu_apsp(torch_dev, w, np.inf)
    b = gpu_apsp(torch_dev, w, np.inf)
    assert np.array_equal(a.view(np.int32), b.view(np.int32))


def test_two_streams_two_matrices(torch_dev):
    torch, dev = torch_dev
    w1 = gg.erdos_renyi(700, 0.01, 1, 100, 1)
    w2 = gg.complete(650, 1, 100, 2)
    t1 = torch.from_numpy(w1).to(dev)
    t2 = torch.from_numpy(w2).to(dev)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        ga.fw(t1, INF)
    with torch.cuda.stream(s2):
        ga.fw(t2, INF)
    torch.cuda.synchronize()
    assert np.array_equal(t1.cpu().numpy(), oracle.fw_i32(w1))
    assert np.array_equal(t2.cpu().numpy(), oracle.fw_i32(w2))


def test_timed_variant_counts_launches(torch_dev):
    torch, dev = torch_dev
    n = 1000
    w = gg.erdos_renyi(n, 0.01, 1, 100, 5)
    t = torch.from_numpy(w).to(dev)
    nb = (n + 127) // 128
    with ga.int32_arith(ga.APSP_ARITH_F32_WHEN_EXACT):
        ms, cnt, arith = ga.fw_timed(t, INF)
    # later Phase 1s run inside Phase-3 launches; kind 3 is the scan before the
    # rounds and the last pivot row and column's conversion after them
    assert cnt == [1, nb, nb, 2]
    assert all(x > 0 for x in ms)
    assert arith == 1            # 999 * 100 <= 2^24: binary32 arithmetic
    assert np.array_equal(t.cpu().numpy(), oracle.fw_i32(w))
    t = torch.from_numpy(w).to(dev)
    ms, cnt, arith = ga.fw_timed(t, INF)   # auto: 49 tiles, binary32 when exact
    assert cnt == [1, nb, nb, 2] and arith == 1
    assert np.array_equal(t.cpu().numpy(), oracle.fw_i32(w))
    ws = gg.erdos_renyi(300, 0.05, 1, 100, 5)
    t = torch.from_numpy(ws).to(dev)
    ms, cnt, arith = ga.fw_timed(t, INF)   # auto: 4 tiles, too few for the scan to pay
    assert cnt == [1, 3, 3, 0] and arith == 0
    assert np.array_equal(t.cpu().numpy(), oracle.fw_i32(ws))
    wf = gg.complete_f32(300, 3)
    tf = torch.from_numpy(wf).to(dev)
    ms, cnt, arith = ga.fw_timed(tf)
    assert cnt == [1, 3, 3, 0] and arith == 1


def test_release_events_then_measure_again(torch_dev):
    """The pooled timing events (timed calls and the launch trace) can be
    released and are created again by the next measurement call."""
    torch, dev = torch_dev
    w = gg.erdos_renyi(300, 0.05, 1, 100, 6)
    want = oracle.fw_i32(w)
    for _ in range(2):
        t = torch.from_numpy(w).to(dev)
        ms, cnt, arith = ga.fw_timed(t, INF)
        assert cnt[2] == 3 and np.array_equal(t.cpu().numpy(), want)
        assert ga.apsp_trace_begin(64) == ga.APSP_OK
        assert ga.apsp_release_events() == ga.APSP_ERR_INVALID_VALUE   # a trace is open
        t = torch.from_numpy(w).to(dev)
        ga.fw(t, INF)
        st, phase_ms, launches, dropped = ga.apsp_trace_end()
        assert st == ga.APSP_OK and launches[2] == 3 and dropped == 0
        assert np.array_equal(t.cpu().numpy(), want)
        assert ga.apsp_release_events() == ga.APSP_OK


# ---- int32 matrices: binary32 vs int32 arithmetic --------------------------

LIM = 1 << 24


def _arith_of(torch_dev, w, inf, mode=ga.APSP_ARITH_F32_WHEN_EXACT):
    torch, dev = torch_dev
    t = torch.from_numpy(w).to(dev)
    with ga.int32_arith(mode):
        _, _, arith = ga.fw_timed(t, inf)
    return arith, t.cpu().numpy()


def test_int32_policy_forces_int_arithmetic(torch_dev):
    w = gg.complete(300, 1, 1000, 12)
    arith, got = _arith_of(torch_dev, w, INF, ga.APSP_ARITH_INT32)
    assert arith == 0 and np.array_equal(got, oracle.fw_i32(w))
    arith, got = _arith_of(torch_dev, w, INF, ga.APSP_ARITH_F32_WHEN_EXACT)
    assert arith == 1 and np.array_equal(got, oracle.fw_i32(w))


@pytest.mark.parametrize("n,want", [(384, 0), (385, 1), (513, 1)])
def test_auto_policy_boundary(torch_dev, n, want):
    """Under the default policy an exact int32 matrix computes in binary32
    from nine Phase-3 tiles (n > 384) on, and in int32 without the scan
    below; the result is the oracle's either way."""
    print(f"case auto policy n={n}", flush=True)
    torch, dev = torch_dev
    w = gg.erdos_renyi(n, 0.05, 1, 1000, 70 + n)
    t = torch.from_numpy(w).to(dev)
    ms, cnt, arith = ga.fw_timed(t, INF)
    nb = (n + 127) // 128
    assert arith == want
    assert cnt == [1, nb, nb, 2 if want else 0]
    assert np.array_equal(t.cpu().numpy(), oracle.fw_i32(w))


def test_rounds_resume_in_binary32(torch_dev):
    torch, dev = torch_dev
    n = 300
    w = gg.erdos_renyi(n, 0.02, 1, 100, 18)
    t = torch.from_numpy(w).to(dev)
    with ga.int32_arith(ga.APSP_ARITH_F32_WHEN_EXACT):
        ga.fw_rounds(t, 0, 1, INF)
        torch.cuda.synchronize()
        assert np.array_equal(t.cpu().numpy(), oracle.fw_i32(w, k_end=128))
        ga.fw_rounds(t, 1, 3, INF)
        torch.cuda.synchronize()
    assert np.array_equal(t.cpu().numpy(), oracle.fw_i32(w))


@pytest.mark.parametrize("case", ["complete_at_limit", "ring_at_bound", "big_weights",
                                  "ring_over_bound", "negative_free_small_inf",
                                  "complete_over_limit"])
def test_int32_arithmetic_choice_and_exactness(torch_dev, case):
    print(f"case arith {case}", flush=True)
    rng = np.random.default_rng(7)
    if case == "complete_at_limit":          # weights up to 2^24, no inf: binary32
        n = 300
        w = rng.integers(LIM - 5000, LIM + 1, size=(n, n)).astype(np.int32)
        np.fill_diagonal(w, 0)
        want_arith = 1
        inf = INF
    elif case == "ring_at_bound":            # (n-1) * w == 2^24 exactly: binary32
        n = 257
        w = gg.ring(n, LIM // 256)
        want_arith, inf = 1, INF
    elif case == "ring_over_bound":          # (n-1) * w > 2^24 with inf: int32
        n = 258
        w = gg.ring(n, LIM // 256)
        want_arith, inf = 0, INF
    elif case == "big_weights":              # a weight above 2^24: int32
        n = 200
        w = gg.erdos_renyi(n, 0.05, 1, 100, 3)
        w[3, 7] = (1 << 28) + 1
        want_arith, inf = 0, INF
    elif case == "negative_free_small_inf":  # small sentinel; sums may exceed it
        n = 150
        w = gg.erdos_renyi(n, 0.03, 1, 60, 9, inf=100)
        want_arith, inf = 1, 100
    else:                                    # complete, one weight 2^24 + 1: int32
        n = 130
        w = gg.complete(n, 1, 1000, 4)
        w[5, 9] = LIM + 1
        want_arith, inf = 0, INF
    arith, got = _arith_of(torch_dev, w, inf)
    assert arith == want_arith
    assert np.array_equal(got, oracle.fw_i32(w)), case


def test_tensor_wrapper_errors(torch_dev):
    torch, dev = torch_dev
    with pytest.raises(ValueError):
        ga.fw(torch.zeros((4, 4), dtype=torch.float64, device=dev))
    with pytest.raises(ValueError):
        ga.fw(torch.zeros((4, 3), dtype=torch.int32, device=dev))
    with pytest.raises(ga.APSPError):
        ga.fw(torch.zeros((4, 4), dtype=torch.int32, device=dev), inf=0)


def test_minplus_ceiling_diagnostic(torch_dev):
    # the register-only core runs between half and twice the spec peaks
    st, r32 = ga.apsp_minplus_ceiling(0)
    assert st == ga.APSP_OK and 0.5 * 2.62e13 < r32 < 2.0 * 2.62e13
    st, rf = ga.apsp_minplus_ceiling(1)
    assert st == ga.APSP_OK and 0.5 * 5.24e13 < rf < 2.0 * 5.24e13
    assert ga.apsp_minplus_ceiling(5)[0] == ga.APSP_ERR_INVALID_VALUE
    # at a given wave count: every count runs, and no count beats twice the
    # best of the even ones
    for arith, best in ((0, r32), (1, rf)):
        for w in (1, 2, 3, 4):
            st, r = ga.apsp_minplus_ceiling_waves(arith, w)
            assert st == ga.APSP_OK and 0 < r < 2.0 * best, (arith, w, r)
    for bad in ((0, 0), (0, 5), (3, 2)):
        assert ga.apsp_minplus_ceiling_waves(*bad)[0] == ga.APSP_ERR_INVALID_VALUE


def test_trace_across_calls_counts_every_launch(torch_dev):
    # three asynchronous calls under one trace record exactly three times the
    # launches (and launch groups) of one synchronised timed call, and the
    # results are unchanged
    print("case trace across calls", flush=True)
    torch, dev = torch_dev
    n = 1000
    w = gg.erdos_renyi(n, 0.01, 1, 100, 41)
    want = oracle.fw_i32(w)
    s = torch.cuda.current_stream().cuda_stream
    per_call = {}
    for mode in (ga.APSP_ARITH_AUTO, ga.APSP_ARITH_F32_WHEN_EXACT):
        with ga.int32_arith(mode):
            one = torch.from_numpy(w).to(dev)
            st, _, cnt1, _ = ga.apsp_fw_timed_i32(one.data_ptr(), n, n, INF, s)
            assert st == ga.APSP_OK
            per_call[mode] = sum(cnt1)
            ts = [torch.from_numpy(w).to(dev) for _ in range(3)]
            torch.cuda.synchronize()
            assert ga.apsp_trace_begin(1000) == ga.APSP_OK
            assert ga.apsp_trace_begin(10) == ga.APSP_ERR_INVALID_VALUE  # already on
            for t in ts:
                assert ga.apsp_fw_i32(t.data_ptr(), n, n, INF, s) == ga.APSP_OK
            st, ms, cnt, dropped = ga.apsp_trace_end()
            assert st == ga.APSP_OK and dropped == 0
            assert cnt == [3 * c for c in cnt1] and all(x >= 0 for x in ms) and ms[2] > 0
            for t in ts:
                assert np.array_equal(t.cpu().numpy(), want)
    # a trace smaller than the launches keeps the first ones and counts the rest
    t = torch.from_numpy(w).to(dev)
    assert ga.apsp_trace_begin(5) == ga.APSP_OK
    assert ga.apsp_fw_i32(t.data_ptr(), n, n, INF, s) == ga.APSP_OK
    st, ms, cnt, dropped = ga.apsp_trace_end()
    assert st == ga.APSP_OK and sum(cnt) == 5 and dropped == per_call[ga.APSP_ARITH_AUTO] - 5
    assert np.array_equal(t.cpu().numpy(), want)
