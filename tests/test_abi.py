"""C-ABI library checks that need no GPU: it loads, exports every symbol the
header declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import graph_all_pairs_amd as ga
from graph_all_pairs_amd import _build

HEADER = os.path.join(_build.ROOT, "include", "apsp.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_build.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return ga.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(apsp_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(ga.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(_build.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_library_is_built_for_gfx950_only():
    # the offload bundle carries a gfx950 code object and no other target
    data = open(_build.LIB_PATH, "rb").read()
    assert b"gfx950" in data
    for other in (b"gfx942", b"gfx90a", b"gfx1100", b"sm_"):
        assert other + b"\x00" not in data and b"amdgcn-amd-amdhsa--" + other not in data


def test_status_strings_and_version(lib):
    assert ga.apsp_status_string(0) == "APSP_OK"
    for s in (1, 2, 3):
        assert ga.apsp_status_string(s).startswith("APSP_ERR")
    assert "unknown" in ga.apsp_status_string(99)
    assert ga.apsp_version() >= 100
    assert ga.apsp_pivot_block(1000) == 128


FAKE = 0x10000  # never dereferenced: every case below is rejected first


@pytest.mark.parametrize("args", [
    (FAKE, -1, 4, 100),            # n < 0
    (0, 4, 4, 100),                # null pointer with n > 0
    (FAKE, 8, 7, 100),             # ld < n
    (FAKE + 2, 4, 4, 100),         # not 4-byte aligned
    (FAKE, 4, 4, 0),               # inf < 1
    (FAKE, 4, 4, 0x40000000),      # inf + inf would overflow int32
    (FAKE, 4, 4, -5),
    (FAKE, (1 << 31) + 1, (1 << 31) + 1, 100),  # too large
])
def test_i32_argument_errors(lib, args):
    assert ga.apsp_fw_i32(*args, 0) == ga.APSP_ERR_INVALID_VALUE
    assert ga.apsp_fw_i32_noalloc(*args, 0) == ga.APSP_ERR_INVALID_VALUE


@pytest.mark.parametrize("inf", [0.0, -1.0, float("nan"), -float("inf")])
def test_f32_bad_inf(lib, inf):
    assert ga.apsp_fw_f32(FAKE, 4, 4, inf, 0) == ga.APSP_ERR_INVALID_VALUE


def test_round_range_errors(lib):
    # 300 vertices -> 3 rounds of 128
    assert ga.apsp_fw_rounds_i32(FAKE, 300, 300, 100, -1, 1) == ga.APSP_ERR_INVALID_VALUE
    assert ga.apsp_fw_rounds_i32(FAKE, 300, 300, 100, 2, 1) == ga.APSP_ERR_INVALID_VALUE
    assert ga.apsp_fw_rounds_i32(FAKE, 300, 300, 100, 0, 4) == ga.APSP_ERR_INVALID_VALUE
    assert ga.apsp_fw_rounds_f32(FAKE, 300, 300, 1.0, 0, 4) == ga.APSP_ERR_INVALID_VALUE


@pytest.mark.parametrize("args", [
    (FAKE, -1, 4, 4, 16, 100),         # batch < 0
    (FAKE, 3, -1, 4, 16, 100),         # n < 0
    (FAKE, 3, 129, 129, 129 * 129, 100),  # n > 128
    (0, 3, 4, 4, 16, 100),             # null pointer
    (FAKE, 3, 8, 7, 64, 100),          # ld < n
    (FAKE, 3, 4, 4, 15, 100),          # stride < (n-1)*ld + n: graphs overlap
    (FAKE, 3, 4, 8, 27, 100),          # same with padded rows
    (FAKE + 2, 3, 4, 4, 16, 100),      # not 4-byte aligned
    (FAKE, 3, 4, 4, 16, 0),            # bad inf
    (FAKE, 3, 4, 4, 16, 0x40000000),
    (FAKE, 1 << 40, 4, 4, 1 << 40, 100),  # last graph not addressable
])
def test_batched_argument_errors(lib, args):
    assert ga.apsp_fw_batched_i32(*args, 0) == ga.APSP_ERR_INVALID_VALUE


def test_batched_f32_bad_inf_and_no_ops(lib):
    for inf in (0.0, -1.0, float("nan")):
        assert ga.apsp_fw_batched_f32(FAKE, 3, 4, 4, 16, inf, 0) == ga.APSP_ERR_INVALID_VALUE
    # empty batches and empty graphs touch nothing, whatever the pointer
    assert ga.apsp_fw_batched_i32(0, 0, 4, 4, 16, 100, 0) == ga.APSP_OK
    assert ga.apsp_fw_batched_i32(0, 5, 0, 1, 1, 100, 0) == ga.APSP_OK
    assert ga.apsp_fw_batched_f32(0, 0, 128, 128, 128 * 128, 1.0, 0) == ga.APSP_OK
    # the smallest legal stride: (n-1)*ld + n
    assert ga.apsp_fw_batched_i32(0, 3, 4, 8, 28, 100, 0) == ga.APSP_ERR_INVALID_VALUE  # null


def test_arith_policy_setter(lib):
    assert ga.apsp_get_int32_arith() == ga.APSP_ARITH_AUTO
    assert ga.apsp_set_int32_arith(7) == ga.APSP_ERR_INVALID_VALUE
    with ga.int32_arith(ga.APSP_ARITH_INT32):
        assert ga.apsp_get_int32_arith() == ga.APSP_ARITH_INT32
    assert ga.apsp_get_int32_arith() == ga.APSP_ARITH_AUTO


def test_release_events_without_pooled_events_is_a_no_op(lib):
    # nothing is pooled in a process that made no measurement call, so the
    # call returns at once (no HIP call, works without a GPU)
    assert ga.apsp_release_events() == ga.APSP_OK
    assert ga.apsp_release_events() == ga.APSP_OK


def test_empty_is_a_no_op(lib):
    assert ga.apsp_fw_i32(0, 0, 1, 100, 0) == ga.APSP_OK
    assert ga.apsp_fw_i32_noalloc(0, 0, 1, 100, 0) == ga.APSP_OK
    assert ga.apsp_fw_f32(0, 0, 1, 1.0, 0) == ga.APSP_OK
    assert ga.apsp_fw_rounds_i32(FAKE, 300, 300, 100, 1, 1) == ga.APSP_OK


def test_timed_variant_validates_too(lib):
    st, ms, cnt, arith = ga.apsp_fw_timed_i32(0, 4, 4, 100)
    assert st == ga.APSP_ERR_INVALID_VALUE
    st, ms, cnt, arith = ga.apsp_fw_timed_f32(FAKE, 4, 3, 1.0)
    assert st == ga.APSP_ERR_INVALID_VALUE


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        ga.load(str(tmp_path / "nope.so"))


def test_single_hip_runtime_in_process(lib):
    # torch and libapsp.so must share one libamdhip64 (see graph_all_pairs_amd.load)
    maps = open("/proc/self/maps").read().splitlines()
    paths = {ln.split()[-1] for ln in maps if "libamdhip64" in ln}
    assert len(paths) == 1, paths


@pytest.mark.parametrize("args", [
    # row_ptr, col, w, n, nnz, d, ld, inf
    (FAKE, FAKE, FAKE, -1, 4, FAKE, 4, 100),          # n < 0
    (FAKE, FAKE, FAKE, 4, -1, FAKE, 4, 100),          # nnz < 0
    (0, FAKE, FAKE, 4, 4, FAKE, 4, 100),              # null row_ptr
    (FAKE, 0, FAKE, 4, 4, FAKE, 4, 100),              # null col with edges
    (FAKE, FAKE, 0, 4, 4, FAKE, 4, 100),              # null weights with edges
    (FAKE, FAKE, FAKE, 4, 4, 0, 4, 100),              # null output
    (FAKE, FAKE, FAKE, 8, 4, FAKE, 7, 100),           # ld < n
    (FAKE + 4, FAKE, FAKE, 4, 4, FAKE, 4, 100),       # row_ptr not 8-byte aligned
    (FAKE, FAKE + 2, FAKE, 4, 4, FAKE, 4, 100),       # col not 4-byte aligned
    (FAKE, FAKE, FAKE, 4, 4, FAKE + 1, 4, 100),       # d not 4-byte aligned
    (FAKE, FAKE, FAKE, 4, 4, FAKE, 4, 0),             # inf < 1
    (FAKE, FAKE, FAKE, 4, 4, FAKE, 4, 0x40000000),    # inf too large
    (FAKE, FAKE, FAKE, 1 << 31, 4, FAKE, 1 << 31, 100),  # n too large
    (FAKE, FAKE, FAKE, 4, 1 << 31, FAKE, 4, 100),     # nnz too large
])
def test_johnson_argument_errors(lib, args):
    assert ga.apsp_johnson_i32(*args, 0, -1, 0) == ga.APSP_ERR_INVALID_VALUE
    st, ms, counts = ga.apsp_johnson_timed_i32(*args, 0, -1, 0)
    assert st == ga.APSP_ERR_INVALID_VALUE and counts == [0, 0, 0, 0]


def test_johnson_empty_graph_is_a_no_op(lib):
    assert ga.apsp_johnson_i32(0, 0, 0, 0, 0, 0, 1, 100, 0, -1, 0) == ga.APSP_OK


def test_status_strings_for_negative_weights(lib):
    assert "NEGATIVE_CYCLE" in ga.apsp_status_string(ga.APSP_ERR_NEGATIVE_CYCLE)
    assert "RANGE" in ga.apsp_status_string(ga.APSP_ERR_RANGE)


@pytest.mark.parametrize("args", [
    (FAKE, -1, 4, 100), (0, 4, 4, 100), (FAKE, 8, 7, 100), (FAKE + 2, 4, 4, 100),
    (FAKE, 4, 4, 0), (FAKE, 4, 4, 0x40000000),
])
def test_signed_argument_errors(lib, args):
    assert ga.apsp_fw_signed_i32(*args, 0) == ga.APSP_ERR_INVALID_VALUE


def test_signed_f32_bad_inf_and_empty(lib):
    for inf in (0.0, -1.0, float("nan")):
        assert ga.apsp_fw_signed_f32(FAKE, 4, 4, inf, 0) == ga.APSP_ERR_INVALID_VALUE
    assert ga.apsp_fw_signed_i32(0, 0, 1, 100, 0) == ga.APSP_OK
    assert ga.apsp_fw_signed_f32(0, 0, 1, 1.0, 0) == ga.APSP_OK


def test_trace_argument_errors(lib):
    assert ga.apsp_trace_begin(0) == ga.APSP_ERR_INVALID_VALUE
    assert ga.apsp_trace_begin(-5) == ga.APSP_ERR_INVALID_VALUE
    assert ga.apsp_trace_begin((1 << 24) + 1) == ga.APSP_ERR_INVALID_VALUE
    st, ms, cnt, dropped = ga.apsp_trace_end()        # none is on
    assert st == ga.APSP_ERR_INVALID_VALUE and cnt == [0, 0, 0, 0] and dropped == 0


@pytest.mark.parametrize("args", [
    # C, ldc, A, lda, B, ldb, m, n, k, inf
    (FAKE, 8, FAKE, 8, FAKE, 8, -1, 8, 8, 100),       # m < 0
    (FAKE, 8, FAKE, 8, FAKE, 8, 8, 8, -1, 100),       # k < 0
    (0, 8, FAKE, 8, FAKE, 8, 8, 8, 8, 100),           # null C
    (FAKE, 8, 0, 8, FAKE, 8, 8, 8, 8, 100),           # null A
    (FAKE, 8, FAKE, 8, 0, 8, 8, 8, 8, 100),           # null B
    (FAKE, 7, FAKE, 8, FAKE, 8, 8, 8, 8, 100),        # ldc < n
    (FAKE, 8, FAKE, 7, FAKE, 8, 8, 8, 8, 100),        # lda < k
    (FAKE, 8, FAKE, 8, FAKE, 7, 8, 8, 8, 100),        # ldb < n
    (FAKE + 2, 8, FAKE, 8, FAKE, 8, 8, 8, 8, 100),    # misaligned
    (FAKE, 8, FAKE, 8, FAKE, 8, 8, 8, 8, 0),          # bad inf
    (FAKE, 8, FAKE, 8, FAKE, 8, 8, 8, 8, 0x40000000),
])
def test_gemm_argument_errors(lib, args):
    assert ga.apsp_minplus_gemm_i32(*args, 0) == ga.APSP_ERR_INVALID_VALUE


def test_gemm_empty_is_a_no_op_and_f32_inf(lib):
    assert ga.apsp_minplus_gemm_i32(0, 1, 0, 1, 0, 1, 0, 5, 5, 100, 0) == ga.APSP_OK
    assert ga.apsp_minplus_gemm_f32(0, 1, 0, 1, 0, 1, 5, 5, 0, 1.0, 0) == ga.APSP_OK
    for inf in (0.0, -1.0, float("nan")):
        assert ga.apsp_minplus_gemm_f32(FAKE, 8, FAKE, 8, FAKE, 8, 8, 8, 8, inf, 0) == \
            ga.APSP_ERR_INVALID_VALUE


@pytest.mark.parametrize("args", [
    (FAKE, -1, 4, 100, 0), (0, 4, 4, 100, 0), (FAKE, 8, 7, 100, 0), (FAKE + 2, 4, 4, 100, 0),
    (FAKE, 4, 4, 0, 0), (FAKE, 4, 4, 100, -1),
])
def test_host_argument_errors(lib, args):
    st, blk = ga.apsp_fw_host_i32(*args)
    assert st == ga.APSP_ERR_INVALID_VALUE and blk == 0
    assert ga.apsp_fw_host_i32(0, 0, 1, 100)[0] == ga.APSP_OK


def _plan_by_search(n, budget):
    """What the host-resident call should choose, by plain search over the
    multiples of 128: in-core when the matrix fits; else the largest S whose
    buffers fit with one or two panel sets (two when S2 >= min(S1, 4096)),
    lowered to the smallest S with the same number of outer rounds."""
    ldr = (n + 3) // 4 * 4
    n128 = (n + 127) // 128 * 128
    if 4 * n * ldr <= budget:
        return ga.APSP_OK, n128, 0

    def need(S, sets):
        return 4 * (sets * (S * ldr + n * S) + 4 * S * S)

    def largest(sets):
        best = 0
        for S in range(128, n128 + 1, 128):
            if need(S, sets) <= budget:
                best = S
        return best
    s1, s2 = largest(1), largest(2)
    if s1 == 0:
        return ga.APSP_ERR_RANGE, 0, 0
    sets, top = (2, s2) if s2 and s2 >= min(s1, 4096) else (1, s1)
    rounds = -(-n // top)
    S = 128
    while -(-n // S) > rounds:
        S += 128
    assert need(S, sets) <= budget
    return ga.APSP_OK, S, sets


@pytest.mark.parametrize("n", [1, 5, 127, 128, 129, 1000, 4099, 32768, 100_003])
@pytest.mark.parametrize("frac", [0.0, 0.01, 0.05, 0.2, 0.5, 0.75, 0.99, 1.0, 2.0])
def test_host_plan_matches_a_plain_search(lib, n, frac):
    ldr = (n + 3) // 4 * 4
    budget = max(1, int(frac * 4 * n * ldr))
    want = _plan_by_search(n, budget)
    assert ga.apsp_fw_host_plan(n, 4, budget) == want


def test_host_plan_named_cases(lib):
    n = 32768
    # 3 GiB for a 4 GiB matrix: two sets, 7 balanced rounds
    st, S, sets = ga.apsp_fw_host_plan(n, 4, 3 << 30)
    assert (st, sets) == (ga.APSP_OK, 2) and S % 128 == 0 and -(-n // S) == 7
    # exactly the matrix: in-core
    assert ga.apsp_fw_host_plan(n, 4, 4 * n * n) == (ga.APSP_OK, n, 0)
    # a tight budget keeps one set at a larger S
    st, S, sets = ga.apsp_fw_host_plan(n, 4, 4 * (2 * 1024 * n + 4 * 1024 * 1024))
    assert (st, S, sets) == (ga.APSP_OK, 1024, 1)
    assert ga.apsp_fw_host_plan(n, 4, 1000)[0] == ga.APSP_ERR_RANGE
    assert ga.apsp_fw_host_plan(0, 4, 0) == (ga.APSP_OK, 0, 0)
    for args in ((-1, 4, 100), (5, 8, 100), (5, 4, -1), (2**31 + 1, 4, 100)):
        assert ga.apsp_fw_host_plan(*args)[0] == ga.APSP_ERR_INVALID_VALUE


def test_path_walker_on_host_memory(lib):
    import numpy as np
    # successors of the hand-worked example (tests/golden/hand4_fw.txt)
    nxt = np.array([[0, 1, 1, 1], [-1, 1, 2, 2], [-1, 3, 2, 3], [-1, 1, 1, 3]], dtype=np.int32)
    assert ga.path(nxt, 0, 3) == [0, 1, 2, 3]
    assert ga.path(nxt, 2, 1) == [2, 3, 1]
    assert ga.path(nxt, 1, 1) == [1]
    assert ga.path(nxt, 1, 0) == []
    # too small an output buffer: the length is still returned
    buf = np.zeros(2, dtype=np.int32)
    assert ga.apsp_path(nxt.ctypes.data, 4, 4, 0, 3, buf.ctypes.data, 2) == 4
    assert buf.tolist() == [0, 1]
    # bad arguments and a successor cycle
    assert ga.apsp_path(nxt.ctypes.data, 4, 4, 0, 4, 0, 0) == -2
    assert ga.apsp_path(0, 4, 4, 0, 1, 0, 0) == -2
    loop = np.array([[0, 1, 1], [0, 1, 0], [-1, -1, 2]], dtype=np.int32)
    assert ga.apsp_path(loop.ctypes.data, 3, 3, 0, 2, 0, 0) == -3
    with pytest.raises(ValueError):
        ga.path(loop, 0, 2)


@pytest.mark.parametrize("fn", ["apsp_successors_i32", "apsp_fw_paths_i32"])
def test_successor_argument_errors(lib, fn):
    f = getattr(ga, fn)
    if fn == "apsp_successors_i32":
        bad = [(FAKE, 4, FAKE, 4, FAKE, 4, -1, 100), (0, 4, FAKE, 4, FAKE, 4, 4, 100),
               (FAKE, 3, FAKE, 4, FAKE, 4, 4, 100), (FAKE, 4, FAKE, 4, FAKE + 2, 4, 4, 100),
               (FAKE, 4, FAKE, 4, FAKE, 4, 4, 0)]
    else:
        bad = [(FAKE, 4, FAKE, 4, -1, 100), (0, 4, FAKE, 4, 4, 100), (FAKE, 4, FAKE, 3, 4, 100),
               (FAKE, 4, FAKE, 4, 4, 0x40000000)]
    for args in bad:
        assert f(*args, 0) == ga.APSP_ERR_INVALID_VALUE


def test_ceiling_at_wave_count_rejects_bad_arguments():
    # checked before any HIP call
    for arith, w in ((0, 0), (1, 5), (-1, 2), (3, 2)):
        assert ga.apsp_minplus_ceiling_waves(arith, w)[0] == ga.APSP_ERR_INVALID_VALUE
