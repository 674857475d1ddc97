#!/usr/bin/env python3
"""Throughput bench: blocked Floyd-Warshall APSP on one MI355X.

One step = one full all-pairs shortest-path call (every round: Phase 1,
Phase 2, Phase 3) over its own fresh copy of the seeded synthetic matrix,
which is resident in HBM before the timed region starts.

Prints ONE JSON line:
  value        relaxations/s = n^3 / (wall time per step), n = logical size
  roofline     the Phase-3 kernel (the hot loop): algorithmic relaxations per
               launch / its average launch duration (HIP events recorded on
               the kernel's stream around every launch of the last two calls
               of the timed region), against the VALU min-plus peak of the
               arithmetic the call used
  cpu_baseline the CPU oracle (plain Floyd-Warshall) timed on this host on a
               bounded sample of the same workload: its first k pivots

With --workload batch-... (many independent graphs of n <= 128, see
graphgen.BATCH_WORKLOADS) a step is one apsp_fw_batched_* call over the whole
batch; value = batch * n^3 / (wall time per step), and the roofline entry
describes the batched kernel (one launch per step, timed with events on its
stream).

With --workload shard-<workload>-p<P> a step is one GPU's share of one round's
Phase 3 when the matrix is split into P block rows (the multi-GPU design): the
(n/P) x n slab updated through apsp_minplus_gemm; value = its relaxations/s.

With --workload johnson-... (sparse graphs, see graphgen.JOHNSON_WORKLOADS) a
step is one apsp_johnson_timed_i32 call (CSR on the device, dense n x n
distances out); value = n^3 / (wall time per step), the rate a dense
Floyd-Warshall would need to match it, and the same matrix is also timed
through apsp_fw_i32 (apsp_fw_signed_i32 when some weight is negative).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "APSP min-plus relaxations/s (n^3/time) at n=8192; % of VALU roofline"
METRIC_BATCHED = "batched APSP min-plus relaxations/s (batch*n^3/time); % of VALU roofline"
METRIC_JOHNSON = ("Johnson APSP on a sparse graph: n^3/time (the relaxations/s a dense "
                  "Floyd-Warshall would need for the same answer)")
DEFAULT_WORKLOAD = "complete-8192-i32"

# MI355X VALU peaks (256 CUs, 2.4 GHz).  A relaxation (one add, one min)
# costs 1.5 VALU instructions when two candidates share one three-input min
# (v_add, v_add, v_min3 per pair).
#  - binary32 adds/mins issue at 128 lanes per clock per CU (the rate behind
#    the published 157.3 TFLOP/s fp32 vector figure, FMA = 2 flops):
#    7.86e13 lane-instructions/s -> 5.24e13 relaxations/s;
#  - int32: the VOP2 add issues at 64 lanes per clock per CU, but the
#    kernels write it in its VOP3 encoding, which co-issues: the
#    register-only int32 mix with it measures above 2.62e13 relaxations/s
#    (3.5e13).  So the int32 roof is the same dual-issue rate, 5.24e13.
INSTR_PER_RELAX = 1.5
VALU_LANE_OPS = {"f32": 256 * 128 * 2.4e9, "int32": 256 * 128 * 2.4e9}
PEAK_RELAX = {k: v / INSTR_PER_RELAX for k, v in VALU_LANE_OPS.items()}
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def phase3_relaxations_per_round(n: int, B: int) -> list[int]:
    """Algorithmic (logical-n) relaxations done by Phase 3 in each round:
    rows and columns outside pivot block K, times the pivots in block K."""
    out = []
    nb = (n + B - 1) // B
    for K in range(nb):
        bk = min(B, n - K * B)
        out.append((n - bk) * (n - bk) * bk)
    return out


def source_sha(names=("apsp.hip", "minplus.h")) -> str:
    """SHA-256 over the kernel sources a counter summary was taken on."""
    h = hashlib.sha256()
    for name in names:
        h.update(open(os.path.join(ROOT, "graph_all_pairs_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def read_traffic(workload: str, per_launch_relax: float, kernel: str = "phase3",
                 source=("apsp.hip", "minplus.h")):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, when it was taken on the current kernel
    source; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_hbm_traffic_{workload}.md")
    if not os.path.exists(p):
        return None
    txt = open(p).read()
    m_sha = re.search(r"kernel source sha256:\s*([0-9a-f]{64})", txt)
    m_b = re.search(r"HBM bytes per launch \(scaled\):\s*([0-9.eE+]+)", txt)
    if not m_sha or not m_b or m_sha.group(1) != source_sha(source):
        return None
    return float(m_b.group(1))


def cpu_baseline(w, target_s: float):
    """Time the oracle's plain Floyd-Warshall on the first k pivots."""
    import numpy as np
    import oracle
    orc = oracle.default()
    n = w.shape[0]
    f64 = w.dtype != np.int32

    def run(k):
        a = w.astype(np.float64) if f64 else np.array(w, copy=True)
        t0 = time.perf_counter()
        (orc.lib.oracle_fw_f64 if f64 else orc.lib.oracle_fw_i32)(a.ctypes.data, n, a.shape[1], k)
        return time.perf_counter() - t0

    probe = min(n, 64)
    per_pivot = run(probe) / probe
    k = int(max(1, min(n, target_s / max(per_pivot, 1e-9))))
    dt = run(k)
    if dt < 0.6 * target_s and k < n:  # the short probe over-estimated the per-pivot time
        k = int(max(1, min(n, k * target_s / max(dt, 1e-9))))
        dt = run(k)
    return {
        "value": k * n * n / dt,
        "unit": "relaxations/s",
        "cores": orc.threads(),
        "kind": "oracle",
        "sample": f"plain Floyd-Warshall (k outermost, OpenMP over rows) on the same "
                  f"{n}x{n} matrix, first {k} of {n} pivots ({k * n * n:.3e} relaxations) "
                  f"in {dt:.2f} s; rate = relaxations / time",
    }


def cpu_baseline_batched(w, target_s: float):
    """Time the oracle's per-graph Floyd-Warshall on the first graphs."""
    import numpy as np
    import oracle
    orc = oracle.default()
    batch, n = w.shape[0], w.shape[1]
    f64 = w.dtype != np.int32

    def run(k):
        a = w[:k].astype(np.float64) if f64 else np.array(w[:k], copy=True)
        t0 = time.perf_counter()
        (orc.lib.oracle_fw_batched_f64 if f64 else orc.lib.oracle_fw_batched_i32)(
            a.ctypes.data, k, n, a.shape[2], n * a.shape[2])
        return time.perf_counter() - t0

    probe = min(batch, 256)
    per_graph = run(probe) / probe
    k = int(max(1, min(batch, target_s / max(per_graph, 1e-12))))
    dt = run(k)
    return {
        "value": k * n ** 3 / dt,
        "unit": "relaxations/s",
        "cores": orc.threads(),
        "kind": "oracle",
        "sample": f"plain Floyd-Warshall per graph (OpenMP over graphs) on the first {k} of "
                  f"{batch} graphs of the same batch, n = {n} ({k * n ** 3:.3e} relaxations) "
                  f"in {dt:.2f} s; rate = relaxations / time",
    }


def bench_batched(args) -> int:
    """Many small graphs: one apsp_fw_batched_* launch per step."""
    import numpy as np
    import torch

    import graph_all_pairs_amd as ga
    import graphgen as gg

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = gg.BATCH_WORKLOADS[args.workload]
    t0 = time.perf_counter()
    w = gg.make_batch_workload(args.workload, ld=args.ld)
    batch, n, ld = w.shape
    sha = hashlib.sha256(np.ascontiguousarray(w).tobytes()).hexdigest()
    log(f"workload {args.workload}: batch={batch} n={n} ld={ld} built in "
        f"{time.perf_counter() - t0:.1f} s sha256={sha[:16]}")
    is_int = w.dtype == np.int32
    inf = gg.INF_I32 if is_int else float("inf")
    fn = ga.apsp_fw_batched_i32 if is_int else ga.apsp_fw_batched_f32

    pristine = torch.from_numpy(w).to(dev)
    copies = [torch.empty_like(pristine) for _ in range(args.warmup + args.steps)]
    for c in copies:
        c.copy_(pristine)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def step(t):
        st = fn(t.data_ptr(), batch, n, ld, n * ld, inf, sptr)
        if st != ga.APSP_OK:
            raise ga.APSPError(st, "apsp_fw_batched")

    for i in range(args.warmup):
        step(copies[i])
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    # One kernel launch per step on torch's current stream: events recorded
    # on that stream around each launch time the kernel itself.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    wall0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(copies[args.warmup + i])
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    kern_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    ms_per_step = 1e3 * wall / args.steps
    relax = float(batch) * n ** 3
    value = relax / (wall / args.steps)
    arith = "int32" if is_int else "f32"
    achieved = relax / (kern_ms * 1e-3)
    peak = PEAK_RELAX[arith]
    log(f"timed {args.steps} steps: wall {wall * 1e3:.1f} ms, kernel {kern_ms:.3f} ms/launch")
    roofline = {
        "bound": "alu",
        "kernel": "fw_batched",
        "achieved": achieved / 1e12,
        "peak": peak / 1e12,
        "unit": "Trelax/s",
        "frac": achieved / peak,
        "traffic": read_traffic(args.workload, relax, kernel="batched",
                                source=("batched.hip", "minplus.h")),
        "relax_per_launch": relax,
        "avg_launch_ms": kern_ms,
        "launches": args.steps,
    }
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline_batched(w, args.cpu_seconds)
        log(f"cpu baseline {cpu['value']:.3e} relax/s on {cpu['cores']} threads")
    rec = {
        "metric": METRIC_BATCHED,
        "value": value,
        "unit": "relaxations/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": arith,
        "data": "synthetic",
        "config": {
            "workload": args.workload, "batch": batch, "n": n, "ld": ld,
            "seed": spec["seed"], "matrix_dtype": arith, "input_sha256": sha,
            "graphs_per_s": batch / (wall / args.steps),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


def cpu_baseline_johnson(w, csr, target_s: float):
    """Time the oracle's single-source routine on the first sources: Dijkstra
    rows (non-negative weights) or Bellman-Ford rows (negative weights)."""
    import numpy as np
    import oracle
    import graphgen as gg
    orc = oracle.default()
    n = w.shape[0]
    neg = bool((csr[2] < 0).any())

    def run(k):
        t0 = time.perf_counter()
        if neg:
            orc.bf_rows_csr(*csr, n, np.arange(k), gg.INF_I32)
        else:
            orc.sssp_rows_i32(w, gg.INF_I32, np.arange(k))
        return time.perf_counter() - t0

    probe = min(n, 2 * orc.threads())
    per_src = run(probe) / probe
    k = int(max(1, min(n, target_s / max(per_src, 1e-9))))
    dt = run(k)
    how = "Bellman-Ford over CSR" if neg else "Dijkstra on the dense matrix"
    return {
        "value": float(n) ** 3 / (dt * n / k),
        "unit": "relaxations/s",
        "cores": orc.threads(),
        "kind": "oracle",
        "sample": f"{how}, one source per thread (OpenMP), first {k} of {n} sources in "
                  f"{dt:.2f} s; the all-pairs time is extrapolated to n sources and the rate "
                  f"reported as n^3 / time, like the GPU value",
    }


def bench_johnson(args) -> int:
    """Sparse graphs: one synchronous apsp_johnson_timed_i32 call per step."""
    import numpy as np
    import torch

    import graph_all_pairs_amd as ga
    import graphgen as gg

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    w = gg.make_johnson_workload(args.workload)
    n = w.shape[0]
    csr = gg.csr_from_dense(w, gg.INF_I32)
    nnz = len(csr[1])
    sha = gg.sha256_matrix(w, n)
    neg = bool((csr[2] < 0).any())
    log(f"workload {args.workload}: n={n} nnz={nnz} negative weights={neg} built in "
        f"{time.perf_counter() - t0:.1f} s sha256={sha[:16]}")
    rp, col, wt = (torch.from_numpy(np.ascontiguousarray(x, dtype=dt)).to(dev)
                   for x, dt in zip(csr, (np.int64, np.int32, np.int32)))
    out = torch.empty((n, n), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        ga.johnson(rp, col, wt, out=out)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")
    phase_ms = [0.0] * 4
    counts = [0] * 4
    wall0 = time.perf_counter()
    for _ in range(args.steps):
        _, ms, cnt = ga.johnson(rp, col, wt, out=out, timed=True)
        for i in range(4):
            phase_ms[i] += ms[i]
            counts[i] += cnt[i]
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = 1e3 * wall / args.steps
    value = float(n) ** 3 / (wall / args.steps)
    per = [x / args.steps for x in phase_ms]
    cnt = [x / args.steps for x in counts]
    log(f"timed {args.steps} steps: {ms_per_step:.2f} ms/step; ms by phase [validate, "
        f"bellman-ford, reweight, search] {[round(x, 3) for x in per]}; counts per call "
        f"[bf rounds, steps, removed, relaxations] {cnt}")

    # The blocked Floyd-Warshall on the same dense matrix (its negative-weight
    # entry when some weight is negative), for comparison.
    d = torch.from_numpy(w).to(dev)
    ref = torch.empty_like(d)
    times = []
    for _ in range(2):
        ref.copy_(d)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        (ga.fw_signed if neg else ga.fw)(ref, gg.INF_I32)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t1)
    fw_ms = 1e3 * min(times)
    same = bool(torch.equal(ref, out))
    log(f"blocked Floyd-Warshall on the same matrix: {fw_ms:.2f} ms, results equal: {same}")
    if not same:
        raise RuntimeError("Johnson and Floyd-Warshall disagree")
    del d, ref

    # The search kernel: algorithmic HBM bytes per launch are the n x n
    # result written once plus the graph read once (packed edges, offsets).
    search_ms = per[3]
    alg_bytes = 4.0 * n * n + 8.0 * nnz + 8.0 * (n + 1)
    achieved = alg_bytes / (search_ms * 1e-3) / 1e9
    relax = cnt[3]
    roofline = {
        "bound": "hbm",
        "kernel": "jo_sssp",
        "achieved": achieved,
        "peak": 8000.0,
        "unit": "GB/s",
        "frac": achieved / 8000.0,
        "traffic": None,
        "avg_launch_ms": search_ms,
        "launches": args.steps,
        "bytes_per_launch": alg_bytes,
        "edge_relaxations_per_launch": relax,
        "edge_relaxations_per_s": relax / (search_ms * 1e-3),
        "relaxations_per_edge_per_source": relax / (float(n) * nnz),
        "steps_per_source": cnt[1] / n,
        "note": "latency bound: each search step waits on two dependent memory loads and "
                "three barriers; no throughput roof is near",
    }
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline_johnson(w, csr, args.cpu_seconds)
        log(f"cpu baseline {cpu['value']:.3e} n^3/s on {cpu['cores']} threads")
    rec = {
        "metric": METRIC_JOHNSON,
        "value": value,
        "unit": "relaxations/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "n": n, "nnz": nnz, "negative_weights": neg,
            "input_sha256": sha, "fw_ms_per_call": fw_ms,
            "fw_entry": "apsp_fw_signed_i32" if neg else "apsp_fw_i32",
            "speedup_vs_fw": fw_ms / ms_per_step,
        },
        "ms_per_step_by_phase": dict(zip(["validate", "bellman_ford", "reweight", "search"], per)),
        "counts_per_step": dict(zip(["bellman_ford_rounds", "search_steps", "removed",
                                     "edge_relaxations"], cnt)),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


def host_pcie_bytes(n, S, sets, scanned):
    """Bytes the host-resident call moves over PCIe: the exactness scan (which
    also loads the first round's panels), the panels in (every round with one
    set, else the first round when not scanned) and back, and the super-tiles
    in and out (with two sets, the next pivot row's and column's stay)."""
    e = 4
    total = e * n * n if scanned else 0
    for K0 in range(0, n, S):
        sk = min(S, n - K0)
        if sets == 1 and not (K0 == 0 and scanned) or sets == 2 and K0 == 0 and not scanned:
            total += e * 2 * sk * n
        total += e * (sk * n + (n - sk) * sk)
        rest = n - sk
        total += e * rest * rest
        K1 = K0 + S
        nxt = min(S, n - K1) if K1 < n else 0
        stay = (nxt * rest + (rest - nxt) * nxt) if sets == 2 else 0
        total += e * (rest * rest - stay)
    return total


def bench_host(args) -> int:
    """Host-resident matrix: one apsp_fw_host_i32 call per step within the
    workload's device budget (the matrix does not fit in it), on a fresh copy
    of the pinned matrix."""
    import numpy as np
    import torch

    import graph_all_pairs_amd as ga
    import graphgen as gg

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = gg.HOST_WORKLOADS[args.workload]
    n, budget = spec["n"], spec["device_budget"]
    st, S, sets = ga.apsp_fw_host_plan(n, 4, budget)
    if st != ga.APSP_OK or sets == 0:
        raise RuntimeError(f"workload {args.workload}: plan {st, S, sets} is not out-of-core")
    t0 = time.perf_counter()
    pristine = torch.empty((n, n), dtype=torch.int32, pin_memory=True)
    gg.complete(n, spec["wlo"], spec["whi"], spec["seed"], out=pristine.numpy())
    work = torch.empty_like(pristine).pin_memory()
    sha = gg.sha256_matrix(pristine.numpy(), n)
    log(f"workload {args.workload}: n={n} ({4 * n * n / 2**30:.1f} GiB pinned host matrix), "
        f"device budget {budget / 2**30:.2f} GiB (outer block {S}, {sets} panel set(s)); built in "
        f"{time.perf_counter() - t0:.1f} s sha256={sha[:16]}")
    s = torch.cuda.current_stream().cuda_stream

    def step():
        work.copy_(pristine)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        st, blk = ga.apsp_fw_host_i32(work.data_ptr(), n, n, gg.INF_I32, budget, s)
        dt = time.perf_counter() - t1
        if st != ga.APSP_OK:
            raise ga.APSPError(st, "apsp_fw_host_i32")
        return dt, blk

    for _ in range(args.warmup):
        step()
    times = []
    for _ in range(args.steps):
        dt, blk = step()
        times.append(dt)
    wall = sum(times)
    ms_per_step = 1e3 * wall / args.steps
    value = float(n) ** 3 / (wall / args.steps)
    log(f"timed {args.steps} steps: {ms_per_step:.1f} ms/step (outer block {blk})")
    if blk != S:
        raise RuntimeError(f"outer block {blk} differs from the plan's {S}")

    # The same matrix in device memory, in-core, for comparison.
    d = pristine.to(dev)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ga.fw(d, gg.INF_I32)
    torch.cuda.synchronize()
    in_core_ms = 1e3 * (time.perf_counter() - t1)
    same = bool(torch.equal(d.cpu(), work))
    log(f"in-core apsp_fw_i32 on the same matrix: {in_core_ms:.1f} ms; results equal: {same}")
    if not same:
        raise RuntimeError("host-resident and in-core results differ")
    del d
    moved = float(host_pcie_bytes(n, S, sets, scanned=ga.apsp_get_int32_arith() != ga.APSP_ARITH_INT32))
    peak = PEAK_RELAX["f32"]
    roofline = {
        "bound": "alu",
        "kernel": "mp_gemm (whole job: products, closures and PCIe transfers overlapped)",
        "achieved": value / 1e12,
        "peak": peak / 1e12,
        "unit": "Trelax/s",
        "frac": value / peak,
        "traffic": None,
        "pcie_bytes_per_step": moved,
        "pcie_gb_per_s": moved / (wall / args.steps) / 1e9,
        "note": "whole-job rate (products, closures and PCIe transfers together)",
    }
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(pristine.numpy(), args.cpu_seconds)
        log(f"cpu baseline {cpu['value']:.3e} relax/s on {cpu['cores']} threads")
    rec = {
        "metric": "host-resident APSP min-plus relaxations/s (n^3/time), matrix in pinned host memory",
        "value": value,
        "unit": "relaxations/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "n": n, "seed": spec["seed"], "outer_block": S,
                   "panel_sets": sets, "device_budget_bytes": budget, "matrix_dtype": "int32", "input_sha256": sha,
                   "in_core_ms": in_core_ms},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    # Give the pinned host blocks back while the HIP runtime is whole: torch's
    # pinned-memory cache would otherwise free them from a static destructor
    # at process exit.
    del pristine, work
    torch.cuda.synchronize()
    if hasattr(torch._C, "_host_emptyCache"):
        torch._C._host_emptyCache()
    return 0


def parse_shard(name: str):
    """shard-<workload>-p<P> -> (workload, P), else None."""
    m = re.fullmatch(r"shard-(.+)-p(\d+)", name)
    return (m.group(1), int(m.group(2))) if m else None


def bench_shard(args) -> int:
    """One GPU's share of one round's Phase 3 when the matrix is split into P
    block rows, one per GPU: the (n/P) x n slab takes C <- min(C, A (x) B)
    with A its n/P x B pivot columns and B the B x n pivot-row panel that
    the owner of block row K broadcasts.  It runs through apsp_minplus_gemm
    (the Phase-3 register tiling, C resident for the whole depth) at that
    shape, on the workload's values, in the arithmetic the in-core call
    uses (binary32 for an int32 matrix whose entries are exact there).  A
    step is one slab update, timed with HIP events on its stream."""
    import numpy as np
    import torch

    import graph_all_pairs_amd as ga
    import graphgen as gg

    base, P = parse_shard(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = gg.make_workload(base)
    n = w.shape[0]
    B = ga.apsp_pivot_block(n)
    nb = (n + B - 1) // B
    if P < 1 or n % P or (n // P) % B:
        raise SystemExit(f"bench.py: {n} rows do not split into {P} block rows of whole pivot blocks")
    rows = n // P
    K = nb // 2  # a middle round; the kernel's work does not depend on the values
    f32 = w.dtype != np.int32 or (
        bool(((w == gg.INF_I32) | ((w >= 0) & (w <= 1 << 24))).all()))
    if w.dtype == np.int32 and f32:
        wf = np.where(w == gg.INF_I32, np.float32(np.inf), w.astype(np.float32))
    else:
        wf = w
    full = torch.from_numpy(np.ascontiguousarray(wf[:, :n]))
    p = P // 2  # the GPU whose slab is measured
    c0 = full[p * rows:(p + 1) * rows].to(dev)
    a = full[p * rows:(p + 1) * rows, K * B:(K + 1) * B].contiguous().to(dev)
    b = full[K * B:(K + 1) * B].contiguous().to(dev)
    del full
    arith = "f32" if c0.dtype == torch.float32 else "int32"
    steps = max(args.steps, 200)  # a slab update takes tens of microseconds
    cs = [c0.clone() for _ in range(min(steps + args.warmup, 16))]
    torch.cuda.synchronize()
    for i in range(args.warmup):
        ga.minplus_gemm(cs[i % len(cs)], a, b)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        ga.minplus_gemm(cs[i % len(cs)], a, b)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = e0.elapsed_time(e1) / steps
    relax = rows * n * B
    achieved = relax / (ms * 1e-3)
    peak = PEAK_RELAX[arith]
    log(f"{args.workload}: slab {rows} x {n}, depth {B} (round {K} of {nb}), {arith}: "
        f"{ms * 1e3:.1f} us per slab update, {achieved / 1e12:.2f} Trelax/s")
    # What the other GPUs would wait for: the B x n pivot-row panel on one xGMI link.
    panel_bytes = B * n * 4
    roofline = {
        "bound": "alu", "kernel": "mp_gemm", "achieved": achieved / 1e12,
        "peak": peak / 1e12, "unit": "Trelax/s", "frac": achieved / peak, "traffic": None,
        "relax_per_launch": relax, "avg_launch_ms": ms, "launches": steps,
    }
    st_c, ceil = ga.apsp_minplus_ceiling(1 if arith == "f32" else 0)
    if st_c == ga.APSP_OK:
        roofline["ceiling_measured"] = ceil / 1e12
        roofline["frac_of_ceiling"] = achieved / ceil
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.default()
        sub = rows  # the whole slab: about a second of CPU work
        ch = c0[:sub].cpu().numpy().astype(np.float64 if arith == "f32" else np.int64)
        ah = a[:sub].cpu().numpy().astype(ch.dtype)
        bh = b.cpu().numpy().astype(ch.dtype)
        t0 = time.perf_counter()
        if arith == "f32":
            orc.minplus(ch, ah, bh)
        else:
            orc.minplus(ch, ah, bh, gg.INF_I32)
        dt = time.perf_counter() - t0
        cpu = {"value": sub * n * B / dt, "unit": "relaxations/s", "cores": orc.threads(),
               "kind": "oracle",
               "sample": f"the oracle's min-plus product on {sub} of the {rows} slab rows "
                         f"({sub * n * B:.3e} relaxations) in {dt:.2f} s"}
    rec = {
        "metric": "one GPU's share of one Floyd-Warshall round: slab min-plus update, "
                  "relaxations/s",
        "value": achieved, "unit": "relaxations/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "strong", "vs_baseline": None, "dtype": arith, "data": "synthetic",
        "config": {"workload": args.workload, "matrix": base, "n": n, "gpus_in_design": P,
                   "slab_rows": rows, "depth": B, "round": K,
                   "panel_bytes_broadcast": panel_bytes,
                   "panel_ms_on_one_xgmi_link": panel_bytes / 153e9 * 1e3,
                   "wall_ms_per_step": 1e3 * wall / steps},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_paths(args) -> int:
    """Distances plus successors.  A dense int32 workload whose weights fit the
    key form (see apsp_fw_paths_i32) runs one apsp_fw_paths_i32 call per
    step: the rounds on keys value << s | first hop, in int32 arithmetic, with
    no successor pass; the roofline entry is that call's Phase-3 kernel
    (fw_keys_phase3), from the launch trace, against the dual-issue VALU rate.
    Any other workload runs one apsp_fw_i32 and one apsp_successors_i32 call
    per step (what apsp_fw_paths_i32 does for it); the roofline entry is the
    successor pass (its kernels between HIP events on its stream).  Dense
    weights run an argmin product, bound by the int32 VALU: with packed keys
    (non-negative weights and distances whose largest finite sum is below inf
    and 2^(31 - ceil(log2 n))) at 1.5 instructions per candidate, like the
    min-plus product, else at 4 (add, compare, two selects); sparse weights
    run the neighbour-list kernel, n candidates per edge, each reading 4 bytes
    of D (bound by memory: reported against HBM, although most reads hit L2
    and the MALL)."""
    import numpy as np
    import torch

    import graph_all_pairs_amd as ga
    import graphgen as gg

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    base = args.workload[len("paths-"):]
    w = gg.make_workload(base)
    n = w.shape[0]
    sha = gg.sha256_matrix(w, n)
    log(f"workload {args.workload}: successors of {base}, n={n}")
    tw = torch.from_numpy(w).to(dev)
    copies = [tw.clone() for _ in range(1 + args.warmup + args.steps)]
    nxt = torch.empty((n, n), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream

    # Which form the library takes for this matrix: one call on a spare copy.
    if ga.apsp_fw_paths_i32(copies[0].data_ptr(), n, nxt.data_ptr(), n, n, gg.INF_I32, s) \
            != ga.APSP_OK:
        raise RuntimeError("apsp_fw_paths_i32 failed")
    torch.cuda.synchronize()
    keys = ga.apsp_fw_paths_last_form() == 1
    copies = copies[1:]
    B = ga.apsp_pivot_block(n)
    nb = (n + B - 1) // B

    def step(d, evs=None):
        if keys:
            if ga.apsp_fw_paths_i32(d.data_ptr(), n, nxt.data_ptr(), n, n, gg.INF_I32, s) \
                    != ga.APSP_OK:
                raise RuntimeError("apsp_fw_paths_i32 failed")
            return
        if ga.apsp_fw_i32(d.data_ptr(), n, n, gg.INF_I32, s) != ga.APSP_OK:
            raise RuntimeError("apsp_fw_i32 failed")
        if evs:
            evs[0].record(stream)
        if ga.apsp_successors_i32(tw.data_ptr(), n, d.data_ptr(), n, nxt.data_ptr(), n, n,
                                  gg.INF_I32, s) != ga.APSP_OK:
            raise RuntimeError("apsp_successors_i32 failed")
        if evs:
            evs[1].record(stream)

    for i in range(args.warmup):
        step(copies[i])
    torch.cuda.synchronize()
    n_traced = min(2, args.steps) if keys else 0
    launches_per_call = 2 * nb + 8
    if keys:
        for _ in range(2):  # create the trace's event pool outside the region
            if ga.apsp_trace_begin(n_traced * launches_per_call) != ga.APSP_OK:
                raise RuntimeError("apsp_trace_begin failed")
            ga.apsp_trace_end()
        torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    wall0 = time.perf_counter()
    for i in range(args.steps):
        if keys and i == args.steps - n_traced:
            st = ga.apsp_trace_begin(n_traced * launches_per_call)
            if st != ga.APSP_OK:
                raise ga.APSPError(st, "apsp_trace_begin")
        step(copies[args.warmup + i], evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = 1e3 * wall / args.steps
    edges = int((w[:n, :n] < gg.INF_I32).sum() - np.count_nonzero(np.diag(w[:n, :n]) < gg.INF_I32))
    sparse = edges <= n * n // 16
    succ_ms = None
    if keys:
        st, phase_ms, launches, dropped = ga.apsp_trace_end()
        if st != ga.APSP_OK or dropped:
            raise RuntimeError(f"launch trace failed: status {st}, {dropped} launches not recorded")
        p3_relax = sum(phase3_relaxations_per_round(n, B)) * n_traced
        p3_launch = launches[2]
        p3_ms_avg = phase_ms[2] / max(p3_launch, 1)
        relax_per_launch = p3_relax / max(p3_launch, 1)
        achieved = relax_per_launch / (p3_ms_avg * 1e-3) if p3_ms_avg > 0 else 0.0
        peak = PEAK_RELAX["int32"]
        st_c, ceil = ga.apsp_minplus_ceiling(0)
        st_w, at3 = ga.apsp_minplus_ceiling_waves(0, 3)
        roofline = {"bound": "alu", "kernel": "fw_keys_phase3",
                    "achieved": achieved / 1e12, "peak": peak / 1e12, "unit": "Trelax/s",
                    "frac": achieved / peak,
                    "traffic": read_traffic(args.workload, relax_per_launch),
                    "relax_per_launch": relax_per_launch, "avg_launch_ms": p3_ms_avg,
                    "launches": p3_launch,
                    "ceiling_measured": ceil / 1e12 if st_c == ga.APSP_OK else None,
                    "ceiling_at_kernel_occupancy": (
                        {"waves_per_simd": 3, "value": at3 / 1e12, "frac": achieved / at3}
                        if st_w == ga.APSP_OK and at3 > 0 else None),
                    "note": "the rounds on successor keys (value << s | first hop) in int32 "
                            "arithmetic: two VOP3 adds and one v_min3_i32 per pair of pivots, "
                            "as the int32 Phase 3; peak: the dual-issue VALU rate / 1.5; "
                            "ceiling_measured: the register-only int32 replica"}
        log(f"timed {args.steps} steps: {ms_per_step:.2f} ms/step, one pass on successor keys; "
            f"traced ms/call by kind {[round(x / n_traced, 3) for x in phase_ms]}")
    elif sparse:
        succ_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
        # Algorithmic HBM bytes: W and D read once, the successor matrix written
        # once.  The kernel loads a D row per edge (4 bytes per candidate); those
        # loads are mostly served by L2 and the last-level cache, so they are
        # reported as a gather rate, not priced against HBM.
        moved = 3 * 4.0 * n * n
        gathered = 4.0 * edges * n
        roofline = {"bound": "hbm", "kernel": "successors_sparse",
                    "achieved": moved / (succ_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": moved / (succ_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": None,
                    "avg_launch_ms": succ_ms, "launches": args.steps, "edges": edges,
                    "candidates_per_s": edges * float(n) / (succ_ms * 1e-3),
                    "gather_GBps": gathered / (succ_ms * 1e-3) / 1e9,
                    "note": "achieved: W and D read once, successors written once (12 n^2 bytes); "
                            "gather_GBps: 4 bytes of D per candidate, n candidates per edge"}
    else:
        succ_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
        # The library's choice between its two dense kernels, from the same facts.
        d = copies[-1]
        wf, df_ = tw[tw < gg.INF_I32], d[d < gg.INF_I32]
        shift = max(0, (n - 1).bit_length())
        wmax = int(wf.max()) if wf.numel() else 0
        dmax = int(df_.max()) if df_.numel() else 0
        packed = (bool(wf.numel() == 0 or int(wf.min()) >= 0) and
                  bool(df_.numel() == 0 or int(df_.min()) >= 0) and
                  max(wmax, 0) + max(dmax, 0) < min(gg.INF_I32, 1 << (31 - shift)))
        achieved = float(n) ** 3 / (succ_ms * 1e-3)
        if packed:
            # Unsigned saturating adds and v_min3_u32 issue above the 64-lane
            # int32 rate (the register-only replica of this mix measures it), so
            # the roof is the dual-issue VALU rate, as for binary32.
            peak = VALU_LANE_OPS["f32"] / INSTR_PER_RELAX
            st_c, ceil = ga.apsp_minplus_ceiling(2)
            roofline = {"bound": "alu", "kernel": "successors_packed",
                        "achieved": achieved / 1e12, "peak": peak / 1e12, "unit": "Tcandidates/s",
                        "frac": achieved / peak, "traffic": None, "avg_launch_ms": succ_ms,
                        "launches": args.steps,
                        "ceiling_measured": ceil / 1e12 if st_c == ga.APSP_OK else None,
                        "note": "peak: VALU dual-issue rate (256 CUs x 128 lanes x 2.4 GHz) / 1.5 "
                                "instructions per candidate (two unsigned saturating adds and one "
                                "v_min3_u32 per pair of candidates); ceiling_measured: a "
                                "register-only replica of that mix on this device"}
        else:
            peak = VALU_LANE_OPS["int32"] / 4.0
            roofline = {"bound": "alu", "kernel": "successors",
                        "achieved": achieved / 1e12, "peak": peak / 1e12, "unit": "Tcandidates/s",
                        "frac": achieved / peak, "traffic": None, "avg_launch_ms": succ_ms,
                        "launches": args.steps,
                        "note": "peak: dual-issue VALU rate / 4 instructions per candidate "
                                "(add, compare, two selects)"}
    if not keys:
        log(f"timed {args.steps} steps: {ms_per_step:.1f} ms/step, successor pass {succ_ms:.2f} ms "
            f"({'neighbour lists' if sparse else 'dense product'}, {edges} edges)")
    rec = {
        "metric": "APSP distances plus successor matrix, n^3/time",
        "value": float(n) ** 3 / (wall / args.steps),
        "unit": "relaxations/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "strong", "vs_baseline": None, "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": args.workload, "n": n, "input_sha256": sha,
                   "form": "successor keys, one pass" if keys else "rounds, then successor pass",
                   "successor_ms": succ_ms,
                   "fw_ms": None if keys else ms_per_step - succ_ms},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--ld", type=int, default=None, help="leading dimension (default n)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--int32-arith", choices=("auto", "f32", "int32"), default="auto",
                    help="arithmetic policy of int32 calls: auto (default), binary32 when exact, "
                         "or int32 forced")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is designed but not implemented)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import graph_all_pairs_amd as ga
    import graphgen as gg

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.workload in gg.BATCH_WORKLOADS:
        return bench_batched(args)
    if args.workload in gg.JOHNSON_WORKLOADS:
        return bench_johnson(args)
    if args.workload in gg.HOST_WORKLOADS:
        return bench_host(args)
    if args.workload.startswith("paths-") and args.workload[len("paths-"):] in gg.WORKLOADS:
        return bench_paths(args)
    shard = parse_shard(args.workload)
    if shard is not None and shard[0] in gg.WORKLOADS:
        return bench_shard(args)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    policy = {"auto": ga.APSP_ARITH_AUTO, "f32": ga.APSP_ARITH_F32_WHEN_EXACT,
              "int32": ga.APSP_ARITH_INT32}[args.int32_arith]
    if ga.apsp_set_int32_arith(policy) != ga.APSP_OK:
        raise RuntimeError("apsp_set_int32_arith failed")

    spec = gg.WORKLOADS[args.workload]
    t0 = time.perf_counter()
    w = gg.make_workload(args.workload, ld=args.ld)
    n, ld = w.shape[0], w.shape[1]
    sha = gg.sha256_matrix(w, n)
    log(f"workload {args.workload}: n={n} ld={ld} built in {time.perf_counter() - t0:.1f} s "
        f"sha256={sha[:16]}")
    is_int = w.dtype == np.int32
    inf = gg.INF_I32 if is_int else float("inf")
    B = ga.apsp_pivot_block(n)
    nb = (n + B - 1) // B

    pristine = torch.from_numpy(w).to(dev)
    copies = [torch.empty_like(pristine) for _ in range(args.warmup + args.steps)]
    for c in copies:
        c.copy_(pristine)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    timed_fn = ga.apsp_fw_timed_i32 if is_int else ga.apsp_fw_timed_f32
    plain_fn = ga.apsp_fw_i32 if is_int else ga.apsp_fw_f32

    # The arithmetic an int32 call takes depends only on the matrix: learn it
    # from one synchronised timed call during the warm-up.
    arith_code = None
    for i in range(args.warmup):
        if i == 0:
            st, _, _, arith_code = timed_fn(copies[i].data_ptr(), n, ld, inf, sptr)
        else:
            st = plain_fn(copies[i].data_ptr(), n, ld, inf, sptr)
        if st != ga.APSP_OK:
            raise ga.APSPError(st, "apsp_fw warm-up")
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    # Timed region: K asynchronous calls back to back, one synchronisation
    # at the end.  The library's launch trace records HIP events around every
    # launch of the last few calls on the calls' stream (no synchronisation
    # in between); the per-kind times are read after the region.  Event
    # markers cost about 4 us of idle GPU time per launch, so only a sample
    # of the calls carries them (the Phase-3 average comes from 64 launches
    # per traced call).
    launches_per_call = 2 * nb + 8
    n_traced = min(2, args.steps)
    for _ in range(2):  # create the trace's event pool outside the region
        if ga.apsp_trace_begin(n_traced * launches_per_call) != ga.APSP_OK:
            raise RuntimeError("apsp_trace_begin failed")
        ga.apsp_trace_end()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        if i == args.steps - n_traced:
            st = ga.apsp_trace_begin(n_traced * launches_per_call)
            if st != ga.APSP_OK:
                raise ga.APSPError(st, "apsp_trace_begin")
        st = plain_fn(copies[args.warmup + i].data_ptr(), n, ld, inf, sptr)
        if st != ga.APSP_OK:
            raise ga.APSPError(st, "apsp_fw")
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    st, phase_ms, launches, dropped = ga.apsp_trace_end()
    if st != ga.APSP_OK or dropped:
        raise RuntimeError(f"launch trace failed: status {st}, {dropped} launches not recorded")
    if arith_code is None:  # no warm-up: one extra synchronised call outside the region
        scratch = torch.empty_like(pristine)
        scratch.copy_(pristine)
        _, _, _, arith_code = timed_fn(scratch.data_ptr(), n, ld, inf, sptr)
        del scratch
    ms_per_step = 1e3 * wall / args.steps
    value = float(n) ** 3 / (wall / args.steps)
    arith = "f32" if arith_code == 1 else "int32"
    log(f"timed {args.steps} steps: wall {wall * 1e3:.1f} ms; traced calls: ms/call by kind "
        f"[phase1, phase2, phase3, int32 scan and panel conversion] "
        f"{[round(x / n_traced, 3) for x in phase_ms]}, arithmetic {arith}")

    # Phase-3 roofline: algorithmic relaxations per launch / mean launch time.
    p3_relax = sum(phase3_relaxations_per_round(n, B)) * n_traced
    p3_launch = launches[2]
    p3_ms_avg = phase_ms[2] / max(p3_launch, 1)
    relax_per_launch = p3_relax / max(p3_launch, 1)
    achieved = relax_per_launch / (p3_ms_avg * 1e-3) if p3_ms_avg > 0 else 0.0
    # Counter summaries are kept per workload and, when the policy is not the
    # default, per forced arithmetic.
    profile_key = args.workload + ("" if args.int32_arith == "auto" else f"-{args.int32_arith}arith")
    traffic = read_traffic(profile_key, relax_per_launch)
    peak = PEAK_RELAX["int32" if arith == "int32" else "f32"]
    roofline = {
        "bound": "alu",
        "kernel": "fw_phase3",
        "achieved": achieved / 1e12,
        "peak": peak / 1e12,
        "unit": "Trelax/s",
        "frac": achieved / peak,
        "traffic": traffic,
        "relax_per_launch": relax_per_launch,
        "avg_launch_ms": p3_ms_avg,
        "launches": p3_launch,
    }

    # Register-only replica of the Phase-3 inner step, both arithmetics.
    ceilings = {}
    for name, code in (("int32", 0), ("f32", 1)):
        st_c, c = ga.apsp_minplus_ceiling(code)
        if st_c == ga.APSP_OK:
            ceilings[name] = c
    if ceilings:
        log("register-only min-plus ceilings (Trelax/s): "
            + ", ".join(f"{k} {v / 1e12:.2f}" for k, v in ceilings.items()))
    own = ceilings.get("int32" if arith == "int32" else "f32")
    if own:
        roofline["ceiling_measured"] = own / 1e12
        roofline["frac_of_ceiling"] = achieved / own
    roofline["ceilings_measured"] = {k: v / 1e12 for k, v in ceilings.items()}
    # The same replica at the Phase-3 kernels' own occupancy, 3 waves per
    # SIMD: the double issue pairs waves, so one of three runs single-issue.
    st_w, at3 = ga.apsp_minplus_ceiling_waves(0 if arith == "int32" else 1, 3)
    if st_w == ga.APSP_OK and at3 > 0:
        roofline["ceiling_at_kernel_occupancy"] = {
            "waves_per_simd": 3, "value": at3 / 1e12, "frac": achieved / at3}
        log(f"register-only ceiling at 3 waves per SIMD: {at3 / 1e12:.2f} Trelax/s "
            f"(Phase 3 at {achieved / at3:.2f} of it)")

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(w, args.cpu_seconds)
        log(f"cpu baseline {cpu['value']:.3e} relax/s on {cpu['cores']} threads")

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "relaxations/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": arith,
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "n": n, "ld": ld, "seed": spec["seed"], "pivot_block": B, "rounds": nb,
            "matrix_dtype": "int32" if is_int else "f32",
            "int32_arith_policy": args.int32_arith,
            "input_sha256": sha,
        },
        "ms_per_step_by_kind": dict(zip(["phase1", "phase2", "phase3", "scan_convert"],
                                        [x / n_traced for x in phase_ms])),
        "traced_steps": n_traced,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
