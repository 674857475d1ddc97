// Johnson's all-pairs shortest paths for sparse digraphs (negative weights
// allowed, negative cycles detected), dense n x n distances out.
//
// Method: the page "Johnson's APSP in Glushkov algorithmic algebras" (CEUR
// Vol-1631, pp. 105-112), operators extendGraph, BellmanFord, UpdateWeights,
// D(q) and to(D, i):
//   1. a new vertex q gets a 0-weight edge to every vertex, and Bellman-Ford
//      from q gives h(v), the shortest distance from q (h <= 0); an edge that
//      can still be relaxed after |V| - 1 rounds means a negative cycle;
//   2. every edge is reweighted to w'(u,v) = w(u,v) + h(u) - h(v) >= 0, which
//      keeps shortest paths shortest;
//   3. a single-source search on w' runs from every vertex i;
//   4. d(i, j) = D'(j) - h(i) + h(j).
//
// gfx950 design:
//  * Bellman-Ford runs in vertex-frontier rounds: round r relaxes the
//    out-edges of the vertices whose h dropped in round r - 1 (all vertices
//    in round 1, the state right after q's edges), one wave per vertex with
//    the lanes striding its adjacency; h is int64 and lowered with global
//    atomic min.  A vertex improved during a round is re-examined in the next,
//    so after round k every h(v) is at most the shortest walk from q with k
//    real edges: without a negative cycle round |V| changes nothing, and a
//    change in round |V| is the page's condition cnc.  The host checks the
//    per-round change flags after every few rounds and stops at the first
//    quiet round.
//  * The per-source search follows the delta-stepping scheme of the page
//    "Delta-stepping SSSP on CPU and GPU" (CEUR Vol-1662, Algorithm 1, its
//    buckets of width delta) with the threshold rule of the Johnson page's
//    parallel ExtractMin (every unsettled vertex within delta of the smallest
//    tentative distance is taken together).  One workgroup owns one source at
//    a time and keeps that source's whole tentative-distance row in LDS (4n
//    bytes), so every relaxation is an LDS atomic min.  A vertex whose
//    distance drops is marked in an LDS bitmap.  Each step removes the marked
//    vertices with distance <= T into a queue and relaxes all of their
//    out-edges (light and heavy together); when no marked vertex is <= T,
//    T moves to (smallest marked distance) + delta.  With w' >= 0 the
//    search ends when nothing is marked, and each distance is then final.
//  * The edges of the removed vertices are spread over the workgroup by
//    adjacency length: groups of G lanes take short adjacencies (up to 8G
//    edges, G from the average degree), whole waves take the long ones.  A
//    balanced split of all edges by a prefix sum and a per-chunk binary
//    search was tried first and was 1.3-2.5x slower: its extra barriers and
//    dependent LDS reads lengthen every step, and the search is latency
//    bound, not work bound (about 1.03-1.3 relaxations per edge per source).
//  * Reweighted edges are packed as (target, w') pairs, one 8-byte load per
//    edge; the packed array (8 bytes per edge) stays in the L2/MALL while the
//    sources stream through.  Sources are handed out by an atomic counter.
//  * The result row is transformed back (step 4) while it is written out,
//    coalesced, straight from LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "apsp.h"
#include "detail.h"

namespace {

constexpr int kSsspThreads = 512;           // per-source search workgroup
constexpr int kSsspWaves = kSsspThreads / 64;
#ifndef APSP_JO_MAX_QCAP
#define APSP_JO_MAX_QCAP 4096
#endif
constexpr int kMaxQcap = APSP_JO_MAX_QCAP;  // queue entries
constexpr int kQueueBytes = 6;              // LDS per queue entry: vertex + half a hub slot
constexpr uint32_t kUnreached = 0xFFFFFFFFu;
constexpr int kBfRoundsPerCheck = 8;
#ifndef APSP_JO_HUB_UNROLL
#define APSP_JO_HUB_UNROLL 4
#endif
constexpr int kHubUnroll = APSP_JO_HUB_UNROLL;  // edge loads in flight per lane on a hub
#ifndef APSP_JO_HUB_MUL
#define APSP_JO_HUB_MUL 8     // a hub has more than APSP_JO_HUB_MUL * G edges
#endif
#ifndef APSP_JO_ENTRIES
#define APSP_JO_ENTRIES 2     // queued vertices a lane group relaxes at a time
#endif
#ifndef APSP_JO_G
#define APSP_JO_G 0           // lanes per edge chunk; 0 = by average degree
#endif
#ifndef APSP_JO_FORCE_GD
#define APSP_JO_FORCE_GD 0    // 1: distances in global memory even when the row fits LDS
#endif
#ifndef APSP_JO_WG_PER_CU
#define APSP_JO_WG_PER_CU 0   // search workgroups per CU; 0 = as many as LDS allows (<= 2)
#endif

// Device flag bits.
constexpr int32_t kBadCsr = 1;        // malformed CSR or a weight outside (-inf, inf)
constexpr int32_t kHasNegative = 2;   // some edge weight < 0
constexpr int32_t kOutOfRange = 4;    // a potential or a result outside (-inf, inf)
constexpr int32_t kNegReweight = 8;   // a reweighted edge < 0 (cannot happen without a cycle)
constexpr int32_t kIterCap = 16;      // a search hit its step limit (cannot happen for w' >= 0)

struct Stats {
  int32_t flags;
  uint32_t max_w;              // largest reweighted edge
  unsigned long long sum_w;    // sum of reweighted edges
  int32_t work;                // next source to hand out
  int32_t pad;
  unsigned long long steps;    // search steps, summed over sources
  unsigned long long removed;  // vertices removed from the marks, summed
  unsigned long long edges;    // edge relaxations, summed
};

// ---------------------------------------------------------------------------
// Validation: row_ptr[0] = 0, non-decreasing, row_ptr[n] = nnz; targets in
// [0, n); weights in (-inf, inf).  Also records whether any weight is < 0.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) jo_check(const int64_t* __restrict__ row_ptr,
                                                const int32_t* __restrict__ col,
                                                const int32_t* __restrict__ w, int64_t n,
                                                int64_t nnz, int32_t inf, Stats* st) {
  int32_t fl = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t u = t0; u <= n; u += stride) {
    const int64_t a = row_ptr[u];
    if (u == 0 && a != 0) fl |= kBadCsr;
    if (u == n && a != nnz) fl |= kBadCsr;
    if (u < n && row_ptr[u + 1] < a) fl |= kBadCsr;
  }
  for (int64_t e = t0; e < nnz; e += stride) {
    const int32_t c = col[e];
    const int32_t x = w[e];
    if (c < 0 || (int64_t)c >= n) fl |= kBadCsr;
    if (x >= inf || x <= -inf) fl |= kBadCsr;
    if (x < 0) fl |= kHasNegative;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) fl |= __shfl_xor(fl, o);
  if ((threadIdx.x & 63) == 0 && fl) atomicOr(&st->flags, fl);
}

__global__ void __launch_bounds__(256) jo_init(int64_t* __restrict__ h64, uint8_t* __restrict__ act,
                                               int32_t* __restrict__ changed, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n + 2; v += stride) {
    if (v < n) {
      h64[v] = 0;
      act[v] = 0;       // parity 0: written by odd rounds
      act[n + v] = 1;   // parity 1: read by round 1 (every vertex was reached from q)
    }
    changed[v] = 0;
  }
}

// One Bellman-Ford round r >= 1: one wave per vertex u with act[r & 1][u].
__global__ void __launch_bounds__(256) jo_bf_round(const int64_t* __restrict__ row_ptr,
                                                   const int32_t* __restrict__ col,
                                                   const int32_t* __restrict__ w, int64_t n,
                                                   int64_t* h64, uint8_t* act,
                                                   int32_t* changed, int64_t r) {
  if (r > 1 && __hip_atomic_load(&changed[r - 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0)
    return;  // the previous round was quiet: converged
  const int64_t u = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x & 63;
  if (u >= n) return;
  uint8_t* cur = act + (r & 1) * n;
  uint8_t* nxt = act + ((r + 1) & 1) * n;
  if (cur[u] == 0) return;
  const int64_t hu = __hip_atomic_load(&h64[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (lane == 0) cur[u] = 0;
  const int64_t e1 = row_ptr[u + 1];
  bool any = false;
  for (int64_t e = row_ptr[u] + lane; e < e1; e += 64) {
    const int32_t v = col[e];
    const int64_t cand = hu + (int64_t)w[e];
    if (cand < __hip_atomic_load(&h64[v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
      const long long old = atomicMin(reinterpret_cast<long long*>(&h64[v]), (long long)cand);
      if (cand < old) {
        nxt[v] = 1;
        any = true;
      }
    }
  }
  if (any) changed[r] = 1;
}

// h (int32) from the int64 potentials; a potential <= -inf is out of range.
__global__ void __launch_bounds__(256) jo_potentials(const int64_t* __restrict__ h64,
                                                     int32_t* __restrict__ h32,
                                                     int32_t* __restrict__ h_out, int64_t n,
                                                     int32_t inf, Stats* st) {
  int32_t fl = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n; v += stride) {
    int64_t x = h64[v];
    if (x <= -(int64_t)inf) {
      fl |= kOutOfRange;
      x = 0;
    }
    h32[v] = (int32_t)x;
    if (h_out) h_out[v] = (int32_t)x;
  }
  if (fl) atomicOr(&st->flags, fl);
}

// w'(u, v) = w + h(u) - h(v), packed with its target; one wave per vertex.
__global__ void __launch_bounds__(256) jo_reweight(const int64_t* __restrict__ row_ptr,
                                                   const int32_t* __restrict__ col,
                                                   const int32_t* __restrict__ w, int64_t n,
                                                   const int32_t* __restrict__ h32,
                                                   int2* __restrict__ ew, Stats* st) {
  const int64_t u = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x & 63;
  uint32_t mx = 0;
  unsigned long long sum = 0;
  int32_t fl = 0;
  if (u < n) {
    const int64_t hu = h32[u];
    const int64_t e1 = row_ptr[u + 1];
    for (int64_t e = row_ptr[u] + lane; e < e1; e += 64) {
      const int32_t v = col[e];
      int64_t x = (int64_t)w[e] + hu - (int64_t)h32[v];
      if (x < 0) {
        fl |= kNegReweight;
        x = 0;
      }
      if (x > 0x7FFFFFFF) {
        fl |= kOutOfRange;
        x = 0x7FFFFFFF;
      }
      ew[e] = make_int2(v, (int32_t)x);
      mx = max(mx, (uint32_t)x);
      sum += (unsigned long long)x;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    sum += __shfl_xor(sum, o);
    fl |= __shfl_xor(fl, o);
  }
  if (lane == 0) {
    if (mx) atomicMax(&st->max_w, mx);
    if (sum) atomicAdd(&st->sum_w, sum);
    if (fl) atomicOr(&st->flags, fl);
  }
}

// ---------------------------------------------------------------------------
// Per-source search (steps 3 and 4).  A step is remove -> relax -> hubs,
// with a barrier after each:
//   remove   marked vertices with distance <= T leave the bitmap for the
//            queue (at most qcap per step; the rest stay marked);
//   relax    each group of G lanes fetches the adjacency [row_ptr[u],
//            row_ptr[u+1]) of a queued vertex and relaxes it whole when it
//            has up to 8G edges, two vertices at a time (up to 8 edge loads
//            in flight per lane, then strides of G); a longer adjacency (a
//            hub) is listed;
//   hubs     one wave per listed hub, the waves in parallel.
// Dynamic LDS (32-bit words): dist[n4] tentative distances (kUnreached = not
// reached), mark[nw4] the bitmap of vertices whose distance dropped since
// they were last removed, qv[qcap] the queued vertices and big[qcap / 2]
// the queue positions of the hubs.  With the list full, a hub's group
// relaxes the rest of it.  Fetching the ranges inside the relax loop
// instead of in a phase of their own keeps the queue at 6 bytes per entry,
// so more vertices fit a step (BA-16000: 38 steps per source instead of 48).
// Held to four waves per SIMD (<= 128 VGPRs) so that two 512-thread
// workgroups share a CU; wider unrolling of the hub loop crossed that limit
// and halved the throughput.
// ---------------------------------------------------------------------------
//
// GD (a row too long for LDS): the tentative distances live in the source's
// own output row in global memory instead, reinterpreted as uint32 until
// the row is transformed back.  Only this workgroup touches that row; its
// reads are L2-coherent atomic loads (an L1 line could be stale after
// another wave's L2 atomic) and its updates L2 atomics.  The bitmap and the
// queue stay in LDS.
template <int G, bool GD>
__global__ void __launch_bounds__(kSsspThreads) __attribute__((amdgpu_waves_per_eu(4)))
jo_sssp(const int64_t* __restrict__ row_ptr, const int2* __restrict__ ew, int32_t n,
         const int32_t* __restrict__ h32, int32_t* __restrict__ d, int64_t ld, int32_t inf,
         uint32_t delta, int32_t qcap, int64_t step_cap, Stats* st) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const int32_t n4 = (n + 3) & ~3;
  const int32_t nw = (n + 31) >> 5;
  const int32_t nw4 = (nw + 3) & ~3;
  uint32_t* dist = smem;  // GD: set to the source's row below
  uint32_t* mark = smem + (GD ? 0 : n4);
  uint32_t* qv = mark + nw4;
  uint32_t* big = qv + qcap;
  const uint32_t hcap = (uint32_t)qcap / 2;
  __shared__ uint32_t ctl[2][4];  // per step parity: queue count, smallest marked distance > T, hubs
  __shared__ int32_t s_src;
  constexpr uint32_t kBig = APSP_JO_HUB_MUL * G;
  constexpr uint32_t kGroups = kSsspThreads / G;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const uint32_t grp = (uint32_t)(tid / G), gl = (uint32_t)(tid % G);
  int32_t err = 0;
  unsigned long long n_steps = 0, n_removed = 0, n_edges = 0;

  auto dget = [&](uint32_t v) -> uint32_t {
    if constexpr (GD) return __hip_atomic_load(&dist[v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return dist[v];
  };
  auto dset = [&](uint32_t v, uint32_t x) {
    if constexpr (GD) __hip_atomic_store(&dist[v], x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else dist[v] = x;
  };
  auto relax = [&](uint32_t du, int2 x) {
    const uint32_t v = (uint32_t)x.x;
    uint32_t nd = du + (uint32_t)x.y;
    if (nd < du) nd = kUnreached;  // saturate instead of wrapping
    if (nd < dget(v)) {
      const uint32_t old = atomicMin(&dist[v], nd);
      if (nd < old) atomicOr(&mark[v >> 5], 1u << (v & 31));
    }
  };

  for (;;) {
    if (tid == 0) s_src = atomicAdd(&st->work, 1);
    __syncthreads();
    const int32_t s = s_src;
    if (s >= n) break;
    if constexpr (GD) dist = reinterpret_cast<uint32_t*>(d + (int64_t)s * ld);

    for (int32_t v = tid; v < n; v += kSsspThreads) dset(v, kUnreached);
    for (int32_t x = tid; x < nw; x += kSsspThreads) mark[x] = 0;
    if (tid < 8) ctl[tid >> 2][tid & 3] = (tid & 3) == 1 ? kUnreached : 0u;
    __syncthreads();
    if (tid == 0) {
      dset(s, 0);
      mark[s >> 5] = 1u << (s & 31);
    }
    __syncthreads();

    uint32_t T = delta;
    int par = 0;
    int64_t steps = 0;
    for (;;) {
      // -- remove ---------------------------------------------------------
      uint32_t lmin = kUnreached;
      // Queue slots are claimed once per wave (a scan over the lanes' counts
      // and one LDS atomic), not once per mark word.
      for (int32_t x0 = 0; x0 < nw; x0 += kSsspThreads) {
        const int32_t x = x0 + tid;
        uint32_t bits = 0, take = 0;
        if (x < nw) {
          bits = mark[x];
          for (uint32_t b = bits; b; b &= b - 1) {
            const int i = __builtin_ctz(b);
            const uint32_t dv = dget(x * 32 + i);
            if (dv <= T) take |= 1u << i;
            else lmin = min(lmin, dv);
          }
        }
        const uint32_t c = (uint32_t)__builtin_popcount(take);
        uint32_t incl = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t y = (uint32_t)__shfl_up((int)incl, o);
          if (lane >= o) incl += y;
        }
        const uint32_t wtot = (uint32_t)__shfl((int)incl, 63);
        if (wtot == 0) continue;
        uint32_t wbase = 0;
        if (lane == 63) wbase = atomicAdd(&ctl[par][0], wtot);
        wbase = (uint32_t)__shfl((int)wbase, 63);
        if (take == 0) continue;
        const uint32_t base = wbase + incl - c;
        if (base >= (uint32_t)qcap) continue;
        uint32_t k = base, kept = 0;
        for (uint32_t b = take; b && k < (uint32_t)qcap; b &= b - 1) {
          const int i = __builtin_ctz(b);
          qv[k++] = x * 32 + i;
          kept |= 1u << i;
        }
        mark[x] = bits & ~kept;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) lmin = min(lmin, (uint32_t)__shfl_xor((int)lmin, o));
      if (lane == 0 && lmin != kUnreached) atomicMin(&ctl[par][1], lmin);
      __syncthreads();
      const uint32_t qn = min(ctl[par][0], (uint32_t)qcap);
      const uint32_t smin = ctl[par][1];
      if (tid == 0) {
        ctl[par ^ 1][0] = 0;
        ctl[par ^ 1][1] = kUnreached;
        ctl[par ^ 1][2] = 0;
        n_steps += 1;
        n_removed += qn;
      }
      if (++steps > step_cap) {
        err |= kIterCap;
        __syncthreads();
        break;
      }
      if (qn == 0) {
        if (smin == kUnreached) break;
        T = smin > kUnreached - 1 - delta ? kUnreached - 1 : smin + delta;
        par ^= 1;
        __syncthreads();
        continue;
      }

      // -- relax: each group fetches its vertices' edge ranges itself --------
      // A hub (more than kBig edges) goes to the hub list for a whole wave;
      // when the list is full, its group relaxes it like any other: four
      // loads per lane, then the rest in strides of G.
      constexpr int kE = APSP_JO_ENTRIES;
      for (uint32_t i0 = grp; i0 < qn; i0 += kE * kGroups) {
        int2 x[kE][4];
        uint32_t du[kE], rest_a[kE], rest_b[kE];
        bool ok[kE][4];
#pragma unroll
        for (int m = 0; m < kE; ++m) {
          const uint32_t i = i0 + m * kGroups;
          uint32_t a = 0, b = 0;
          rest_a[m] = rest_b[m] = 0;
          if (i < qn) {
            const uint32_t u = qv[i];
            a = (uint32_t)row_ptr[u];
            b = (uint32_t)row_ptr[u + 1];
            if (gl == 0) n_edges += b - a;
            if (b - a > kBig) {
              uint32_t slot = 0;
              if (gl == 0) slot = atomicAdd(&ctl[par][2], 1u);
              slot = (uint32_t)__shfl((int)slot, lane - (int)gl);
              if (slot < hcap) {
                if (gl == 0) big[slot] = i;
                b = a;  // relaxed by a wave below
              }
            }
            if (b - a > 4 * G) {  // the group's four loads per lane, then strides
              rest_a[m] = a + 4 * G;
              rest_b[m] = b;
              b = a + 4 * G;
            }
            du[m] = dget(u);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t e = a + gl + j * G;
            ok[m][j] = e < b;
            if (ok[m][j]) x[m][j] = ew[e];
          }
        }
#pragma unroll
        for (int m = 0; m < kE; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (ok[m][j]) relax(du[m], x[m][j]);
#pragma unroll
        for (int m = 0; m < kE; ++m)
          for (uint32_t e = rest_a[m] + gl; e < rest_b[m]; e += G) relax(du[m], ew[e]);
      }
      __syncthreads();
      const uint32_t nbig = min(ctl[par][2], hcap);
      par ^= 1;
      // -- hubs: one wave per long adjacency, the waves in parallel -----------
      for (uint32_t h = (uint32_t)(tid >> 6); h < nbig; h += kSsspWaves) {
        const uint32_t u = qv[big[h]];
        const uint32_t a = (uint32_t)row_ptr[u], b = (uint32_t)row_ptr[u + 1];
        const uint32_t du = dget(u);
        for (uint32_t e0 = a + (uint32_t)lane; e0 < b; e0 += kHubUnroll * 64) {
          int2 x[kHubUnroll];
          bool ok[kHubUnroll];
#pragma unroll
          for (int j = 0; j < kHubUnroll; ++j) {
            const uint32_t e = e0 + j * 64;
            ok[j] = e < b;
            if (ok[j]) x[j] = ew[e];
          }
#pragma unroll
          for (int j = 0; j < kHubUnroll; ++j)
            if (ok[j]) relax(du, x[j]);
        }
      }
      __syncthreads();
    }

    const int64_t hs = h32[s];
    int32_t* row = d + (int64_t)s * ld;
    for (int32_t v = tid; v < n; v += kSsspThreads) {
      const uint32_t dv = dget(v);  // GD: the same word as row[v], read before it is written
      int32_t out = inf;
      if (dv != kUnreached) {
        const int64_t x = (int64_t)dv + (int64_t)h32[v] - hs;
        if (x >= inf || x <= -(int64_t)inf) err |= kOutOfRange;
        else out = (int32_t)x;
      }
      row[v] = out;
    }
    __syncthreads();
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    err |= __shfl_xor(err, o);
    n_edges += __shfl_xor(n_edges, o);
  }
  if (lane == 0) {
    if (err) atomicOr(&st->flags, err);
    if (n_edges) atomicAdd(&st->edges, n_edges);
  }
  if (tid == 0 && n_steps) {
    atomicAdd(&st->steps, n_steps);
    atomicAdd(&st->removed, n_removed);
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
struct Timing {
  hipEvent_t ev[8] = {};
  bool on = false;
};

constexpr int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

int device_lds_limits(int* per_block, int* per_cu, int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return APSP_ERR_NO_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return APSP_ERR_NO_DEVICE;
  *per_block = (int)prop.sharedMemPerBlock;
  *per_cu = (int)prop.maxSharedMemoryPerMultiProcessor;
  if (*per_cu < *per_block) *per_cu = *per_block;
  *cus = prop.multiProcessorCount;
  return APSP_OK;
}

// A failed HIP call: keep its error for apsp_last_hip_error.
int hip_failed() {
  (void)apsp_detail_launch_status();
  return APSP_ERR_LAUNCH;
}

template <int G>
int launch_sssp(const int64_t* row_ptr, const int2* ew, int32_t n, const int32_t* h32, int32_t* d,
                int64_t ld, int32_t inf, uint32_t delta, int32_t qcap, size_t lds, int grid,
                bool gd, Stats* st, hipStream_t s) {
  const void* fn = gd ? reinterpret_cast<const void*>(&jo_sssp<G, true>)
                      : reinterpret_cast<const void*>(&jo_sssp<G, false>);
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return hip_failed();
  const int64_t step_cap = 64 * (int64_t)n + 4096;
  if (gd)
    hipLaunchKernelGGL((jo_sssp<G, true>), dim3(grid), dim3(kSsspThreads), lds, s, row_ptr, ew, n, h32,
                       d, ld, inf, delta, qcap, step_cap, st);
  else
    hipLaunchKernelGGL((jo_sssp<G, false>), dim3(grid), dim3(kSsspThreads), lds, s, row_ptr, ew, n,
                       h32, d, ld, inf, delta, qcap, step_cap, st);
  return apsp_detail_launch_status();
}

int sync_read(hipStream_t s, void* host, const void* dev, size_t bytes) {
  if (hipMemcpyAsync(host, dev, bytes, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return hip_failed();
  return APSP_OK;
}

int run_johnson(const int64_t* row_ptr, const int32_t* col, const int32_t* w, int64_t n,
                int64_t nnz, int32_t* d, int64_t ld, int32_t inf, int32_t* h_out, int32_t delta,
                void* stream, double* phase_ms, int64_t* counts) {
  if (phase_ms)
    for (int i = 0; i < 4; ++i) phase_ms[i] = 0.0;
  if (counts)
    for (int i = 0; i < 4; ++i) counts[i] = 0;
  if (n < 0 || nnz < 0) return APSP_ERR_INVALID_VALUE;
  if (n == 0) return APSP_OK;
  if (n > 0x7FFFFFFE || nnz > 0x7FFFFFFF) return APSP_ERR_INVALID_VALUE;
  if (row_ptr == nullptr || d == nullptr || (nnz > 0 && (col == nullptr || w == nullptr)))
    return APSP_ERR_INVALID_VALUE;
  if (ld < n || ld > INT64_MAX / 4 / n) return APSP_ERR_INVALID_VALUE;
  if (inf < 1 || inf > 0x3FFFFFFF) return APSP_ERR_INVALID_VALUE;
  if (reinterpret_cast<uintptr_t>(row_ptr) % 8 || reinterpret_cast<uintptr_t>(col) % 4 ||
      reinterpret_cast<uintptr_t>(w) % 4 || reinterpret_cast<uintptr_t>(d) % 4 ||
      reinterpret_cast<uintptr_t>(h_out) % 4)
    return APSP_ERR_INVALID_VALUE;
  int st = apsp_detail_check_device();
  if (st != APSP_OK) return st;

  // LDS for one search workgroup: the row, the bitmap and the queue.
  int lds_block = 0, lds_cu = 0, cus = 0;
  st = device_lds_limits(&lds_block, &lds_cu, &cus);
  if (st != APSP_OK) return st;
  const int64_t n4 = (n + 3) & ~int64_t(3);
  const int64_t nw4 = (((n + 31) >> 5) + 3) & ~int64_t(3);
  int32_t qcap = 0;
  int per_cu = 0;
  bool gd = false;
  // Two 512-thread search workgroups fit a CU by registers (four waves per
  // SIMD); LDS decides between two and one.  A row that does not fit at all
  // moves to global memory (GD), leaving the bitmap and the queue in LDS.
  for (int pass = APSP_JO_FORCE_GD; pass < 2 && qcap == 0; ++pass) {
    gd = pass == 1;
    const int64_t fixed = 4 * ((gd ? 0 : n4) + nw4) + 1024;  // + static LDS and slack
    for (int k = APSP_JO_WG_PER_CU ? APSP_JO_WG_PER_CU : 2; k >= 1 && qcap == 0; k /= 2) {
      const int64_t budget = std::min<int64_t>(lds_cu / k, lds_block);
      const int64_t q = std::min<int64_t>(kMaxQcap, (budget - fixed) / kQueueBytes) & ~int64_t(63);
      if (q >= 256 || (k == 1 && q >= 64)) {
        qcap = (int32_t)q;
        per_cu = k;
      }
    }
  }
  if (qcap == 0) return APSP_ERR_RANGE;  // not even the bitmap fits in one workgroup's LDS
  const size_t lds = (size_t)(4 * ((gd ? 0 : n4) + nw4) + (int64_t)kQueueBytes * qcap);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t off_stats = 0;
  const int64_t off_h64 = align256(sizeof(Stats));
  const int64_t off_h32 = off_h64 + align256(8 * n);
  const int64_t off_act = off_h32 + align256(4 * n);
  const int64_t off_chg = off_act + align256(2 * n);
  const int64_t off_ew = off_chg + align256(4 * (n + 2));
  const int64_t bytes = off_ew + align256(8 * std::max<int64_t>(nnz, 1));
  char* scratch = nullptr;
  if (hipMallocAsync(reinterpret_cast<void**>(&scratch), (size_t)bytes, s) != hipSuccess)
    return hip_failed();
  Stats* dst = reinterpret_cast<Stats*>(scratch + off_stats);
  int64_t* h64 = reinterpret_cast<int64_t*>(scratch + off_h64);
  int32_t* h32 = reinterpret_cast<int32_t*>(scratch + off_h32);
  uint8_t* act = reinterpret_cast<uint8_t*>(scratch + off_act);
  int32_t* changed = reinterpret_cast<int32_t*>(scratch + off_chg);
  int2* ew = reinterpret_cast<int2*>(scratch + off_ew);

  Timing tm;
  if (phase_ms) {
    tm.on = true;
    for (auto& e : tm.ev)
      if (hipEventCreate(&e) != hipSuccess) tm.on = false;
  }
  auto mark = [&](int i) {
    if (tm.on) (void)hipEventRecord(tm.ev[i], s);
  };

  int rc = APSP_OK;
  Stats hs{};
  const unsigned vgrid = (unsigned)std::min<int64_t>((n + 3) / 4, int64_t(1) << 30);
  const unsigned egrid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((std::max(nnz, n + 1) + 255) / 256, 4096));
  do {
    // 1. validate the graph
    mark(0);
    (void)hipMemsetAsync(dst, 0, sizeof(Stats), s);
    hipLaunchKernelGGL(jo_check, dim3(egrid), dim3(256), 0, s, row_ptr, col, w, n, nnz, inf, dst);
    hipLaunchKernelGGL(jo_init, dim3((unsigned)std::min<int64_t>((n + 257) / 256, 4096)), dim3(256),
                       0, s, h64, act, changed, n);
    mark(1);
    if ((rc = apsp_detail_launch_status()) != APSP_OK) break;
    if ((rc = sync_read(s, &hs, dst, sizeof(Stats))) != APSP_OK) break;
    if (hs.flags & kBadCsr) {
      rc = APSP_ERR_INVALID_VALUE;
      break;
    }

    // 2. potentials: Bellman-Ford from the added vertex (skipped when no
    //    weight is negative: then h = 0 is already the answer)
    mark(2);
    int64_t rounds = 0;
    if (hs.flags & kHasNegative) {
      int32_t last = 1;
      while (rounds < n && last != 0) {
        const int64_t r_end = std::min<int64_t>(n, rounds + kBfRoundsPerCheck);
        for (int64_t r = rounds + 1; r <= r_end; ++r)
          hipLaunchKernelGGL(jo_bf_round, dim3(vgrid), dim3(256), 0, s, row_ptr, col, w, n, h64,
                             act, changed, r);
        if ((rc = apsp_detail_launch_status()) != APSP_OK) break;
        rounds = r_end;
        if ((rc = sync_read(s, &last, changed + rounds, sizeof(int32_t))) != APSP_OK) break;
      }
      if (rc != APSP_OK) break;
      if (last != 0) {  // round n still relaxed an edge
        rc = APSP_ERR_NEGATIVE_CYCLE;
        if (counts) counts[0] = rounds;
        break;
      }
    }
    if (counts) counts[0] = rounds;
    hipLaunchKernelGGL(jo_potentials, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 4096)),
                       dim3(256), 0, s, h64, h32, h_out, n, inf, dst);
    mark(3);

    // 3. reweight and pack the edges
    mark(4);
    hipLaunchKernelGGL(jo_reweight, dim3(vgrid), dim3(256), 0, s, row_ptr, col, w, n, h32, ew, dst);
    mark(5);
    if ((rc = apsp_detail_launch_status()) != APSP_OK) break;
    if ((rc = sync_read(s, &hs, dst, sizeof(Stats))) != APSP_OK) break;
    if (hs.flags & kOutOfRange) {
      rc = APSP_ERR_RANGE;
      break;
    }
    if (hs.flags & kNegReweight) {  // impossible once Bellman-Ford converged
      rc = APSP_ERR_NEGATIVE_CYCLE;
      break;
    }

    // 4. a search from every source, rows transformed back as they are written
    uint32_t dl = 0;
    if (delta >= 0) {
      dl = (uint32_t)delta;
    }
    const double avg_deg = std::max(1.0, (double)nnz / (double)n);
    if (delta < 0) {
      // Automatic: six mean reweighted edges per average degree (the width
      // shrinks as more edges leave each vertex, as in delta-stepping's
      // analysis).  Measured on the sparse workloads (BA n = 16000, ER n =
      // 2048 and n = 8192) this lies within a few percent of the fastest
      // width of a sweep from 16 to 256.
      const double mean = nnz > 0 ? (double)hs.sum_w / (double)nnz : 1.0;
      dl = (uint32_t)std::min(1e9, std::max(1.0, 6.0 * mean / avg_deg));
    }
    const int grid = (int)std::min<int64_t>(n, (int64_t)cus * per_cu);
    mark(6);
    // Lanes per adjacency: short adjacencies (<= 8G edges) go to groups of G
    // lanes, longer ones to whole waves; G = 8 up to an average degree of 32,
    // then the smallest power of two with 4G >= the average degree.
    const int gsel = APSP_JO_G       ? APSP_JO_G
                     : avg_deg <= 32.0  ? 8
                     : avg_deg <= 64.0  ? 16
                     : avg_deg <= 128.0 ? 32
                                        : 64;
    if (gsel == 4)
      rc = launch_sssp<4>(row_ptr, ew, (int32_t)n, h32, d, ld, inf, dl, qcap, lds, grid, gd, dst, s);
    else if (gsel == 8)
      rc = launch_sssp<8>(row_ptr, ew, (int32_t)n, h32, d, ld, inf, dl, qcap, lds, grid, gd, dst, s);
    else if (gsel == 16)
      rc = launch_sssp<16>(row_ptr, ew, (int32_t)n, h32, d, ld, inf, dl, qcap, lds, grid, gd, dst, s);
    else if (gsel == 32)
      rc = launch_sssp<32>(row_ptr, ew, (int32_t)n, h32, d, ld, inf, dl, qcap, lds, grid, gd, dst, s);
    else
      rc = launch_sssp<64>(row_ptr, ew, (int32_t)n, h32, d, ld, inf, dl, qcap, lds, grid, gd, dst, s);
    mark(7);
    if (rc != APSP_OK) break;
    if ((rc = sync_read(s, &hs, dst, sizeof(Stats))) != APSP_OK) break;
    if (hs.flags & kOutOfRange) rc = APSP_ERR_RANGE;
    else if (hs.flags & kIterCap) rc = APSP_ERR_LAUNCH;
    if (counts) {
      counts[1] = (int64_t)hs.steps;
      counts[2] = (int64_t)hs.removed;
      counts[3] = (int64_t)hs.edges;
    }
  } while (false);

  (void)hipStreamSynchronize(s);
  if (tm.on) {
    if (rc == APSP_OK) {
      for (int i = 0; i < 4; ++i) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, tm.ev[2 * i], tm.ev[2 * i + 1]) == hipSuccess)
          phase_ms[i] = ms;
      }
    }
    for (auto& e : tm.ev) (void)hipEventDestroy(e);
  }
  (void)hipFreeAsync(scratch, s);
  (void)hipStreamSynchronize(s);
  return rc;
}

}  // namespace

extern "C" {

int apsp_johnson_i32(const int64_t* row_ptr, const int32_t* col, const int32_t* w, int64_t n,
                     int64_t nnz, int32_t* d, int64_t ld, int32_t inf, int32_t* h,
                     int32_t delta, void* stream) {
  return run_johnson(row_ptr, col, w, n, nnz, d, ld, inf, h, delta, stream, nullptr, nullptr);
}

int apsp_johnson_timed_i32(const int64_t* row_ptr, const int32_t* col, const int32_t* w,
                           int64_t n, int64_t nnz, int32_t* d, int64_t ld, int32_t inf,
                           int32_t* h, int32_t delta, void* stream, double* phase_ms,
                           int64_t* counts) {
  double local[4];
  return run_johnson(row_ptr, col, w, n, nnz, d, ld, inf, h, delta, stream,
                     phase_ms ? phase_ms : local, counts);
}

}  // extern "C"
