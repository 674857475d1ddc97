// Path reconstruction: the successor (first-hop) matrix of all-pairs
// shortest paths, from the weights and the final distances.
//
// For i != j, nxt[i][j] is the smallest vertex u != i that minimises
// w(i, u) + d(u, j) -- the first hop of a shortest path, by Bellman's
// equation d(i, j) = min over u != i of w(i, u) + d(u, j) (a shortest path
// from i leaves i through some first edge).  nxt[i][i] = i, and -1 where j is
// unreachable from i.  This is the relaxation RelaxEdge of the page
// "Johnson's APSP in Glushkov algorithmic algebras" applied once more to the
// final distances, keeping the argument of the minimum; the result does not
// depend on the order in which the blocked rounds found the distances, so it
// is unique.  Following nxt from i reaches j along a path of total weight
// d(i, j) when every weight is positive (each hop lowers the remaining
// distance).
//
// gfx950 design: the min-plus product W (x) D of the product kernel
// (gemm.hip) with the minimum's argument tracked: a 256-thread workgroup owns
// a 128 x 128 tile of (value, index) pairs as 8 x 8 micro-tiles in
// registers, W's rows and D's rows stream through LDS in 16-deep chunks
// (double buffered), u runs in increasing order and a candidate replaces the
// pair only when strictly smaller, so the smallest u wins ties.  W[i][i] is
// staged as inf (u != i).  Per candidate: add, compare, two selects.  For
// int32 inputs in a bounded range a second dense kernel packs value and index
// into one key and runs at the min-plus product's instruction count (see
// successors_packed); the range is checked on the device.
//
// Sparse weights.  Only u with w(i, u) < inf can win (any other candidate is
// >= inf and never replaces the running value, which starts at inf), so for
// a matrix with at most n^2 / 16 finite off-diagonal weights a second kernel
// tries only the neighbours of i: one workgroup per row gathers the row's
// neighbours into LDS in increasing u (2048 at a time), then streams row u
// of D for each of them, 4 columns per thread, with the same strict
// comparison.  The result is the same matrix.  A row with more neighbours
// takes several gathers; between them the running value of a column is
// recomputed from the stored index with the same single add.  A count kernel
// adds up the finite weights into 8 bytes of stream-ordered scratch, and both
// kernels read it and return at once unless they are the one for this
// matrix, so the choice costs no host synchronisation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "apsp.h"
#include "detail.h"
#include "minplus.h"

namespace {

using namespace apsp_dev;

constexpr int kT = 128;
constexpr int kThreads = 256;
constexpr int kR = 8;
constexpr int kThr = kT / kR;
constexpr int kKC = 16;
constexpr int kLd = kT + 4;
constexpr int kGroupStride = kT / (kR / 4);
constexpr int kLoads = kT * kKC / 4 / kThreads;

template <typename T, bool VEC>
__device__ __forceinline__ void ld4(const T* __restrict__ p, int64_t ld, int64_t rows, int64_t cols,
                                    int64_t r, int64_t c, T inf, T (&v)[4]) {
  const T* q = p + r * ld + c;
  if (r < rows && c + 3 < cols) {
    if (VEC) {
      load4(q, v);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = q[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (r < rows && c + e < cols) ? q[e] : inf;
  }
}

// Device-side facts that choose the kernel: the number of finite
// off-diagonal weights, and the range of the finite weights and distances.
struct SuccStats {
  unsigned long long edges;
  int32_t wmin, wmax, dmin, dmax;
};

template <typename T>
__device__ __forceinline__ void wave_minmax(int32_t& lo, int32_t& hi) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = min(lo, __shfl_xor(lo, o));
    hi = max(hi, __shfl_xor(hi, o));
  }
}

// The statistics scans leave one partial per workgroup (no same-address
// atomics: thousands of them serialise in L2) and one workgroup folds them.
constexpr int kStatParts = 1024;

// (c, lo, hi) summed / ranged over the workgroup; thread 0 holds the result.
__device__ __forceinline__ void block_stats(unsigned long long& c, int32_t& lo, int32_t& hi) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  wave_minmax<int32_t>(lo, hi);
  __shared__ unsigned long long sc[16];
  __shared__ int32_t slo[16], shi[16];
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sc[wv] = c; slo[wv] = lo; shi[wv] = hi; }
  __syncthreads();
  if (threadIdx.x == 0)
    for (int k = 1; k < (int)(blockDim.x >> 6); ++k) {
      c += sc[k];
      lo = min(lo, slo[k]);
      hi = max(hi, shi[k]);
    }
}

// Visits row r's entries (c, v) of an n x n matrix, 16-byte quads with four
// in flight per thread when VEC (16-byte aligned rows), else one at a time.
template <typename T, bool VEC, typename F>
__device__ __forceinline__ void scan_row(const T* __restrict__ row, int64_t n, F&& visit) {
  const int64_t full = VEC ? n / 4 : 0;  // quads wholly inside the row
  int64_t q = threadIdx.x;
  for (; q + 3 * blockDim.x < full; q += 4 * blockDim.x) {
    T v[4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) load4(row + (q + k * blockDim.x) * 4, v[k]);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) visit((q + k * blockDim.x) * 4 + e, v[k][e]);
  }
  for (; q < full; q += blockDim.x) {
    T v[4];
    load4(row + q * 4, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) visit(q * 4 + e, v[e]);
  }
  for (int64_t c = full * 4 + threadIdx.x; c < n; c += blockDim.x) visit(c, row[c]);
}

// The finite off-diagonal weights w[i][u] < inf, u != i: their number and,
// for int32, their range.
template <typename T, bool VEC>
__global__ void __launch_bounds__(256) succ_count(const T* __restrict__ W, int64_t ldw, int64_t n,
                                                  T inf, SuccStats* __restrict__ part) {
  uint32_t c = 0;
  int32_t lo = INT32_MAX, hi = INT32_MIN;
  for (int64_t i = blockIdx.x; i < n; i += gridDim.x)
    scan_row<T, VEC>(W + i * ldw, n, [&](int64_t u, T v) {
      const bool f = u != i && v < inf;
      c += f;
      if constexpr (std::is_same_v<T, int32_t>) {
        lo = f ? min(lo, v) : lo;
        hi = f ? max(hi, v) : hi;
      }
    });
  unsigned long long cc = c;
  block_stats(cc, lo, hi);
  if (threadIdx.x == 0) {
    part[blockIdx.x].edges = cc;
    part[blockIdx.x].wmin = lo;
    part[blockIdx.x].wmax = hi;
  }
}

// The range of the finite distances (int32, dense graphs only).
template <bool VEC>
__global__ void __launch_bounds__(256) succ_dstats(const int32_t* __restrict__ D, int64_t ldd,
                                                   int64_t n, int32_t inf,
                                                   const SuccStats* __restrict__ st,
                                                   SuccStats* __restrict__ part,
                                                   unsigned long long max_sparse) {
  if (st->edges <= max_sparse) return;  // the sparse kernel takes this matrix
  int32_t lo = INT32_MAX, hi = INT32_MIN;
  for (int64_t u = blockIdx.x; u < n; u += gridDim.x)
    scan_row<int32_t, VEC>(D + u * ldd, n, [&](int64_t, int32_t v) {
      const bool f = v < inf;
      lo = f ? min(lo, v) : lo;
      hi = f ? max(hi, v) : hi;
    });
  unsigned long long none = 0;
  block_stats(none, lo, hi);
  if (threadIdx.x == 0) {
    part[blockIdx.x].dmin = lo;
    part[blockIdx.x].dmax = hi;
  }
}

// Folds the first `parts` partials into *st: the weight statistics (DIST
// false), or the distance range of a dense matrix (DIST true).
template <bool DIST>
__global__ void __launch_bounds__(256) succ_fold(const SuccStats* __restrict__ part, int parts,
                                                 SuccStats* __restrict__ st,
                                                 unsigned long long max_sparse) {
  if (DIST && st->edges <= max_sparse) return;
  unsigned long long c = 0;
  int32_t lo = INT32_MAX, hi = INT32_MIN;
  for (int k = threadIdx.x; k < parts; k += blockDim.x) {
    c += DIST ? 0 : part[k].edges;
    lo = min(lo, DIST ? part[k].dmin : part[k].wmin);
    hi = max(hi, DIST ? part[k].dmax : part[k].wmax);
  }
  block_stats(c, lo, hi);
  if (threadIdx.x == 0) {
    if (DIST) {
      st->dmin = lo;
      st->dmax = hi;
    } else {
      *st = SuccStats{c, lo, hi, INT32_MAX, INT32_MIN};
    }
  }
}

// Packed keys apply when every finite weight and distance is >= 0 and the
// largest finite weight plus the largest finite distance is below both inf
// and 2^(31 - shift): then (w + d) << shift | u < 2^31 for every finite
// candidate, no finite candidate reaches inf, and 2^31 marks "no edge".
__device__ __forceinline__ bool succ_packable(const SuccStats* st, int32_t inf, int shift) {
  if (st->wmin < 0 || st->dmin < 0) return false;
  const int64_t sum = (int64_t)max(st->wmax, 0) + (int64_t)max(st->dmax, 0);
  return sum < (int64_t)inf && sum < (int64_t(1) << (31 - shift));
}

template <typename T, bool VEC>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
successors(const T* __restrict__ W, int64_t ldw, const T* __restrict__ D, int64_t ldd,
           int32_t* __restrict__ nxt, int64_t ldn, int64_t n, T inf, uint32_t tiles_per_row,
           const SuccStats* __restrict__ st, unsigned long long max_sparse, int shift) {
  if (st->edges <= max_sparse) return;  // the sparse kernel takes this matrix
  if constexpr (std::is_same_v<T, int32_t>)
    if (succ_packable(st, inf, shift)) return;  // the packed kernel takes it
  __shared__ __attribute__((aligned(16))) T lds[4 * kKC * kLd];
  T* sA = lds;                  // [2][kKC][kLd]: sA[t][row] = W[row0 + row][u0 + t]
  T* sB = lds + 2 * kKC * kLd;  // [2][kKC][kLd]: sB[t][col] = D[u0 + t][col0 + col]
  const int tid = threadIdx.x;
  const int tc = tid % kThr, tr = tid / kThr;
  const int64_t row0 = (int64_t)(blockIdx.x / tiles_per_row) * kT;
  const int64_t col0 = (int64_t)(blockIdx.x % tiles_per_row) * kT;

  T val[kR][kR];
  int32_t idx[kR][kR];
#pragma unroll
  for (int i = 0; i < kR; ++i)
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      val[i][j] = inf;
      idx[i][j] = -1;
    }

  T ga[kLoads][4], gb[kLoads][4];
  auto fetch = [&](int64_t u0) {
#pragma unroll
    for (int l = 0; l < kLoads; ++l) {
      const int q = tid + l * kThreads;
      const int r = q / (kKC / 4), uq = q % (kKC / 4);
      ld4<T, VEC>(W, ldw, n, n, row0 + r, u0 + uq * 4, inf, ga[l]);
#pragma unroll
      for (int e = 0; e < 4; ++e)  // u != i: the vertex itself is never its own first hop
        if (row0 + r == u0 + uq * 4 + e) ga[l][e] = inf;
      const int ur = q / (kT / 4), cq = q % (kT / 4);
      ld4<T, VEC>(D, ldd, n, n, u0 + ur, col0 + cq * 4, inf, gb[l]);
    }
  };
  auto stash = [&](int buf) {
    T* a = sA + buf * kKC * kLd;
    T* b = sB + buf * kKC * kLd;
#pragma unroll
    for (int l = 0; l < kLoads; ++l) {
      const int q = tid + l * kThreads;
      const int r = q / (kKC / 4), uq = q % (kKC / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[(uq * 4 + e) * kLd + r] = ga[l][e];
      const int ur = q / (kT / 4), cq = q % (kT / 4);
      store4(b + ur * kLd + cq * 4, gb[l]);
    }
  };

  const int64_t chunks = (n + kKC - 1) / kKC;
  fetch(0);
  stash(0);
  __syncthreads();
#pragma unroll 1
  for (int64_t c = 0; c < chunks; ++c) {
    const int buf = (int)(c & 1);
    if (c + 1 < chunks) fetch((c + 1) * kKC);
    const T* a = sA + buf * kKC * kLd;
    const T* b = sB + buf * kKC * kLd;
    const int32_t u0 = (int32_t)(c * kKC);
#pragma unroll 2
    for (int t = 0; t < kKC; ++t) {
      T av[kR], bv[kR];
#pragma unroll
      for (int gi = 0; gi < kR / 4; ++gi) {
        T v[4];
        load4(a + t * kLd + gi * kGroupStride + tr * 4, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) av[gi * 4 + i] = v[i];
        load4(b + t * kLd + gi * kGroupStride + tc * 4, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[gi * 4 + j] = v[j];
      }
      const int32_t u = u0 + t;
#pragma unroll
      for (int i = 0; i < kR; ++i)
#pragma unroll
        for (int j = 0; j < kR; ++j) {
          const T cand = av[i] + bv[j];
          const bool better = cand < val[i][j];
          val[i][j] = better ? cand : val[i][j];
          idx[i][j] = better ? u : idx[i][j];
        }
    }
    if (c + 1 < chunks) stash(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int gi = 0; gi < kR / 4; ++gi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = row0 + gi * kGroupStride + tr * 4 + i;
      if (r >= n) continue;
#pragma unroll
      for (int gj = 0; gj < kR / 4; ++gj)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t col = col0 + gj * kGroupStride + tc * 4 + j;
          if (col >= n) continue;
          // unreachable: no candidate below inf
          const int32_t s = r == col ? (int32_t)r : (val[gi * 4 + i][gj * 4 + j] < inf ? idx[gi * 4 + i][gj * 4 + j] : -1);
          nxt[r * ldn + col] = s;
        }
    }
}

// Dense successors with packed keys (int32, see succ_packable): the operand
// staged for (i, u) is w(i, u) << shift, for (u, j) it is d(u, j) << shift | u,
// "no edge" (and u = i) is 2^31, and a candidate is their unsigned sum,
// saturated.  Its minimum over u is (the least w + d) << shift | (the
// smallest u that reaches it) -- the same argmin and tie rule as the kernel
// above -- at the instruction cost of the min-plus product: two saturating
// adds and one three-input minimum per pair of candidates.
constexpr uint32_t kNoEdge = 0x80000000u;

template <bool VEC>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
successors_packed(const int32_t* __restrict__ W, int64_t ldw, const int32_t* __restrict__ D,
                  int64_t ldd, int32_t* __restrict__ nxt, int64_t ldn, int64_t n, int32_t inf,
                  uint32_t tiles_per_row, const SuccStats* __restrict__ st,
                  unsigned long long max_sparse, int shift) {
  if (st->edges <= max_sparse || !succ_packable(st, inf, shift)) return;
  // Keys are kept as their int32 bit patterns (the vector LDS helpers take
  // int32) and read back as uint32.
  __shared__ __attribute__((aligned(16))) int32_t lds[4 * kKC * kLd];
  int32_t* sA = lds;                  // [2][kKC][kLd]: key of W[row0 + row][u0 + t]
  int32_t* sB = lds + 2 * kKC * kLd;  // [2][kKC][kLd]: key of D[u0 + t][col0 + col]
  const int tid = threadIdx.x;
  const int tc = tid % kThr, tr = tid / kThr;
  const int64_t row0 = (int64_t)(blockIdx.x / tiles_per_row) * kT;
  const int64_t col0 = (int64_t)(blockIdx.x % tiles_per_row) * kT;

  uint32_t acc[kR][kR];
#pragma unroll
  for (int i = 0; i < kR; ++i)
#pragma unroll
    for (int j = 0; j < kR; ++j) acc[i][j] = 0xFFFFFFFFu;

  int32_t ga[kLoads][4], gb[kLoads][4];
  auto fetch = [&](int64_t u0) {
#pragma unroll
    for (int l = 0; l < kLoads; ++l) {
      const int q = tid + l * kThreads;
      const int r = q / (kKC / 4), uq = q % (kKC / 4);
      ld4<int32_t, VEC>(W, ldw, n, n, row0 + r, u0 + uq * 4, inf, ga[l]);
#pragma unroll
      for (int e = 0; e < 4; ++e)  // u != i: the vertex itself is never its own first hop
        if (row0 + r == u0 + uq * 4 + e) ga[l][e] = inf;
      const int ur = q / (kT / 4), cq = q % (kT / 4);
      ld4<int32_t, VEC>(D, ldd, n, n, u0 + ur, col0 + cq * 4, inf, gb[l]);
    }
  };
  auto stash = [&](int buf, int64_t u0) {
    int32_t* a = sA + buf * kKC * kLd;
    int32_t* b = sB + buf * kKC * kLd;
#pragma unroll
    for (int l = 0; l < kLoads; ++l) {
      const int q = tid + l * kThreads;
      const int r = q / (kKC / 4), uq = q % (kKC / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        a[(uq * 4 + e) * kLd + r] =
            (int32_t)(ga[l][e] < inf ? (uint32_t)ga[l][e] << shift : kNoEdge);
      const int ur = q / (kT / 4), cq = q % (kT / 4);
      const uint32_t u = (uint32_t)(u0 + ur);
      int32_t v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = (int32_t)(gb[l][e] < inf ? ((uint32_t)gb[l][e] << shift) | u : kNoEdge);
      store4(b + ur * kLd + cq * 4, v);
    }
  };

  const int64_t chunks = (n + kKC - 1) / kKC;
  fetch(0);
  stash(0, 0);
  __syncthreads();
#pragma unroll 1
  for (int64_t c = 0; c < chunks; ++c) {
    const int buf = (int)(c & 1);
    if (c + 1 < chunks) fetch((c + 1) * kKC);
    const int32_t* a = sA + buf * kKC * kLd;
    const int32_t* b = sB + buf * kKC * kLd;
#pragma unroll 1
    for (int t = 0; t < kKC; t += 2) {
      uint32_t a0[kR], b0[kR], a1[kR], b1[kR];
#pragma unroll
      for (int gi = 0; gi < kR / 4; ++gi) {
        int32_t v[4];
        load4(a + t * kLd + gi * kGroupStride + tr * 4, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) a0[gi * 4 + i] = v[i];
        load4(a + (t + 1) * kLd + gi * kGroupStride + tr * 4, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) a1[gi * 4 + i] = v[i];
        load4(b + t * kLd + gi * kGroupStride + tc * 4, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) b0[gi * 4 + j] = v[j];
        load4(b + (t + 1) * kLd + gi * kGroupStride + tc * 4, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) b1[gi * 4 + j] = v[j];
      }
#pragma unroll
      for (int i = 0; i < kR; ++i)
#pragma unroll
        for (int j = 0; j < kR; ++j)
          acc[i][j] = min(acc[i][j], min(__builtin_elementwise_add_sat(a0[i], b0[j]),
                                         __builtin_elementwise_add_sat(a1[i], b1[j])));
    }
    if (c + 1 < chunks) stash(buf ^ 1, (c + 1) * kKC);
    __syncthreads();
  }

  const uint32_t mask = (1u << shift) - 1u;
#pragma unroll
  for (int gi = 0; gi < kR / 4; ++gi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = row0 + gi * kGroupStride + tr * 4 + i;
      if (r >= n) continue;
#pragma unroll
      for (int gj = 0; gj < kR / 4; ++gj)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t col = col0 + gj * kGroupStride + tc * 4 + j;
          if (col >= n) continue;
          const uint32_t k = acc[gi * 4 + i][gj * 4 + j];
          nxt[r * ldn + col] = r == col ? (int32_t)r : (k < kNoEdge ? (int32_t)(k & mask) : -1);
        }
    }
}

constexpr int kSThreads = 256;
constexpr int kSeg = kSThreads * 4;  // row entries gathered, and columns relaxed, per step
constexpr int kCap = 2 * kSeg;       // neighbours held in LDS at a time

template <typename T, bool VEC>
__global__ void __launch_bounds__(kSThreads)
successors_sparse(const T* __restrict__ W, int64_t ldw, const T* __restrict__ D, int64_t ldd,
                  int32_t* __restrict__ nxt, int64_t ldn, int64_t n, T inf,
                  const SuccStats* __restrict__ st, unsigned long long max_sparse) {
  if (st->edges > max_sparse) return;  // a dense kernel takes this matrix
  __shared__ int32_t lu[kCap];
  __shared__ T lw[kCap];
  __shared__ int32_t wsum[kSThreads / 64];
  const int64_t i = blockIdx.x;
  const T* wrow = W + i * ldw;
  int32_t* nrow = nxt + i * ldn;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int64_t p = 0;  // first row entry not gathered yet
  bool first = true;
  for (;;) {
    // Gather the neighbours in [p, ...) until the next segment would overflow
    // the list; a segment holds at most kSeg <= kCap of them, so p advances.
    int32_t cnt = 0;
    while (p < n) {
      const int64_t u0 = p + tid * 4;
      T v[4];
      ld4<T, VEC>(W, ldw, n, n, i, u0, inf, v);
      bool f[4];
      int c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[e] = u0 + e < n && u0 + e != i && v[e] < inf;
        c += f[e];
      }
      int x = c;  // inclusive scan over the wave
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      if (lane == 63) wsum[wv] = x;
      __syncthreads();
      int base = 0, total = 0;
#pragma unroll
      for (int k = 0; k < kSThreads / 64; ++k) {
        const int sk = wsum[k];
        base += k < wv ? sk : 0;
        total += sk;
      }
      __syncthreads();  // wsum is rewritten by the next segment
      if (cnt + total > kCap) break;
      int pos = cnt + base + x - c;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (f[e]) {
          lu[pos] = (int32_t)(u0 + e);
          lw[pos] = v[e];
          ++pos;
        }
      cnt += total;
      p += kSeg;
    }
    __syncthreads();  // the list is complete
    const bool last = p >= n;
    for (int64_t j0 = 0; j0 < n; j0 += kSeg) {
      const int64_t j = j0 + tid * 4;
      if (j >= n) continue;
      T bv[4];
      int32_t bu[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bv[e] = inf;
        bu[e] = -1;
        if (!first && j + e < n) {
          bu[e] = nrow[j + e];
          if (bu[e] >= 0) bv[e] = wrow[bu[e]] + D[(int64_t)bu[e] * ldd + j + e];
        }
      }
#pragma unroll 4
      for (int32_t t = 0; t < cnt; ++t) {
        const int32_t u = lu[t];
        const T wu = lw[t];
        T dv[4];
        ld4<T, VEC>(D, ldd, n, n, u, j, inf, dv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const T cand = wu + dv[e];
          const bool better = cand < bv[e];
          bv[e] = better ? cand : bv[e];
          bu[e] = better ? u : bu[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j + e < n)
          nrow[j + e] = !last ? bu[e] : (j + e == i ? (int32_t)i : (bv[e] < inf ? bu[e] : -1));
    }
    if (last) break;
    first = false;
    __syncthreads();  // the list is rebuilt
  }
}

template <typename T>
bool inf_ok(T inf);
template <>
bool inf_ok<int32_t>(int32_t inf) { return inf >= 1 && inf <= 0x3FFFFFFF; }
template <>
bool inf_ok<float>(float inf) { return inf > 0.0f; }

template <typename T>
bool mat_ok(const void* p, int64_t n, int64_t ld, size_t elem) {
  return p != nullptr && ld >= n && reinterpret_cast<uintptr_t>(p) % elem == 0 &&
         ld <= INT64_MAX / (int64_t)elem / n;
}

template <typename T>
int run_successors(const T* w, int64_t ldw, const T* d, int64_t ldd, int32_t* nxt, int64_t ldn,
                   int64_t n, T inf, void* stream) {
  if (n < 0 || !inf_ok<T>(inf)) return APSP_ERR_INVALID_VALUE;
  if (n == 0) return APSP_OK;
  if (n >= (int64_t(1) << 31) || !mat_ok<T>(w, n, ldw, sizeof(T)) ||
      !mat_ok<T>(d, n, ldd, sizeof(T)) || !mat_ok<int32_t>(nxt, n, ldn, sizeof(int32_t)))
    return APSP_ERR_INVALID_VALUE;
  const int64_t tpr = (n + kT - 1) / kT;
  if (tpr * tpr > (int64_t(1) << 31)) return APSP_ERR_INVALID_VALUE;
  int st = apsp_detail_check_device();
  if (st != APSP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const auto al16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  const bool vec = al16(w) && al16(d) && ldw % 4 == 0 && ldd % 4 == 0;
  // stats[0]: the folded statistics; stats[1 .. parts]: per-workgroup partials.
  const int parts = (int)std::min<int64_t>(n, kStatParts);
  SuccStats* stats = nullptr;
  if (hipMallocAsync(reinterpret_cast<void**>(&stats), sizeof(SuccStats) * (1 + parts), s) !=
      hipSuccess) {
    (void)apsp_detail_launch_status();
    return APSP_ERR_LAUNCH;
  }
  const unsigned long long max_sparse = (unsigned long long)n * (unsigned long long)n / 16;
  int shift = 0;  // bits that hold a vertex index: n <= 2^shift
  while ((int64_t(1) << shift) < n) ++shift;
  SuccStats* part = stats + 1;
  const bool wvec = al16(w) && ldw % 4 == 0, dvec = al16(d) && ldd % 4 == 0;
  if (wvec)
    hipLaunchKernelGGL((succ_count<T, true>), dim3(parts), dim3(256), 0, s, w, ldw, n, inf, part);
  else
    hipLaunchKernelGGL((succ_count<T, false>), dim3(parts), dim3(256), 0, s, w, ldw, n, inf, part);
  hipLaunchKernelGGL(succ_fold<false>, dim3(1), dim3(256), 0, s, part, parts, stats, max_sparse);
  if constexpr (std::is_same_v<T, int32_t>) {
    if (dvec)
      hipLaunchKernelGGL(succ_dstats<true>, dim3(parts), dim3(256), 0, s, d, ldd, n, inf, stats,
                         part, max_sparse);
    else
      hipLaunchKernelGGL(succ_dstats<false>, dim3(parts), dim3(256), 0, s, d, ldd, n, inf, stats,
                         part, max_sparse);
    hipLaunchKernelGGL(succ_fold<true>, dim3(1), dim3(256), 0, s, part, parts, stats, max_sparse);
  }
  const dim3 grid((unsigned)(tpr * tpr));
  if (vec) {
    hipLaunchKernelGGL((successors<T, true>), grid, dim3(kThreads), 0, s, w, ldw, d, ldd, nxt, ldn,
                       n, inf, (uint32_t)tpr, stats, max_sparse, shift);
    if constexpr (std::is_same_v<T, int32_t>)
      hipLaunchKernelGGL((successors_packed<true>), grid, dim3(kThreads), 0, s, w, ldw, d, ldd, nxt,
                         ldn, n, inf, (uint32_t)tpr, stats, max_sparse, shift);
    hipLaunchKernelGGL((successors_sparse<T, true>), dim3((unsigned)n), dim3(kSThreads), 0, s, w, ldw,
                       d, ldd, nxt, ldn, n, inf, stats, max_sparse);
  } else {
    hipLaunchKernelGGL((successors<T, false>), grid, dim3(kThreads), 0, s, w, ldw, d, ldd, nxt,
                       ldn, n, inf, (uint32_t)tpr, stats, max_sparse, shift);
    if constexpr (std::is_same_v<T, int32_t>)
      hipLaunchKernelGGL((successors_packed<false>), grid, dim3(kThreads), 0, s, w, ldw, d, ldd,
                         nxt, ldn, n, inf, (uint32_t)tpr, stats, max_sparse, shift);
    hipLaunchKernelGGL((successors_sparse<T, false>), dim3((unsigned)n), dim3(kSThreads), 0, s, w,
                       ldw, d, ldd, nxt, ldn, n, inf, stats, max_sparse);
  }
  const int st_launch = apsp_detail_launch_status();
  (void)hipFreeAsync(stats, s);
  return st_launch;
}

// ---------------------------------------------------------------------------
// Distances and successors in one pass of the rounds (int32, dense).
//
// For a dense int32 matrix with weights >= 0, a zero diagonal and a bounded
// range, the rounds run on keys v << s | h (s the bit width of n): each
// entry then ends as its shortest distance and the smallest first hop of a
// shortest path, which is the successor defined above (the smallest u != i
// with w(i, u) + d(u, j) = d(i, j): every such u starts a shortest walk, and
// every shortest walk's first hop is such a u).  That replaces the n^3
// successor product by a split of the keys.  Walks that begin with the
// diagonal entry carry the hop 2^s - 1, which loses every tie, so a first
// hop is never i itself.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int32_t key_of(int32_t w, int64_t i, int64_t j, int32_t inf, int sb,
                                          int32_t none) {
  const uint32_t hop = i == j ? (1u << sb) - 1u : (uint32_t)j;
  return w >= inf ? none : (int32_t)(((uint32_t)w << sb) | hop);
}

// The diagonal's range (into st->dmin, st->dmax), one workgroup.
__global__ void __launch_bounds__(256) keys_diag(const int32_t* __restrict__ d, int64_t ld,
                                                 int64_t n, SuccStats* __restrict__ st) {
  int32_t lo = INT32_MAX, hi = INT32_MIN;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int32_t v = d[i * ld + i];
    lo = min(lo, v);
    hi = max(hi, v);
  }
  unsigned long long none = 0;
  block_stats(none, lo, hi);
  if (threadIdx.x == 0) {
    st->dmin = lo;
    st->dmax = hi;
  }
}

// Weights to keys in place; "no edge" (>= inf) becomes none = 2^30 - 2^s.
template <bool VEC>
__global__ void __launch_bounds__(256) keys_pack(int32_t* __restrict__ d, int64_t ld, int64_t n,
                                                 int32_t inf, int sb) {
  const int32_t none = (int32_t)((1u << 30) - (1u << sb));
  const int64_t quads = VEC ? n / 4 : 0;
  for (int64_t i = blockIdx.x; i < n; i += gridDim.x) {
    int32_t* row = d + i * ld;
    for (int64_t q = threadIdx.x; q < quads; q += blockDim.x) {
      int32_t v[4];
      load4(row + q * 4, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = key_of(v[e], i, q * 4 + e, inf, sb, none);
      store4(row + q * 4, v);
    }
    for (int64_t j = quads * 4 + threadIdx.x; j < n; j += blockDim.x)
      row[j] = key_of(row[j], i, j, inf, sb, none);
  }
}

// Keys to distances (in place) and successors.
__device__ __forceinline__ void key_split(int32_t k, int64_t i, int64_t j, int32_t inf, int sb,
                                          int32_t none, int32_t& dist, int32_t& hop) {
  const int32_t v = k >> sb;
  const bool reach = k < none && v < inf;
  dist = reach ? v : inf;
  hop = i == j ? (int32_t)i : (reach ? (int32_t)(k & (int32_t)((1u << sb) - 1u)) : -1);
}

template <bool VEC>
__global__ void __launch_bounds__(256) keys_split(int32_t* __restrict__ d, int64_t ld,
                                                  int32_t* __restrict__ nxt, int64_t ldn,
                                                  int64_t n, int32_t inf, int sb) {
  const int32_t none = (int32_t)((1u << 30) - (1u << sb));
  const int64_t quads = VEC ? n / 4 : 0;
  for (int64_t i = blockIdx.x; i < n; i += gridDim.x) {
    int32_t* row = d + i * ld;
    int32_t* out = nxt + i * ldn;
    for (int64_t q = threadIdx.x; q < quads; q += blockDim.x) {
      int32_t v[4], h[4];
      load4(row + q * 4, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) key_split(v[e], i, q * 4 + e, inf, sb, none, v[e], h[e]);
      store4(row + q * 4, v);
      store4(out + q * 4, h);
    }
    for (int64_t j = quads * 4 + threadIdx.x; j < n; j += blockDim.x) {
      int32_t dv, hv;
      key_split(row[j], i, j, inf, sb, none, dv, hv);
      row[j] = dv;
      out[j] = hv;
    }
  }
}

}  // namespace

extern "C" int apsp_fw_i32(int32_t* d, int64_t n, int64_t ld, int32_t inf, void* stream);
extern "C" int apsp_fw_f32(float* d, int64_t n, int64_t ld, float inf, void* stream);

namespace {

// Whether the one-pass key form applies to the int32 weights d: they are
// dense (more than n^2/16 finite off-diagonal entries, where the separate
// pass would run the n^3 product), none is negative, the diagonal is zero,
// and every value the rounds can store stays below 2^(30-s) - 1 -- it is
// at most the largest weight when no off-diagonal entry is inf, else at
// most n - 1 times it (a shortest path is simple).  Reads the statistics
// back, so the stream is synchronised once.
int keys_choice(const int32_t* d, int64_t ld, int64_t n, int32_t inf, hipStream_t s, bool* use) {
  *use = false;
  if (n >= (int64_t(1) << 29)) return APSP_OK;
  // A stream under graph capture cannot be synchronised: keep the form that
  // decides on the device.
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
    (void)apsp_detail_launch_status();
    return APSP_ERR_LAUNCH;
  }
  if (cs != hipStreamCaptureStatusNone) return APSP_OK;
  const int parts = (int)std::min<int64_t>(n, kStatParts);
  SuccStats* stats = nullptr;
  if (hipMallocAsync(reinterpret_cast<void**>(&stats), sizeof(SuccStats) * (1 + parts), s) !=
      hipSuccess) {
    (void)apsp_detail_launch_status();
    return APSP_ERR_LAUNCH;
  }
  SuccStats* part = stats + 1;
  if (reinterpret_cast<uintptr_t>(d) % 16 == 0 && ld % 4 == 0)
    hipLaunchKernelGGL((succ_count<int32_t, true>), dim3(parts), dim3(256), 0, s, d, ld, n, inf,
                       part);
  else
    hipLaunchKernelGGL((succ_count<int32_t, false>), dim3(parts), dim3(256), 0, s, d, ld, n, inf,
                       part);
  hipLaunchKernelGGL(succ_fold<false>, dim3(1), dim3(256), 0, s, part, parts, stats, 0ull);
  hipLaunchKernelGGL(keys_diag, dim3(1), dim3(256), 0, s, d, ld, n, stats);
  SuccStats h{};
  int st = apsp_detail_launch_status();
  if (st == APSP_OK &&
      (hipMemcpyAsync(&h, stats, sizeof(SuccStats), hipMemcpyDeviceToHost, s) != hipSuccess ||
       hipStreamSynchronize(s) != hipSuccess)) {
    (void)apsp_detail_launch_status();
    st = APSP_ERR_LAUNCH;
  }
  (void)hipFreeAsync(stats, s);
  if (st != APSP_OK) return st;
  const unsigned long long nn = (unsigned long long)n;
  const int sb = 32 - __builtin_clz((unsigned)n);
  const int64_t lim = (int64_t(1) << (30 - sb)) - 1;
  const int64_t wmax = h.edges ? h.wmax : 0;
  const int64_t bound = h.edges == nn * (nn - 1) ? wmax : (n - 1) * wmax;
  *use = h.edges > nn * nn / 16 && (h.edges == 0 || h.wmin >= 0) && h.dmin == 0 &&
         h.dmax == 0 && bound < lim;
  return APSP_OK;
}

// The form the last apsp_fw_paths_i32 call of this thread took: 1 keys, 0 the
// separate successor pass, -1 none yet (or the call failed before choosing).
thread_local int g_paths_form = -1;

// Distances in place plus successors.  int32 weights for which the key form
// applies take one pass of the rounds on keys; otherwise the weights are
// kept in stream-ordered scratch for the successor pass after the rounds.
template <typename T>
int run_fw_paths(T* d, int64_t ld, int32_t* nxt, int64_t ldn, int64_t n, T inf, void* stream) {
  if constexpr (std::is_same_v<T, int32_t>) g_paths_form = -1;
  if (n < 0 || !inf_ok<T>(inf)) return APSP_ERR_INVALID_VALUE;
  if (n == 0) return APSP_OK;
  if (!mat_ok<T>(d, n, ld, sizeof(T)) || !mat_ok<int32_t>(nxt, n, ldn, sizeof(int32_t)) ||
      n >= (int64_t(1) << 31))
    return APSP_ERR_INVALID_VALUE;
  int st = apsp_detail_check_device();
  if (st != APSP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if constexpr (std::is_same_v<T, int32_t>) {
    bool use = false;
    st = keys_choice(d, ld, n, inf, s, &use);
    if (st != APSP_OK) return st;
    g_paths_form = use ? 1 : 0;
    if (use) {
      const int sb = 32 - __builtin_clz((unsigned)n);
      const dim3 rows((unsigned)std::min<int64_t>(n, 4096));
      const bool dv = reinterpret_cast<uintptr_t>(d) % 16 == 0 && ld % 4 == 0;
      const bool nv = dv && reinterpret_cast<uintptr_t>(nxt) % 16 == 0 && ldn % 4 == 0;
      if (dv) hipLaunchKernelGGL(keys_pack<true>, rows, dim3(256), 0, s, d, ld, n, inf, sb);
      else hipLaunchKernelGGL(keys_pack<false>, rows, dim3(256), 0, s, d, ld, n, inf, sb);
      st = apsp_detail_launch_status();
      if (st == APSP_OK) st = apsp_detail_fw_keys(d, n, ld, stream);
      if (st != APSP_OK) return st;
      if (nv) hipLaunchKernelGGL(keys_split<true>, rows, dim3(256), 0, s, d, ld, nxt, ldn, n, inf, sb);
      else hipLaunchKernelGGL(keys_split<false>, rows, dim3(256), 0, s, d, ld, nxt, ldn, n, inf, sb);
      return apsp_detail_launch_status();
    }
  }
  const int64_t ldw = (n + 3) & ~int64_t(3);
  T* w = nullptr;
  if (hipMallocAsync(reinterpret_cast<void**>(&w), (size_t)(ldw * n * sizeof(T)), s) != hipSuccess) {
    (void)apsp_detail_launch_status();
    return APSP_ERR_LAUNCH;
  }
  if (hipMemcpy2DAsync(w, ldw * sizeof(T), d, ld * sizeof(T), n * sizeof(T), n,
                       hipMemcpyDeviceToDevice, s) != hipSuccess) {
    (void)apsp_detail_launch_status();
    (void)hipFreeAsync(w, s);
    return APSP_ERR_LAUNCH;
  }
  if constexpr (std::is_same_v<T, int32_t>) st = apsp_fw_i32(d, n, ld, inf, stream);
  else st = apsp_fw_f32(d, n, ld, inf, stream);
  if (st == APSP_OK) st = run_successors<T>(w, ldw, d, ld, nxt, ldn, n, inf, stream);
  (void)hipFreeAsync(w, s);
  return st;
}

}  // namespace

extern "C" {

int apsp_fw_paths_i32(int32_t* d, int64_t ld, int32_t* nxt, int64_t ldn, int64_t n, int32_t inf,
                      void* stream) {
  return run_fw_paths<int32_t>(d, ld, nxt, ldn, n, inf, stream);
}

int apsp_fw_paths_f32(float* d, int64_t ld, int32_t* nxt, int64_t ldn, int64_t n, float inf,
                      void* stream) {
  return run_fw_paths<float>(d, ld, nxt, ldn, n, inf, stream);
}

int apsp_fw_paths_last_form(void) { return g_paths_form; }


int apsp_successors_i32(const int32_t* w, int64_t ldw, const int32_t* d, int64_t ldd,
                        int32_t* nxt, int64_t ldn, int64_t n, int32_t inf, void* stream) {
  return run_successors<int32_t>(w, ldw, d, ldd, nxt, ldn, n, inf, stream);
}

int apsp_successors_f32(const float* w, int64_t ldw, const float* d, int64_t ldd, int32_t* nxt,
                        int64_t ldn, int64_t n, float inf, void* stream) {
  return run_successors<float>(w, ldw, d, ldd, nxt, ldn, n, inf, stream);
}

int64_t apsp_path(const int32_t* nxt, int64_t ldn, int64_t n, int64_t i, int64_t j, int32_t* path,
                  int64_t cap) {
  if (nxt == nullptr || n <= 0 || ldn < n || i < 0 || i >= n || j < 0 || j >= n || cap < 0 ||
      (cap > 0 && path == nullptr))
    return -2;
  if (nxt[i * ldn + j] < 0) return -1;  // j unreachable from i
  int64_t len = 0, v = i;
  for (;;) {
    if (len < cap) path[len] = (int32_t)v;
    ++len;
    if (v == j) return len;
    if (len > n) return -3;  // no progress within n hops: a zero-weight cycle
    const int32_t u = nxt[v * ldn + j];
    if (u < 0 || u >= n) return -3;
    v = u;
  }
}

}  // extern "C"
