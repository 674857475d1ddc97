// Min-plus matrix product C <- min(C, A (x) B), (A (x) B)[i][j] = min_t
// A[i][t] + B[t][j], for operands in separate buffers and of any depth.
//
// This is the operation inside Phases 2 and 3 of the blocked Floyd-Warshall
// of the page "Katz and Kider" (thesis section 4.6, Algorithms 17 and 18: a
// block updated from the pivot row and pivot column blocks), taken out of the
// single-matrix setting so that it can run on blocks that do not share one
// device buffer -- the building block of the host-resident (out-of-core)
// blocked Floyd-Warshall (host.hip), whose outer blocks are far deeper than
// one 128-pivot round.
//
// gfx950 design: the same register tiling as the in-core Phase 3 -- a
// 256-thread workgroup owns a 128 x 128 tile of C as an 8 x 8 micro-tile per
// thread, held in registers for the whole depth k; A and B stream through
// LDS in 16-deep chunks, double buffered, A stored k-major so every operand
// fetch is one 128-bit LDS read; two candidates share one three-input min.
// C is read and written once per product, whatever k is, so the product is
// VALU bound once k is a few hundred.  Tiles are handed to XCDs in contiguous
// ranges walked in bands of 8 tile rows, so neighbouring workgroups share A
// and B panels through their XCD's L2.
// Out-of-range rows and columns load as inf and are never stored; along the
// depth both operands read inf there, and inf + inf never improves C.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "apsp.h"
#include "detail.h"
#include "minplus.h"

namespace {

using namespace apsp_dev;

constexpr int kT = 128;         // C tile edge
constexpr int kThreads = 256;
constexpr int kR = 8;           // micro-tile edge
constexpr int kThr = kT / kR;   // 16 threads per tile dimension
constexpr int kKC = 16;         // depth per LDS chunk
constexpr int kLd = kT + 4;     // LDS row stride (elements), keeps 16-byte alignment
constexpr int kGroupStride = kT / (kR / 4);  // 64: distance between a thread's 4-wide groups
constexpr int kQuads = kT * kKC / 4;         // 512 quads per operand chunk
constexpr int kLoads = kQuads / kThreads;    // 2 quad loads per thread per operand
constexpr uint32_t kXcds = 8;
constexpr uint32_t kBand = 8;

// Four elements [c, c+4) of row r of a rows x cols operand (leading dimension
// ld); anything outside reads as inf.
template <typename T, bool VEC, bool EDGE>
__device__ __forceinline__ void opload4(const T* __restrict__ p, int64_t ld, int64_t rows,
                                        int64_t cols, int64_t r, int64_t c, T inf, T (&v)[4]) {
  const T* q = p + r * ld + c;
  if (!EDGE || (r < rows && c + 3 < cols)) {
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

template <typename T, bool VEC, bool EDGE>
__device__ __forceinline__ void opstore4(T* __restrict__ p, int64_t ld, int64_t rows,
                                         int64_t cols, int64_t r, int64_t c, const T (&v)[4]) {
  T* q = p + r * ld + c;
  if (!EDGE || (r < rows && c + 3 < cols)) {
    if (VEC) {
      store4(q, v);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = v[e];
    }
  } else if (r < rows) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c + e < cols) q[e] = v[e];
  }
}

// Tile L of an mt x nt grid -> (tile row, tile column): XCD x takes the
// contiguous range of L, walked band by band (kBand tile rows), column by
// column inside a band.
__device__ __forceinline__ void tile_of(uint32_t b, uint32_t mt, uint32_t nt, uint32_t& ti,
                                        uint32_t& tj) {
  const uint32_t total = mt * nt;
  const uint32_t x = b % kXcds, j = b / kXcds;
  const uint32_t q = total / kXcds, rem = total % kXcds;
  const uint32_t L = x * q + min(x, rem) + j;
  const uint32_t g = L / (kBand * nt);
  const uint32_t base = g * kBand;
  const uint32_t rows = min(kBand, mt - base);
  const uint32_t r = L - g * kBand * nt;
  ti = base + r % rows;
  tj = r / rows;
}

template <typename T, bool VEC, bool EDGE>
__device__ __forceinline__ void gemm_tile(T* __restrict__ C, int64_t ldc, const T* __restrict__ A,
                                          int64_t lda, const T* __restrict__ B, int64_t ldb,
                                          int64_t m, int64_t n, int64_t k, T inf, int64_t row0,
                                          int64_t col0, T* __restrict__ lds) {
  T* sA = lds;                  // [2][kKC][kLd], k-major: sA[t][row]
  T* sB = lds + 2 * kKC * kLd;  // [2][kKC][kLd]: sB[t][col]
  const int tid = threadIdx.x;
  const int tc = tid % kThr, tr = tid / kThr;
  const T* At = A + row0 * lda;   // this tile's rows of A
  const T* Bt = B + col0;         // this tile's columns of B
  T* Ct = C + row0 * ldc + col0;
  const int64_t mr = m - row0, nc = n - col0;  // valid rows / columns of the tile

  T acc[kR][kR];
#pragma unroll
  for (int gi = 0; gi < kR / 4; ++gi)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int gj = 0; gj < kR / 4; ++gj) {
        T v[4];
        opload4<T, VEC, EDGE>(Ct, ldc, mr, nc, gi * kGroupStride + tr * 4 + i,
                              gj * kGroupStride + tc * 4, inf, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[gi * 4 + i][gj * 4 + j] = v[j];
      }

  T ga[kLoads][4], gb[kLoads][4];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int l = 0; l < kLoads; ++l) {
      const int q = tid + l * kThreads;
      const int r = q / (kKC / 4), kq = q % (kKC / 4);
      opload4<T, VEC, EDGE>(At, lda, mr, k, r, k0 + kq * 4, inf, ga[l]);
      const int kr = q / (kT / 4), cq = q % (kT / 4);
      opload4<T, VEC, EDGE>(Bt, ldb, k, nc, k0 + kr, cq * 4, inf, gb[l]);
    }
  };
  auto stash = [&](int buf) {
    T* a = sA + buf * kKC * kLd;
    T* b = sB + buf * kKC * kLd;
#pragma unroll
    for (int l = 0; l < kLoads; ++l) {
      const int q = tid + l * kThreads;
      const int r = q / (kKC / 4), kq = q % (kKC / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[(kq * 4 + e) * kLd + r] = ga[l][e];
      const int kr = q / (kT / 4), cq = q % (kT / 4);
      store4(b + kr * kLd + cq * 4, gb[l]);
    }
  };

  const int64_t chunks = (k + kKC - 1) / kKC;
  fetch(0);
  stash(0);
  __syncthreads();
#pragma unroll 1
  for (int64_t c = 0; c < chunks; ++c) {
    const int buf = (int)(c & 1);
    if (c + 1 < chunks) fetch((c + 1) * kKC);
    const T* a = sA + buf * kKC * kLd;
    const T* b = sB + buf * kKC * kLd;
#pragma unroll
    for (int t = 0; t < kKC; t += 2) {
      T a0[kR], a1[kR], b0[kR], b1[kR];
#pragma unroll
      for (int gi = 0; gi < kR / 4; ++gi) {
        T v[4];
        load4(a + t * kLd + gi * kGroupStride + tr * 4, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) a0[gi * 4 + i] = v[i];
        load4(a + (t + 1) * kLd + gi * kGroupStride + tr * 4, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) a1[gi * 4 + i] = v[i];
      }
#pragma unroll
      for (int gj = 0; gj < kR / 4; ++gj) {
        T v[4];
        load4(b + t * kLd + gj * kGroupStride + tc * 4, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) b0[gj * 4 + j] = v[j];
        load4(b + (t + 1) * kLd + gj * kGroupStride + tc * 4, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) b1[gj * 4 + j] = v[j];
      }
#pragma unroll
      for (int i = 0; i < kR; ++i)
#pragma unroll
        for (int j = 0; j < kR; ++j)
          acc[i][j] = mp_relax2(acc[i][j], a0[i], b0[j], a1[i], b1[j]);
    }
    if (c + 1 < chunks) stash(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int gi = 0; gi < kR / 4; ++gi)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int gj = 0; gj < kR / 4; ++gj) {
        T v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = acc[gi * 4 + i][gj * 4 + j];
        opstore4<T, VEC, EDGE>(Ct, ldc, mr, nc, gi * kGroupStride + tr * 4 + i,
                               gj * kGroupStride + tc * 4, v);
      }
}

// One workgroup per 128 x 128 tile of C.  Interior tiles with a depth that
// is a multiple of the LDS chunk take the unpredicated path.
template <typename T, bool VEC>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
mp_gemm(T* __restrict__ C, int64_t ldc, const T* __restrict__ A, int64_t lda,
        const T* __restrict__ B, int64_t ldb, int64_t m, int64_t n, int64_t k, T inf,
        uint32_t mt, uint32_t nt) {
  __shared__ __attribute__((aligned(16))) T lds[4 * kKC * kLd];
  uint32_t ti, tj;
  tile_of(blockIdx.x, mt, nt, ti, tj);
  const int64_t row0 = (int64_t)ti * kT, col0 = (int64_t)tj * kT;
  if (row0 + kT <= m && col0 + kT <= n && k % kKC == 0)
    gemm_tile<T, VEC, false>(C, ldc, A, lda, B, ldb, m, n, k, inf, row0, col0, lds);
  else
    gemm_tile<T, VEC, true>(C, ldc, A, lda, B, ldb, m, n, k, inf, row0, col0, lds);
}

template <typename T>
bool inf_ok(T inf);
template <>
bool inf_ok<int32_t>(int32_t inf) { return inf >= 1 && inf <= 0x3FFFFFFF; }
template <>
bool inf_ok<float>(float inf) { return inf > 0.0f; }

template <typename T>
bool operand_ok(const void* p, int64_t rows, int64_t cols, int64_t ld) {
  if (rows == 0 || cols == 0) return true;
  if (p == nullptr || ld < cols || reinterpret_cast<uintptr_t>(p) % sizeof(T)) return false;
  return rows - 1 <= (INT64_MAX / (int64_t)sizeof(T) - cols) / ld;
}

template <typename T>
int run_gemm(T* C, int64_t ldc, const T* A, int64_t lda, const T* B, int64_t ldb, int64_t m,
             int64_t n, int64_t k, T inf, void* stream) {
  if (m < 0 || n < 0 || k < 0 || !inf_ok<T>(inf)) return APSP_ERR_INVALID_VALUE;
  if (m == 0 || n == 0 || k == 0) return APSP_OK;
  if (!operand_ok<T>(C, m, n, ldc) || !operand_ok<T>(A, m, k, lda) || !operand_ok<T>(B, k, n, ldb))
    return APSP_ERR_INVALID_VALUE;
  const int64_t mt = (m + kT - 1) / kT, nt = (n + kT - 1) / kT;
  if (mt * nt > (int64_t(1) << 31)) return APSP_ERR_INVALID_VALUE;
  int st = apsp_detail_check_device();
  if (st != APSP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const auto al16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  const bool vec = al16(C) && al16(A) && al16(B) && ldc % 4 == 0 && lda % 4 == 0 && ldb % 4 == 0;
  const dim3 grid((unsigned)(mt * nt));
  if (vec)
    hipLaunchKernelGGL((mp_gemm<T, true>), grid, dim3(kThreads), 0, s, C, ldc, A, lda, B, ldb, m,
                       n, k, inf, (uint32_t)mt, (uint32_t)nt);
  else
    hipLaunchKernelGGL((mp_gemm<T, false>), grid, dim3(kThreads), 0, s, C, ldc, A, lda, B, ldb, m,
                       n, k, inf, (uint32_t)mt, (uint32_t)nt);
  return apsp_detail_launch_status();
}

}  // namespace

// Library-internal entry for the host-resident driver (no argument checks).
int apsp_detail_gemm_i32(int32_t* C, int64_t ldc, const int32_t* A, int64_t lda, const int32_t* B,
                         int64_t ldb, int64_t m, int64_t n, int64_t k, int32_t inf,
                         void* stream) {
  return run_gemm<int32_t>(C, ldc, A, lda, B, ldb, m, n, k, inf, stream);
}
int apsp_detail_gemm_f32(float* C, int64_t ldc, const float* A, int64_t lda, const float* B,
                         int64_t ldb, int64_t m, int64_t n, int64_t k, float inf, void* stream) {
  return run_gemm<float>(C, ldc, A, lda, B, ldb, m, n, k, inf, stream);
}

extern "C" {

int apsp_minplus_gemm_i32(int32_t* C, int64_t ldc, const int32_t* A, int64_t lda,
                          const int32_t* B, int64_t ldb, int64_t m, int64_t n, int64_t k,
                          int32_t inf, void* stream) {
  return run_gemm<int32_t>(C, ldc, A, lda, B, ldb, m, n, k, inf, stream);
}

int apsp_minplus_gemm_f32(float* C, int64_t ldc, const float* A, int64_t lda, const float* B,
                          int64_t ldb, int64_t m, int64_t n, int64_t k, float inf, void* stream) {
  return run_gemm<float>(C, ldc, A, lda, B, ldb, m, n, k, inf, stream);
}

}  // extern "C"
