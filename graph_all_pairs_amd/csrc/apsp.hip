// Blocked Floyd-Warshall all-pairs shortest paths for gfx950 (MI355X).
//
// Method: the blocked Floyd-Warshall of the page "Katz and Kider" (thesis
// section 4.6, Algorithms 16-18, Figures 4.2-4.5).  The n x n distance matrix
// is cut into B x B pivot blocks; round K
//   Phase 1  closes the diagonal block D_KK (Floyd-Warshall inside the block);
//   Phase 2  updates the pivot-row blocks D_KJ and pivot-column blocks D_IK;
//   Phase 3  updates every other block D_IJ from D_IK and D_KJ;
// and the next round takes the next diagonal block.
//
// gfx950 design (what differs from the page's 16 x 16 CUDA design):
//  * B = 128.  Phase 3 gives each 256-thread workgroup a 128 x 128 output tile
//    held in registers as an 8 x 8 micro-tile per thread; the 128 x 128 pivot
//    column/row operands stream through LDS in k-chunks, double buffered, the
//    column operand stored k-major so that every operand fetch is a 128-bit
//    LDS read with no bank conflict.  Per pair of pivots each output costs two
//    adds and one three-input min (v_add_u32 / v_add_f32 + v_min3).
//  * Phase 2 is computed with the closed diagonal block:
//      D_KJ <- min(D_KJ, D_KK* (x) D_KJ),   D_IK <- min(D_IK, D_IK (x) D_KK*),
//    where (x) is the min-plus product.  Both sides equal the shortest
//    distances through intermediates in blocks <= K, so this is the same
//    result as the page's in-place pivot loop (exact for integers), and it
//    turns Phase 2 into the same barrier-free product kernel as Phase 3.  Each
//    Phase-2 workgroup owns all B rows (row panel) or all B columns (column
//    panel) of its tile, so the operand it reads from its own tile is never
//    written by another workgroup.
//  * Phase 1 keeps the block in registers in the same 8 x 8-per-thread layout;
//    only pivot row t and pivot column t travel through LDS, in ping-pong
//    buffers, with one barrier per pivot.  The page runs Phase 1 on a single
//    multiprocessor while the rest of the GPU waits; here the Phase 1 of
//    round K+1 is done by the workgroup that computes tile (K+1, K+1) in
//    round K's Phase-3 launch, right after that tile's update, so it overlaps
//    the rest of Phase 3 (only the first round has a Phase-1 launch).
//  * Phase 3 hands each XCD a contiguous, banded range of tiles so the pivot
//    panels a workgroup reads are shared through that XCD's L2.
//  * Ragged n: rows and columns >= n behave as isolated vertices -- loads
//    return inf, stores are suppressed -- so nothing outside the leading
//    n x n block is read or written.
//  * The page's skipPrimaryBlock equations (Figures 4.2, 4.3) become the index
//    map j' -> j' + (j' >= K) on the workgroup id.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "apsp.h"
#include "detail.h"
#include "minplus.h"

namespace {

using namespace apsp_dev;

constexpr int kB = 128;        // pivot block edge
constexpr int kThreads = 256;  // Phase 2/3 workgroup size
#ifndef APSP_KC
#define APSP_KC 16
#endif
#ifndef APSP_P2_TILE
#define APSP_P2_TILE 32
#endif
constexpr int kKC = APSP_KC;   // pivots per LDS chunk
constexpr int kPad = 4;        // LDS row padding (elements), keeps 16-B alignment
constexpr int kWavesP3 = 3;    // waves per SIMD targeted by Phase 3 (<= 168 VGPRs): a
                               // third wave per SIMD keeps the VALU fed while the
                               // others wait on LDS (measured faster than two waves
                               // with software-pipelined operand reads)
constexpr int kWavesP2 = 4;    // waves per SIMD targeted by Phase 2 (<= 128 VGPRs)
constexpr int kP3PerCu = 2;    // Phase-3 tiles per CU below which signed int32 calls prefer int32
constexpr int kF32MinTiles = 9;  // Phase-3 tiles below which int32 calls stay in int32

// ---------------------------------------------------------------------------
// Min-plus tile update  C <- min(C, A (x) B)  for one workgroup.
//   C = D[row0 .. row0+TM) x [col0 .. col0+TN)
//   A = D[row0 .. row0+TM) x [kb0 .. kb0+kB)      (pivot columns)
//   B = D[kb0 .. kb0+kB)  x [col0 .. col0+TN)     (pivot rows)
// Thread layout: (TM/RM) x (TN/RN) = 256 threads, each holding an RM x RN
// micro-tile made of (RM/4) x (RN/4) blocks of 4 x 4 spaced TM/(RM/4) rows
// and TN/(RN/4) columns apart.  The C tile stays in registers for the whole
// kB-deep update and is written once at the end, so a tile may alias A or B.
// ---------------------------------------------------------------------------
template <typename T, int TM, int TN, int RM, int RN>
struct TileShape {
  static constexpr int kThrCols = TN / RN;
  static constexpr int kThrRows = TM / RM;
  static_assert(kThrCols * kThrRows == kThreads, "256 threads per tile");
  static constexpr int kGroupRowStride = TM / (RM / 4);
  static constexpr int kGroupColStride = TN / (RN / 4);
  static constexpr int kLdA = TM + kPad;  // sA[k][row]
  static constexpr int kLdB = TN + kPad;  // sB[k][col]
  static constexpr int kQuadsA = TM * kKC / 4;
  static constexpr int kQuadsB = kKC * TN / 4;
  static constexpr int kLoadsA = (kQuadsA + kThreads - 1) / kThreads;
  static constexpr int kLoadsB = (kQuadsB + kThreads - 1) / kThreads;
  static constexpr int kLdsElems = 2 * kKC * (kLdA + kLdB);
};

// ---------------------------------------------------------------------------
// An int32 matrix computed in binary32 is converted on the fly: the loads of
// the first round read int32 entries and convert them (the sentinel becomes
// +infinity), the stores of the last round convert back (see i32_to_f32 and
// f32_to_i32).  The flags say which accesses of a launch convert.
// ---------------------------------------------------------------------------
constexpr int kConvC = 1;      // the C tile's loads
constexpr int kConvA = 2;      // the A operand's loads (Phase 2 column pieces: the piece itself)
constexpr int kConvB = 4;      // the B operand's loads (Phase 2 row pieces: the piece itself)
constexpr int kConvOut = 8;    // every store of the launch
constexpr int kConvDiag = 16;  // Phase 3: workgroup 0 also converts block (K, K) back

// gload4, converting int32 entries to binary32 when cv is set.  Elements
// outside the matrix read as inf32, which converts to +infinity.
template <typename T, bool VEC, bool EDGE>
__device__ __forceinline__ void gload4x(const T* __restrict__ d, int64_t ld, int64_t n,
                                        int64_t row, int64_t col, T inf, T (&v)[4], bool cv,
                                        int32_t inf32) {
  if constexpr (std::is_same_v<T, float>) {
    if (cv) {
      int32_t r[4];
      gload4<int32_t, VEC, EDGE>(reinterpret_cast<const int32_t*>(d), ld, n, row, col, inf32, r);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = i32_to_f32(r[e], inf32);
      return;
    }
  }
  gload4<T, VEC, EDGE>(d, ld, n, row, col, inf, v);
}

template <typename T, bool VEC, bool EDGE>
__device__ __forceinline__ void gstore4x(T* __restrict__ d, int64_t ld, int64_t n, int64_t row,
                                         int64_t col, const T (&v)[4], bool cv, int32_t inf32) {
  if constexpr (std::is_same_v<T, float>) {
    if (cv) {
      int32_t r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = f32_to_i32(v[e], inf32);
      gstore4<int32_t, VEC, EDGE>(reinterpret_cast<int32_t*>(d), ld, n, row, col, r);
      return;
    }
  }
  gstore4<T, VEC, EDGE>(d, ld, n, row, col, v);
}

// C tile <-> registers, in the micro-tile layout described above.
template <typename T, int TM, int TN, int RM, int RN, bool VEC, bool EDGE>
__device__ __forceinline__ void load_tile(const T* __restrict__ d, int64_t n, int64_t ld, T inf,
                                          int64_t row0, int64_t col0, T (&acc)[RM][RN],
                                          int tid = threadIdx.x, bool cv = false,
                                          int32_t inf32 = 0) {
  using S = TileShape<T, TM, TN, RM, RN>;
  const int tc = tid % S::kThrCols;
  const int tr = tid / S::kThrCols;
#pragma unroll
  for (int gi = 0; gi < RM / 4; ++gi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = row0 + gi * S::kGroupRowStride + tr * 4 + i;
#pragma unroll
      for (int gj = 0; gj < RN / 4; ++gj) {
        T v[4];
        gload4x<T, VEC, EDGE>(d, ld, n, row, col0 + gj * S::kGroupColStride + tc * 4, inf, v, cv,
                              inf32);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[gi * 4 + i][gj * 4 + j] = v[j];
      }
    }
}

template <typename T, int TM, int TN, int RM, int RN, bool VEC, bool EDGE>
__device__ __forceinline__ void store_tile(T* __restrict__ d, int64_t n, int64_t ld,
                                           int64_t row0, int64_t col0, const T (&acc)[RM][RN],
                                           int tid = threadIdx.x, bool cv = false,
                                           int32_t inf32 = 0) {
  using S = TileShape<T, TM, TN, RM, RN>;
  const int tc = tid % S::kThrCols;
  const int tr = tid / S::kThrCols;
#pragma unroll
  for (int gi = 0; gi < RM / 4; ++gi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = row0 + gi * S::kGroupRowStride + tr * 4 + i;
#pragma unroll
      for (int gj = 0; gj < RN / 4; ++gj) {
        T v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = acc[gi * 4 + i][gj * 4 + j];
        gstore4x<T, VEC, EDGE>(d, ld, n, row, col0 + gj * S::kGroupColStride + tc * 4, v, cv,
                               inf32);
      }
    }
}

// Loads the C tile into acc and applies acc <- min(acc, A (x) B) over the kB
// pivots of block kb0; acc stays in registers (the caller stores it).
// Per pair of pivots each accumulator takes one mp_relax2 (two adds, one
// three-input min).
// Chunks c_begin .. c_begin + c_count - 1 of kKC pivots are applied (all
// kB pivots by default); tid is the thread's index within the 256 threads
// that share `lds`.  Ends with a barrier after its last LDS reads.
// MASK: successor keys; the B operand (pivot rows) is staged with its low
// bits cleared (AND with km), so each sum keeps A's first hop.
template <typename T, int TM, int TN, int RM, int RN, bool VEC, bool EDGE, bool MASK = false>
__device__ __forceinline__ void minplus_update(const T* __restrict__ d, int64_t n, int64_t ld,
                                               T inf, int64_t row0, int64_t col0, int64_t kb0,
                                               T* __restrict__ lds, T (&acc)[RM][RN],
                                               int c_begin = 0, int c_count = kB / kKC,
                                               int tid = threadIdx.x, int conv = 0,
                                               int32_t inf32 = 0, T km = T(0)) {
  using S = TileShape<T, TM, TN, RM, RN>;
  T* sA = lds;                              // [2][kKC][kLdA]
  T* sB = lds + 2 * kKC * S::kLdA;          // [2][kKC][kLdB]

  const int tc = tid % S::kThrCols;
  const int tr = tid / S::kThrCols;

  // Prefetch registers for one chunk of A and B.
  T ga[S::kLoadsA][4];
  T gb[S::kLoadsB][4];

  auto fetch = [&](int chunk) {
    const int64_t k0 = kb0 + (int64_t)chunk * kKC;
#pragma unroll
    for (int l = 0; l < S::kLoadsA; ++l) {
      const int q = tid + l * kThreads;
      if (S::kQuadsA % kThreads == 0 || q < S::kQuadsA) {
        const int r = q / (kKC / 4), kq = q % (kKC / 4);
        gload4x<T, VEC, EDGE>(d, ld, n, row0 + r, k0 + kq * 4, inf, ga[l], conv & kConvA, inf32);
      }
    }
#pragma unroll
    for (int l = 0; l < S::kLoadsB; ++l) {
      const int q = tid + l * kThreads;
      if (S::kQuadsB % kThreads == 0 || q < S::kQuadsB) {
        const int kr = q / (TN / 4), cq = q % (TN / 4);
        gload4x<T, VEC, EDGE>(d, ld, n, k0 + kr, col0 + cq * 4, inf, gb[l], conv & kConvB, inf32);
      }
    }
  };
  auto stash = [&](int buf) {
    T* a = sA + buf * kKC * S::kLdA;
    T* b = sB + buf * kKC * S::kLdB;
#pragma unroll
    for (int l = 0; l < S::kLoadsA; ++l) {
      const int q = tid + l * kThreads;
      if (S::kQuadsA % kThreads == 0 || q < S::kQuadsA) {
        const int r = q / (kKC / 4), kq = q % (kKC / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[(kq * 4 + e) * S::kLdA + r] = ga[l][e];
      }
    }
#pragma unroll
    for (int l = 0; l < S::kLoadsB; ++l) {
      const int q = tid + l * kThreads;
      if (S::kQuadsB % kThreads == 0 || q < S::kQuadsB) {
        const int kr = q / (TN / 4), cq = q % (TN / 4);
        if constexpr (MASK) {
#pragma unroll
          for (int e = 0; e < 4; ++e) gb[l][e] &= km;
        }
        store4(b + kr * S::kLdB + cq * 4, gb[l]);
      }
    }
  };

  fetch(c_begin);
  load_tile<T, TM, TN, RM, RN, VEC, EDGE>(d, n, ld, inf, row0, col0, acc, tid, conv & kConvC,
                                          inf32);
  stash(0);
  __syncthreads();

#pragma unroll 1
  for (int c = 0; c < c_count; ++c) {
    const int buf = c & 1;
    if (c + 1 < c_count) fetch(c_begin + c + 1);
    const T* a = sA + buf * kKC * S::kLdA;
    const T* b = sB + buf * kKC * S::kLdB;
#pragma unroll
    for (int k = 0; k < kKC; k += 2) {
      T a0[RM], b0[RN], a1[RM], b1[RN];
#pragma unroll
      for (int gi = 0; gi < RM / 4; ++gi) {
        T v[4];
        load4(a + k * S::kLdA + gi * S::kGroupRowStride + tr * 4, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) a0[gi * 4 + i] = v[i];
        load4(a + (k + 1) * S::kLdA + gi * S::kGroupRowStride + tr * 4, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) a1[gi * 4 + i] = v[i];
      }
#pragma unroll
      for (int gj = 0; gj < RN / 4; ++gj) {
        T v[4];
        load4(b + k * S::kLdB + gj * S::kGroupColStride + tc * 4, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) b0[gj * 4 + j] = v[j];
        load4(b + (k + 1) * S::kLdB + gj * S::kGroupColStride + tc * 4, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) b1[gj * 4 + j] = v[j];
      }
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j)
          acc[i][j] = mp_relax2(acc[i][j], a0[i], b0[j], a1[i], b1[j]);
    }
    if (c + 1 < c_count) stash(buf ^ 1);
    __syncthreads();
  }
}


// Phase-2 panel tiles: the row panel is split into kB x kP2 tiles, the column
// panel into kP2 x kB tiles.
constexpr int kP2 = APSP_P2_TILE;
using P2Row = TileShape<int32_t, kB, kP2, 4, 4>;
using P2Col = TileShape<int32_t, kP2, kB, 4, 4>;
using P3 = TileShape<int32_t, kB, kB, 8, 8>;
constexpr int kLdsP2 = P2Row::kLdsElems > P2Col::kLdsElems ? P2Row::kLdsElems : P2Col::kLdsElems;
constexpr int kLdsP3 = P3::kLdsElems;
constexpr int kLdsClose = 8 * kB;  // two pivot columns + two pivot rows, two buffers

// The kB x kB block of a 256-thread workgroup in the Phase-3 layout.
template <typename T, bool MASK = false>
__device__ __forceinline__ void close_block(T (&acc)[8][8], T* __restrict__ lds, T km = T(0)) {
  close_block_t<T, kB, 8, MASK>(acc, lds, km);
}

// The same closure one pivot per step (d <- min(d, d[x][t] + d[t][y]), one
// barrier per pivot), for the next-round Phase 1 fused into the Phase-3
// kernel.  There the pair-step version above made the Phase-3 tile loop
// itself about 4 % slower (measured at n = 8192, also with the fused path
// switched off, so the cost lies in the compiled kernel, not in the closure's
// run time); the fused closure is off the critical path at large n.
template <typename T, bool MASK = false>
__device__ __forceinline__ void close_block_seq(T (&acc)[8][8], T* __restrict__ lds,
                                                T km = T(0)) {
  T* colv = lds;            // [2][kB]: column t at every row
  T* rowv = lds + 2 * kB;   // [2][kB]: row t at every column
  const int tc = threadIdx.x % 16;
  const int tr = threadIdx.x / 16;

  // publish pivot 0: column 0 lives in group gj = 0, lane tc = 0, slot 0
  if (tc == 0) {
    T v0[4] = {acc[0][0], acc[1][0], acc[2][0], acc[3][0]};
    T v1[4] = {acc[4][0], acc[5][0], acc[6][0], acc[7][0]};
    store4(&colv[tr * 4], v0);
    store4(&colv[64 + tr * 4], v1);
  }
  if (tr == 0) {
    T v0[4] = {acc[0][0], acc[0][1], acc[0][2], acc[0][3]};
    T v1[4] = {acc[0][4], acc[0][5], acc[0][6], acc[0][7]};
    if constexpr (MASK) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v0[e] &= km;
        v1[e] &= km;
      }
    }
    store4(&rowv[tc * 4], v0);
    store4(&rowv[64 + tc * 4], v1);
  }
  __syncthreads();

  // pivot t = 64 * g + 4 * q + c: group g, owner lane q, slot c
#pragma unroll
  for (int g = 0; g < 2; ++g) {
#pragma unroll 1
    for (int q = 0; q < 16; ++q) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int p = c & 1;  // (64g + 4q + c) & 1
        T a[8], b[8];
        {
          T v[4];
          load4(&colv[p * kB + tr * 4], v);
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] = v[i];
          load4(&colv[p * kB + 64 + tr * 4], v);
#pragma unroll
          for (int i = 0; i < 4; ++i) a[4 + i] = v[i];
          load4(&rowv[p * kB + tc * 4], v);
#pragma unroll
          for (int j = 0; j < 4; ++j) b[j] = v[j];
          load4(&rowv[p * kB + 64 + tc * 4], v);
#pragma unroll
          for (int j = 0; j < 4; ++j) b[4 + j] = v[j];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = mp_min(acc[i][j], a[i] + b[j]);

        // publish pivot t + 1 into the other buffer
        auto publish = [&](int owner, int slot) {
          T* cv = colv + (p ^ 1) * kB;
          T* rv = rowv + (p ^ 1) * kB;
          if (tc == owner) {
            T v0[4] = {acc[0][slot], acc[1][slot], acc[2][slot], acc[3][slot]};
            T v1[4] = {acc[4][slot], acc[5][slot], acc[6][slot], acc[7][slot]};
            store4(&cv[tr * 4], v0);
            store4(&cv[64 + tr * 4], v1);
          }
          if (tr == owner) {
            T v0[4] = {acc[slot][0], acc[slot][1], acc[slot][2], acc[slot][3]};
            T v1[4] = {acc[slot][4], acc[slot][5], acc[slot][6], acc[slot][7]};
            if constexpr (MASK) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                v0[e] &= km;
                v1[e] &= km;
              }
            }
            store4(&rv[tc * 4], v0);
            store4(&rv[64 + tc * 4], v1);
          }
        };
        if (c < 3) {
          publish(q, g * 4 + c + 1);
        } else if (q < 15) {
          publish(q + 1, g * 4);
        } else if (g == 0) {
          publish(0, 4);
        }
        __syncthreads();
      }
    }
  }
}

// Standalone Phase 1 (first round of a call): one workgroup of kP1Threads
// threads, a 4 x 4 micro-tile each (32 x 32 threads over the 128 x 128
// block), closing the block two pivots per barrier.  It is one workgroup
// alone on the GPU, so it runs 16 waves rather than the Phase-3 layout's 4:
// each pivot pair's work spreads over four waves per SIMD.  conv: kConvC
// converts the block on load, kConvOut on store.
constexpr int kP1Threads = 1024;
template <typename T, bool VEC, bool EDGE, bool MASK = false>
__device__ __forceinline__ void phase1_wide(T* __restrict__ d, int64_t n, int64_t ld, T inf,
                                            int64_t base, T* __restrict__ lds, int conv,
                                            int32_t inf32, T km = T(0)) {
  constexpr int kThr = kB / 4;
  static_assert(kThr * kThr == kP1Threads, "4 x 4 per thread");
  const int tc = threadIdx.x % kThr, tr = threadIdx.x / kThr;
  T acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    gload4x<T, VEC, EDGE>(d, ld, n, base + tr * 4 + i, base + tc * 4, inf, acc[i],
                          conv & kConvC, inf32);
  close_block_t<T, kB, 4, MASK>(acc, lds, km);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    gstore4x<T, VEC, EDGE>(d, ld, n, base + tr * 4 + i, base + tc * 4, acc[i],
                           (conv & kConvOut) != 0, inf32);
}

template <typename T, bool VEC, bool MASK = false>
__device__ __forceinline__ void phase1_body(T* __restrict__ d, int64_t n, int64_t ld, T inf,
                                            int64_t K, T* __restrict__ lds, int conv,
                                            int32_t inf32, T km = T(0)) {
  const int64_t base = K * kB;
  if (base + kB <= n)
    phase1_wide<T, VEC, false, MASK>(d, n, ld, inf, base, lds, conv, inf32, km);
  else
    phase1_wide<T, VEC, true, MASK>(d, n, ld, inf, base, lds, conv, inf32, km);
}

// ---------------------------------------------------------------------------
// Phase 2: pivot-row tiles (blocks 0 .. nr-1) then pivot-column tiles.
//
// A Phase-2 piece (kB x kP2 or kP2 x kB, kB pivots) has too little work per
// thread for its 4 x 4 micro-tile to keep the VALU fed: 2048 relaxations
// per thread in a row, two waves per SIMD.  So each 512-thread workgroup
// splits the pivot depth between its two halves: threads 0-255 apply pivot
// chunks 0-3, threads 256-511 chunks 4-7, each half from its own LDS
// buffers and starting from the same tile.  The second half then hands its
// accumulators over LDS and the first stores the elementwise minimum, which
// is min(C, A (x) B) over all kB pivots (min is exact and order-free, so the
// result is the same bit for bit as one half applying all pivots).
// ---------------------------------------------------------------------------
constexpr int kP2Threads = 2 * kThreads;
template <typename T, int TM, int TN, bool VEC, bool EDGE, bool MASK = false>
__device__ __forceinline__ void p2_halves(T* __restrict__ d, int64_t n, int64_t ld, T inf,
                                          int64_t row0, int64_t col0, int64_t kb0,
                                          T* __restrict__ lds, int conv, int32_t inf32,
                                          T km = T(0)) {
  using S = TileShape<T, TM, TN, 4, 4>;
  constexpr int kHalf = kB / kKC / 2;  // chunks per half
  const int half = threadIdx.x / kThreads;
  const int tid = threadIdx.x % kThreads;
  T acc[4][4];
  minplus_update<T, TM, TN, 4, 4, VEC, EDGE, MASK>(d, n, ld, inf, row0, col0, kb0,
                                                   lds + half * S::kLdsElems, acc, half * kHalf,
                                                   kHalf, tid, conv, inf32, km);
  // Both halves passed minplus_update's final barrier: the LDS is free.
  constexpr int kLdR = TN + kPad;
  static_assert(TM * kLdR <= 2 * S::kLdsElems, "the hand-over fits the LDS");
  const int tc = tid % S::kThrCols, tr = tid / S::kThrCols;
  if (half == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) store4(lds + (tr * 4 + i) * kLdR + tc * 4, acc[i]);
  }
  __syncthreads();
  if (half == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      T v[4];
      load4(lds + (tr * 4 + i) * kLdR + tc * 4, v);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mp_min(acc[i][j], v[j]);
    }
    store_tile<T, TM, TN, 4, 4, VEC, EDGE>(d, n, ld, row0, col0, acc, tid, conv & kConvOut,
                                           inf32);
  }
}

template <typename T, int TM, int TN, bool VEC, bool MASK = false>
__device__ __forceinline__ void p2_piece(T* __restrict__ d, int64_t n, int64_t ld, T inf,
                                         int64_t row0, int64_t col0, int64_t kb0,
                                         T* __restrict__ lds, int conv, int32_t inf32,
                                         T km = T(0)) {
  if (row0 + TM <= n && col0 + TN <= n && kb0 + kB <= n)
    p2_halves<T, TM, TN, VEC, false, MASK>(d, n, ld, inf, row0, col0, kb0, lds, conv, inf32, km);
  else
    p2_halves<T, TM, TN, VEC, true, MASK>(d, n, ld, inf, row0, col0, kb0, lds, conv, inf32, km);
}

// conv: kConvC converts the piece's own entries on load (as C and as its
// operand: B of a row piece, A of a column piece; D_KK is already binary32),
// kConvOut converts on store.
template <typename T, bool VEC, bool MASK = false>
__device__ __forceinline__ void phase2_body(T* __restrict__ d, int64_t n, int64_t ld, T inf,
                                            int64_t K, int64_t nb, T* __restrict__ lds, int conv,
                                            int32_t inf32, T km = T(0)) {
  const int own = (conv & kConvC) ? kConvC : 0;
  constexpr int kSub = kB / kP2;
  const int64_t nr = (nb - 1) * kSub;
  int64_t b = blockIdx.x;
  const int64_t kb0 = K * kB;
  if (b < nr) {
    const int64_t jp = b / kSub, sub = b % kSub;
    const int64_t J = jp + (jp >= K);
    const int64_t col0 = J * kB + sub * kP2;
    if (col0 >= n) return;
    p2_piece<T, kB, kP2, VEC, MASK>(d, n, ld, inf, kb0, col0, kb0, lds,
                                    own | (own ? kConvB : 0) | (conv & kConvOut), inf32, km);
  } else {
    b -= nr;
    const int64_t ip = b / kSub, sub = b % kSub;
    const int64_t I = ip + (ip >= K);
    const int64_t row0 = I * kB + sub * kP2;
    if (row0 >= n) return;
    p2_piece<T, kP2, kB, VEC, MASK>(d, n, ld, inf, row0, kb0, kb0, lds,
                                    own | (own ? kConvA : 0) | (conv & kConvOut), inf32, km);
  }
}

// ---------------------------------------------------------------------------
// Phase 3: every tile (I, J) with I != K and J != K; m = nb - 1 tiles a side.
//
// Work order.  The hardware hands workgroup b to XCD b % 8 (8 XCDs, each
// with its own L2).  Each XCD is given a contiguous range of the tile
// sequence, and the sequence walks bands of kBand tile rows column by column,
// so the workgroups resident on one XCD share a few pivot-column panels
// (rows I) and pivot-row panels (columns J) through that XCD's L2.
//
// Next-round Phase 1.  When fuse_next is set, workgroup 0 takes tile
// (K+1, K+1): after its Phase-3 update it closes the block in registers
// (Phase 1 of round K+1) before storing it.  No other workgroup of this
// launch reads that tile, and round K+1 starts with Phase 2.
// ---------------------------------------------------------------------------
constexpr uint32_t kXcds = 8;
constexpr uint32_t kBand = 8;

__device__ __forceinline__ void p3_decode(uint32_t L, uint32_t m, uint32_t& ip, uint32_t& jp) {
  const uint32_t g = L / (kBand * m);
  const uint32_t base = g * kBand;
  const uint32_t rows = min(kBand, m - base);
  const uint32_t r = L - g * kBand * m;
  ip = base + r % rows;
  jp = r / rows;
}

__device__ __forceinline__ uint32_t p3_encode(uint32_t ip, uint32_t jp, uint32_t m) {
  const uint32_t g = ip / kBand;
  const uint32_t base = g * kBand;
  const uint32_t rows = min(kBand, m - base);
  return g * kBand * m + jp * rows + (ip - base);
}

// The launch's last, partial wave of tiles.  With R workgroups resident
// per CU the tiles run in waves of R x CUs; when the tile count leaves a
// short last wave, that wave would hold the whole launch for one more tile
// time while most CUs idle.  The host keeps the first `full` tiles whole
// and hands each remaining tile to four workgroups, one 64 x 64 quarter
// each (all kB pivots, 4 x 4 accumulators per thread): the dispatcher
// starts them as the last whole tiles free their slots, and a quarter takes
// a fraction of a tile's time.  Workgroups b < full take whole tiles,
// b >= full quarter (b - full) % 4 of tile full + (b - full) / 4.
//
// conv: kConvC converts the C tile on load (first round), kConvOut the
// stores (last round).  The body can also convert its pivot operands
// (kConvA, kConvB) and, in workgroup 0, send block (K, K) back (kConvDiag);
// the round schedule no longer asks for those (the last round keeps its
// pivot row and column in binary32 and converts them after Phase 3), but
// taking that code out of this shared body made the kernels every other
// round runs 1.5 % slower, so it stays.
template <typename T, bool VEC, bool PAIR_CLOSE = false, bool MASK = false>
__device__ __forceinline__ void phase3_body(T* __restrict__ d, int64_t n, int64_t ld, T inf,
                                            int64_t K, int64_t nb, int fuse_next, uint32_t full,
                                            T* __restrict__ lds, int conv, int32_t inf32,
                                            T km = T(0)) {
  const uint32_t m = (uint32_t)(nb - 1);
  const uint32_t b = blockIdx.x;
  const uint32_t kp = (uint32_t)K;  // tile (K+1, K+1) is (kp, kp) in the skipped grid
  const int tid = threadIdx.x;
  const int cin = conv & (kConvC | kConvA | kConvB);
  const bool cout = (conv & kConvOut) != 0;
  const int64_t kb0 = K * kB;
  const uint32_t ls = fuse_next ? p3_encode(kp, kp, m) : 0;
  if (b >= full) {
    const uint32_t p = b - full;
    uint32_t L = full + p / 4;
    if (fuse_next && L == ls) L = 0;  // tile 0 went to workgroup 0 (full >= 1 then)
    uint32_t ip, jp;
    p3_decode(L, m, ip, jp);
    const int64_t I = ip + (ip >= kp), J = jp + (jp >= kp);
    const int64_t row0 = I * kB + (p % 4 / 2) * (kB / 2), col0 = J * kB + (p % 2) * (kB / 2);
    if (row0 >= n || col0 >= n) return;
    T acc[4][4];
    if (row0 + kB / 2 <= n && col0 + kB / 2 <= n && kb0 + kB <= n) {
      minplus_update<T, kB / 2, kB / 2, 4, 4, VEC, false, MASK>(d, n, ld, inf, row0, col0, kb0,
                                                                lds, acc, 0, kB / kKC, tid, cin,
                                                                inf32, km);
      store_tile<T, kB / 2, kB / 2, 4, 4, VEC, false>(d, n, ld, row0, col0, acc, tid, cout,
                                                      inf32);
    } else {
      minplus_update<T, kB / 2, kB / 2, 4, 4, VEC, true, MASK>(d, n, ld, inf, row0, col0, kb0,
                                                               lds, acc, 0, kB / kKC, tid, cin,
                                                               inf32, km);
      store_tile<T, kB / 2, kB / 2, 4, 4, VEC, true>(d, n, ld, row0, col0, acc, tid, cout,
                                                     inf32);
    }
    return;
  }
  const uint32_t x = b % kXcds, j = b / kXcds;
  const uint32_t q = full / kXcds, rem = full % kXcds;
  uint32_t L = x * q + min(x, rem) + j;
  const bool special = fuse_next && L == 0;
  if (fuse_next) {
    if (L == 0) L = ls;
    else if (L == ls) L = 0;
  }
  uint32_t ip, jp;
  p3_decode(L, m, ip, jp);
  const int64_t I = ip + (ip >= kp), J = jp + (jp >= kp);
  const int64_t row0 = I * kB, col0 = J * kB;

  T acc[8][8];
  const bool interior = row0 + kB <= n && col0 + kB <= n && kb0 + kB <= n;
  if (interior) {
    minplus_update<T, kB, kB, 8, 8, VEC, false, MASK>(d, n, ld, inf, row0, col0, kb0, lds, acc,
                                                      0, kB / kKC, tid, cin, inf32, km);
    if (special) {
      if constexpr (PAIR_CLOSE) close_block<T, MASK>(acc, lds, km);
      else close_block_seq<T, MASK>(acc, lds, km);
    }
    store_tile<T, kB, kB, 8, 8, VEC, false>(d, n, ld, row0, col0, acc, tid, cout, inf32);
  } else {
    minplus_update<T, kB, kB, 8, 8, VEC, true, MASK>(d, n, ld, inf, row0, col0, kb0, lds, acc,
                                                     0, kB / kKC, tid, cin, inf32, km);
    if (special) {
      if constexpr (PAIR_CLOSE) close_block<T, MASK>(acc, lds, km);
      else close_block_seq<T, MASK>(acc, lds, km);
    }
    store_tile<T, kB, kB, 8, 8, VEC, true>(d, n, ld, row0, col0, acc, tid, cout, inf32);
  }
  if ((conv & kConvDiag) && b == 0) {
    // Block (K, K) back to int32, in place (it holds binary32 bits).
    if (kb0 + kB <= n) {
      load_tile<T, kB, kB, 8, 8, VEC, false>(d, n, ld, inf, kb0, kb0, acc, tid);
      store_tile<T, kB, kB, 8, 8, VEC, false>(d, n, ld, kb0, kb0, acc, tid, true, inf32);
    } else {
      load_tile<T, kB, kB, 8, 8, VEC, true>(d, n, ld, inf, kb0, kb0, acc, tid);
      store_tile<T, kB, kB, 8, 8, VEC, true>(d, n, ld, kb0, kb0, acc, tid, true, inf32);
    }
  }
}

// ---------------------------------------------------------------------------
// int32 matrices in binary32 arithmetic.
//
// gfx950 issues binary32 adds and mins at twice the rate of int32 adds and
// mins, so an int32 matrix is computed in binary32 whenever that is exact.
// It is exact when every finite entry is an integer in [0, 2^24] and every
// shortest distance -- and every distance restricted to intermediate vertices
// below some pivot, which bounds each value the blocked recurrence stores --
// is at most 2^24.  Then each value the recurrence keeps is the exact integer
// (a candidate that realises a value <= 2^24 sums two exact values whose
// exact sum is representable; any other candidate is >= that value even
// after rounding, since rounding is monotone and 2^24 is representable).
// The distance bound holds when no off-diagonal entry is inf (each distance
// is at most the direct edge, hence at most the largest weight), or when
// (n - 1) times the largest finite weight is at most 2^24 (a shortest path
// is simple).  A scan kernel records the largest finite entry and two flags
// in a small stream-ordered scratch; every later kernel of the call reads
// them and takes the binary32 or the int32 body.  Entries equal to inf
// become +infinity and come back as inf; finite results are clamped to inf,
// which is what int32 arithmetic would store when a sum is not below inf.
// ---------------------------------------------------------------------------
constexpr int32_t kFlagHasInf = 1;     // some off-diagonal entry equals inf
constexpr int32_t kFlagNotExact = 2;   // a negative entry, or a finite one above 2^24
constexpr int64_t kExactLimit = int64_t(1) << 24;
constexpr int kScanBlocks = 2048;

__device__ __forceinline__ bool f32_exact(const int32_t* __restrict__ s, int64_t n) {
  if (s == nullptr) return false;
  const int32_t maxw = s[0];
  const int32_t flags = s[1];
  if (flags & kFlagNotExact) return false;
  if (!(flags & kFlagHasInf)) return true;
  return (n - 1) * (int64_t)maxw <= kExactLimit;
}

__global__ void __launch_bounds__(64) scan_zero(int32_t* __restrict__ s) {
  if (threadIdx.x < 2) s[threadIdx.x] = 0;
}

template <bool VEC>
__global__ void __launch_bounds__(kThreads) scan_i32(const int32_t* __restrict__ d, int64_t n,
                                                     int64_t ld, int32_t inf,
                                                     int32_t* __restrict__ s) {
  int32_t mx = 0, fl = 0;
  auto visit = [&](int32_t v, int64_t r, int64_t c) {
    if (v == inf) {
      if (r != c) fl |= kFlagHasInf;
    } else {
      if (v < 0 || v > kExactLimit) fl |= kFlagNotExact;
      mx = max(mx, v);
    }
  };
  const int64_t quads = (n + 3) / 4;
  const int64_t full = VEC ? n / 4 : 0;  // quads wholly inside the row
  for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
    const int32_t* row = d + r * ld;
    int64_t q = threadIdx.x;
    // Four quads in flight per thread before any is visited.
    for (; q + 3 * kThreads < full; q += 4 * kThreads) {
      int32_t v[4][4];
#pragma unroll
      for (int k = 0; k < 4; ++k) load4(row + (q + k * kThreads) * 4, v[k]);
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) visit(v[k][e], r, (q + k * kThreads) * 4 + e);
    }
    for (; q < quads; q += kThreads) {
      const int64_t c = q * 4;
      if (VEC && c + 3 < n) {
        int32_t v[4];
        load4(row + c, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) visit(v[e], r, c + e);
      } else {
        for (int e = 0; e < 4 && c + e < n; ++e) visit(row[c + e], r, c + e);
      }
    }
  }
  // Workgroup reduction, then at most one atomic pair per workgroup: the
  // stored values only grow, so a workgroup whose result is already covered
  // by what it reads skips the atomic (thousands of workgroups would
  // otherwise serialise on the same two words).
  __shared__ int32_t red[2][kThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mx = max(mx, __shfl_xor(mx, o));
    fl |= __shfl_xor(fl, o);
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x / 64] = mx;
    red[1][threadIdx.x / 64] = fl;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) {
      mx = max(mx, red[0][w]);
      fl |= red[1][w];
    }
    const int32_t cur_mx = __hip_atomic_load(&s[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int32_t cur_fl = __hip_atomic_load(&s[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (mx > cur_mx) atomicMax(&s[0], mx);
    if (fl & ~cur_fl) atomicOr(&s[1], fl);
  }
}

// ---------------------------------------------------------------------------
// Kernels.  fw_phase* run one element type; fw_phase*_i32 serve int32
// matrices and take the binary32 body when the call's scan says it is exact,
// converting on the first round's loads and the last round's stores as
// `conv` says (see kConvC).  Only the CONV instances convert: the rounds in
// between run instances with no conversion code in their loops.
// ---------------------------------------------------------------------------
template <typename T, bool VEC>
__global__ void __launch_bounds__(kP1Threads) fw_phase1(T* __restrict__ d, int64_t n, int64_t ld,
                                                      T inf, int64_t K) {
  __shared__ __attribute__((aligned(16))) T lds[kLdsClose];
  phase1_body<T, VEC>(d, n, ld, inf, K, lds, 0, 0);
}

template <typename T, bool VEC>
__global__ void __launch_bounds__(kP2Threads) __attribute__((amdgpu_waves_per_eu(kWavesP2)))
fw_phase2(T* __restrict__ d, int64_t n, int64_t ld, T inf, int64_t K, int64_t nb) {
  __shared__ __attribute__((aligned(16))) T lds[2 * kLdsP2];
  phase2_body<T, VEC>(d, n, ld, inf, K, nb, lds, 0, 0);
}

template <typename T, bool VEC, bool PC>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesP3)))
fw_phase3(T* __restrict__ d, int64_t n, int64_t ld, T inf, int64_t K, int64_t nb, int fuse_next,
          uint32_t full) {
  __shared__ __attribute__((aligned(16))) T lds[kLdsP3];
  phase3_body<T, VEC, PC>(d, n, ld, inf, K, nb, fuse_next, full, lds, 0, 0);
}

template <bool VEC, bool CONV>
__global__ void __launch_bounds__(kP1Threads) fw_phase1_i32(int32_t* __restrict__ d, int64_t n,
                                                          int64_t ld, int32_t inf, int64_t K,
                                                          int conv,
                                                          const int32_t* __restrict__ s) {
  __shared__ __attribute__((aligned(16))) int32_t lds[kLdsClose];
  if (f32_exact(s, n))
    phase1_body<float, VEC>(reinterpret_cast<float*>(d), n, ld, __builtin_inff(), K,
                            reinterpret_cast<float*>(lds), CONV ? conv : 0, inf);
  else
    phase1_body<int32_t, VEC>(d, n, ld, inf, K, lds, 0, 0);
}

template <bool VEC, bool CONV>
__global__ void __launch_bounds__(kP2Threads) __attribute__((amdgpu_waves_per_eu(kWavesP2)))
fw_phase2_i32(int32_t* __restrict__ d, int64_t n, int64_t ld, int32_t inf, int64_t K, int64_t nb,
              int conv, const int32_t* __restrict__ s) {
  __shared__ __attribute__((aligned(16))) int32_t lds[2 * kLdsP2];
  if (f32_exact(s, n))
    phase2_body<float, VEC>(reinterpret_cast<float*>(d), n, ld, __builtin_inff(), K, nb,
                            reinterpret_cast<float*>(lds), CONV ? conv : 0, inf);
  else
    phase2_body<int32_t, VEC>(d, n, ld, inf, K, nb, lds, 0, 0);
}

template <bool VEC, bool CONV, bool PC>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesP3)))
fw_phase3_i32(int32_t* __restrict__ d, int64_t n, int64_t ld, int32_t inf, int64_t K, int64_t nb,
              int fuse_next, uint32_t full, int conv, const int32_t* __restrict__ s) {
  __shared__ __attribute__((aligned(16))) int32_t lds[kLdsP3];
  if (f32_exact(s, n))
    phase3_body<float, VEC, PC>(reinterpret_cast<float*>(d), n, ld, __builtin_inff(), K, nb,
                                fuse_next, full, reinterpret_cast<float*>(lds),
                                CONV ? conv : 0, inf);
  else
    phase3_body<int32_t, VEC, PC>(d, n, ld, inf, K, nb, fuse_next, full, lds, 0, 0);
}

// ---------------------------------------------------------------------------
// Successor keys: distances and first hops in one pass of the rounds.
//
// The matrix holds int32 keys v << s | h, with s the bit width of n (so
// 2^s > n and h = 2^s - 1 names no vertex) and "no edge" the key
// 2^30 - 2^s.  For a pivot k the sum (a << s | h) + (b << s) =
// (a + b) << s | h stands for the walk i -> k -> j with the first hop h of
// its i -> k part, and the minimum of keys orders by value, then by first
// hop.  So the blocked recurrence, run unchanged on keys with the low s bits
// of every pivot-row operand cleared, leaves in each entry the smallest
// (distance, first hop) over the walks it has seen, which at the end is the
// shortest distance and the smallest first hop of a shortest path: the
// successor of the page "Study of Betweenness Centrality Algorithms in GPU"
// (predecessor arrays), with the same tie rule as the separate successor
// pass.  Keys stay exact and below 2^31 when every value the recurrence
// stores is below 2^(30-s) - 1; the caller checks that before choosing
// this path.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int32_t key_mask(int64_t n) {
  const int s = 32 - __clz((int)n);  // 1 <= n < 2^29 on this path
  return (int32_t)(~((1u << s) - 1u));
}

template <bool VEC>
__global__ void __launch_bounds__(kP1Threads) fw_keys_phase1(int32_t* __restrict__ d, int64_t n,
                                                           int64_t ld, int32_t inf, int64_t K) {
  __shared__ __attribute__((aligned(16))) int32_t lds[kLdsClose];
  phase1_body<int32_t, VEC, true>(d, n, ld, inf, K, lds, 0, 0, key_mask(n));
}

template <bool VEC>
__global__ void __launch_bounds__(kP2Threads) __attribute__((amdgpu_waves_per_eu(kWavesP2)))
fw_keys_phase2(int32_t* __restrict__ d, int64_t n, int64_t ld, int32_t inf, int64_t K,
               int64_t nb) {
  __shared__ __attribute__((aligned(16))) int32_t lds[2 * kLdsP2];
  phase2_body<int32_t, VEC, true>(d, n, ld, inf, K, nb, lds, 0, 0, key_mask(n));
}

template <bool VEC>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesP3)))
fw_keys_phase3(int32_t* __restrict__ d, int64_t n, int64_t ld, int32_t inf, int64_t K,
               int64_t nb, int fuse_next, uint32_t full) {
  __shared__ __attribute__((aligned(16))) int32_t lds[kLdsP3];
  phase3_body<int32_t, VEC, false, true>(d, n, ld, inf, K, nb, fuse_next, full, lds, 0, 0,
                                         key_mask(n));
}

// After the last round of a binary32 call: round K's pivot row and column
// (block (K, K) included) back to int32, in place.  That round's Phase 2
// left them in binary32, so its Phase 3 read its operands without a
// conversion in the pivot loop, and converted every other block on store.
// Workgroup r takes matrix row r: the whole row inside the pivot block,
// else its kB entries in the pivot columns.
__global__ void __launch_bounds__(kThreads) pivot_panels_to_i32(int32_t* __restrict__ d,
                                                                int64_t n, int64_t ld,
                                                                int32_t inf, int64_t K,
                                                                const int32_t* __restrict__ s) {
  if (!f32_exact(s, n)) return;
  const int64_t r = blockIdx.x;
  const int64_t k0 = K * kB, k1 = k0 + kB < n ? k0 + kB : n;
  const bool pivot_row = r >= k0 && r < k1;
  const int64_t c0 = pivot_row ? 0 : k0, c1 = pivot_row ? n : k1;
  int32_t* row = d + r * ld;
  for (int64_t c = c0 + threadIdx.x; c < c1; c += kThreads)
    row[c] = f32_to_i32(__int_as_float(row[c]), inf);
}

// ---------------------------------------------------------------------------
// Negative weights in the dense matrix (the setting of the Johnson's-APSP
// page, where Floyd-Warshall must not treat "no edge" as a number).
//
// No guard is needed in the min-plus loops.  Let W be the largest |weight|
// over finite off-diagonal entries and assume no negative cycle.
//  * binary32: "no edge" becomes +infinity, and +inf plus any finite value
//    is +inf, which is exactly the guard.  Every value the recurrence keeps
//    is a walk length between -(n-1)W and (n-1)W, so when (n-1)W <= 2^24
//    each is an exactly representable integer and, as for non-negative
//    weights, the rounded minimum over the candidates is the exact one.
//  * int32: "no edge" stays the number inf = M.  In the complete graph with
//    weight M on non-edges, a simple path that uses a non-edge weighs at
//    least M - (n-2)W, and a cycle that uses one weighs at least
//    M - (n-1)W > 0, so that graph has no negative cycle either.  Its
//    shortest distances equal the true ones (at most (n-1)W) on reachable
//    pairs when M > (2n-3)W, and exceed (n-1)W on the others.  The plain
//    recurrence computes them without overflow (values stay in
//    [-(n-1)W, M], sums in [-2(n-1)W, 2M]); a final pass maps every value
//    above (n-1)W back to inf.  With no non-edge at all the same holds when
//    (n-1)W < 2^30.
// A negative cycle shows as some d(i, i) < 0 after the rounds (a stored
// value never increases, so a negative diagonal stays negative).
// ---------------------------------------------------------------------------
constexpr int32_t kSgHasInf = 1;      // an off-diagonal entry equals inf
constexpr int32_t kSgBadEntry = 2;    // a diagonal entry != 0, or an entry outside (-inf, inf]
struct SignedScan {
  int32_t maxabs;     // largest |finite off-diagonal entry|
  int32_t flags;
  int32_t neg_cycle;  // some d(i, i) < 0 after the rounds
  int32_t pad;
};

__global__ void __launch_bounds__(64) signed_zero(SignedScan* __restrict__ s) {
  if (threadIdx.x == 0) *s = SignedScan{0, 0, 0, 0};
}

template <bool VEC>
__global__ void __launch_bounds__(kThreads) scan_signed_i32(const int32_t* __restrict__ d,
                                                            int64_t n, int64_t ld, int32_t inf,
                                                            SignedScan* __restrict__ s) {
  int32_t mx = 0, fl = 0;
  auto visit = [&](int32_t v, int64_t r, int64_t c) {
    if (r == c) {
      if (v != 0) fl |= kSgBadEntry;
    } else if (v == inf) {
      fl |= kSgHasInf;
    } else if (v > inf || v <= -inf) {
      fl |= kSgBadEntry;
    } else {
      mx = max(mx, v < 0 ? -v : v);
    }
  };
  const int64_t quads = (n + 3) / 4;
  for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
    const int32_t* row = d + r * ld;
    for (int64_t q = threadIdx.x; q < quads; q += kThreads) {
      const int64_t c = q * 4;
      if (VEC && c + 3 < n) {
        int32_t v[4];
        load4(row + c, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) visit(v[e], r, c + e);
      } else {
        for (int e = 0; e < 4 && c + e < n; ++e) visit(row[c + e], r, c + e);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mx = max(mx, __shfl_xor(mx, o));
    fl |= __shfl_xor(fl, o);
  }
  if ((threadIdx.x & 63) == 0) {
    if (mx) atomicMax(&s->maxabs, mx);
    if (fl) atomicOr(&s->flags, fl);
  }
}

// In place: int32 entries <-> binary32 (inf <-> +infinity).  Back from
// binary32, anything >= inf (including +inf) is inf; values below -2^31
// (possible only after a negative cycle) saturate.
template <bool VEC, bool TO_F32>
__global__ void __launch_bounds__(kThreads) signed_convert(int32_t* __restrict__ d, int64_t n,
                                                           int64_t ld, int32_t inf) {
  auto conv = [&](int32_t v) -> int32_t {
    if (TO_F32) return __float_as_int(i32_to_f32(v, inf));
    return f32_to_i32(__int_as_float(v), inf);
  };
  const int64_t quads = (n + 3) / 4;
  for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
    int32_t* row = d + r * ld;
    for (int64_t q = threadIdx.x; q < quads; q += kThreads) {
      const int64_t c = q * 4;
      if (VEC && c + 3 < n) {
        int32_t v[4];
        load4(row + c, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = conv(v[e]);
        store4(row + c, v);
      } else {
        for (int e = 0; e < 4 && c + e < n; ++e) row[c + e] = conv(row[c + e]);
      }
    }
  }
}

// In place: every value above thr becomes inf (the int32 form above).
template <bool VEC>
__global__ void __launch_bounds__(kThreads) signed_clamp(int32_t* __restrict__ d, int64_t n,
                                                         int64_t ld, int32_t inf, int32_t thr) {
  const int64_t quads = (n + 3) / 4;
  for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
    int32_t* row = d + r * ld;
    for (int64_t q = threadIdx.x; q < quads; q += kThreads) {
      const int64_t c = q * 4;
      if (VEC && c + 3 < n) {
        int32_t v[4];
        load4(row + c, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = v[e] > thr ? inf : v[e];
        store4(row + c, v);
      } else {
        for (int e = 0; e < 4 && c + e < n; ++e) row[c + e] = row[c + e] > thr ? inf : row[c + e];
      }
    }
  }
}

// float32 matrices: the caller's sentinel <-> +infinity, in place.
template <bool TO_INF>
__global__ void __launch_bounds__(kThreads) signed_sentinel_f32(float* __restrict__ d, int64_t n,
                                                                int64_t ld, float inf) {
  for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
    float* row = d + r * ld;
    for (int64_t c = threadIdx.x; c < n; c += kThreads) {
      const float v = row[c];
      if (TO_INF ? v == inf : v >= inf) row[c] = TO_INF ? __builtin_inff() : inf;
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(kThreads) diag_negative(const T* __restrict__ d, int64_t n,
                                                          int64_t ld, SignedScan* __restrict__ s) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    if (d[i * ld + i] < T(0)) s->neg_cycle = 1;
}

// ---------------------------------------------------------------------------
// Scratch for apsp_fw_i32_noalloc: the scan result of an int32 call (two
// words) in a file-scope device array, so that entry point allocates
// nothing.  Every call of it on one GPU shares that GPU's copy; each call
// clears the two words (scan_zero) before its scan writes them.
// ---------------------------------------------------------------------------
constexpr int kNoAllocScratchWords = 64;  // 256 bytes; an int32 call needs 2
static __device__ __align__(256) int32_t scratch[kNoAllocScratchWords];

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
thread_local int g_last_hip_error = 0;
std::atomic<int> g_int32_arith{APSP_ARITH_AUTO};

// Per-device cache: 0 = unknown, 1 = gfx950, 2 = other.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];
std::atomic<int> g_dev_cus[kMaxDevices];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return APSP_ERR_NO_DEVICE;
  if (dev < kMaxDevices) {
    int s = g_dev_state[dev].load(std::memory_order_relaxed);
    if (s == 1) return APSP_OK;
    if (s == 2) return APSP_ERR_NO_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return APSP_ERR_NO_DEVICE;
  const char* a = prop.gcnArchName;
  const bool ok = a[0] == 'g' && a[1] == 'f' && a[2] == 'x' && a[3] == '9' && a[4] == '5' &&
                  a[5] == '0' && (a[6] == '\0' || a[6] == ':');
  if (dev < kMaxDevices) {
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_dev_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  }
  return ok ? APSP_OK : APSP_ERR_NO_DEVICE;
}

// Compute units of the current device (known once check_device succeeded).
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
    const int c = g_dev_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  return 256;
}

// Device address of `scratch` on the current device, looked up once per
// device (each GPU holds its own copy of the array at its own address).  In
// host code the array's name is only a host-side stand-in; this address is
// what kernels and copies take.
std::atomic<int32_t*> g_noalloc_scratch[kMaxDevices];

int noalloc_scratch(int32_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    g_last_hip_error = (int)hipGetLastError();
    return APSP_ERR_NO_DEVICE;
  }
  int32_t* p = g_noalloc_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* addr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || addr == nullptr) {
      g_last_hip_error = (int)(e != hipSuccess ? e : hipErrorInvalidSymbol);
      (void)hipGetLastError();
      return APSP_ERR_LAUNCH;
    }
    p = static_cast<int32_t*>(addr);
    g_noalloc_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return APSP_OK;
}

template <typename T>
bool inf_ok(T inf);
template <>
bool inf_ok<int32_t>(int32_t inf) { return inf >= 1 && inf <= 0x3FFFFFFF; }
template <>
bool inf_ok<float>(float inf) { return inf > 0.0f; }  // false for NaN

template <typename T>
int validate(const T* d, int64_t n, int64_t ld, T inf) {
  if (n < 0) return APSP_ERR_INVALID_VALUE;
  if (n == 0) return APSP_OK;
  if (d == nullptr) return APSP_ERR_INVALID_VALUE;
  if (ld < n) return APSP_ERR_INVALID_VALUE;
  if ((reinterpret_cast<uintptr_t>(d) % sizeof(T)) != 0) return APSP_ERR_INVALID_VALUE;
  if (n > (int64_t(1) << 31)) return APSP_ERR_INVALID_VALUE;
  if (ld > INT64_MAX / (int64_t)sizeof(T) / n) return APSP_ERR_INVALID_VALUE;
  if (!inf_ok<T>(inf)) return APSP_ERR_INVALID_VALUE;
  return APSP_OK;
}

// Launch kinds reported by the timed entry points.
enum { kKindPhase1 = 0, kKindPhase2 = 1, kKindPhase3 = 2, kKindScan = 3, kKinds = 4 };

struct PhaseTimer {
  // Events bracketing each launch: ev[2*i] before, ev[2*i+1] after launch i.
  // Launches beyond `cap` are not recorded (counted in `dropped`).
  hipEvent_t* ev = nullptr;
  int* kind = nullptr;
  int64_t cap = 0, used = 0, dropped = 0;
  hipStream_t s = nullptr;
  void mark(int k, bool before) {
    if (used >= cap) {
      if (!before) ++dropped;
      return;
    }
    if (before) {
      (void)hipEventRecord(ev[2 * used], s);
      kind[used] = k;
    } else {
      (void)hipEventRecord(ev[2 * used + 1], s);
      ++used;
    }
  }
};

// Launch tracing across calls (apsp_trace_begin / apsp_trace_end): while it
// is on, every Floyd-Warshall call of this thread records events around its
// launches into one pooled buffer, with no synchronisation; the totals are
// read once at the end.
struct Trace {
  bool on = false;
  int dev = -1;
  hipEvent_t* ev = nullptr;  // 2 * cap events, owned by the event pool
  int* kind = nullptr;
  int64_t cap = 0, used = 0, dropped = 0;
};
thread_local Trace g_trace;

int launch_status() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return APSP_ERR_LAUNCH;
  }
  return APSP_OK;
}

// Launches the converting instance of an int32 phase kernel when `mask`
// asks for a conversion, else the plain one; both take (args..., conv, scan).
template <typename K, typename... A>
void launch_i32(K plain, K conv, int64_t grid, int threads, hipStream_t s, int mask,
                const int32_t* scan, A... args) {
  if (mask)
    hipLaunchKernelGGL(conv, dim3((unsigned)grid), dim3(threads), 0, s, args..., mask, scan);
  else
    hipLaunchKernelGGL(plain, dim3((unsigned)grid), dim3(threads), 0, s, args..., 0, scan);
}

// Rounds [r0, r1).  For int32 matrices `scan_buf` (may be null) holds the
// scan result that selects binary32 or int32 arithmetic inside the kernels.
// In binary32 the matrix is converted on the way: round r0 reads every
// block once before any other access (block (r0, r0) in Phase 1, its pivot
// row and column in Phase 2, the rest in Phase 3), so those loads convert;
// Phase 3 of round r1 - 1 writes every block outside its pivot row and
// column once after its last read, so its stores convert; that round's
// Phase 2 keeps the pivot row and column in binary32 (Phase 3 reads them as
// operands), and pivot_panels_to_i32 converts them, block (K, K) included,
// after the last Phase 3.
template <typename T, bool VEC, bool KEYS = false>
void enqueue_rounds(T* d, int64_t n, int64_t ld, T inf, int64_t r0, int64_t r1, hipStream_t s,
                    const int32_t* scan_buf, PhaseTimer* tm) {
  static_assert(!KEYS || std::is_same_v<T, int32_t>, "successor keys are int32");
  const int64_t nb = (n + kB - 1) / kB;
  const int conv_first = scan_buf ? kConvC : 0;
  const int conv_last = scan_buf ? kConvOut : 0;

  auto mark = [&](int k, bool before) {
    if (tm) tm->mark(k, before);
  };
  // Round r0 closes its diagonal block on its own; every later round's
  // Phase 1 runs inside the previous round's Phase-3 launch.
  // An int32 matrix with no scan computes in int32 throughout and runs the
  // plain int32 kernels: without the binary32 body beside it, the int32
  // Phase 3 keeps more of its values in registers (18 spilled VGPRs instead
  // of 32, and no spilled SGPRs) and the call is about 1 % faster.
  bool dual = false;
  if constexpr (std::is_same_v<T, int32_t>) dual = scan_buf != nullptr;
  mark(kKindPhase1, true);
  if constexpr (std::is_same_v<T, int32_t>) {
    if (dual)
      launch_i32(fw_phase1_i32<VEC, false>, fw_phase1_i32<VEC, true>, 1, kP1Threads, s,
                 conv_first | (nb == 1 ? conv_last : 0), scan_buf, d, n, ld, inf, r0);
  }
  if constexpr (KEYS)
    hipLaunchKernelGGL((fw_keys_phase1<VEC>), dim3(1), dim3(kP1Threads), 0, s, d, n, ld, inf, r0);
  else if (!dual)
    hipLaunchKernelGGL((fw_phase1<T, VEC>), dim3(1), dim3(kP1Threads), 0, s, d, n, ld, inf, r0);
  mark(kKindPhase1, false);
  // Phase-3 grid: whole tiles, then the quarters of a short last wave.
  const int64_t tiles = (nb - 1) * (nb - 1);
  const int64_t slots = (int64_t)kWavesP3 * device_cus();
  int64_t whole = tiles;
  if (tiles % slots != 0 && 4 * (tiles % slots) <= slots) whole = tiles - tiles % slots;
  // Workgroup 0 takes a whole tile: it closes block (K+1, K+1) after the
  // update, or converts block (K, K) back in the last round.
  const uint32_t full3 = (uint32_t)(whole > 0 ? whole : 1);
  const int64_t g3 = tiles > 0 ? full3 + 4 * (tiles - full3) : 0;
  // Below about one and a half waves of tiles, workgroup 0's update and
  // closure of the next diagonal block is the longest chain of the launch,
  // so in binary32 it closes the block two pivots per barrier (measured
  // 4-7 % faster per launch at n = 2048 and 4096).  Above, the closure is off
  // the critical path and the kernel with the one-pivot closure keeps the
  // faster tile loop (the pair-step kernel was 6 % slower at n = 5120); the
  // int32 body gains nothing from it (its pair-step kernel spills more).
  const bool pair_close = 2 * tiles < 3 * slots && (!std::is_same_v<T, int32_t> || dual);
  for (int64_t K = r0; K < r1 && nb > 1; ++K) {
    const int64_t g2 = 2 * (nb - 1) * (kB / kP2);
    mark(kKindPhase2, true);
    if constexpr (std::is_same_v<T, int32_t>) {
      if (dual)
        launch_i32(fw_phase2_i32<VEC, false>, fw_phase2_i32<VEC, true>, g2, kP2Threads, s,
                   K == r0 ? conv_first : 0 /* the last round's panels stay binary32 */, scan_buf,
                   d, n, ld, inf, K, nb);
    }
    if constexpr (KEYS)
      hipLaunchKernelGGL((fw_keys_phase2<VEC>), dim3((unsigned)g2), dim3(kP2Threads), 0, s, d, n,
                         ld, inf, K, nb);
    else if (!dual)
      hipLaunchKernelGGL((fw_phase2<T, VEC>), dim3((unsigned)g2), dim3(kP2Threads), 0, s, d, n, ld,
                         inf, K, nb);
    mark(kKindPhase2, false);
    const int fuse = K + 1 < r1 ? 1 : 0;
    mark(kKindPhase3, true);
    const int mask3 = (K == r0 ? conv_first : 0) | (K + 1 == r1 ? conv_last : 0);
    if constexpr (std::is_same_v<T, int32_t>) {
      if (dual) {
        if (pair_close)
          launch_i32(fw_phase3_i32<VEC, false, true>, fw_phase3_i32<VEC, true, true>, g3, kThreads,
                     s, mask3, scan_buf, d, n, ld, inf, K, nb, fuse, full3);
        else
          launch_i32(fw_phase3_i32<VEC, false, false>, fw_phase3_i32<VEC, true, false>, g3,
                     kThreads, s, mask3, scan_buf, d, n, ld, inf, K, nb, fuse, full3);
      }
    }
    if constexpr (KEYS) {
      hipLaunchKernelGGL((fw_keys_phase3<VEC>), dim3((unsigned)g3), dim3(kThreads), 0, s, d, n,
                         ld, inf, K, nb, fuse, full3);
    } else if (!dual) {
      if (pair_close)
        hipLaunchKernelGGL((fw_phase3<T, VEC, true>), dim3((unsigned)g3), dim3(kThreads), 0, s, d,
                           n, ld, inf, K, nb, fuse, full3);
      else
        hipLaunchKernelGGL((fw_phase3<T, VEC, false>), dim3((unsigned)g3), dim3(kThreads), 0, s,
                           d, n, ld, inf, K, nb, fuse, full3);
    }
    mark(kKindPhase3, false);
  }
  if constexpr (std::is_same_v<T, int32_t>) {
    if (scan_buf && nb > 1) {
      mark(kKindScan, true);
      hipLaunchKernelGGL(pivot_panels_to_i32, dim3((unsigned)n), dim3(kThreads), 0, s, d, n, ld,
                         inf, r1 - 1, scan_buf);
      mark(kKindScan, false);
    }
  }
}

// The scan that picks the arithmetic of an int32 call, then its rounds.
template <bool VEC>
void enqueue_i32(int32_t* d, int64_t n, int64_t ld, int32_t inf, int64_t r0, int64_t r1,
                 hipStream_t s, int32_t* scan_buf, PhaseTimer* tm) {
  const int64_t rows = n < kScanBlocks ? n : kScanBlocks;
  if (scan_buf) {
    if (tm) tm->mark(kKindScan, true);
    hipLaunchKernelGGL(scan_zero, dim3(1), dim3(64), 0, s, scan_buf);
    hipLaunchKernelGGL((scan_i32<VEC>), dim3((unsigned)rows), dim3(kThreads), 0, s, d, n, ld, inf,
                       scan_buf);
    if (tm) tm->mark(kKindScan, false);
  }
  enqueue_rounds<int32_t, VEC>(d, n, ld, inf, r0, r1, s, scan_buf, tm);
}

// Validates, then enqueues rounds [r0, r1).  For int32 the scan result is
// copied to scan_out (host, when non-null; valid after the stream has
// synchronised) before the stream-ordered scratch is released.
template <typename T>
int run(T* d, int64_t n, int64_t ld, T inf, int64_t r0, int64_t r1, void* stream,
        PhaseTimer* tm, int32_t* scan_out, int32_t* fixed_scan_buf = nullptr) {
  int st = validate<T>(d, n, ld, inf);
  if (st != APSP_OK) return st;
  const int64_t nb = n == 0 ? 0 : (n + kB - 1) / kB;
  if (r0 < 0 || r1 < r0 || r1 > nb) return APSP_ERR_INVALID_VALUE;
  if (n == 0 || r0 == r1) return APSP_OK;
  st = check_device();
  if (st != APSP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  PhaseTimer trace_tm;
  if (!tm && g_trace.on) {
    trace_tm.ev = g_trace.ev + 2 * g_trace.used;
    trace_tm.kind = g_trace.kind + g_trace.used;
    trace_tm.cap = g_trace.cap - g_trace.used;
    tm = &trace_tm;
  }
  if (tm) tm->s = s;
  const bool vec = (ld % 4 == 0) && (reinterpret_cast<uintptr_t>(d) % 16 == 0);
  struct TraceCommit {  // fold the launches of this call into the trace
    PhaseTimer* t;
    ~TraceCommit() {
      if (t) {
        g_trace.used += t->used;
        g_trace.dropped += t->dropped;
      }
    }
  } commit{tm == &trace_tm ? &trace_tm : nullptr};
  if constexpr (std::is_same_v<T, int32_t>) {
    // Binary32 pays from nine Phase-3 tiles (n > 384) on: measured against
    // int32 arithmetic, 1.5 % faster per call at n = 512, 7-9 % at n = 1024
    // to 2048 (there each round waits on workgroup 0's closure, which is
    // shorter in binary32), and 2 % slower at n = 384, where the scan costs
    // more than three rounds save.  Smaller matrices stay in int32 and skip
    // the scan.  The scan result lives in a few bytes of stream-ordered
    // scratch; without it the call stays in int32.
    int32_t* scan_buf = nullptr;
    const int64_t tiles = (nb - 1) * (nb - 1);
    const int policy = g_int32_arith.load(std::memory_order_relaxed);
    const bool try_f32 = policy == APSP_ARITH_F32_WHEN_EXACT ||
                         (policy == APSP_ARITH_AUTO && tiles >= kF32MinTiles);
    if (try_f32) {
      if (fixed_scan_buf) {
        scan_buf = fixed_scan_buf;
      } else if (hipMallocAsync(reinterpret_cast<void**>(&scan_buf), 256, s) != hipSuccess) {
        scan_buf = nullptr;
        (void)hipGetLastError();
      }
    }
    if (vec) enqueue_i32<true>(d, n, ld, inf, r0, r1, s, scan_buf, tm);
    else enqueue_i32<false>(d, n, ld, inf, r0, r1, s, scan_buf, tm);
    if (scan_buf) {
      if (scan_out)
        (void)hipMemcpyAsync(scan_out, scan_buf, 2 * sizeof(int32_t), hipMemcpyDeviceToHost, s);
      if (scan_buf != fixed_scan_buf) (void)hipFreeAsync(scan_buf, s);
    }
  } else {
    (void)scan_out;
    if (vec) enqueue_rounds<T, true>(d, n, ld, inf, r0, r1, s, nullptr, tm);
    else enqueue_rounds<T, false>(d, n, ld, inf, r0, r1, s, nullptr, tm);
  }
  return launch_status();
}

// Every round on successor keys (see key_mask), in place on s.  The caller
// has validated the matrix and checked that the keys stay exact.
int run_keys(int32_t* d, int64_t n, int64_t ld, hipStream_t s) {
  const int64_t nb = (n + kB - 1) / kB;
  const int sb = 32 - __builtin_clz((unsigned)n);
  const int32_t inf_key = (int32_t)((1u << 30) - (1u << sb));
  PhaseTimer trace_tm;
  PhaseTimer* tm = nullptr;
  if (g_trace.on) {
    trace_tm.ev = g_trace.ev + 2 * g_trace.used;
    trace_tm.kind = g_trace.kind + g_trace.used;
    trace_tm.cap = g_trace.cap - g_trace.used;
    trace_tm.s = s;
    tm = &trace_tm;
  }
  const bool vec = (ld % 4 == 0) && (reinterpret_cast<uintptr_t>(d) % 16 == 0);
  if (vec) enqueue_rounds<int32_t, true, true>(d, n, ld, inf_key, 0, nb, s, nullptr, tm);
  else enqueue_rounds<int32_t, false, true>(d, n, ld, inf_key, 0, nb, s, nullptr, tm);
  if (tm) {
    g_trace.used += trace_tm.used;
    g_trace.dropped += trace_tm.dropped;
  }
  return launch_status();
}

// Timing events are created once per thread and device and reused, so the
// measured calls do not pay for event creation.  Timing-only events carry
// no system-scope fence (no cache writeback between the kernels they
// bracket).  They live until apsp_release_events() on the owning thread (the
// Python binding calls it at interpreter exit); no static destructor makes a
// HIP call, so nothing of the library runs after the HIP runtime has begun
// to shut down.
struct EventPool {
  hipEvent_t* ev = nullptr;
  int64_t size = 0;
};
thread_local EventPool g_event_pool[kMaxDevices];

hipEvent_t* grow_pool(EventPool* pools, int64_t count) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  EventPool& p = pools[dev];
  if (p.size >= count) return p.ev;
  hipEvent_t* ev = new hipEvent_t[count];
  for (int64_t i = 0; i < p.size; ++i) ev[i] = p.ev[i];
  int64_t made = p.size;
  for (; made < count; ++made)
    if (hipEventCreateWithFlags(&ev[made], hipEventDisableSystemFence) != hipSuccess) break;
  delete[] p.ev;
  p.ev = ev;
  p.size = made;
  return made >= count ? ev : nullptr;
}

// The timed entry points and the cross-call trace keep separate pools, so a
// timed call made while a trace is on cannot move the trace's events.
thread_local EventPool g_trace_pool[kMaxDevices];

hipEvent_t* pooled_events(int64_t count) { return grow_pool(g_event_pool, count); }

template <typename T>
int run_timed(T* d, int64_t n, int64_t ld, T inf, void* stream, double* phase_ms,
              int64_t* phase_launch, int* arith) {
  int st = validate<T>(d, n, ld, inf);
  if (st != APSP_OK) return st;
  if (phase_ms) for (int p = 0; p < kKinds; ++p) phase_ms[p] = 0.0;
  if (phase_launch) for (int p = 0; p < kKinds; ++p) phase_launch[p] = 0;
  if (arith) *arith = std::is_same_v<T, int32_t> ? 0 : 1;
  if (n == 0) return APSP_OK;
  st = check_device();
  if (st != APSP_OK) return st;
  const int64_t nb = (n + kB - 1) / kB;
  PhaseTimer tm;
  tm.cap = 3 * nb + 4;
  tm.ev = pooled_events(2 * tm.cap);
  if (tm.ev == nullptr) {
    g_last_hip_error = (int)hipGetLastError();
    return APSP_ERR_LAUNCH;
  }
  tm.kind = new int[tm.cap];
  int32_t scan[2] = {0, -1};
  st = run<T>(d, n, ld, inf, 0, nb, stream, &tm, scan);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess && st == APSP_OK) {
    g_last_hip_error = (int)hipGetLastError();
    st = APSP_ERR_LAUNCH;
  }
  if (st == APSP_OK) {
    for (int64_t i = 0; i < tm.used; ++i) {
      float ms = 0.f;
      (void)hipEventElapsedTime(&ms, tm.ev[2 * i], tm.ev[2 * i + 1]);
      const int p = tm.kind[i];
      if (phase_ms) phase_ms[p] += ms;
      if (phase_launch) phase_launch[p] += 1;
    }
    if (arith && std::is_same_v<T, int32_t>) {
      // Same decision the kernels took (see f32_exact).
      const bool exact = scan[1] >= 0 && !(scan[1] & kFlagNotExact) &&
                         (!(scan[1] & kFlagHasInf) || (n - 1) * (int64_t)scan[0] <= kExactLimit);
      *arith = exact ? 1 : 0;
    }
  }
  delete[] tm.kind;
  return st;
}

// A failed HIP call: keep its error for apsp_last_hip_error.
int hip_failed() {
  g_last_hip_error = (int)hipGetLastError();
  return APSP_ERR_LAUNCH;
}

int sync_read(hipStream_t s, void* host, const void* dev, size_t bytes) {
  if (hipMemcpyAsync(host, dev, bytes, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return hip_failed();
  return APSP_OK;
}

// Negative weights, int32 matrix (see the kernels above).  Synchronous.
int run_signed_i32(int32_t* d, int64_t n, int64_t ld, int32_t inf, void* stream, int* arith_out) {
  if (arith_out) *arith_out = -1;
  int st = validate<int32_t>(d, n, ld, inf);
  if (st != APSP_OK || n == 0) return st;
  st = check_device();
  if (st != APSP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool vec = (ld % 4 == 0) && (reinterpret_cast<uintptr_t>(d) % 16 == 0);
  const int64_t nb = (n + kB - 1) / kB;
  const unsigned rows = (unsigned)(n < kScanBlocks ? n : kScanBlocks);
  SignedScan* sc = nullptr;
  if (hipMallocAsync(reinterpret_cast<void**>(&sc), sizeof(SignedScan), s) != hipSuccess)
    return hip_failed();
  SignedScan h{};
  int rc = APSP_OK;
  do {
    hipLaunchKernelGGL(signed_zero, dim3(1), dim3(64), 0, s, sc);
    if (vec) hipLaunchKernelGGL((scan_signed_i32<true>), dim3(rows), dim3(kThreads), 0, s, d, n, ld, inf, sc);
    else hipLaunchKernelGGL((scan_signed_i32<false>), dim3(rows), dim3(kThreads), 0, s, d, n, ld, inf, sc);
    if ((rc = launch_status()) != APSP_OK || (rc = sync_read(s, &h, sc, sizeof(h))) != APSP_OK) break;
    if (h.flags & kSgBadEntry) {
      rc = APSP_ERR_INVALID_VALUE;
      break;
    }
    const int64_t W = h.maxabs;
    const bool has_inf = (h.flags & kSgHasInf) != 0;
    const int policy = g_int32_arith.load(std::memory_order_relaxed);
    const int64_t tiles = (nb - 1) * (nb - 1);
    const bool exact_f32 = (n - 1) * W <= kExactLimit && policy != APSP_ARITH_INT32;
    const bool prefer_f32 = policy == APSP_ARITH_F32_WHEN_EXACT ||
                            (policy == APSP_ARITH_AUTO && tiles >= (int64_t)kP3PerCu * device_cus());
    const bool i32_ok = has_inf ? (2 * n - 3) * W < (int64_t)inf : (n - 1) * W < (int64_t(1) << 30);
    if (!exact_f32 && !i32_ok) {
      rc = APSP_ERR_RANGE;
      break;
    }
    const bool f32 = exact_f32 && (prefer_f32 || !i32_ok);
    if (arith_out) *arith_out = f32 ? 1 : 0;
    if (f32) {
      float* fd = reinterpret_cast<float*>(d);
      if (vec) {
        hipLaunchKernelGGL((signed_convert<true, true>), dim3(rows), dim3(kThreads), 0, s, d, n, ld, inf);
        enqueue_rounds<float, true>(fd, n, ld, __builtin_inff(), 0, nb, s, nullptr, nullptr);
        hipLaunchKernelGGL((signed_convert<true, false>), dim3(rows), dim3(kThreads), 0, s, d, n, ld, inf);
      } else {
        hipLaunchKernelGGL((signed_convert<false, true>), dim3(rows), dim3(kThreads), 0, s, d, n, ld, inf);
        enqueue_rounds<float, false>(fd, n, ld, __builtin_inff(), 0, nb, s, nullptr, nullptr);
        hipLaunchKernelGGL((signed_convert<false, false>), dim3(rows), dim3(kThreads), 0, s, d, n, ld, inf);
      }
    } else {
      const int32_t thr = (int32_t)((n - 1) * W);
      if (vec) {
        enqueue_rounds<int32_t, true>(d, n, ld, inf, 0, nb, s, nullptr, nullptr);
        if (has_inf) hipLaunchKernelGGL((signed_clamp<true>), dim3(rows), dim3(kThreads), 0, s, d, n, ld, inf, thr);
      } else {
        enqueue_rounds<int32_t, false>(d, n, ld, inf, 0, nb, s, nullptr, nullptr);
        if (has_inf) hipLaunchKernelGGL((signed_clamp<false>), dim3(rows), dim3(kThreads), 0, s, d, n, ld, inf, thr);
      }
    }
    const unsigned dg = (unsigned)std::min<int64_t>((n + kThreads - 1) / kThreads, 1024);
    hipLaunchKernelGGL((diag_negative<int32_t>), dim3(dg), dim3(kThreads), 0, s, d, n, ld, sc);
    if ((rc = launch_status()) != APSP_OK || (rc = sync_read(s, &h, sc, sizeof(h))) != APSP_OK) break;
    if (h.neg_cycle) rc = APSP_ERR_NEGATIVE_CYCLE;
  } while (false);
  (void)hipFreeAsync(sc, s);
  (void)hipStreamSynchronize(s);
  return rc;
}

// Negative weights, float32 matrix: the sentinel becomes +infinity for the
// rounds, which makes every sum through it +infinity.  Synchronous.
int run_signed_f32(float* d, int64_t n, int64_t ld, float inf, void* stream) {
  int st = validate<float>(d, n, ld, inf);
  if (st != APSP_OK || n == 0) return st;
  st = check_device();
  if (st != APSP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool vec = (ld % 4 == 0) && (reinterpret_cast<uintptr_t>(d) % 16 == 0);
  const int64_t nb = (n + kB - 1) / kB;
  const unsigned rows = (unsigned)(n < kScanBlocks ? n : kScanBlocks);
  SignedScan* sc = nullptr;
  if (hipMallocAsync(reinterpret_cast<void**>(&sc), sizeof(SignedScan), s) != hipSuccess)
    return hip_failed();
  SignedScan h{};
  int rc = APSP_OK;
  do {
    hipLaunchKernelGGL(signed_zero, dim3(1), dim3(64), 0, s, sc);
    const bool finite = inf != __builtin_inff();
    if (finite)
      hipLaunchKernelGGL((signed_sentinel_f32<true>), dim3(rows), dim3(kThreads), 0, s, d, n, ld, inf);
    if (vec) enqueue_rounds<float, true>(d, n, ld, __builtin_inff(), 0, nb, s, nullptr, nullptr);
    else enqueue_rounds<float, false>(d, n, ld, __builtin_inff(), 0, nb, s, nullptr, nullptr);
    if (finite)
      hipLaunchKernelGGL((signed_sentinel_f32<false>), dim3(rows), dim3(kThreads), 0, s, d, n, ld, inf);
    const unsigned dg = (unsigned)std::min<int64_t>((n + kThreads - 1) / kThreads, 1024);
    hipLaunchKernelGGL((diag_negative<float>), dim3(dg), dim3(kThreads), 0, s, d, n, ld, sc);
    if ((rc = launch_status()) != APSP_OK || (rc = sync_read(s, &h, sc, sizeof(h))) != APSP_OK) break;
    if (h.neg_cycle) rc = APSP_ERR_NEGATIVE_CYCLE;
  } while (false);
  (void)hipFreeAsync(sc, s);
  (void)hipStreamSynchronize(s);
  return rc;
}

}  // namespace

// Library-internal host helpers for the other translation units.
int apsp_detail_check_device() { return check_device(); }
int apsp_detail_fw_keys(int32_t* d, int64_t n, int64_t ld, void* stream) {
  if (d == nullptr || n < 1 || n >= (int64_t(1) << 29) || ld < n) return APSP_ERR_INVALID_VALUE;
  return run_keys(d, n, ld, reinterpret_cast<hipStream_t>(stream));
}
int apsp_detail_launch_status() { return launch_status(); }

extern "C" {

int apsp_fw_i32(int32_t* d, int64_t n, int64_t ld, int32_t inf, void* stream) {
  const int64_t nb = n > 0 ? (n + kB - 1) / kB : 0;
  return run<int32_t>(d, n, ld, inf, 0, nb, stream, nullptr, nullptr);
}

int apsp_fw_f32(float* d, int64_t n, int64_t ld, float inf, void* stream) {
  const int64_t nb = n > 0 ? (n + kB - 1) / kB : 0;
  return run<float>(d, n, ld, inf, 0, nb, stream, nullptr, nullptr);
}

int apsp_fw_i32_noalloc(int32_t* d, int64_t n, int64_t ld, int32_t inf, void* stream) {
  int st = validate<int32_t>(d, n, ld, inf);
  if (st != APSP_OK || n == 0) return st;
  if ((st = check_device()) != APSP_OK) return st;
  static_assert(2 <= kNoAllocScratchWords, "the scan result fits the static scratch");
  int32_t* sc = nullptr;
  if ((st = noalloc_scratch(&sc)) != APSP_OK) return st;
  const int64_t nb = (n + kB - 1) / kB;
  return run<int32_t>(d, n, ld, inf, 0, nb, stream, nullptr, nullptr, sc);
}

int apsp_fw_rounds_i32(int32_t* d, int64_t n, int64_t ld, int32_t inf, int64_t round_begin,
                       int64_t round_end, void* stream) {
  return run<int32_t>(d, n, ld, inf, round_begin, round_end, stream, nullptr, nullptr);
}

int apsp_fw_rounds_f32(float* d, int64_t n, int64_t ld, float inf, int64_t round_begin,
                       int64_t round_end, void* stream) {
  return run<float>(d, n, ld, inf, round_begin, round_end, stream, nullptr, nullptr);
}

int apsp_fw_timed_i32(int32_t* d, int64_t n, int64_t ld, int32_t inf, void* stream,
                      double* phase_ms, int64_t* phase_launch, int* arith) {
  return run_timed<int32_t>(d, n, ld, inf, stream, phase_ms, phase_launch, arith);
}

int apsp_fw_timed_f32(float* d, int64_t n, int64_t ld, float inf, void* stream,
                      double* phase_ms, int64_t* phase_launch, int* arith) {
  return run_timed<float>(d, n, ld, inf, stream, phase_ms, phase_launch, arith);
}

int apsp_fw_signed_i32(int32_t* d, int64_t n, int64_t ld, int32_t inf, void* stream) {
  return run_signed_i32(d, n, ld, inf, stream, nullptr);
}

int apsp_fw_signed_f32(float* d, int64_t n, int64_t ld, float inf, void* stream) {
  return run_signed_f32(d, n, ld, inf, stream);
}

int apsp_trace_begin(int64_t max_launches) {
  if (max_launches <= 0 || max_launches > (int64_t(1) << 24)) return APSP_ERR_INVALID_VALUE;
  if (g_trace.on) return APSP_ERR_INVALID_VALUE;
  int st = check_device();
  if (st != APSP_OK) return st;
  hipEvent_t* ev = grow_pool(g_trace_pool, 2 * max_launches);
  if (ev == nullptr) return hip_failed();
  int dev = 0;
  (void)hipGetDevice(&dev);
  delete[] g_trace.kind;
  g_trace.kind = new int[max_launches];
  g_trace.ev = ev;
  g_trace.cap = max_launches;
  g_trace.used = g_trace.dropped = 0;
  g_trace.dev = dev;
  g_trace.on = true;
  return APSP_OK;
}

int apsp_trace_end(double* phase_ms, int64_t* phase_launch, int64_t* dropped) {
  if (phase_ms) for (int p = 0; p < kKinds; ++p) phase_ms[p] = 0.0;
  if (phase_launch) for (int p = 0; p < kKinds; ++p) phase_launch[p] = 0;
  if (dropped) *dropped = 0;
  if (!g_trace.on) return APSP_ERR_INVALID_VALUE;
  g_trace.on = false;
  int rc = APSP_OK;
  int cur = 0;
  (void)hipGetDevice(&cur);
  if (cur != g_trace.dev) (void)hipSetDevice(g_trace.dev);
  if (g_trace.used > 0 && hipEventSynchronize(g_trace.ev[2 * g_trace.used - 1]) != hipSuccess)
    rc = hip_failed();
  for (int64_t i = 0; rc == APSP_OK && i < g_trace.used; ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_trace.ev[2 * i], g_trace.ev[2 * i + 1]) != hipSuccess) {
      rc = hip_failed();
      break;
    }
    const int p = g_trace.kind[i];
    if (phase_ms) phase_ms[p] += ms;
    if (phase_launch) phase_launch[p] += 1;
  }
  if (dropped) *dropped = g_trace.dropped;
  if (cur != g_trace.dev) (void)hipSetDevice(cur);
  return rc;
}

int apsp_release_events(void) {
  if (g_trace.on) return APSP_ERR_INVALID_VALUE;
  bool any = false;
  for (int dev = 0; dev < kMaxDevices; ++dev)
    any = any || g_event_pool[dev].size > 0 || g_trace_pool[dev].size > 0;
  delete[] g_trace.kind;
  g_trace = Trace{};
  if (!any) return APSP_OK;  // nothing pooled: no HIP call at all
  int cur = 0;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  int rc = APSP_OK;
  for (EventPool* pools : {g_event_pool, g_trace_pool}) {
    for (int dev = 0; dev < kMaxDevices; ++dev) {
      EventPool& p = pools[dev];
      if (p.size == 0) continue;
      if (hipSetDevice(dev) != hipSuccess) {
        rc = hip_failed();
        continue;
      }
      for (int64_t i = 0; i < p.size; ++i)
        if (hipEventDestroy(p.ev[i]) != hipSuccess && rc == APSP_OK) rc = hip_failed();
      delete[] p.ev;
      p.ev = nullptr;
      p.size = 0;
    }
  }
  if (have_cur) (void)hipSetDevice(cur);
  return rc;
}

int apsp_set_int32_arith(int mode) {
  if (mode != APSP_ARITH_AUTO && mode != APSP_ARITH_F32_WHEN_EXACT && mode != APSP_ARITH_INT32)
    return APSP_ERR_INVALID_VALUE;
  g_int32_arith.store(mode, std::memory_order_relaxed);
  return APSP_OK;
}

int apsp_get_int32_arith(void) { return g_int32_arith.load(std::memory_order_relaxed); }

int64_t apsp_pivot_block(int64_t n) {
  (void)n;
  return kB;
}

const char* apsp_status_string(int status) {
  switch (status) {
    case APSP_OK: return "APSP_OK";
    case APSP_ERR_INVALID_VALUE: return "APSP_ERR_INVALID_VALUE: invalid argument";
    case APSP_ERR_NO_DEVICE: return "APSP_ERR_NO_DEVICE: current device is not gfx950";
    case APSP_ERR_LAUNCH: return "APSP_ERR_LAUNCH: kernel launch failed";
    case APSP_ERR_NEGATIVE_CYCLE: return "APSP_ERR_NEGATIVE_CYCLE: the graph has a negative cycle";
    case APSP_ERR_RANGE: return "APSP_ERR_RANGE: a value is outside the representable range";
    default: return "APSP: unknown status";
  }
}

int apsp_last_hip_error(void) { return g_last_hip_error; }

int apsp_version(void) { return 100; }

}  // extern "C"
