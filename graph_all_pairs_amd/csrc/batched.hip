// Batched all-pairs shortest paths for many small graphs, one workgroup per
// graph.
//
// The page "Loops into zones" (section "Many small graphs") parallelises a
// graph algorithm over many independent small graphs by making each graph
// one GPU block: the outer level runs graphs that never interact, the inner
// level is one graph.  Here the inner level is Floyd-Warshall on a graph of
// n <= 128 vertices, which is exactly one diagonal-block closure of the
// blocked method (Phase 1 of the page "Katz and Kider", thesis section 4.6,
// Algorithm 16): the graph's matrix is loaded into registers, closed two
// pivots per barrier, and stored.
//
// Size classes: the padded edge NB is n rounded up to a multiple of 8 (at
// least 16), with an RT x RT micro-tile per thread and (NB/RT)^2 threads:
//   NB = 16, 24, 32:      RT = 4, 16 / 36 / 64 threads (one wave per graph);
//   NB = 40, 48, ..., 128: RT = 8, 25 ... 256 threads (1 to 4 waves).
// A graph costs NB/2 pivot-pair steps of the same per-thread work, and the
// waves it occupies set how many graphs share a CU, so every multiple of 8
// is its own class (n = 100 runs as NB = 104: 3 waves and 52 steps, against
// 4 waves and 64 steps at NB = 128).
// Rows and columns n .. NB-1 are isolated vertices: they load as inf and are
// never stored, so the closure of the padded block restricted to [0, n) is
// the closure of the graph.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "apsp.h"
#include "detail.h"
#include "minplus.h"

namespace {

using namespace apsp_dev;

constexpr int64_t kMaxBatchedN = 128;
constexpr int64_t kMaxGrid = int64_t(1) << 20;  // workgroups; more graphs loop

// One quad (row, col .. col+3) of a graph; rows and columns >= n read as
// inf and are never written.  A quad that straddles column n loads each
// element from a clamped in-range address and then selects inf, and stores
// through clamped addresses (an out-of-range element rewrites element n-1 of
// its row with that element's own value), so a quad costs a branch or two,
// not one per element: with a branch per element the compiler kept 64 lane
// masks per thread alive across the closure and spilled them, and the
// graphs whose n is not a multiple of 8 ran 14 % slower than the next
// multiple of 8.
template <typename T, bool VEC, bool EDGE>
__device__ __forceinline__ void bload4(const T* __restrict__ m, int64_t ld, int64_t n,
                                       int64_t row, int64_t col, T inf, T (&v)[4]) {
  if (!EDGE || (row < n && col + 3 < n)) {
    gload4<T, VEC, false>(m, ld, n, row, col, inf, v);
    return;
  }
  if (row >= n || col >= n) {  // the whole quad is padding
    v[0] = v[1] = v[2] = v[3] = inf;
    return;
  }
  const T* p = m + row * ld;
  const int64_t c1 = col + 1 < n ? col + 1 : n - 1, c2 = col + 2 < n ? col + 2 : n - 1;
  const T x0 = p[col], x1 = p[c1], x2 = p[c2];
  v[0] = x0;
  v[1] = col + 1 < n ? x1 : inf;
  v[2] = col + 2 < n ? x2 : inf;
  v[3] = inf;  // col + 3 >= n here
}

// Written with named values rather than a loop over the quad: a loop that
// indexes the quad made the compiler move it into LDS.
template <typename T, bool VEC, bool EDGE>
__device__ __forceinline__ void bstore4(T* __restrict__ m, int64_t ld, int64_t n, int64_t row,
                                        int64_t col, const T (&v)[4]) {
  if (!EDGE || (row < n && col + 3 < n)) {
    gstore4<T, VEC, false>(m, ld, n, row, col, v);
    return;
  }
  if (row >= n || col >= n) return;
  const T v0 = v[0], v1 = v[1], v2 = v[2];
  const T last = col + 2 < n ? v2 : (col + 1 < n ? v1 : v0);  // element n - 1
  T* p = m + row * ld;
  p[col] = v0;
  p[col + 1 < n ? col + 1 : n - 1] = col + 1 < n ? v1 : last;
  p[col + 2 < n ? col + 2 : n - 1] = col + 2 < n ? v2 : last;
}

template <int NB, int RT>
struct BatchShape {
  static constexpr int kThr = NB / RT;          // threads per dimension
  static constexpr int kThreads = kThr * kThr;
  static constexpr int G = RT / 4;              // 4-wide groups per thread
  static constexpr int S = NB / G;              // distance between groups
};

// VEC: 16-byte aligned quads (d, ld and stride all allow it); EDGE: n < NB.
// Waves per SIMD for the 8 x 8 micro-tile kernels, measured on 8192 graphs:
// 3 when n is the class edge (fits 168 VGPRs without spills; 4 waves were
// 1-3 % slower), 4 when n < NB (128 VGPRs, at most 2 spills except 14 for
// binary32 NB = 64): their boundary loads and stores leave gaps that a
// fourth wave fills, 3-10 % faster than 3 waves at n = 44, 98, 100, 118.
template <typename T, int NB, int RT, bool VEC, bool EDGE>
__global__ void __launch_bounds__((NB / RT) * (NB / RT))
__attribute__((amdgpu_waves_per_eu(RT == 8 ? (EDGE ? 4 : 3) : 1)))
fw_batched(T* __restrict__ d, int64_t batch, int64_t n, int64_t ld, int64_t stride, T inf) {
  using S = BatchShape<NB, RT>;
  __shared__ __attribute__((aligned(16))) T lds[8 * NB];
  const int tc = threadIdx.x % S::kThr;
  const int tr = threadIdx.x / S::kThr;
  for (int64_t g = blockIdx.x; g < batch; g += gridDim.x) {
    T* m = d + g * stride;
    T acc[RT][RT];
    // The per-element addresses and bounds are recomputed for every graph
    // (the opaque copies stop the compiler hoisting them out of the graph
    // loop, where they would stay live across the closure and spill).
    int tr_l = tr, tc_l = tc;
    int64_t n_l = n;
    asm volatile("" : "+v"(tr_l), "+v"(tc_l), "+s"(n_l));
#pragma unroll
    for (int gi = 0; gi < S::G; ++gi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = gi * S::S + tr_l * 4 + i;
#pragma unroll
        for (int gj = 0; gj < S::G; ++gj) {
          T v[4];
          bload4<T, VEC, EDGE>(m, ld, n_l, row, gj * S::S + tc_l * 4, inf, v);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[gi * 4 + i][gj * 4 + j] = v[j];
        }
      }
    // The closure ends with a barrier after its last LDS reads, so the next
    // graph may publish into the buffers right away.
    close_block_t<T, NB, RT>(acc, lds);
    tr_l = tr;
    tc_l = tc;
    n_l = n;
    asm volatile("" : "+v"(tr_l), "+v"(tc_l), "+s"(n_l));
#pragma unroll
    for (int gi = 0; gi < S::G; ++gi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = gi * S::S + tr_l * 4 + i;
#pragma unroll
        for (int gj = 0; gj < S::G; ++gj) {
          T v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = acc[gi * 4 + i][gj * 4 + j];
          bstore4<T, VEC, EDGE>(m, ld, n_l, row, gj * S::S + tc_l * 4, v);
        }
      }
  }
}

// f(integral_constant<int, s>) for s = 0, 1, ..., in order.
template <int... S, typename F>
__device__ __forceinline__ void for_each_slot(std::integer_sequence<int, S...>, F&& f) {
  (f(std::integral_constant<int, S>{}), ...);
}

// One wave closes one graph of NB = 8 R vertices (NB <= 88), with no
// barrier between waves: lane (lr, lc) = (lane / 8, lane % 8) holds the
// elements (8 ri + lr, 8 cj + lc), ri, cj < R.  Pivot pairs (t, t + 1) come in
// increasing order and each element sees the same operations as in
// close_block_t, so the results are bit-identical to that closure.  A
// published pivot vector v is stored as p[8][16], v[8 q + r] at p[r][q], so a
// lane reads its R values from one 16-aligned run.
template <typename T, int NB, bool EDGE>
__global__ void __launch_bounds__(64)
__attribute__((amdgpu_waves_per_eu(2)))
fw_batched_wave(T* __restrict__ d, int64_t batch, int64_t n, int64_t ld, int64_t stride, T inf) {
  static_assert(NB % 8 == 0 && NB <= 88, "eight lanes per dimension; the tile fits two waves/SIMD");
  constexpr int R = NB / 8;
  // [buffer][column t, column t+1, row t, row t+1][8][16]
  __shared__ __attribute__((aligned(16))) T lds[2][4][128];
  const int lr = threadIdx.x >> 3, lc = threadIdx.x & 7;
  for (int64_t g = blockIdx.x; g < batch; g += gridDim.x) {
    T* m = d + g * stride;
    T acc[R][R];
    // As in fw_batched: per-graph copies keep the bounds from being hoisted
    // out of the graph loop, and out-of-range elements load from a clamped
    // address and are replaced by inf, with no branch per element.
    int lr_l = lr, lc_l = lc;
    int64_t n_l = n;
    asm volatile("" : "+v"(lr_l), "+v"(lc_l), "+s"(n_l));
#pragma unroll
    for (int ri = 0; ri < R; ++ri) {
      if constexpr (!EDGE) {
        // element (8 ri + lr, 8 cj + lc) at row[8 cj]
        const T* row = m + (int64_t)(8 * ri + lr) * ld + lc;
#pragma unroll
        for (int cj = 0; cj < R; ++cj) acc[ri][cj] = row[8 * cj];
      } else {
        const int i = 8 * ri + lr_l;
        const T* row = m + (int64_t)(i < n_l ? i : n_l - 1) * ld;
#pragma unroll
        for (int cj = 0; cj < R; ++cj) {
          const int64_t c = 8 * cj + lc_l;
          const T x = row[c < n_l ? c : n_l - 1];
          acc[ri][cj] = (i < n_l && c < n_l) ? x : inf;
        }
      }
    }
    // Pivots 8 s + owner and 8 s + owner + 1 into buffer buf.
    auto publish = [&](int buf, int owner, auto slot) {
      constexpr int s = decltype(slot)::value;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (lc == owner + h) {
#pragma unroll
          for (int ri = 0; ri < R; ++ri) lds[buf][h][lr * 16 + ri] = acc[ri][s];
        }
        if (lr == owner + h) {
#pragma unroll
          for (int cj = 0; cj < R; ++cj) lds[buf][2 + h][lc * 16 + cj] = acc[s][cj];
        }
      }
    };
    publish(0, 0, std::integral_constant<int, 0>{});
    __syncthreads();
    int buf = 0;
    for_each_slot(std::make_integer_sequence<int, R>{}, [&](auto slot) {
        constexpr int s = decltype(slot)::value;
#pragma unroll 1
        for (int c = 0; c < 4; ++c) {
          const int t1 = 8 * s + 2 * c + 1;
          const T* base = &lds[buf][0][0];
          T b0[R], b1[R];
#pragma unroll
          for (int k = 0; k < R; ++k) {
            b0[k] = base[256 + lc * 16 + k];
            b1[k] = base[384 + lc * 16 + k];
          }
          const int q1 = (t1 & 7) * 16 + (t1 >> 3);
          const T d_t_t1 = base[256 + q1];  // D[t][t+1]
          const T d_t1_t = base[q1];        // D[t+1][t]
#pragma unroll
          for (int k = 0; k < R; ++k) b1[k] = mp_min(b1[k], mp_add(d_t1_t, b0[k]));
          // The column values are read one row at a time: the tile and the row
          // vectors already hold most of the registers.
#pragma unroll
          for (int ri = 0; ri < R; ++ri) {
            const T a0 = base[lr * 16 + ri];
            const T a1 = mp_min(base[128 + lr * 16 + ri], mp_add(a0, d_t_t1));
#pragma unroll
            for (int cj = 0; cj < R; ++cj)
              acc[ri][cj] = mp_relax2(acc[ri][cj], a0, b0[cj], a1, b1[cj]);
          }
          buf ^= 1;
          if (c < 3) {
            publish(buf, 2 * c + 2, std::integral_constant<int, s>{});
          } else if constexpr (s + 1 < R) {
            publish(buf, 0, std::integral_constant<int, s + 1>{});
          }
          __syncthreads();
        }
    });
    // Recompute the addresses here rather than keep the loads' row pointers
    // live through the closure.
    int lr_s = lr, lc_s = lc;
    int64_t n_s = n;
    asm volatile("" : "+v"(lr_s), "+v"(lc_s), "+s"(n_s));
#pragma unroll
    for (int ri = 0; ri < R; ++ri) {
      const int i = 8 * ri + lr_s;
      T* row = m + (int64_t)i * ld + lc_s;
#pragma unroll
      for (int cj = 0; cj < R; ++cj)
        if (!EDGE || (i < n_s && 8 * cj + lc_s < n_s)) row[8 * cj] = acc[ri][cj];
    }
  }
}

template <typename T>
bool inf_ok(T inf);
template <>
bool inf_ok<int32_t>(int32_t inf) { return inf >= 1 && inf <= 0x3FFFFFFF; }
template <>
bool inf_ok<float>(float inf) { return inf > 0.0f; }  // false for NaN

template <typename T, int NB, int RT>
void launch(T* d, int64_t batch, int64_t n, int64_t ld, int64_t stride, T inf, bool vec,
            hipStream_t s) {
  const dim3 grid((unsigned)(batch < kMaxGrid ? batch : kMaxGrid));
  const dim3 block(BatchShape<NB, RT>::kThreads);
  if (n == NB) {
    if (vec) hipLaunchKernelGGL((fw_batched<T, NB, RT, true, false>), grid, block, 0, s, d, batch, n, ld, stride, inf);
    else hipLaunchKernelGGL((fw_batched<T, NB, RT, false, false>), grid, block, 0, s, d, batch, n, ld, stride, inf);
  } else {
    if (vec) hipLaunchKernelGGL((fw_batched<T, NB, RT, true, true>), grid, block, 0, s, d, batch, n, ld, stride, inf);
    else hipLaunchKernelGGL((fw_batched<T, NB, RT, false, true>), grid, block, 0, s, d, batch, n, ld, stride, inf);
  }
}

// The one-wave kernel where it measured faster than the workgroup closure
// (8192 complete graphs): NB = 72 by 1.3-1.4x in both types, NB = 80 by 1.1x
// in int32.  At NB = 88 the two tie; at NB = 96 and 104 the tile needs one
// wave per SIMD and runs 0.7-0.9x.
template <typename T, int NB>
constexpr bool kWaveClass = NB == 72 || (NB == 80 && std::is_same_v<T, int32_t>);

template <typename T, int NB>
void launch_class(T* d, int64_t batch, int64_t n, int64_t ld, int64_t stride, T inf, bool vec,
                  hipStream_t s) {
  if constexpr (!kWaveClass<T, NB>) {
    launch<T, NB, 8>(d, batch, n, ld, stride, inf, vec, s);
  } else {
    const dim3 grid((unsigned)(batch < kMaxGrid ? batch : kMaxGrid));
    if (n == NB)
      hipLaunchKernelGGL((fw_batched_wave<T, NB, false>), grid, dim3(64), 0, s, d, batch, n, ld,
                         stride, inf);
    else
      hipLaunchKernelGGL((fw_batched_wave<T, NB, true>), grid, dim3(64), 0, s, d, batch, n, ld,
                         stride, inf);
  }
}

template <typename T>
int run_batched(T* d, int64_t batch, int64_t n, int64_t ld, int64_t stride, T inf,
                void* stream) {
  if (batch < 0 || n < 0 || n > kMaxBatchedN) return APSP_ERR_INVALID_VALUE;
  if (batch == 0 || n == 0) return APSP_OK;
  if (d == nullptr || ld < n) return APSP_ERR_INVALID_VALUE;
  if ((reinterpret_cast<uintptr_t>(d) % sizeof(T)) != 0) return APSP_ERR_INVALID_VALUE;
  // Graph g occupies elements [g*stride, g*stride + (n-1)*ld + n); graphs
  // must not overlap and the last one must be addressable.
  const int64_t span = (n - 1) * ld + n;
  if (stride < span) return APSP_ERR_INVALID_VALUE;
  if (batch > 1 && stride > (INT64_MAX / (int64_t)sizeof(T) - span) / (batch - 1))
    return APSP_ERR_INVALID_VALUE;
  if (!inf_ok<T>(inf)) return APSP_ERR_INVALID_VALUE;
  int st = apsp_detail_check_device();
  if (st != APSP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool vec = (reinterpret_cast<uintptr_t>(d) % 16 == 0) && ld % 4 == 0 && stride % 4 == 0;
  switch ((n + 7) / 8) {
    case 1:
    case 2: launch<T, 16, 4>(d, batch, n, ld, stride, inf, vec, s); break;
    case 3: launch<T, 24, 4>(d, batch, n, ld, stride, inf, vec, s); break;
    case 4: launch<T, 32, 4>(d, batch, n, ld, stride, inf, vec, s); break;
    case 5: launch<T, 40, 8>(d, batch, n, ld, stride, inf, vec, s); break;
    case 6: launch<T, 48, 8>(d, batch, n, ld, stride, inf, vec, s); break;
    case 7: launch<T, 56, 8>(d, batch, n, ld, stride, inf, vec, s); break;
    case 8: launch<T, 64, 8>(d, batch, n, ld, stride, inf, vec, s); break;
    case 9: launch_class<T, 72>(d, batch, n, ld, stride, inf, vec, s); break;
    case 10: launch_class<T, 80>(d, batch, n, ld, stride, inf, vec, s); break;
    case 11: launch<T, 88, 8>(d, batch, n, ld, stride, inf, vec, s); break;
    case 12: launch<T, 96, 8>(d, batch, n, ld, stride, inf, vec, s); break;
    case 13: launch<T, 104, 8>(d, batch, n, ld, stride, inf, vec, s); break;
    case 14: launch<T, 112, 8>(d, batch, n, ld, stride, inf, vec, s); break;
    case 15: launch<T, 120, 8>(d, batch, n, ld, stride, inf, vec, s); break;
    default: launch<T, 128, 8>(d, batch, n, ld, stride, inf, vec, s); break;
  }
  return apsp_detail_launch_status();
}

}  // namespace

extern "C" {

int apsp_fw_batched_i32(int32_t* d, int64_t batch, int64_t n, int64_t ld, int64_t stride,
                        int32_t inf, void* stream) {
  return run_batched<int32_t>(d, batch, n, ld, stride, inf, stream);
}

int apsp_fw_batched_f32(float* d, int64_t batch, int64_t n, int64_t ld, int64_t stride,
                        float inf, void* stream) {
  return run_batched<float>(d, batch, n, ld, stride, inf, stream);
}

}  // extern "C"
