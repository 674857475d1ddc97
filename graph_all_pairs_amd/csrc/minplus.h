// Device building blocks shared by the blocked Floyd-Warshall kernels and
// the batched small-graph kernels: the min-plus element operations, 128-bit
// tile element access with edge predication, and the in-register closure of
// one diagonal block (Phase 1 of the page "Katz and Kider", thesis section
// 4.6, Algorithm 16).
#ifndef APSP_MINPLUS_H
#define APSP_MINPLUS_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace apsp_dev {

// ---------------------------------------------------------------------------
// Element operations.  int32: wrap-free because every value is <= inf <=
// 2^30 - 1.  float32: IEEE add and min (no NaN by precondition).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int32_t mp_min(int32_t a, int32_t b) { return min(a, b); }
__device__ __forceinline__ float mp_min(float a, float b) {
  float r;  // no NaN by precondition, so no canonicalising fminf
  asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// A candidate sum.  int32: the wrapping add written in its VOP3 encoding.
// With it the add, add, min3 mix issues about 1.4x faster on gfx950 than
// with the VOP2 form the compiler picks for a + b (a register-only replica
// measures 35 against 25-26 T relaxations/s); the result is the same add.
__device__ __forceinline__ int32_t mp_add(int32_t a, int32_t b) {
  int32_t r;
  asm("v_add_u32_e64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float mp_add(float a, float b) { return a + b; }

// min(a, b, c) as one v_min3.  Written as an instruction so that the compiler
// keeps one three-input min per pair of candidates instead of re-balancing
// the chain into two-input mins.
__device__ __forceinline__ int32_t mp_min3(int32_t a, int32_t b, int32_t c) {
  int32_t r;
  asm("v_min3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float mp_min3(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// One min-plus step of an accumulator over two pivots:
//   acc <- min(acc, a0 + b0, a1 + b1).
// binary32: plain adds (the compiler interleaves them freely) and one v_min3.
// int32: the two adds in their VOP3 encoding and one v_min3_i32, issued in
// this order (volatile keeps the three together, so no more than two sums
// are live per accumulator and the register allocation stays that of the
// plain code).  Measured in the Phase-3 tile loop at n = 8192: 355 us per
// launch with the compiler's VOP2 add, 281 us with unordered VOP3 adds, 278
// us with this sequence; the arithmetic is the same wrapping add.
__device__ __forceinline__ float mp_relax2(float acc, float a0, float b0, float a1, float b1) {
  return mp_min3(acc, a0 + b0, a1 + b1);
}
__device__ __forceinline__ int32_t mp_relax2(int32_t acc, int32_t a0, int32_t b0, int32_t a1,
                                             int32_t b1) {
  int32_t t0, t1, r;
  asm volatile("v_add_u32_e64 %0, %1, %2" : "=v"(t0) : "v"(a0), "v"(b0));
  asm volatile("v_add_u32_e64 %0, %1, %2" : "=v"(t1) : "v"(a1), "v"(b1));
  asm volatile("v_min3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(acc), "v"(t0), "v"(t1));
  return r;
}

// An int32 matrix computed in binary32 (only when that is exact): entry in,
// and result back.  "No edge" (the sentinel inf) becomes +infinity.  Back,
// the value is compared with inf as an integer, not as (float)inf: 2^24 + 1
// rounds to 2^24 in binary32, so a float comparison would turn an exact
// distance of 2^24 into inf.  +infinity, and anything not below 2^31, is
// inf; values not above -2^31 (only after a negative cycle) saturate, and
// NaN goes there too.
__device__ __forceinline__ float i32_to_f32(int32_t v, int32_t inf) {
  return v == inf ? __builtin_inff() : (float)v;
}
__device__ __forceinline__ int32_t f32_to_i32(float f, int32_t inf) {
  if (!(f > -2147483648.0f)) return INT32_MIN;
  if (!(f < 2147483648.0f)) return inf;
  const int32_t v = (int32_t)f;
  return v >= inf ? inf : v;
}

template <typename T> struct Vec4;
template <> struct Vec4<int32_t> { using type = int4; };
template <> struct Vec4<float> { using type = float4; };

template <typename T>
__device__ __forceinline__ void load4(const T* __restrict__ p, T (&v)[4]) {
  using V = typename Vec4<T>::type;
  V x = *reinterpret_cast<const V*>(p);
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}

template <typename T>
__device__ __forceinline__ void store4(T* __restrict__ p, const T (&v)[4]) {
  using V = typename Vec4<T>::type;
  V x; x.x = v[0]; x.y = v[1]; x.z = v[2]; x.w = v[3];
  *reinterpret_cast<V*>(p) = x;
}

// Four consecutive elements of row `row`, columns col .. col+3, of the
// matrix; out-of-range elements read as inf.  VEC: one 128-bit load when the
// whole quad is in range.  EDGE=false promises the quad is in range.
template <typename T, bool VEC, bool EDGE>
__device__ __forceinline__ void gload4(const T* __restrict__ d, int64_t ld, int64_t n,
                                       int64_t row, int64_t col, T inf, T (&v)[4]) {
  const T* p = d + row * ld + col;
  if (!EDGE) {
    if (VEC) { load4(p, v); }
    else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = p[e];
    }
  } else {
    if (row < n && col + 3 < n) {
      if (VEC) { load4(p, v); }
      else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = p[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (row < n && col + e < n) ? p[e] : inf;
    }
  }
}

template <typename T, bool VEC, bool EDGE>
__device__ __forceinline__ void gstore4(T* __restrict__ d, int64_t ld, int64_t n,
                                        int64_t row, int64_t col, const T (&v)[4]) {
  T* p = d + row * ld + col;
  if (!EDGE) {
    if (VEC) { store4(p, v); }
    else {
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = v[e];
    }
  } else {
    if (row < n && col + 3 < n) {
      if (VEC) { store4(p, v); }
      else {
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = v[e];
      }
    } else if (row < n) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (col + e < n) p[e] = v[e];
    }
  }
}

// ---------------------------------------------------------------------------
// Phase 1 on an NB x NB block held in registers, RT x RT elements per thread
// (for NB = 128, RT = 8 this is the Phase-3 layout of a 256-thread
// workgroup): Floyd-Warshall over the block's own pivots t = 0 .. NB-1, in
// order, two pivots per step.
//
// With D the block before pivot t, the plain recurrence gives after pivots t
// and t+1
//   D1[x][y] = min(D[x][y], D[x][t] + D[t][y])
//   D2[x][y] = min(D1[x][y], D1[x][t+1] + D1[t+1][y])
//            = min(D[x][y], D[x][t] + D[t][y], D1[x][t+1] + D1[t+1][y]),
// and the only D1 values that takes are column t+1 and row t+1:
//   D1[x][t+1] = min(D[x][t+1], D[x][t] + D[t][t+1]),
//   D1[t+1][y] = min(D[t+1][y], D[t+1][t] + D[t][y]).
// So a step publishes columns t, t+1 and rows t, t+1 of D to LDS, every
// thread forms D1's column and row entries for its own 8 rows and 8 columns,
// and each element takes one three-input min.  Every stored value is the
// same expression, evaluated the same way, as in the one-pivot-at-a-time
// recurrence, so float results equal the plain sequential Floyd-Warshall on
// the block bit for bit.  Ping-pong LDS buffers: one barrier per pivot pair.
// ---------------------------------------------------------------------------
//
// Generic in the block edge NB and the micro-tile edge RT (a multiple of 4):
// a workgroup of (NB/RT)^2 threads, thread (tr, tc) holding rows and columns
// g*S + 4*tr + i and g*S + 4*tc + j for g < RT/4, i, j < 4, S = NB/(RT/4).
// LDS: 8*NB elements.
//
// MASK (int32 successor keys, value << s | first hop): every value taken
// from a pivot row -- the second operand of a sum -- has its low s bits
// cleared (AND with km), so a sum keeps the first operand's first hop.
template <typename T, int NB, int RT, bool MASK = false>
__device__ __forceinline__ void close_block_t(T (&acc)[RT][RT], T* __restrict__ lds,
                                              T km = T(0)) {
  static_assert(RT % 4 == 0 && NB % RT == 0, "micro-tile of 4x4 groups");
  constexpr int G = RT / 4;          // 4-wide groups per thread and dimension
  constexpr int S = NB / G;          // distance between a thread's groups
  constexpr int kThr = NB / RT;      // threads per dimension
  // lds: [2 buffers][4][NB] = column t, column t+1, row t, row t+1
  const int tc = threadIdx.x % kThr;
  const int tr = threadIdx.x / kThr;

  // Pivot t = S g + 4 q + c lives in register slot s = 4 g + c of the
  // threads with tc == q (its column) and tr == q (its row).
  auto publish = [&](int buf, int owner, int slot) {
    T* base = lds + buf * 4 * NB;
    if (tc == owner) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
          T v[4] = {acc[4 * gi][slot + h], acc[4 * gi + 1][slot + h], acc[4 * gi + 2][slot + h],
                    acc[4 * gi + 3][slot + h]};
          store4(&base[h * NB + gi * S + tr * 4], v);
        }
    }
    if (tr == owner) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int gj = 0; gj < G; ++gj) {
          T v[4] = {acc[slot + h][4 * gj], acc[slot + h][4 * gj + 1], acc[slot + h][4 * gj + 2],
                    acc[slot + h][4 * gj + 3]};
          if constexpr (MASK) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] &= km;
          }
          store4(&base[(2 + h) * NB + gj * S + tc * 4], v);
        }
    }
  };

  publish(0, 0, 0);
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll 1
    for (int q = 0; q < kThr; ++q) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int t = S * g + 4 * q + 2 * cc;  // first pivot of the pair
        const T* base = lds + cc * 4 * NB;     // pair index (S g + 4 q)/2 + cc has parity cc
        T a0[RT], a1[RT], b0[RT], b1[RT];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          T v[4];
          load4(&base[tr * 4 + S * h], v);
#pragma unroll
          for (int i = 0; i < 4; ++i) a0[4 * h + i] = v[i];
          load4(&base[NB + tr * 4 + S * h], v);
#pragma unroll
          for (int i = 0; i < 4; ++i) a1[4 * h + i] = v[i];
          load4(&base[2 * NB + tc * 4 + S * h], v);
#pragma unroll
          for (int j = 0; j < 4; ++j) b0[4 * h + j] = v[j];
          load4(&base[3 * NB + tc * 4 + S * h], v);
#pragma unroll
          for (int j = 0; j < 4; ++j) b1[4 * h + j] = v[j];
        }
        const T d_t_t1 = base[2 * NB + t + 1];  // D[t][t+1]
        T d_t1_t = base[t + 1];                 // D[t+1][t]
        // D[t+1][t] + D[t][y] forms a pivot-row value (row t+1 after pivot t)
        if constexpr (MASK) d_t1_t &= km;
#pragma unroll
        for (int i = 0; i < RT; ++i) a1[i] = mp_min(a1[i], mp_add(a0[i], d_t_t1));
#pragma unroll
        for (int j = 0; j < RT; ++j) b1[j] = mp_min(b1[j], mp_add(d_t1_t, b0[j]));
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
          for (int j = 0; j < RT; ++j) acc[i][j] = mp_relax2(acc[i][j], a0[i], b0[j], a1[i], b1[j]);

        // publish the next pair into the other buffer
        if (cc == 0) {
          publish(1, q, 4 * g + 2);
        } else if (q + 1 < kThr) {
          publish(0, q + 1, 4 * g);
        } else if (g + 1 < G) {
          publish(0, 0, 4 * (g + 1));
        }
        __syncthreads();
      }
    }
  }
}

}  // namespace apsp_dev

#endif  // APSP_MINPLUS_H
