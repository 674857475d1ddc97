// Empirical VALU ceiling of the min-plus core on the current device.
//
// A register-only replica of the Phase-3 inner step: each thread holds an
// 8 x 8 block of accumulators and, per pair of pivots, forms two candidate
// sums per accumulator and folds them in with one three-input min -- the
// same add, add, min3 instruction mix as the tile kernel, but with operands
// already in registers (no LDS, no global memory, no barriers).  It runs at
// 2 and at 4 waves per SIMD and reports the faster: binary32's double issue
// rate needs more than one wave per SIMD, and an odd wave count leaves part
// of it unused, so this is the most the tile kernel's instruction stream can
// reach on this device and clock.  It is reported next to the peak derived
// from unit counts and clock.  A third mix replicates the successor
// product's packed keys: two unsigned saturating adds and one unsigned
// three-input min per pair of candidates.  apsp_minplus_ceiling_waves runs
// it at one given wave count (1 to 4 per SIMD).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "apsp.h"

namespace {

__device__ __forceinline__ int32_t ceil_min3(int32_t a, int32_t b, int32_t c) {
  int32_t r;
  asm("v_min3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float ceil_min3(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ uint32_t ceil_min3(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_min3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// A candidate sum: binary32, or saturating for the unsigned packed
// (sum, index) keys of the successor product.
template <typename T>
__device__ __forceinline__ T ceil_add(T a, T b) {
  if constexpr (std::is_same_v<T, uint32_t>) {
    return __builtin_elementwise_add_sat(a, b);
  } else {
    return a + b;
  }
}

// One accumulator over two candidates, in the tile kernels' instruction
// order: for int32 the two VOP3 adds and the v_min3_i32 are issued in
// sequence (as the kernels' volatile sequence does); otherwise as written.
template <typename T>
__device__ __forceinline__ T ceil_relax2(T acc, T a0, T b0, T a1, T b1) {
  if constexpr (std::is_same_v<T, int32_t>) {
    int32_t t0, t1, r;
    asm volatile("v_add_u32_e64 %0, %1, %2" : "=v"(t0) : "v"(a0), "v"(b0));
    asm volatile("v_add_u32_e64 %0, %1, %2" : "=v"(t1) : "v"(a1), "v"(b1));
    asm volatile("v_min3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(acc), "v"(t0), "v"(t1));
    return r;
  } else {
    return ceil_min3(acc, ceil_add(a0, b0), ceil_add(a1, b1));
  }
}

template <typename T>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
minplus_core(T* __restrict__ out, int iters) {
  T acc[8][8], a0[8], a1[8], b0[8], b1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a0[i] = (T)(threadIdx.x + i);
    a1[i] = (T)(2 * threadIdx.x + i);
    b0[i] = (T)(3 * i);
    b1[i] = (T)(5 * i + 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = (T)(1000000 + 8 * i + j);
  }
  for (int it = 0; it < iters; ++it) {
    // Opaque to the compiler: the sums cannot be hoisted out of the loop.
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(a0[i]), "+v"(a1[i]), "+v"(b0[i]), "+v"(b1[i]));
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = ceil_relax2(acc[i][j], a0[i], b0[j], a1[i], b1[j]);
  }
  T s = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) s = s + acc[i][j];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

template <typename T>
int measure(int waves_per_simd, double* relax_per_s) {
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return APSP_ERR_NO_DEVICE;
  // A 256-thread workgroup puts one wave on each of a CU's 4 SIMDs.
  const int blocks = waves_per_simd * prop.multiProcessorCount;
  const int iters = 4000;
  T* out = nullptr;
  if (hipMalloc(&out, (size_t)blocks * 256 * sizeof(T)) != hipSuccess) return APSP_ERR_LAUNCH;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int st = APSP_OK;
  float ms = 0.f;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) st = APSP_ERR_LAUNCH;
  if (st == APSP_OK) {
    hipLaunchKernelGGL((minplus_core<T>), dim3(blocks), dim3(256), 0, 0, out, iters / 8);  // warm-up
    (void)hipEventRecord(e0, 0);
    hipLaunchKernelGGL((minplus_core<T>), dim3(blocks), dim3(256), 0, 0, out, iters);
    (void)hipEventRecord(e1, 0);
    if (hipEventSynchronize(e1) != hipSuccess || hipGetLastError() != hipSuccess ||
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess || ms <= 0.f)
      st = APSP_ERR_LAUNCH;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(out);
  if (st == APSP_OK && relax_per_s)
    *relax_per_s = (double)blocks * 256.0 * iters * 128.0 / (ms * 1e-3);
  return st;
}

template <typename T>
int measure_best(double* relax_per_s) {
  double best = 0.0;
  for (int w : {2, 4}) {
    double r = 0.0;
    const int st = measure<T>(w, &r);
    if (st != APSP_OK) return st;
    if (r > best) best = r;
  }
  *relax_per_s = best;
  return APSP_OK;
}

}  // namespace

extern "C" int apsp_minplus_ceiling(int arith, double* relax_per_s) {
  if (relax_per_s == nullptr || arith < 0 || arith > 2) return APSP_ERR_INVALID_VALUE;
  if (arith == 2) return measure_best<uint32_t>(relax_per_s);
  return arith == 1 ? measure_best<float>(relax_per_s) : measure_best<int32_t>(relax_per_s);
}

// The same replica at a given number of waves per SIMD.  The double rate
// pairs two waves of a SIMD, so an odd count leaves one wave single-issue:
// this is the rate a kernel resident at that count can reach.
extern "C" int apsp_minplus_ceiling_waves(int arith, int waves_per_simd, double* relax_per_s) {
  if (relax_per_s == nullptr || arith < 0 || arith > 2 || waves_per_simd < 1 ||
      waves_per_simd > 4)
    return APSP_ERR_INVALID_VALUE;
  if (arith == 2) return measure<uint32_t>(waves_per_simd, relax_per_s);
  return arith == 1 ? measure<float>(waves_per_simd, relax_per_s)
                    : measure<int32_t>(waves_per_simd, relax_per_s);
}
