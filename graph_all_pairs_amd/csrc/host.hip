// All-pairs shortest paths of a matrix held in host memory: the blocked
// Floyd-Warshall of the page "Katz and Kider" (thesis section 4.6) with a
// second, outer level of blocking, for graphs larger than device memory
// (its section 4.6.1 names the limit: the whole graph must sit in global
// memory).
//
// Outer round KK takes pivots [K0, K0 + S) for an outer block S (a multiple
// of 128 sized to the device budget) and runs the same three phases on S x S
// super-blocks:
//   Phase 1  the diagonal super-block D_KK is closed on the device by the
//            in-core blocked Floyd-Warshall (apsp_fw_*, S/128 rounds);
//   Phase 2  the pivot-row panel D_KJ <- min(D_KJ, D*_KK (x) D_KJ) and the
//            pivot-column panel D_IK <- min(D_IK, D_IK (x) D*_KK), as min-plus
//            products with the closed block (the same reading as the in-core
//            Phase 2: both equal the shortest distances through blocks <= K);
//   Phase 3  every other super-tile D_IJ <- min(D_IJ, D_IK (x) D_KJ), depth S.
// The two panels (S x n and n x S) stay in HBM for the round; the other
// super-tiles stream host -> device -> host.  Per round the matrix crosses
// PCIe once each way, for n^2 S relaxations: S / 8 relaxations per byte
// moved (1024 at S = 8192), so with the transfers overlapped the products
// set the pace.
//
// gfx950 / runtime design: the Phase-3 super-tiles go round-robin to three
// slot streams, each with its own device tile buffer, running copy-in ->
// product -> copy-out in order; three slots let one tile's copies overlap
// another's product.  The products are the min-plus product kernel
// (gemm.hip), whose C tile stays in registers over the whole depth S.  An
// int32 matrix is computed in binary32 when that is exact (the condition of
// apsp_fw_i32), decided by a device scan streamed over the matrix first;
// tiles and panels are converted on the device after they arrive and before
// they leave.  All streams keep the default priority.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "apsp.h"
#include "detail.h"
#include "minplus.h"

int apsp_detail_gemm_i32(int32_t* C, int64_t ldc, const int32_t* A, int64_t lda, const int32_t* B,
                         int64_t ldb, int64_t m, int64_t n, int64_t k, int32_t inf, void* stream);
int apsp_detail_gemm_f32(float* C, int64_t ldc, const float* A, int64_t lda, const float* B,
                         int64_t ldb, int64_t m, int64_t n, int64_t k, float inf, void* stream);

namespace {

using namespace apsp_dev;

constexpr int64_t kB = 128;
constexpr int kSlots = 3;
constexpr int64_t kExactLimit = int64_t(1) << 24;

struct HostScan {
  int32_t maxw;   // largest finite entry
  int32_t flags;  // 1: an off-diagonal entry equals inf; 2: an entry < 0 or > 2^24
  int32_t pad[2];
};

__global__ void __launch_bounds__(64) hs_zero(HostScan* s) {
  if (threadIdx.x == 0) *s = HostScan{0, 0, {0, 0}};
}

// Scan of one rows x cols tile whose element (0,0) is matrix element (r0, c0).
__global__ void __launch_bounds__(256) hs_scan(const int32_t* __restrict__ t, int64_t ld,
                                               int64_t rows, int64_t cols, int64_t r0, int64_t c0,
                                               int32_t inf, HostScan* s) {
  int32_t mx = 0, fl = 0;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x)
    for (int64_t c = threadIdx.x; c < cols; c += blockDim.x) {
      const int32_t v = t[r * ld + c];
      if (v == inf) {
        if (r0 + r != c0 + c) fl |= 1;
      } else {
        if (v < 0 || v > kExactLimit) fl |= 2;
        mx = max(mx, v);
      }
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mx = max(mx, __shfl_xor(mx, o));
    fl |= __shfl_xor(fl, o);
  }
  if ((threadIdx.x & 63) == 0) {
    if (mx) atomicMax(&s->maxw, mx);
    if (fl) atomicOr(&s->flags, fl);
  }
}

// In place over a rows x cols tile: int32 <-> binary32 (inf <-> +infinity;
// back from binary32 anything >= inf is inf).
template <bool TO_F32>
__global__ void __launch_bounds__(256) hs_convert(int32_t* __restrict__ t, int64_t ld, int64_t rows,
                                                  int64_t cols, int32_t inf) {
  const float finf = (float)inf;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x)
    for (int64_t c = threadIdx.x; c < cols; c += blockDim.x) {
      int32_t* p = t + r * ld + c;
      if (TO_F32) {
        *p = __float_as_int(*p == inf ? __builtin_inff() : (float)*p);
      } else {
        const float f = __int_as_float(*p);
        *p = f >= finf ? inf : (int32_t)f;
      }
    }
}

int hip_failed() {
  (void)apsp_detail_launch_status();
  return APSP_ERR_LAUNCH;
}

#define HIP_TRY(x)                  \
  do {                              \
    if ((x) != hipSuccess) {        \
      rc = hip_failed();            \
      goto done;                    \
    }                               \
  } while (0)

// 2-D copy of rows x cols elements between buffers with leading dimensions
// (in elements) ld_dst and ld_src.
template <typename E>
hipError_t copy2d(E* dst, int64_t ld_dst, const E* src, int64_t ld_src, int64_t rows, int64_t cols,
                  hipMemcpyKind kind, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  return hipMemcpy2DAsync(dst, ld_dst * sizeof(E), src, ld_src * sizeof(E), cols * sizeof(E),
                          rows, kind, s);
}

unsigned conv_grid(int64_t rows) { return (unsigned)std::min<int64_t>(std::max<int64_t>(rows, 1), 2048); }

// The rounds with compute type CT on matrix element type E (int32 -> int32,
// int32 -> binary32, float -> float).
template <typename E, typename CT>
int run_rounds(E* h, int64_t n, int64_t ldh, E inf, int64_t S, char* dev, hipStream_t s,
               hipStream_t* slot, hipEvent_t* ev) {
  constexpr bool kConv = std::is_same_v<E, int32_t> && std::is_same_v<CT, float>;
  const CT cinf = kConv ? CT(__builtin_inff()) : CT(inf);
  const int64_t ldr = (n + 3) & ~int64_t(3);  // row panel leading dimension
  E* rp = reinterpret_cast<E*>(dev);                  // S x n (pivot rows)
  E* cp = rp + S * ldr;                               // n x S (pivot columns)
  E* tmp = cp + n * S;                                // S x S
  E* sb[kSlots];                                      // S x S per slot
  for (int i = 0; i < kSlots; ++i) sb[i] = tmp + (int64_t)(i + 1) * S * S;
  const int64_t rounds = (n + S - 1) / S;
  int rc = APSP_OK;

  auto conv = [&](E* t, int64_t ld, int64_t rows, int64_t cols, bool to_f32, hipStream_t st) {
    if constexpr (kConv) {
      if (to_f32)
        hipLaunchKernelGGL(hs_convert<true>, dim3(conv_grid(rows)), dim3(256), 0, st, t, ld, rows, cols, inf);
      else
        hipLaunchKernelGGL(hs_convert<false>, dim3(conv_grid(rows)), dim3(256), 0, st, t, ld, rows, cols, inf);
    }
  };
  auto gemm = [&](E* C, int64_t ldc, const E* A, int64_t lda, const E* B, int64_t ldb, int64_t m,
                  int64_t nn, int64_t k, hipStream_t st) -> int {
    if constexpr (std::is_same_v<CT, float>)
      return apsp_detail_gemm_f32(reinterpret_cast<float*>(C), ldc, reinterpret_cast<const float*>(A),
                                  lda, reinterpret_cast<const float*>(B), ldb, m, nn, k, cinf, st);
    else
      return apsp_detail_gemm_i32(C, ldc, A, lda, B, ldb, m, nn, k, cinf, st);
  };

  for (int64_t KK = 0; KK < rounds; ++KK) {
    const int64_t K0 = KK * S, sk = std::min(S, n - K0);
    // -- panels in -----------------------------------------------------------
    HIP_TRY(copy2d(rp, ldr, h + K0 * ldh, ldh, sk, n, hipMemcpyHostToDevice, s));
    HIP_TRY(copy2d(cp, S, h + K0, ldh, n, sk, hipMemcpyHostToDevice, s));
    conv(rp, ldr, sk, n, true, s);
    conv(cp, S, n, sk, true, s);
    // -- Phase 1: close D_KK in place inside the row panel, copy it into the
    //    column panel ----------------------------------------------------------
    {
      int st;
      if constexpr (std::is_same_v<CT, float>)
        st = apsp_fw_f32(reinterpret_cast<float*>(rp + K0), sk, ldr, cinf, s);
      else
        st = apsp_fw_i32(rp + K0, sk, ldr, cinf, s);
      if (st != APSP_OK) {
        rc = st;
        goto done;
      }
    }
    HIP_TRY(copy2d(cp + K0 * S, S, rp + K0, ldr, sk, sk, hipMemcpyDeviceToDevice, s));
    // -- Phase 2: panels as products with the closed block (old panel values
    //    on the right-hand side come from a copy) ------------------------------
    for (int64_t J0 = 0; J0 < n; J0 += S) {
      if (J0 == K0) continue;
      const int64_t wj = std::min(S, n - J0);
      HIP_TRY(copy2d(tmp, S, rp + J0, ldr, sk, wj, hipMemcpyDeviceToDevice, s));
      if ((rc = gemm(rp + J0, ldr, rp + K0, ldr, tmp, S, sk, wj, sk, s)) != APSP_OK) goto done;
    }
    for (int64_t I0 = 0; I0 < n; I0 += S) {
      if (I0 == K0) continue;
      const int64_t hi = std::min(S, n - I0);
      HIP_TRY(copy2d(tmp, S, cp + I0 * S, S, hi, sk, hipMemcpyDeviceToDevice, s));
      if ((rc = gemm(cp + I0 * S, S, tmp, S, rp + K0, ldr, hi, sk, sk, s)) != APSP_OK) goto done;
    }
    HIP_TRY(hipEventRecord(ev[0], s));
    // -- Phase 3: every other super-tile through the slot streams -------------
    {
      int64_t t = 0;
      for (int i = 0; i < kSlots; ++i) HIP_TRY(hipStreamWaitEvent(slot[i], ev[0], 0));
      for (int64_t I0 = 0; I0 < n; I0 += S) {
        if (I0 == K0) continue;
        const int64_t hi = std::min(S, n - I0);
        for (int64_t J0 = 0; J0 < n; J0 += S, ++t) {
          if (J0 == K0) {
            --t;
            continue;
          }
          const int64_t wj = std::min(S, n - J0);
          hipStream_t st = slot[t % kSlots];
          E* b = sb[t % kSlots];
          E* ht = h + I0 * ldh + J0;
          HIP_TRY(copy2d(b, S, ht, ldh, hi, wj, hipMemcpyHostToDevice, st));
          conv(b, S, hi, wj, true, st);
          if ((rc = gemm(b, S, cp + I0 * S, S, rp + J0, ldr, hi, wj, sk, st)) != APSP_OK) goto done;
          conv(b, S, hi, wj, false, st);
          HIP_TRY(copy2d(ht, ldh, b, S, hi, wj, hipMemcpyDeviceToHost, st));
        }
      }
      for (int i = 0; i < kSlots; ++i) {
        HIP_TRY(hipEventRecord(ev[1 + i], slot[i]));
        HIP_TRY(hipStreamWaitEvent(s, ev[1 + i], 0));
      }
    }
    // -- panels out (after every product of the round has read them) ----------
    conv(rp, ldr, sk, n, false, s);
    conv(cp, S, n, sk, false, s);
    HIP_TRY(copy2d(h + K0 * ldh, ldh, rp, ldr, sk, n, hipMemcpyDeviceToHost, s));
    HIP_TRY(copy2d(h + K0, ldh, cp, S, n, sk, hipMemcpyDeviceToHost, s));
    if ((rc = apsp_detail_launch_status()) != APSP_OK) goto done;
  }
done:
  return rc;
}

template <typename E>
bool inf_ok(E inf);
template <>
bool inf_ok<int32_t>(int32_t inf) { return inf >= 1 && inf <= 0x3FFFFFFF; }
template <>
bool inf_ok<float>(float inf) { return inf > 0.0f; }

template <typename E>
int run_host(E* h, int64_t n, int64_t ldh, E inf, int64_t device_bytes, void* stream,
             int64_t* outer_block) {
  if (outer_block) *outer_block = 0;
  if (n < 0 || !inf_ok<E>(inf)) return APSP_ERR_INVALID_VALUE;
  if (n == 0) return APSP_OK;
  if (h == nullptr || ldh < n || reinterpret_cast<uintptr_t>(h) % sizeof(E) != 0 ||
      n > (int64_t(1) << 31) || ldh > INT64_MAX / (int64_t)sizeof(E) / n || device_bytes < 0)
    return APSP_ERR_INVALID_VALUE;
  int rc = apsp_detail_check_device();
  if (rc != APSP_OK) return rc;

  // Outer block: the largest multiple of 128 (at most n rounded up) whose
  // buffers -- two panels, the copy buffer and three slot tiles --
  // fit the budget (default: half of the free device memory).
  int64_t budget = device_bytes;
  if (budget == 0) {
    size_t fr = 0, tot = 0;
    if (hipMemGetInfo(&fr, &tot) != hipSuccess) return hip_failed();
    budget = (int64_t)(fr / 2);
  }
  const int64_t ldr = (n + 3) & ~int64_t(3);
  const int64_t n128 = (n + kB - 1) / kB * kB;
  auto bytes_for = [&](int64_t S) {
    return (int64_t)sizeof(E) * (S * ldr + n * S + (1 + kSlots) * S * S);
  };
  int64_t S = 0;
  for (int64_t c = kB; c <= n128; c += kB) {
    if (bytes_for(c) > budget) break;
    S = c;
  }
  if (S == 0) return APSP_ERR_RANGE;
  if (outer_block) *outer_block = S;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipStream_t slot[kSlots] = {};
  hipEvent_t ev[1 + kSlots] = {};
  char* dev = nullptr;
  HostScan* scan = nullptr;
  HostScan hs{};
  bool f32 = false;
  for (int i = 0; i < kSlots; ++i)
    if (hipStreamCreateWithFlags(&slot[i], hipStreamNonBlocking) != hipSuccess) {
      rc = hip_failed();
      goto cleanup;
    }
  for (auto& e : ev)
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
      rc = hip_failed();
      goto cleanup;
    }
  if (hipMallocAsync(reinterpret_cast<void**>(&dev), (size_t)bytes_for(S), s) != hipSuccess ||
      hipMallocAsync(reinterpret_cast<void**>(&scan), sizeof(HostScan), s) != hipSuccess) {
    rc = hip_failed();
    goto cleanup;
  }

  if constexpr (std::is_same_v<E, int32_t>) {
    // Which arithmetic: stream the matrix through the first slot buffer once.
    const int policy = apsp_get_int32_arith();
    if (policy != APSP_ARITH_INT32) {
      E* buf = reinterpret_cast<E*>(dev) + S * ldr + n * S;
      hipLaunchKernelGGL(hs_zero, dim3(1), dim3(64), 0, s, scan);
      for (int64_t r0 = 0; r0 < n && rc == APSP_OK; r0 += S) {
        const int64_t rows = std::min(S, n - r0);
        for (int64_t c0 = 0; c0 < n; c0 += S) {
          const int64_t cols = std::min(S, n - c0);
          if (copy2d(buf, S, h + r0 * ldh + c0, ldh, rows, cols, hipMemcpyHostToDevice, s) != hipSuccess) {
            rc = hip_failed();
            break;
          }
          hipLaunchKernelGGL(hs_scan, dim3(conv_grid(rows)), dim3(256), 0, s, buf, S, rows, cols,
                             r0, c0, inf, scan);
        }
      }
      if (rc != APSP_OK) goto cleanup;
      if (hipMemcpyAsync(&hs, scan, sizeof(hs), hipMemcpyDeviceToHost, s) != hipSuccess ||
          hipStreamSynchronize(s) != hipSuccess) {
        rc = hip_failed();
        goto cleanup;
      }
      f32 = !(hs.flags & 2) && (!(hs.flags & 1) || (n - 1) * (int64_t)hs.maxw <= kExactLimit);
    }
    if (f32) rc = run_rounds<int32_t, float>(h, n, ldh, inf, S, dev, s, slot, ev);
    else rc = run_rounds<int32_t, int32_t>(h, n, ldh, inf, S, dev, s, slot, ev);
  } else {
    rc = run_rounds<float, float>(h, n, ldh, inf, S, dev, s, slot, ev);
  }

cleanup:
  (void)hipStreamSynchronize(s);
  for (auto& st : slot)
    if (st) (void)hipStreamSynchronize(st);
  if (dev) (void)hipFreeAsync(dev, s);
  if (scan) (void)hipFreeAsync(scan, s);
  (void)hipStreamSynchronize(s);
  for (auto& e : ev)
    if (e) (void)hipEventDestroy(e);
  for (auto& st : slot)
    if (st) (void)hipStreamDestroy(st);
  return rc;
}

}  // namespace

extern "C" {

int apsp_fw_host_i32(int32_t* h, int64_t n, int64_t ld, int32_t inf, int64_t device_bytes,
                     void* stream, int64_t* outer_block) {
  return run_host<int32_t>(h, n, ld, inf, device_bytes, stream, outer_block);
}

int apsp_fw_host_f32(float* h, int64_t n, int64_t ld, float inf, int64_t device_bytes,
                     void* stream, int64_t* outer_block) {
  return run_host<float>(h, n, ld, inf, device_bytes, stream, outer_block);
}

}  // extern "C"
