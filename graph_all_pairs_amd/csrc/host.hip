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
#include <functional>
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
constexpr int kRetryInt32 = -1000;  // private: binary32 turned out not to be exact
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
// back from binary32 anything >= inf is inf, compared as integers).
template <bool TO_F32>
__global__ void __launch_bounds__(256) hs_convert(int32_t* __restrict__ t, int64_t ld, int64_t rows,
                                                  int64_t cols, int32_t inf) {
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x)
    for (int64_t c = threadIdx.x; c < cols; c += blockDim.x) {
      int32_t* p = t + r * ld + c;
      if (TO_F32) *p = __float_as_int(i32_to_f32(*p, inf));
      else *p = f32_to_i32(__int_as_float(*p), inf);
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

// Convert-copy of a rows x cols binary32 tile to int32 (anything >= inf is
// inf), for panels that are written back while still being read as binary32.
__global__ void __launch_bounds__(256) hs_to_i32(int32_t* __restrict__ dst, int64_t ldd,
                                                 const float* __restrict__ src, int64_t lds,
                                                 int64_t rows, int64_t cols, int32_t inf) {
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x)
    for (int64_t c = threadIdx.x; c < cols; c += blockDim.x)
      dst[r * ldd + c] = f32_to_i32(src[r * lds + c], inf);
}

// How the call runs, from n, the element size and the device budget.
struct Plan {
  int64_t S;  // outer block (n rounded up to 128 when in-core)
  int sets;   // 0: the matrix fits, one copy in, in-core rounds, one copy out;
              // 1: one panel set, reloaded every outer round;
              // 2: two panel sets, the next round's panels built in place
};

// Two panel sets pay off once S is past the point where a super-tile's
// product outlasts its transfers (S / 4 relaxations per byte each way against
// tens of GB/s of PCIe and tens of T relaxations/s): from 4096 on, a smaller
// S with two sets beats a larger S with one.
#ifndef APSP_HOST_TWO_SETS_MIN
#define APSP_HOST_TWO_SETS_MIN 4096
#endif
constexpr int64_t kTwoSetsMin = APSP_HOST_TWO_SETS_MIN;

__int128 bytes_for(int64_t n, int64_t esz, int64_t S, int sets) {
  const __int128 ldr = (n + 3) & ~int64_t(3);
  return (__int128)esz * (sets * ((__int128)S * ldr + (__int128)n * S) + (__int128)(1 + kSlots) * S * S);
}

// The largest multiple of 128, at most n rounded up to 128, whose buffers fit
// the budget (0 when none does).
int64_t largest_block(int64_t n, int64_t esz, int64_t budget, int sets) {
  int64_t lo = 0, hi = (n + kB - 1) / kB;  // in units of 128
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (bytes_for(n, esz, mid * kB, sets) <= budget) lo = mid;
    else hi = mid - 1;
  }
  return lo * kB;
}

// The same number of outer rounds with the pivots spread evenly: the
// smallest multiple of 128 that still covers n in ceil(n / S) rounds.
int64_t balanced(int64_t n, int64_t S) {
  const int64_t rounds = (n + S - 1) / S;
  const int64_t per = (n + rounds - 1) / rounds;
  return (per + kB - 1) / kB * kB;
}

int plan_for(int64_t n, int64_t esz, int64_t budget, Plan* p) {
  const int64_t ldr = (n + 3) & ~int64_t(3);
  if ((__int128)esz * n * ldr <= budget) {
    *p = Plan{(n + kB - 1) / kB * kB, 0};
    return APSP_OK;
  }
  const int64_t s1 = largest_block(n, esz, budget, 1);
  if (s1 == 0) return APSP_ERR_RANGE;
  const int64_t s2 = largest_block(n, esz, budget, 2);
  if (s2 > 0 && s2 >= std::min(s1, kTwoSetsMin)) *p = Plan{balanced(n, s2), 2};
  else *p = Plan{balanced(n, s1), 1};
  return APSP_OK;
}

// The rounds with compute type CT on matrix element type E (int32 -> int32,
// int32 -> binary32, float -> float), with `sets` panel sets.  With two
// sets, the super-tiles of the next pivot row and column are computed in
// place in the other set (no copy out and back in), and the parts of the
// next panels that lie in this round's panels are copied across on the
// device.
//
// Streams: `s` runs the panel work (load, closure, Phase 2); three slot
// streams run the Phase-3 super-tiles.  Each round ends with `s` waiting for
// the slots.  Four streams in all: with more than the runtime's hardware
// queues (four by default), two streams would share an in-order queue and
// wait on each other's work.
//
// Copies in one direction leave in the order they were issued, so a panel
// write-back issued during Phase 3 holds back the super-tiles' copies out.
// With one panel set the panels go back (on `s`) after Phase 2, since the
// next round reloads the same buffers.  With two sets a round's panels stay
// untouched until the next round's Phase 3, so they go back during the next
// round's closure and Phase 2 (on the first slot stream, staged through its
// tile buffer), when nothing else leaves the device; the last round's go
// back at the end.
//
// `gate`, when given, is asked once, after round 0's Phase 2 has been issued
// and before anything is written to the host or any Phase-3 work is issued:
// APSP_OK goes on; anything else ends the call with that status
// (kRetryInt32: the binary32 speculation failed, the host matrix is
// untouched).
template <typename E, typename CT>
int run_rounds(E* h, int64_t n, int64_t ldh, E inf, int64_t S, int sets, bool panels_loaded,
               char* dev, hipStream_t s, hipStream_t* slot, hipEvent_t* ev,
               const std::function<int()>* gate) {
  constexpr bool kConv = std::is_same_v<E, int32_t> && std::is_same_v<CT, float>;
  const CT cinf = kConv ? CT(__builtin_inff()) : CT(inf);
  const int64_t ldr = (n + 3) & ~int64_t(3);  // row panel leading dimension
  E* rp[2];                                   // S x n (pivot rows)
  E* cp[2];                                   // n x S (pivot columns)
  rp[0] = reinterpret_cast<E*>(dev);
  cp[0] = rp[0] + S * ldr;
  E* tmp = cp[0] + n * S;                     // S x S
  E* sb[kSlots];                              // S x S per slot
  for (int i = 0; i < kSlots; ++i) sb[i] = tmp + (int64_t)(i + 1) * S * S;
  rp[1] = sb[kSlots - 1] + S * S;
  cp[1] = rp[1] + S * ldr;
  if (sets == 1) {
    rp[1] = rp[0];
    cp[1] = cp[0];
  }
  hipEvent_t ev_start = ev[0], ev_panels = ev[1], ev_wb = ev[2], *ev_slot = ev + 3;
  const int64_t rounds = (n + S - 1) / S;
  int rc = APSP_OK;
  int c = 0;  // panel set of this round

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
  // Device -> host of a rows x cols panel piece (in compute form), through
  // the S x S copy buffer when it must be converted back to int32.
  auto write_piece = [&](E* dst, const E* src, int64_t lds, int64_t rows, int64_t cols, E* stage,
                         hipStream_t st) -> hipError_t {
    if constexpr (kConv) {
      hipLaunchKernelGGL(hs_to_i32, dim3(conv_grid(rows)), dim3(256), 0, st, stage, S,
                         reinterpret_cast<const float*>(src), lds, rows, cols, inf);
      return copy2d(dst, ldh, stage, S, rows, cols, hipMemcpyDeviceToHost, st);
    } else {
      return copy2d(dst, ldh, src, lds, rows, cols, hipMemcpyDeviceToHost, st);
    }
  };
  // Both panels of the round with pivots [P0, P0 + sp) back to the host:
  // the row panel whole, the column panel without the diagonal block.
  auto write_panels = [&](const E* Rp, const E* Cp, int64_t P0, int64_t sp, E* stage,
                          hipStream_t st) -> hipError_t {
    hipError_t e = hipSuccess;
    for (int64_t J0 = 0; J0 < n && e == hipSuccess; J0 += S)
      e = write_piece(h + P0 * ldh + J0, Rp + J0, ldr, sp, std::min(S, n - J0), stage, st);
    for (int64_t I0 = 0; I0 < n && e == hipSuccess; I0 += S)
      if (I0 != P0) e = write_piece(h + I0 * ldh + P0, Cp + I0 * S, S, std::min(S, n - I0), sp, stage, st);
    return e;
  };

  for (int64_t KK = 0; KK < rounds; ++KK) {
    const int64_t K0 = KK * S, sk = std::min(S, n - K0);
    const int64_t K1 = K0 + S, sk1 = std::min(S, n - K1);  // next pivot block (sk1 <= 0: none)
    const int nx = sets == 2 ? 1 - c : c;
    E* const R = rp[c];
    E* const C = cp[c];
    HIP_TRY(hipEventRecord(ev_start, s));
    for (int i = 0; i < kSlots; ++i) HIP_TRY(hipStreamWaitEvent(slot[i], ev_start, 0));
    // -- two sets: the previous round's panels go back now, on the first slot
    //    stream; the other slots, and the copies into the other set below,
    //    wait for them -----------------------------------------------------------
    const bool deferred = sets == 2 && KK > 0;
    if (deferred) {
      HIP_TRY(write_panels(rp[nx], cp[nx], K0 - S, S, sb[0], slot[0]));
      HIP_TRY(hipEventRecord(ev_wb, slot[0]));
      for (int i = 1; i < kSlots; ++i) HIP_TRY(hipStreamWaitEvent(slot[i], ev_wb, 0));
    }
    // -- panels in (first round, or every round with one set) -----------------
    if (KK == 0 || sets == 1) {
      if (!(KK == 0 && panels_loaded)) {
        HIP_TRY(copy2d(R, ldr, h + K0 * ldh, ldh, sk, n, hipMemcpyHostToDevice, s));
        HIP_TRY(copy2d(C, S, h + K0, ldh, n, sk, hipMemcpyHostToDevice, s));
      }
      conv(R, ldr, sk, n, true, s);
      conv(C, S, n, sk, true, s);
    }
    // -- Phase 1: close D_KK in place inside the row panel, copy it into the
    //    column panel ----------------------------------------------------------
    {
      int st;
      if constexpr (std::is_same_v<CT, float>)
        st = apsp_fw_f32(reinterpret_cast<float*>(R + K0), sk, ldr, cinf, s);
      else
        st = apsp_fw_i32(R + K0, sk, ldr, cinf, s);
      if (st != APSP_OK) {
        rc = st;
        goto done;
      }
    }
    HIP_TRY(copy2d(C + K0 * S, S, R + K0, ldr, sk, sk, hipMemcpyDeviceToDevice, s));
    // -- Phase 2: panels as products with the closed block (old panel values
    //    on the right-hand side come from a copy) ------------------------------
    for (int64_t J0 = 0; J0 < n; J0 += S) {
      if (J0 == K0) continue;
      const int64_t wj = std::min(S, n - J0);
      HIP_TRY(copy2d(tmp, S, R + J0, ldr, sk, wj, hipMemcpyDeviceToDevice, s));
      if ((rc = gemm(R + J0, ldr, R + K0, ldr, tmp, S, sk, wj, sk, s)) != APSP_OK) goto done;
    }
    for (int64_t I0 = 0; I0 < n; I0 += S) {
      if (I0 == K0) continue;
      const int64_t hi = std::min(S, n - I0);
      HIP_TRY(copy2d(tmp, S, C + I0 * S, S, hi, sk, hipMemcpyDeviceToDevice, s));
      if ((rc = gemm(C + I0 * S, S, tmp, S, R + K0, ldr, hi, sk, sk, s)) != APSP_OK) goto done;
    }
    // -- the parts of the next panels that lie in this round's panels ---------
    if (sets == 2 && sk1 > 0) {
      if (deferred) HIP_TRY(hipStreamWaitEvent(s, ev_wb, 0));
      HIP_TRY(copy2d(rp[nx] + K0, ldr, C + K1 * S, S, sk1, sk, hipMemcpyDeviceToDevice, s));
      HIP_TRY(copy2d(cp[nx] + K0 * S, S, R + K1, ldr, sk, sk1, hipMemcpyDeviceToDevice, s));
    }
    HIP_TRY(hipEventRecord(ev_panels, s));
    if (KK == 0 && gate != nullptr && (rc = (*gate)()) != APSP_OK) goto done;
    // -- one set: the panels go back while Phase 3 reads them -----------------
    if (sets == 1) HIP_TRY(write_panels(R, C, K0, sk, tmp, s));
    // -- Phase 3: every other super-tile through the slot streams.  A slot's
    //    first tile comes in while the panels are still being computed. -----
    {
      int64_t t = 0;
      for (int64_t I0 = 0; I0 < n; I0 += S) {
        if (I0 == K0) continue;
        const int64_t hi = std::min(S, n - I0);
        for (int64_t J0 = 0; J0 < n; J0 += S) {
          if (J0 == K0) continue;
          const int64_t wj = std::min(S, n - J0);
          hipStream_t st = slot[t % kSlots];
          // Where the tile lives on the device: in place in the next panels
          // (two sets, next pivot row or column), else in the slot buffer.
          E* b = sb[t % kSlots];
          int64_t ldb = S;
          bool stays = false;
          if (sets == 2 && I0 == K1) {
            b = rp[nx] + J0;
            ldb = ldr;
            stays = true;
          } else if (sets == 2 && J0 == K1) {
            b = cp[nx] + I0 * S;
            stays = true;
          }
          E* ht = h + I0 * ldh + J0;
          HIP_TRY(copy2d(b, ldb, ht, ldh, hi, wj, hipMemcpyHostToDevice, st));
          conv(b, ldb, hi, wj, true, st);
          if (t < kSlots) HIP_TRY(hipStreamWaitEvent(st, ev_panels, 0));
          if ((rc = gemm(b, ldb, C + I0 * S, S, R + J0, ldr, hi, wj, sk, st)) != APSP_OK) goto done;
          if (!stays) {
            conv(b, ldb, hi, wj, false, st);
            HIP_TRY(copy2d(ht, ldh, b, ldb, hi, wj, hipMemcpyDeviceToHost, st));
          }
          ++t;
        }
      }
      // Slots that got no tile still order after the panels.
      for (int i = (int)std::min<int64_t>(t, kSlots); i < kSlots; ++i)
        HIP_TRY(hipStreamWaitEvent(slot[i], ev_panels, 0));
      for (int i = 0; i < kSlots; ++i) {
        HIP_TRY(hipEventRecord(ev_slot[i], slot[i]));
        HIP_TRY(hipStreamWaitEvent(s, ev_slot[i], 0));
      }
    }
    if ((rc = apsp_detail_launch_status()) != APSP_OK) goto done;
    // -- two sets, last round: its panels go back now --------------------------
    if (sets == 2 && KK == rounds - 1) HIP_TRY(write_panels(R, C, K0, sk, tmp, s));
    c = nx;
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

int budget_of(int64_t device_bytes, int64_t* budget) {
  if (device_bytes < 0) return APSP_ERR_INVALID_VALUE;
  if (device_bytes > 0) {
    *budget = device_bytes;
    return APSP_OK;
  }
  size_t fr = 0, tot = 0;
  if (hipMemGetInfo(&fr, &tot) != hipSuccess) return hip_failed();
  *budget = (int64_t)(fr / 2);
  return APSP_OK;
}

// The whole matrix fits the budget: one copy in, the in-core rounds, one
// copy out.
template <typename E>
int run_in_core(E* h, int64_t n, int64_t ldh, E inf, hipStream_t s) {
  const int64_t ldr = (n + 3) & ~int64_t(3);
  E* d = nullptr;
  int rc = APSP_OK;
  if (hipMallocAsync(reinterpret_cast<void**>(&d), (size_t)(n * ldr) * sizeof(E), s) != hipSuccess)
    return hip_failed();
  HIP_TRY(copy2d(d, ldr, h, ldh, n, n, hipMemcpyHostToDevice, s));
  if constexpr (std::is_same_v<E, float>) rc = apsp_fw_f32(d, n, ldr, inf, s);
  else rc = apsp_fw_i32(d, n, ldr, inf, s);
  if (rc != APSP_OK) goto done;
  HIP_TRY(copy2d(h, ldh, d, ldr, n, n, hipMemcpyDeviceToHost, s));
done:
  (void)hipFreeAsync(d, s);
  if (hipStreamSynchronize(s) != hipSuccess && rc == APSP_OK) rc = hip_failed();
  return rc;
}

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
  int64_t budget = 0;
  if ((rc = budget_of(device_bytes, &budget)) != APSP_OK) return rc;
  Plan plan{};
  if ((rc = plan_for(n, sizeof(E), budget, &plan)) != APSP_OK) return rc;
  if (outer_block) *outer_block = plan.S;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (plan.sets == 0) return run_in_core<E>(h, n, ldh, inf, s);

  const int64_t S = plan.S;
  const int64_t ldr = (n + 3) & ~int64_t(3);
  hipStream_t slot[kSlots] = {};
  hipEvent_t ev[3 + kSlots] = {};
  char* dev = nullptr;
  HostScan* scan = nullptr;
  HostScan* hs = nullptr;  // pinned, so the copy into it stays asynchronous
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
  if (hipMallocAsync(reinterpret_cast<void**>(&dev), (size_t)bytes_for(n, sizeof(E), S, plan.sets), s) != hipSuccess ||
      hipMallocAsync(reinterpret_cast<void**>(&scan), sizeof(HostScan), s) != hipSuccess) {
    rc = hip_failed();
    goto cleanup;
  }

  if constexpr (std::is_same_v<E, int32_t>) {
    // Which arithmetic.  Round 0's panels are loaded and scanned first; if
    // they already rule binary32 out, the call runs in int32 with no further
    // scan.  Otherwise the rest of the matrix is scanned on the first slot
    // stream (through its tile buffer) while round 0's closure and Phase 2
    // run in binary32 on `s`; before round 0 writes anything to the host,
    // the gate reads the whole scan, and if binary32 is not exact after all
    // the call starts over in int32 (the panels are reloaded).
    const int policy = apsp_get_int32_arith();
    if (policy == APSP_ARITH_INT32) {
      rc = run_rounds<int32_t, int32_t>(h, n, ldh, inf, S, plan.sets, false, dev, s, slot, ev, nullptr);
      goto cleanup;
    }
    if (hipHostMalloc(reinterpret_cast<void**>(&hs), sizeof(HostScan), hipHostMallocDefault) != hipSuccess) {
      hs = nullptr;
      rc = hip_failed();
      goto cleanup;
    }
    {
      E* rp0 = reinterpret_cast<E*>(dev);
      E* cp0 = rp0 + S * ldr;
      E* buf = cp0 + n * S + S * S;  // the first slot's tile buffer
      auto exact = [&](const HostScan& x) {
        return !(x.flags & 2) && (!(x.flags & 1) || (n - 1) * (int64_t)x.maxw <= kExactLimit);
      };
      hipLaunchKernelGGL(hs_zero, dim3(1), dim3(64), 0, s, scan);
      if (copy2d(rp0, ldr, h, ldh, S, n, hipMemcpyHostToDevice, s) != hipSuccess ||
          copy2d(cp0 + S * S, S, h + S * ldh, ldh, n - S, S, hipMemcpyHostToDevice, s) != hipSuccess) {
        rc = hip_failed();
        goto cleanup;
      }
      hipLaunchKernelGGL(hs_scan, dim3(conv_grid(S)), dim3(256), 0, s, rp0, ldr, S, n, int64_t(0),
                         int64_t(0), inf, scan);
      hipLaunchKernelGGL(hs_scan, dim3(conv_grid(n - S)), dim3(256), 0, s, cp0 + S * S, S, n - S, S,
                         S, int64_t(0), inf, scan);
      if (hipMemcpyAsync(hs, scan, sizeof(HostScan), hipMemcpyDeviceToHost, s) != hipSuccess ||
          hipStreamSynchronize(s) != hipSuccess) {
        rc = hip_failed();
        goto cleanup;
      }
      // Row block 0 of the column panel is not loaded: the closed diagonal
      // block is copied there before it is read.
      if (!exact(*hs)) {
        rc = run_rounds<int32_t, int32_t>(h, n, ldh, inf, S, plan.sets, true, dev, s, slot, ev, nullptr);
        goto cleanup;
      }
      for (int64_t r0 = S; r0 < n && rc == APSP_OK; r0 += S)
        for (int64_t c0 = S; c0 < n; c0 += S) {
          const int64_t rows = std::min(S, n - r0), cols = std::min(S, n - c0);
          if (copy2d(buf, S, h + r0 * ldh + c0, ldh, rows, cols, hipMemcpyHostToDevice, slot[0]) != hipSuccess) {
            rc = hip_failed();
            break;
          }
          hipLaunchKernelGGL(hs_scan, dim3(conv_grid(rows)), dim3(256), 0, slot[0], buf, S, rows, cols,
                             r0, c0, inf, scan);
        }
      if (rc != APSP_OK) goto cleanup;
      if (hipMemcpyAsync(hs, scan, sizeof(HostScan), hipMemcpyDeviceToHost, slot[0]) != hipSuccess) {
        rc = hip_failed();
        goto cleanup;
      }
      const std::function<int()> gate = [&]() -> int {
        if (hipStreamSynchronize(slot[0]) != hipSuccess) return hip_failed();
        return exact(*hs) ? APSP_OK : kRetryInt32;
      };
      rc = run_rounds<int32_t, float>(h, n, ldh, inf, S, plan.sets, true, dev, s, slot, ev, &gate);
      if (rc == kRetryInt32) {
        (void)hipStreamSynchronize(s);
        rc = run_rounds<int32_t, int32_t>(h, n, ldh, inf, S, plan.sets, false, dev, s, slot, ev, nullptr);
      }
    }
  } else {
    rc = run_rounds<float, float>(h, n, ldh, inf, S, plan.sets, false, dev, s, slot, ev, nullptr);
  }

cleanup:
  (void)hipStreamSynchronize(s);
  for (auto& st : slot)
    if (st) (void)hipStreamSynchronize(st);
  if (dev) (void)hipFreeAsync(dev, s);
  if (scan) (void)hipFreeAsync(scan, s);
  (void)hipStreamSynchronize(s);
  if (hs) (void)hipHostFree(hs);
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

int apsp_fw_host_plan(int64_t n, int64_t elem_bytes, int64_t device_bytes, int64_t* outer_block,
                      int32_t* panel_sets) {
  if (outer_block) *outer_block = 0;
  if (panel_sets) *panel_sets = 0;
  if (n < 0 || n > (int64_t(1) << 31) || (elem_bytes != 4) || device_bytes < 0)
    return APSP_ERR_INVALID_VALUE;
  if (n == 0) return APSP_OK;
  int64_t budget = 0;
  int rc = budget_of(device_bytes, &budget);
  if (rc != APSP_OK) return rc;
  Plan p{};
  if ((rc = plan_for(n, elem_bytes, budget, &p)) != APSP_OK) return rc;
  if (outer_block) *outer_block = p.S;
  if (panel_sets) *panel_sets = p.sets;
  return APSP_OK;
}

}  // extern "C"
