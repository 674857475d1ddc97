// Library-internal host helpers shared by the translation units of
// libapsp.so (hidden: not part of the C ABI).
#ifndef APSP_DETAIL_H
#define APSP_DETAIL_H

#include <stdint.h>

// APSP_OK when the current device is gfx950, else APSP_ERR_NO_DEVICE
// (cached per device).
__attribute__((visibility("hidden"))) int apsp_detail_check_device();

// APSP_ERR_LAUNCH (recording the hipError_t for apsp_last_hip_error) when
// hipGetLastError reports a failure, else APSP_OK.
__attribute__((visibility("hidden"))) int apsp_detail_launch_status();

// Every Floyd-Warshall round on an int32 matrix of successor keys
// (value << s | first hop, s the bit width of n, "no edge" the key
// 2^30 - 2^s), in place on `stream`; the caller has checked that every
// value the recurrence can store stays below 2^(30-s) - 1.  APSP_OK, or
// APSP_ERR_INVALID_VALUE / APSP_ERR_LAUNCH.
__attribute__((visibility("hidden"))) int apsp_detail_fw_keys(int32_t* d, int64_t n, int64_t ld,
                                                              void* stream);

#endif  // APSP_DETAIL_H
