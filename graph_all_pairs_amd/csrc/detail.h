// Library-internal host helpers shared by the translation units of
// libapsp.so (hidden: not part of the C ABI).
#ifndef APSP_DETAIL_H
#define APSP_DETAIL_H

// APSP_OK when the current device is gfx950, else APSP_ERR_NO_DEVICE
// (cached per device).
__attribute__((visibility("hidden"))) int apsp_detail_check_device();

// APSP_ERR_LAUNCH (recording the hipError_t for apsp_last_hip_error) when
// hipGetLastError reports a failure, else APSP_OK.
__attribute__((visibility("hidden"))) int apsp_detail_launch_status();

#endif  // APSP_DETAIL_H
