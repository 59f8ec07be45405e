// Host-side helpers of the C ABI: status/error reporting and argument checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ringattn.h"

namespace ra {

// Records a formatted message as this thread's last error and returns `st`.
ra_status fail(ra_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears this thread's last error and returns RA_OK.
ra_status ok();

// Checks the last launch on this thread; returns RA_ERR_HIP with the HIP text on failure.
ra_status check_launch(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates an ra_shape (and the seg_ids range) shared by the forward and backward steps.
ra_status validate_step(const ra_shape* s, const int32_t* seg_ids, int64_t seg_len);

}  // namespace ra
