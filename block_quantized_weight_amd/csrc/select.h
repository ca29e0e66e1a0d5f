// Pure host dispatcher: which kernel family and launch shape serves a problem.
// No HIP calls, so it is testable on any host at a fixed compute-unit count.
#pragma once

#include <stdint.h>

#include "../../include/qgemv.h"
#include "launch.h"

namespace qgemv {

// Validation of a descriptor (shape, block size, format, pointers). Returns a
// qgemv_status.
int validate_desc(const qgemv_desc *d);

// The launch for M rows on cu_count compute units. `fast_ok` tells whether the
// pointers meet the streaming / MFMA families' alignment needs; `with_ws` whether a
// workspace is at hand, so that the K range may be split across workgroups.
int select_plan(const qgemv_desc *d, int M, int cu_count, bool fast_ok, uint32_t extra_flags, bool with_ws,
                LaunchCfg *out);

// Whether the pointers of d (and optionally A / Y) satisfy the fast families.
bool pointers_fast_ok(const qgemv_desc *d, const void *A, const void *Y);

}  // namespace qgemv
