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

// Whether the launch walks its work persistently (any grid up to the work units), so
// that a create-time cut to the resident workgroups applies.
bool persistent(const LaunchCfg &c);

// Whether two plans launch the same kernels with the same shape.
bool same_launch(const LaunchCfg &x, const LaunchCfg &y);

// Flag sets (extra to d->flags | env_flags) whose plans for M rows give the automatic
// plan's bits with another launch: out[0] = 0 (the automatic plan), then one per
// distinct launch, at most `max`. See qgemv_tune_candidates.
int tune_candidates(const qgemv_desc *d, int M, int cu_count, bool fast_ok, uint32_t env_flags, bool with_ws,
                    uint32_t *out, int max, int *count);

// Whether the pointers of d (and optionally A / Y) satisfy the fast families.
bool pointers_fast_ok(const qgemv_desc *d, const void *A, const void *Y);

}  // namespace qgemv
