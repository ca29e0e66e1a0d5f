// Pure host dispatcher and descriptor validation for qgemv.
//
// Shape gating follows the pages' lesson that a grid must cover the machine:
// tiling that narrows the grid below a wave of the GPU loses ("[CUDA] Block-scaled
// MatMul decode GEMV", FP4 row-tiling paragraph: tiling is gated on the column grid
// covering a full wave on its own), and a grid just past a whole number of waves
// leaves a nearly empty tail ("[CUDA] Pin FP8 GEMV residency", Description). Here the
// unit is the wave64 and the machine is cu_count compute units (256 on MI355X).
//
// Every parameter that changes per-row arithmetic (the family, the lanes that own a
// column, the K split) is chosen from (format, N, K, block size, flags) only, never
// from M, so a row's result does not depend on how many rows travel with it.
#include "select.h"

#include <stdint.h>

namespace qgemv {

static bool valid_block(int fmt, int bs) {
    if (fmt == QGEMV_FMT_NVFP4) return bs == 16;
    return bs == 16 || bs == 32 || bs == 64 || bs == 128 || bs == 256;
}

int validate_desc(const qgemv_desc *d) {
    if (!d) return QGEMV_E_NULL;
    if (d->struct_size != sizeof(qgemv_desc)) return QGEMV_E_ARG;
    if (d->format < QGEMV_FMT_U4 || d->format > QGEMV_FMT_NVFP4) return QGEMV_E_FORMAT;
    if (d->act_dtype != QGEMV_ACT_F16 && d->act_dtype != QGEMV_ACT_BF16) return QGEMV_E_FORMAT;
    if (!d->W || !d->scales) return QGEMV_E_NULL;
    if ((d->format == QGEMV_FMT_FP8 || d->format == QGEMV_FMT_NVFP4) && d->zero_points) return QGEMV_E_FORMAT;
    if (d->N < 1 || d->K < 1) return QGEMV_E_SHAPE;
    if (!valid_block(d->format, d->block_size)) return QGEMV_E_BLOCK;
    if (d->K % d->block_size) return QGEMV_E_SHAPE;
    const uint32_t known = QGEMV_FLAG_FAMILY_MASK | QGEMV_FLAG_KSPLIT_MASK | QGEMV_FLAG_NO_MFMA;
    if (d->flags & ~known) return QGEMV_E_ARG;
    const uint32_t fam = d->flags & QGEMV_FLAG_FAMILY_MASK;
    if (fam > QGEMV_FAMILY_GENERIC) return QGEMV_E_ARG;
    const uint32_t ks = (d->flags & QGEMV_FLAG_KSPLIT_MASK) >> QGEMV_FLAG_KSPLIT_SHIFT;
    if (ks > 64) return QGEMV_E_ARG;
    return QGEMV_OK;
}

static bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool pointers_fast_ok(const qgemv_desc *d, const void *A, const void *Y) {
    const uintptr_t sa = (d->format == QGEMV_FMT_FP8) ? 4 : (d->format == QGEMV_FMT_NVFP4 ? 1 : 2);
    if (!aligned(d->W, 16) || !aligned(d->scales, sa)) return false;
    if (A && !aligned(A, 16)) return false;
    if (Y && !aligned(Y, 2)) return false;
    return true;
}

// k per 16-byte chunk of codes
static int k_per_chunk(int fmt) { return (fmt == QGEMV_FMT_U4 || fmt == QGEMV_FMT_NVFP4) ? 32 : 16; }

static bool stream_shape_ok(const qgemv_desc *d) {
    // every column's codes start on a 16-byte boundary and split into whole chunks
    if (d->K % k_per_chunk(d->format)) return false;
    // NVFP4 scale pairs are read as two bytes per chunk; U4 with 16-wide blocks
    // reads two scales per chunk
    return true;
}

int select_plan(const qgemv_desc *d, int M, int cu_count, bool fast_ok, uint32_t extra_flags, LaunchCfg *out) {
    int rc = validate_desc(d);
    if (rc) return rc;
    if (!out) return QGEMV_E_NULL;
    if (M < 1 || M > QGEMV_MAX_M) return QGEMV_E_SHAPE;
    if (cu_count < 1) return QGEMV_E_ARG;
    const uint32_t flags = d->flags | extra_flags;

    LaunchCfg c{};
    c.fmt = d->format;
    c.act = d->act_dtype;
    c.ksplit = 1;
    c.waves_per_wg = 4;
    c.lds_bytes = 0;
    c.variant = 0;

    int forced = (int)(flags & QGEMV_FLAG_FAMILY_MASK);
    const bool stream_ok = fast_ok && stream_shape_ok(d);
    int family;
    if (forced == QGEMV_FAMILY_GENERIC || (forced == QGEMV_FAMILY_AUTO && !stream_ok)) {
        family = QGEMV_FAMILY_GENERIC;
    } else if (forced == QGEMV_FAMILY_STREAM || forced == QGEMV_FAMILY_MFMA) {
        if (!stream_ok) return QGEMV_E_ARG;  // a forced fast family needs its preconditions
        family = QGEMV_FAMILY_STREAM;        // matrix family not built yet: stream serves it
    } else {
        family = QGEMV_FAMILY_STREAM;
    }
    c.family = family;

    const int64_t wave_target = 8LL * cu_count;  // two waves per SIMD
    if (family == QGEMV_FAMILY_GENERIC) {
        c.rows_per_pass = M;
        c.passes = 1;
        c.cols_per_wave = 1;
        const int64_t wgs = (d->N + 3) / 4;
        const int64_t cap = 8LL * cu_count;
        c.grid = wgs < cap ? wgs : cap;
    } else {
        c.rows_per_pass = (M == 1) ? 1 : (M == 2 ? 2 : 4);
        c.passes = (M + c.rows_per_pass - 1) / c.rows_per_pass;
        if (d->N >= 4 * wave_target) c.cols_per_wave = 4;
        else if (d->N >= 2 * wave_target) c.cols_per_wave = 2;
        else c.cols_per_wave = 1;
        const int64_t waves = (d->N + c.cols_per_wave - 1) / c.cols_per_wave;
        c.grid = (waves + c.waves_per_wg - 1) / c.waves_per_wg;
    }
    *out = c;
    return QGEMV_OK;
}

}  // namespace qgemv
