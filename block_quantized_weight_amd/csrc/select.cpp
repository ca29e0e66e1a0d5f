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
    return d->K % k_per_chunk(d->format) == 0;
}

// The matrix family walks K in steps of four 16-byte chunks per column, and takes
// 8-bit codes only with fp16 activations (1024 + q is an exact fp16 integer; bf16
// has no room for an offset 8-bit code).
static bool mfma_shape_ok(const qgemv_desc *d) {
    if (d->K % (4 * k_per_chunk(d->format))) return false;
    if (d->format == QGEMV_FMT_U8 && d->act_dtype != QGEMV_ACT_F16) return false;
    return true;
}

// Waves that share one 16-column tile's K range. Chosen from N and K only so that
// the summation order of a row never depends on M: enough waves to fill the
// machine (about eight per CU), no more than one K step of four chunks per wave.
static int mfma_ksplit(const qgemv_desc *d, int cu_count, uint32_t flags) {
    const uint32_t forced = (flags & QGEMV_FLAG_KSPLIT_MASK) >> QGEMV_FLAG_KSPLIT_SHIFT;
    const int64_t tiles = (d->N + 15) / 16;
    const int64_t steps = d->K / (4 * k_per_chunk(d->format));
    int ks = 1;
    if (forced) {
        ks = (int)forced;
    } else {
        while (ks < 16 && tiles * ks < 8LL * cu_count && 2 * ks <= steps) ks *= 2;
    }
    if (ks > 16) ks = 16;
    if (ks > steps) ks = (int)steps;
    return ks < 1 ? 1 : ks;
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

    const int forced = (int)(flags & QGEMV_FLAG_FAMILY_MASK);
    const bool stream_ok = fast_ok && stream_shape_ok(d);
    const bool mfma_ok = fast_ok && mfma_shape_ok(d) && !(flags & QGEMV_FLAG_NO_MFMA);
    int family;
    if (forced == QGEMV_FAMILY_GENERIC) {
        family = QGEMV_FAMILY_GENERIC;
    } else if (forced == QGEMV_FAMILY_STREAM) {
        if (!stream_ok) return QGEMV_E_ARG;  // a forced fast family needs its preconditions
        family = QGEMV_FAMILY_STREAM;
    } else if (forced == QGEMV_FAMILY_MFMA) {
        if (!(fast_ok && mfma_shape_ok(d))) return QGEMV_E_ARG;
        family = QGEMV_FAMILY_MFMA;
    } else if (mfma_ok && M >= 2) {
        family = QGEMV_FAMILY_MFMA;
    } else if (stream_ok) {
        family = QGEMV_FAMILY_STREAM;
    } else {
        family = QGEMV_FAMILY_GENERIC;
    }
    c.family = family;

    const int64_t wave_target = 8LL * cu_count;  // two waves per SIMD
    if (family == QGEMV_FAMILY_MFMA) {
        const int rg = (M + 3) / 4;
        c.rows_per_pass = 4 * rg;
        c.passes = 1;
        c.cols_per_wave = 16;
        c.ksplit = mfma_ksplit(d, cu_count, flags);
        c.waves_per_wg = c.ksplit;
        c.grid = (d->N + 15) / 16;
        c.lds_bytes = c.ksplit > 1 ? c.ksplit * rg * 4 * 64 * 4 : 0;
    } else if (family == QGEMV_FAMILY_GENERIC) {
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
