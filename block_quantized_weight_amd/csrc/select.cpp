// Pure host dispatcher and descriptor validation for qgemv.
//
// Shape gating follows the pages' lesson that a grid must cover the machine:
// tiling that narrows the grid below a wave of the GPU loses ("[CUDA] Block-scaled
// MatMul decode GEMV", FP4 row-tiling paragraph: tiling is gated on the column grid
// covering a full wave on its own), and a grid just past a whole number of waves
// leaves a nearly empty tail ("[CUDA] Pin FP8 GEMV residency", Description). Here the
// unit is the wave64 and the machine is cu_count compute units (256 on MI355X).
//
// Within a kernel family, every parameter that changes per-row arithmetic (the lanes
// that own a column, the K split) is chosen from the weight (format, N, K, block size,
// zero points), the flags and the CU count only, never from M, so a row's bits do not
// depend on how many rows travel with it in that family. The family itself is chosen
// from M as well (the streaming family at M = 1, the matrix family from M = 2 or 3 on
// wide weights, and the fallbacks below), and so are qgemv_run_ws's K parts where this
// M's rows do not fit in LDS, with the K split beside them for long rows; the families
// sum in different fp32 orders, so a row's bits can change where M moves a shape from
// one family or part count to another (all within the same bound). A caller who needs
// the same bits for a row at every M forces one family (and the part count) in the
// flags.
#include "select.h"

#include <initializer_list>

#include <stdint.h>

namespace qgemv {

// LDS of one gfx950 compute unit (bytes).
static const int64_t kLdsBytes = 160 * 1024;

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
    if ((uintptr_t)d->bias % 2) return QGEMV_E_ARG;  // read as 16-bit values
    if (d->N < 1 || d->K < 1) return QGEMV_E_SHAPE;
    if (!valid_block(d->format, d->block_size)) return QGEMV_E_BLOCK;
    if (d->K % d->block_size) return QGEMV_E_SHAPE;
    const uint32_t known = QGEMV_FLAG_FAMILY_MASK | QGEMV_FLAG_KPARTS_MASK | QGEMV_FLAG_KSPLIT_MASK | QGEMV_FLAG_NO_MFMA |
                           QGEMV_FLAG_STAGE_A_OFF | QGEMV_FLAG_STAGE_A_ON | QGEMV_FLAG_RING_OFF |
                           QGEMV_FLAG_RING_ON | QGEMV_FLAG_STREAM_CPW_MASK | QGEMV_FLAG_STREAM_UNR_MASK |
                           QGEMV_FLAG_STREAM_WPC_MASK | QGEMV_FLAG_STREAM_CLASSIC | QGEMV_FLAG_MFMA_DEPTH_MASK |
                           QGEMV_FLAG_STREAM_WIDE_WG | QGEMV_FLAG_STREAM_NWG_MASK | QGEMV_FLAG_NO_RESIDENCY_FIT |
                           QGEMV_FLAG_STREAM_META_CHUNK;
    if (d->flags & ~known) return QGEMV_E_ARG;
    const uint32_t fam = d->flags & QGEMV_FLAG_FAMILY_MASK;
    if (fam > QGEMV_FAMILY_GENERIC) return QGEMV_E_ARG;
    const uint32_t ks = (d->flags & QGEMV_FLAG_KSPLIT_MASK) >> QGEMV_FLAG_KSPLIT_SHIFT;
    if (ks > 8 || (ks & (ks - 1))) return QGEMV_E_ARG;  // 1, 2, 4 or 8: whole tiles per 8-wave workgroup
    if (((d->flags & QGEMV_FLAG_KPARTS_MASK) >> QGEMV_FLAG_KPARTS_SHIFT) > 4) return QGEMV_E_ARG;  // 1..8 parts
    if (((d->flags & QGEMV_FLAG_STREAM_NWG_MASK) >> QGEMV_FLAG_STREAM_NWG_SHIFT) > 4) return QGEMV_E_ARG;
    if (((d->flags & QGEMV_FLAG_MFMA_DEPTH_MASK) >> QGEMV_FLAG_MFMA_DEPTH_SHIFT) > 2) return QGEMV_E_ARG;
    if ((d->flags & QGEMV_FLAG_STAGE_A_OFF) && (d->flags & QGEMV_FLAG_STAGE_A_ON)) return QGEMV_E_ARG;
    if ((d->flags & QGEMV_FLAG_RING_OFF) && (d->flags & QGEMV_FLAG_RING_ON)) return QGEMV_E_ARG;
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

// The matrix family walks K in steps of four 16-byte chunks per column.
static bool mfma_shape_ok(const qgemv_desc *d) { return d->K % (4 * k_per_chunk(d->format)) == 0; }

// Whether the kernels keep per-chunk activation sums (for the zero point's
// -z * sum(a) term): 4-bit codes on bf16 activations only. Every other format with
// zero points forms q - z in its decode.
static bool needs_act_sums(const qgemv_desc *d) {
    return d->format == QGEMV_FMT_U4 && d->act_dtype == QGEMV_ACT_BF16;
}

// Whether the matrix family's DMA ring takes the problem with `slots` 4-step slots per
// wave (16 chunks of each of a tile's 16 columns per slot), and its LDS bytes next to
// abytes of staged activations. The scale (and zero-point) rows must be whole dwords on
// 4-byte aligned arrays. A slot of 64 chunks per column holds whole blocks for every
// block size the formats take.
static bool dma_ring_fits(const qgemv_desc *d, int64_t abytes, bool zpp, int slots, int32_t *lds_out) {
    const int64_t nblk = d->K / d->block_size;
    const int sb = d->format == QGEMV_FMT_FP8 ? 4 : (d->format == QGEMV_FMT_NVFP4 ? 1 : 2);
    if ((nblk * sb) % 4 || (uintptr_t)d->scales % 4) return false;
    if (zpp) {
        const int64_t zrow = d->format == QGEMV_FMT_U4 ? (nblk + 1) / 2 : nblk;
        if (zrow % 4 || (uintptr_t)d->zero_points % 4) return false;
    }
    // slot: 4 KiB of codes, the scale window (4 DMAs of 256 B where 16-wide blocks or
    // FP8 need them, else 2), the zero-point window (256 B); 8 waves x `slots` slots
    const bool wide_meta = d->format == QGEMV_FMT_FP8 || (d->format == QGEMV_FMT_U4 && d->block_size == 16);
    const int64_t slot = 4 * 1024 + 256 * (wide_meta ? 4 : 2) + (zpp ? 256 : 0);
    const int64_t lds = abytes + 8 * (int64_t)slots * slot;
    if (lds > kLdsBytes) return false;
    *lds_out = (int32_t)lds;
    return true;
}

// The matrix family's staged activations for `rows` rows over `sm` K steps: a 64-byte
// zero block, the rows (stride sm x 4 chunks + 8 elements, 2 bytes each, rounded up to
// 16 bytes) and, for 4-bit codes on bf16, one 16-byte activation-sum entry per chunk,
// row group and scale block of the chunk.
static int64_t staged_act_bytes(const qgemv_desc *d, int rows, int64_t sm) {
    const int64_t la = (int64_t)rows * (sm * 4 * k_per_chunk(d->format) + 8) * 2;
    const int hh = (d->format == QGEMV_FMT_U4 && d->block_size == 16) ? 2 : 1;
    return 64 + ((la + 15) & ~15LL) + (needs_act_sums(d) ? 4 * sm * ((rows + 3) / 4) * hh * 16 : 0);
}

// Whether `groups` tile groups of the DMA ring (8 tiles each, no K split) fill enough
// of the CUs for the ring to win: from 3/4 of them for the formats with 32 k per chunk
// (4-bit, NVFP4), from 7/8 for those with 16 (FP8, 8-bit), whose slots hold half the
// arithmetic. Measured on MI355X (ring against the best other plan, cold weights):
// 4-bit on bf16 24576 x 4096 (192 groups) M = 2 / 4 / 8 15.6 / 15.8 / 20.3 us against
// 15.9 / 16.6 / 23.5, 28672 x 4096 (224) M = 4 16.2 against 26.0, 32768 x 4096 (256)
// M = 4 17.2 against 24.6; NVFP4 24576 x 2048 M = 1 / 4 8.5 / 8.8 against 8.9 / 20.4;
// 4-bit on f16 32768 x 2048 M = 2 10.7 against 17.7; FP8 28672 x 4096 (224) M = 3 /
// 4 / 8 28.1 / 28.2 / 28.5 against 30.6 / 30.8 / 40.3, 8-bit 28672 x 4096 M = 4 / 8
// 27.8 / 28.4 against 31.0 / 45.2; with more groups, where the earlier rule took the
// streaming kernel or the register ring: 4-bit on f16 49152 x 2048 M = 2 16.3 against
// 25.2, FP8 49152 x 1024 M = 4 12.8 against 23.6, 8-bit 32768 x 2048 M = 4 14.8 against
// 18.1, 4-bit on bf16 32768 x 16384 M = 2 62.6 against 98.4. But FP8 24576 x 4096 (192
// groups) M = 4 26.9 against 23.9, and 4-bit on bf16 16384 x 4096 (128) M = 2 / 4
// 19.3 / 20.0 against 12.2 / 13.7.
static bool ring_groups_fill(const qgemv_desc *d, int64_t groups, int cu_count) {
    return k_per_chunk(d->format) == 32 ? 4 * groups >= 3LL * cu_count : 8 * groups >= 7LL * cu_count;
}

// Whether the DMA ring takes this weight at every M up to 8: its tile groups fill the
// CUs (above) and eight staged rows fit in LDS next to two slots per wave; or, for
// 4-bit and NVFP4 codes whose tile groups reach 7/8 of the CUs, at every M up to 4,
// where four staged rows fit next to them. Such a weight takes no K split in the
// matrix family (the ring has none, and the split may not depend on M), and the
// register ring takes the rows the ring does not at no loss there (µs, K split 8 ->
// unsplit, 28672 x 8192, ring at M <= 4: 4-bit on bf16 M = 2 / 4 / 8 / 16 38.6 / 39.4
// / 56.0 / 110.6 -> 30.7 / 31.8 / 56.3 / 103.2; NVFP4 33.8 / 35.3 / 51.0 / 100.5 ->
// 27.4 / 28.3 / 41.7 / 76.0), but not with fewer groups (4-bit 24576 x 8192, 192
// groups, M = 8: 39.9 us at a split of 4, 54.9 unsplit) nor for 1-byte codes (FP8
// 28672 x 8192 M = 8: 57.3 at 8, 73.3 unsplit).
static bool ring_band(const qgemv_desc *d, int cu_count) {
    const int64_t groups = ((d->N + 15) / 16 + 7) / 8;
    if (!ring_groups_fill(d, groups, cu_count) || d->K % (4 * k_per_chunk(d->format))) return false;
    const bool zpp = d->zero_points && (d->format == QGEMV_FMT_U4 || d->format == QGEMV_FMT_U8);
    const int64_t steps = d->K / (4 * k_per_chunk(d->format));
    int32_t lds = 0;
    if (dma_ring_fits(d, staged_act_bytes(d, 8, steps), zpp, 2, &lds)) return true;
    return k_per_chunk(d->format) == 32 && 8 * groups >= 7LL * cu_count &&
           dma_ring_fits(d, staged_act_bytes(d, 4, steps), zpp, 2, &lds);
}

// Waves that share one 16-column tile's K range. Chosen from the weight (format, N, K,
// block size, zero points) and the CU count only, so that the summation order of a
// row never depends on M. A workgroup holds 8 / ksplit tiles
// of ksplit waves, so the split sets both the number of workgroups and the K steps
// each wave walks. While the workgroups do not fill the CUs, the split taken is the
// one with the least work on the busiest CU, (workgroups per CU, rounded up) x (K
// steps per wave), ties to the smaller split (a finer one adds LDS reduction for
// nothing); a grid that already fills them is not split further. A split that leaves a wave fewer than 8
// K steps is taken only while the tiles are so few (tiles x ksplit < 4 per CU) that
// the machine is mostly idle: it leaves too few steps to amortize staging the
// activations. Measured on MI355X at M = 8, the old rule (about four waves per CU)
// -> this one: 8-bit 16384 x 4096 37.7 -> 26.0 us (split 1 -> 2), FP8 8192 x 4096
// 18.4 -> 14.0 (2 -> 4), 4-bit 8192 x 4096 16.8 -> 13.5 (2 -> 4), 8-bit 4096 x 4096
// 15.4 -> 14.4 (4 -> 8); a finer split than this rule's measured slower on FP8
// 5120 x 6144 (16.7 us at 4, 19.3 at 8), NVFP4 and 4-bit 4096 x 4096 (10.1 / 12.5 us
// at 4, 12.9 / 13.8 at 8) and 4-bit 12288 x 4096 (17.3 us at 2, 19.1 at 4). At least
// two K steps per wave, and at most 8, the waves of one workgroup. No split where the
// DMA ring takes the weight at every M up to 8: from 9 rows the register ring then runs
// unsplit, which measured about as fast or faster there (4-bit on bf16 24576 x 4096
// M = 12 30.4 us unsplit against 29.3 at 4, M = 16 33.4 against 96.7 with unstaged
// rows; FP8 28672 x 4096 M = 12 42.7 against 52.0 at 8; 8-bit 28672 x 4096 M = 12 / 16
// 39.0 / 41.4 against 56.0 / 131.0).
static int mfma_ksplit(const qgemv_desc *d, int cu_count, uint32_t flags) {
    const uint32_t forced = (flags & QGEMV_FLAG_KSPLIT_MASK) >> QGEMV_FLAG_KSPLIT_SHIFT;
    const int64_t tiles = (d->N + 15) / 16;
    const int64_t steps = d->K / (4 * k_per_chunk(d->format));
    int ks = 1;
    if (forced) {
        ks = (int)forced;
    } else if (!ring_band(d, cu_count)) {
        auto groups = [&](int k) { return (tiles + 8 / k - 1) / (8 / k); };
        auto cost = [&](int k) { return (groups(k) + cu_count - 1) / cu_count * ((steps + k - 1) / k); };
        for (int k = 2; k <= 8 && 2 * k <= steps && groups(ks) < cu_count; k *= 2) {
            const bool allowed = steps >= 8LL * k || tiles * ks < 4LL * cu_count;
            if (allowed && cost(k) < cost(ks)) ks = k;
        }
    }
    if (ks > 8) ks = 8;
    while (ks > 1 && ks > steps) ks /= 2;  // a power of two: whole tiles per workgroup
    return ks;
}

// K parts split across workgroups (qgemv_run_ws only), from (format, N, K, block
// size, flags, CU count), not M (select_plan adds the one case that depends on M). A part count that pushes the grid past one
// workgroup per CU always loses. Within that, measured on MI355X at M = 8 (unsplit ->
// best split): where the tile groups fill at most a quarter of the CUs, parts pay
// (FP8 1024 x 16384, 64 groups: 36.1 -> 15.1 us in 4; 4-bit 512 x 8192, 32 groups:
// 15.8 -> 12.7 us in 4), so the most parts that keep two K steps per wave; where they
// fill up to half, 2 parts pay only with long parts, whose activations then fit the
// LDS (FP8 2048 x 16384: 36.4 -> 19.9 us; FP8 4096 x 8192: 19.1 -> 18.1 us; but
// 4-bit 2048 x 8192, 8 steps per wave and part: 16.5 -> 18.6 us; 8-bit 4096 x 4096:
// 15.4 -> 16.0 us), so only with 16 K steps or more per wave and part. A forced count
// is taken as given, up to one part per K step.
static int mfma_kparts(const qgemv_desc *d, int cu_count, uint32_t flags, int ks, int64_t groups) {
    const int64_t steps = d->K / (4 * k_per_chunk(d->format));
    const uint32_t forced = (flags & QGEMV_FLAG_KPARTS_MASK) >> QGEMV_FLAG_KPARTS_SHIFT;
    int kp = 1;
    if (forced) {
        kp = 1 << (forced - 1);
    } else if (groups * 4 <= cu_count) {
        while (kp < 8 && groups * (2 * kp) <= cu_count && steps >= 2LL * ks * (2 * kp)) kp *= 2;
    } else if (groups * 2 <= cu_count && steps >= 16LL * ks * 2) {
        kp = 2;
    }
    while (kp > 1 && kp > steps) kp /= 2;
    // the kernel indexes the partial tiles [kp, M <= 16, N] with 32-bit offsets
    while (kp > 1 && (int64_t)kp * QGEMV_MAX_M * d->N >= (1LL << 31)) kp /= 2;
    return kp;
}

// Long rows with a workspace: where the unsplit tile groups fill between 1/8 of the CUs
// and all of them, and this M's rows of the whole K do not fit in LDS, the matrix
// family splits K across workgroups only (no split inside one; K parts, below). An
// in-workgroup split stages the activations of the whole K range per 16 x (8 / ksplit)
// columns, and here the rows do not stage at all; K parts stage only their part. Like
// the K parts, this choice depends on M: the K split then does too, so rows of
// qgemv_run_ws's automatic plans are bit-identical across M only where no such rule
// applies (a forced split or part count turns it off). Measured on MI355X with a
// workspace (µs, automatic before -> after): 4-bit 8192 x 28672 M = 8 / 16 124.2 /
// 224.2 -> 60.5 / 83.9 (M = 4 55.9 -> 56.4); FP8 8192 x 28672 M = 4 / 8 / 16 73.3 /
// 129.7 / 226.7 -> 69.3 / 79.7 / 99.9; 4-bit 4096 x 14336 M = 8 / 16 32.4 / 58.5 ->
// 22.1 / 27.1; NVFP4 8192 x 28672 M = 4 / 8 / 16 46.1 / 121.9 / 220.3 -> 38.4 / 43.3 /
// 71.3; NVFP4 24576 x 16384 M = 8 181.7 -> 96.6; at K = 8192, M = 12 / 16 (row passes or
// a split of 4 or 8 before): 4-bit 8192 x 8192 32.2 / 37.2 -> 23.4 / 26.3, 4-bit
// 10240 x 8192 48.0 / 55.9 -> 35.3 / 40.3, 8-bit 8192 x 8192 42.7 / 45.8 -> 32.2 /
// 33.8, FP8 4096 x 8192 24.4 / 28.1 -> 18.5 / 20.4; at K = 6144, M = 16: FP8 5120 x 6144
// 34.3 -> 24.9, 4-bit 8192 x 6144 30.9 -> 23.7. But 8-bit 8192 x 16384 M = 8 69.1 ->
// 73.3 and 8-bit 28672 x 16384 M = 5 183.7 -> 222.7. The parts: one round of
// workgroups, not more (FP8 5120 x 6144 M = 16: 24.9 us in 4 parts, 34.5 in 8; 4-bit
// 10240 x 8192: 40.3 in 2, 46.0 in 4). Where the rows stage, the in-workgroup split
// stays ahead (4-bit 5120 x 16384 M = 4: 24.0 against 38.8 us in 8 parts; FP8
// 5120 x 6144 M = 12: 18.0 against 22.9 in 4).
static bool long_rows(const qgemv_desc *d, int M, int cu_count, uint32_t flags, bool with_ws) {
    if (!with_ws || (flags & (QGEMV_FLAG_KSPLIT_MASK | QGEMV_FLAG_KPARTS_MASK))) return false;
    if (d->K % (4 * k_per_chunk(d->format))) return false;
    const int64_t groups = ((d->N + 15) / 16 + 7) / 8;
    if (groups >= cu_count || groups * 8 < cu_count) return false;
    const int64_t steps = d->K / (4 * k_per_chunk(d->format));
    return staged_act_bytes(d, M < QGEMV_MAX_M ? M : QGEMV_MAX_M, steps) > kLdsBytes;
}

// Whether the persistent streaming kernel takes a round's block metadata as one window
// dword per lane per column (variant bit 3) with unr chunks per lane: 8-bit codes
// only, where the round's scale and zero-point windows are whole dwords within 64 of
// them and the rows are whole dwords on 4-byte aligned arrays (the loads never leave a
// row). Measured on MI355X (A/B, one session): 8-bit 4096 x 4096 M = 1 6.20 -> 5.71 us;
// for the other formats the per-chunk loads were as fast or faster (4-bit lm_head M = 1
// 65.2 against 67.2 us, NVFP4 lm_head M = 1 70.6 against 71.7, FP8 5120 x 6144 M = 1
// and 4 7.53 / 11.82 against 7.68 / 11.97), so they keep them.
static bool stream_meta_window(const qgemv_desc *d, int unr) {
    if (d->format != QGEMV_FMT_U8) return false;
    const int64_t nblk = d->K / d->block_size;
    const int64_t bpr = (64LL * unr * 16) / d->block_size;  // blocks per round
    const int64_t zrow = nblk;
    if (bpr * 2 > 256 || bpr % 4 || (nblk * 2) % 4 || (uintptr_t)d->scales % 4) return false;
    if (zrow % 4 || (uintptr_t)d->zero_points % 4) return false;
    return true;
}

// Whether the persistent streaming kernel may load 4-bit, 8-bit and NVFP4 block
// metadata as the aligned dwords that hold it: every scale and zero-point row is whole
// dwords on a 4-byte aligned array, so no such dword reaches past its row. (FP8 scales
// are dwords already.) Without zero points the zero-point loads read the scale row,
// which is at least as long.
static bool stream_meta_dword(const qgemv_desc *d) {
    const int64_t nblk = d->K / d->block_size;
    if ((uintptr_t)d->scales % 4) return false;
    switch (d->format) {
    case QGEMV_FMT_U4:
        if ((nblk * 2) % 4) return false;
        return !d->zero_points || (((nblk + 1) / 2) % 4 == 0 && (uintptr_t)d->zero_points % 4 == 0);
    case QGEMV_FMT_U8:
        if ((nblk * 2) % 4) return false;
        return !d->zero_points || (nblk % 4 == 0 && (uintptr_t)d->zero_points % 4 == 0);
    case QGEMV_FMT_NVFP4: return nblk % 4 == 0;  // one E4M3 byte per 16 k
    default: return false;
    }
}

// Persistent streaming kernel for M <= 4 rows in one pass (2 or 4 rows per pass for
// M = 2 or 3..4): the activation rows (in the decode's pair order) and per-chunk sums
// of them live in LDS; each wave walks column groups with the next batch of codes in
// flight. Returns false when the staged rows do not fit.
//  - chunks per lane per batch (UNR 2, 3 or 4): the fewest idle load slots over the
//    column's chunks, ties to the larger batch;
//  - columns per wave: 1 while every column can have a wave of its own within ~24
//    resident waves per CU, else 2;
//  - grid: one group per wave when that fits in 24 waves per CU (16 for several
//    rows, whose waves hold more registers), else a persistent grid of as many.
static bool stream1_plan(const qgemv_desc *d, int M, int cu_count, uint32_t flags, LaunchCfg *c) {
    // Eight rows per pass: FP8 codes; and 4-bit (on fp16), 8-bit and NVFP4 codes with
    // K >= 2048, one pass against the classic kernel's two (classic -> one pass at M = 8:
    // 4-bit 1024 x 2048 6.22 -> 5.54 us, M = 5 5.51 -> 4.65; 4-bit 1024 x 4096 9.11 ->
    // 6.21; 8-bit 2048 x 2048 6.88 -> 6.13, 8-bit 1024 x 4096 M = 6 8.34 -> 6.57; NVFP4
    // 2048 x 2048 7.42 -> 6.49; but 4-bit 4096 x 1024 8.48 -> 9.47, whose short columns
    // spend the pass on eight rows' reductions). Not 4-bit codes on bf16, whose per-row
    // activation sums leave the scalar registers no room for eight rows.
    if (M > 8) return false;
    if (M > 4 && d->format != QGEMV_FMT_FP8 &&
        (d->K < 2048 || (d->format == QGEMV_FMT_U4 && d->act_dtype == QGEMV_ACT_BF16)))
        return false;
    const int mt = M == 1 ? 1 : (M == 2 ? 2 : (M <= 4 ? 4 : 8));  // rows per pass (one pass)
    const int kpc = k_per_chunk(d->format);
    const int64_t nch = d->K / kpc;
    const int64_t nch64 = (nch + 63) / 64 * 64;
    const int nd = kpc == 32 ? 16 : 8;
    const int h = (d->format == QGEMV_FMT_NVFP4 || (d->format == QGEMV_FMT_U4 && d->block_size == 16)) ? 2 : 1;
    // The staged rows: one row up to 64 KB (two 4-wave workgroups per CU at the least;
    // past it the classic kernel, which re-reads the activations from L2 per column),
    // several up to the whole LDS. One row of 28672 (57-61 KB) measured on MI355X with
    // the 48 KB bound of before -> 64 KB (classic -> persistent): 4-bit 8192 x 28672
    // 35.4 -> 24.6 us, FP8 53.1 -> 38.6, NVFP4 36.6 -> 23.5, 8-bit 4096 x 28672 34.6 ->
    // 22.2. Several rows past 64 KB run as one round of the widest workgroups (below).
    const int64_t lds = mt * (nch64 * nd * 4 + (needs_act_sums(d) ? nch64 * h * 4 : 0));
    if (lds > (mt == 1 ? 64 * 1024 : kLdsBytes)) return false;
    const int64_t cpl = (nch + 63) / 64;  // chunks per lane per column
    int unr = 0;
    const uint32_t fu = (flags & QGEMV_FLAG_STREAM_UNR_MASK) >> QGEMV_FLAG_STREAM_UNR_SHIFT;
    if (mt > 1) {
        unr = 2;  // several rows: 2 chunks per lane per batch
    } else if (fu) {
        unr = (int)fu + 1;
    } else {
        int64_t best = -1;
        for (int u = 4; u >= 2; --u) {
            const int64_t idle = (cpl + u - 1) / u * u - cpl;
            if (best < 0 || idle < best) best = idle, unr = u;
        }
    }
    const uint32_t fc = (flags & QGEMV_FLAG_STREAM_CPW_MASK) >> QGEMV_FLAG_STREAM_CPW_SHIFT;
    int cpw;
    if (fc) cpw = fc == 3 ? 4 : (int)fc;
    else cpw = (mt > 1 || d->N <= 24LL * cu_count) ? 1 : 2;
    if (mt > 1 && cpw > 2) cpw = 2;
    if (mt == 8) cpw = 1;
    const int64_t groups = (d->N + cpw - 1) / cpw;
    const uint32_t fw = (flags & QGEMV_FLAG_STREAM_WPC_MASK) >> QGEMV_FLAG_STREAM_WPC_SHIFT;
    int64_t wpc;
    if (fw) wpc = 4 * (int64_t)fw;
    else wpc = mt > 1 ? 16 : 24;
    // 16-wave workgroups (one row, one column per wave) when asked for, or when the
    // column groups fill 8..16 waves per CU: one workgroup per CU then stages the
    // activation row once for 16 columns instead of once per 4; past 16 per CU the
    // 16-wave groups no longer spread evenly over the CUs and lose. Not for 8-bit codes:
    // there four 4-wave workgroups per CU with two chunks per lane per batch are faster
    // (cold, steady clocks, 16-wave -> 4-wave x 4 with batches of 2: 8-bit 4096 x 4096
    // 5.50 -> 5.15 us, on bf16 6.37 -> 5.77, 2048 x 4096 4.73 -> 4.44; 4-bit 4096 x 4096
    // the other way, 4.42 -> 4.72; FP8 and NVFP4 even).
    const bool wide_auto = !fc && !fw && groups >= 8LL * cu_count && groups <= 16LL * cu_count;
    const bool u8_quads = wide_auto && mt == 1 && cpw == 1 && d->format == QGEMV_FMT_U8 &&
                          !(flags & QGEMV_FLAG_STREAM_WIDE_WG);
    if (u8_quads) {
        wpc = 16;
        if (!fu) unr = 2;
    }
    int nwg = ((flags & QGEMV_FLAG_STREAM_WIDE_WG) || (wide_auto && !u8_quads)) && mt == 1 && cpw == 1 ? 16 : 4;
    // Several rows: 4, 8, 12 or 16 waves share one staged copy of the rows. The staged
    // rows bound the workgroups resident per CU (res); when 16-wave workgroups would
    // hold every column group at once, the fewest waves per workgroup that do are
    // taken and the grid is one group per wave. (FP8 5120 x 6144 at M = 4: 4-wave
    // workgroups hold 8 waves per CU and run 2.5 rounds, 15.6 us; 12-wave ones hold
    // all 5120 columns, 11.5 us.)
    const uint32_t fn = (flags & QGEMV_FLAG_STREAM_NWG_MASK) >> QGEMV_FLAG_STREAM_NWG_SHIFT;
    int64_t res = kLdsBytes / (lds > 0 ? lds : 1);
    if (res < 1) res = 1;
    const int64_t need = (groups + cu_count - 1) / cu_count;  // column groups per CU
    bool one_round = false;
    // the most waves per workgroup the kernel fits without spilling (kernel side:
    // stream_rows_max_wg)
    const bool u4_two_blocks = d->format == QGEMV_FMT_U4 && d->block_size == 16;
    // (eight rows of 4-bit or NVFP4 codes take 177-184 VGPRs: two waves per SIMD, so at
    // most 8 per workgroup)
    const bool wide8 = mt == 8 && (d->format == QGEMV_FMT_U4 || d->format == QGEMV_FMT_NVFP4);
    const int max_wg = (cpw == 2 || wide8) ? 8 : ((u4_two_blocks && mt == 4) ? 12 : 16);
    if (mt > 1 && fn) {
        nwg = 4 * (int)fn < max_wg ? 4 * (int)fn : max_wg;
    } else if (mt == 8 || lds > 64 * 1024) {
        // eight staged rows, or fewer past 64 KB, leave room for few workgroups per CU:
        // the fewest waves per workgroup that hold the CU's column groups, else the
        // most, one round (16-wave workgroups, one per CU, against 8-wave ones, two, at
        // 115-131 KB of rows: 4-bit 8192 x 28672 M = 2 30.2 against 32.7 us, FP8
        // 4096 x 14336 M = 4 15.3 against 16.5, 8-bit 8192 x 16384 M = 4 34.7 against
        // 38.6)
        nwg = 4;
        while (nwg < max_wg && nwg * res < need) nwg += 4;
        one_round = true;
    } else if (mt > 1 && !fw && max_wg * res >= need) {
        nwg = 4;
        while (nwg * res < need) nwg += 4;
        one_round = true;
    }
    const int64_t wgs = (groups + nwg - 1) / nwg;
    int64_t cap = one_round ? res * cu_count : (int64_t)cu_count * wpc / nwg;
    // One row of 1-byte codes: a grid of every column group, one per wave, which the
    // hardware starts as resident workgroups finish, in place of the persistent walk
    // (variant bit 5; not cut to the resident workgroups at create). Measured on MI355X
    // (persistent -> whole grid, us): 8-bit 151936 x 2048 50.1 -> 48.0, 65536 x 8192
    // 86.0 -> 82.3, 32768 x 4096 23.6 -> 22.5, 12288 x 4096 13.3 -> 12.8; FP8
    // 65536 x 4096 42.0 -> 40.4, 131072 x 2048 42.7 -> 41.3, 16384 x 8192 23.9 -> 23.5,
    // 28672 x 4096 20.1 -> 20.0; but 4-bit codes lose (lm_head 55.9 -> 60.7, 28672 x 4096
    // 13.7 -> 14.4), their wave's walk staying ahead of a new workgroup's activation copy.
    const bool whole = mt == 1 && (d->format == QGEMV_FMT_U8 || d->format == QGEMV_FMT_FP8) && !fw && !fc &&
                       !(flags & QGEMV_FLAG_STREAM_WIDE_WG);
    if (whole) cap = wgs;
    // several rows: a grid past one workgroup per CU is cut to a whole number of them per
    // CU, and the persistent walk carries the rest, so that every CU holds as many
    // workgroups (FP8 5120 x 6144 at M = 4: 640 8-wave workgroups, 2.5 per CU, 11.85 us;
    // 512, two per CU, 10.81)
    if (mt > 1 && !(flags & QGEMV_FLAG_STREAM_NWG_MASK) && wgs < cap && wgs > cu_count) cap = wgs / cu_count * cu_count;
    if (cap < 1) cap = 1;
    c->rows_per_pass = mt;
    c->passes = 1;
    c->cols_per_wave = cpw;
    c->ksplit = 1;
    c->waves_per_wg = nwg;
    c->grid = wgs < cap ? wgs : (cap > 0 ? cap : 1);
    c->lds_bytes = (int)lds;
    c->variant = 1 | ((unr & 3) << 1) | (whole ? 32 : 0);
    if (!(flags & QGEMV_FLAG_STREAM_META_CHUNK)) {
        if (mt < 8 && stream_meta_window(d, unr)) c->variant |= 8;  // (no windows next to eight rows)
        else if (stream_meta_dword(d)) c->variant |= 16;
    }
    return true;
}

// Where the streaming family beats the matrix family (measured on MI355X):
//  - M = 2..4 (the persistent kernel, 2 or 4 rows in one pass): for 8-bit integer
//    and FP8 codes, and for 4-bit codes while the weight is small enough (under
//    64 MB) that the call is latency-bound rather than bandwidth-bound. Wide 4-bit
//    weights take the matrix family's DMA ring from M = 2 (4-bit lm_head, M = 2:
//    90 us against 101 us), and so do all weights whose ring tile groups fill the
//    CUs (ring_band), but 1-byte codes at M = 2, where two rows leave the streaming
//    kernel ahead (FP8 28672 x 4096: 22.1 against 28.0 us; 8-bit 24.0 against 27.4). At M = 3..4, where the matrix family's tile groups fill
//    the CUs, it wins for 4-bit codes and, from 64 MB of codes, for 1-byte ones
//    (streaming -> matrix at M = 4: 4-bit 16384 x 4096 22.9 -> 15.9 us, 4-bit
//    8192 x 4096 12.5 -> 10.9 (M = 3: 11.2 -> 10.3), NVFP4 8192 x 4096 12.7 -> 9.1,
//    8-bit 16384 x 4096 28.4 -> 22.6, FP8 16384 x 4096 25.0 -> 19.5), but not for
//    smaller 1-byte weights (8-bit 8192 x 4096: 14.5 against 14.0-14.6 us at M = 4,
//    12.2 against 14.4 at M = 3; 8-bit 4096 x 4096: 9.8 against 11.5), nor with fewer
//    tile groups (FP8 5120 x 6144, 160: 11.9 against 14.2; 4-bit 4096 x 4096, 128:
//    9.0 against 10.1), nor at M = 2, where two rows leave the streaming kernel
//    ahead (FP8 8192 x 4096: 9.9 against 12.7 us; 4-bit 8192 x 4096: 9.2 against
//    10.2; 8-bit 16384 x 4096: 16.7 against 21.8; only 4-bit 16384 x 4096 is close,
//    16.3 against 15.4). 8-bit 16384 x 4096 at M = 3: 25.2 -> 22.1 us.
//  - M = 5..16 (the multi-pass kernel, 4 rows a pass, the weight re-read from L2):
//    for small weights, N x K <= 4 Mi elements with K <= 4096, where the matrix
//    family has too few tiles to fill the CUs. Matrix -> streaming at M = 8: 4-bit
//    1024 x 2048 9.4 -> 7.1 us (M = 16: 15.2 -> 10.7), 4-bit 2048 x 2048 10.0 -> 9.3,
//    FP8 1024 x 4096 9.7 -> 9.3, 8-bit 1024 x 4096 12.4 -> 10.6, 8-bit 2048 x 2048
//    10.2 -> 9.2, NVFP4 2048 x 2048 8.8 -> 8.2. Past it the matrix family wins (4-bit
//    1536 x 4096: 13.4 against 13.9 us; 4-bit 2048 x 4096: 13.4 against 14.3; FP8
//    2048 x 4096: 10.0 against 11.3), and so it does on longer columns (4-bit
//    512 x 8192: 15.8 against 16.7 us, 12.5 with K parts; FP8 512 x 8192: 13.3
//    against 16.7), whose single wave per column walks too many steps. The same holds
//    with a workspace: K parts on these shapes measured slower than the streaming
//    kernel (FP8 1024 x 4096: 13.3 us).
static bool stream_rows_win(const qgemv_desc *d, int M, bool stream_ok, int cu_count, uint32_t flags) {
    if (!stream_ok || M < 2) return false;
    if (M > 4) return d->K <= 4096 && (int64_t)d->N * d->K <= 4LL * 1024 * 1024;
    const bool bytes = d->format == QGEMV_FMT_U8 || d->format == QGEMV_FMT_FP8;
    // the weights in the DMA ring's band (ring_band), but for 1-byte codes at two rows
    if (ring_band(d, cu_count) && !(flags & QGEMV_FLAG_RING_OFF) && !(bytes && M == 2)) return false;
    const int kpc = k_per_chunk(d->format);
    const int64_t nch64 = (d->K / kpc + 63) / 64 * 64;
    const int h = (d->format == QGEMV_FMT_NVFP4 || (d->format == QGEMV_FMT_U4 && d->block_size == 16)) ? 2 : 1;
    const int mt = M == 2 ? 2 : 4;
    const int64_t lds = mt * (nch64 * (kpc == 32 ? 16 : 8) * 4 + (needs_act_sums(d) ? nch64 * h * 4 : 0));
    if (lds > kLdsBytes) return false;
    // Rows past 64 KB (one round of 16-wave workgroups): the streaming kernel for 1-byte
    // codes, and for 4-bit and NVFP4 codes where one workgroup per CU holds them (past
    // 80 KB). Streaming against the matrix family's plan (us): FP8 4096 x 14336 M = 4
    // 15.3 against 17.7, 8192 x 28672 M = 2 41.0 against 53.8, 65536 x 16384 M = 4 204.9
    // against 269.0; 8-bit 8192 x 16384 M = 3 / 4 32.4 / 34.7 against 40.2 / 40.6; 4-bit
    // on bf16 8192 x 28672 M = 2 30.2 against 38.5, 4096 x 14336 M = 3 / 4 13.8 / 16.0
    // against 16.8 / 17.1, 16384 x 16384 M = 4 46.1 against 48.1 (but NVFP4 16384 x 16384
    // M = 4 41.7 against 38.4). Between 64 and 80 KB of 4-bit rows the matrix family
    // holds on wide weights (4-bit on bf16 24576 x 8192 M = 4 32.2 against 37.0 us,
    // 65536 x 16384 M = 2 113.1 against 123.4).
    if (lds > 64 * 1024) return bytes || lds > kLdsBytes / 2;
    if (M >= 3) {
        // four rows per pass: the matrix family wins once its tile groups fill the CUs,
        // for 1-byte codes only from 64 MB of codes on
        const int ks = mfma_ksplit(d, cu_count, flags);
        const int64_t groups = ((d->N + 15) / 16 + 8 / ks - 1) / (8 / ks);
        if (groups >= cu_count && (!bytes || (int64_t)d->N * d->K >= 64LL * 1024 * 1024)) return false;
    }
    const double wbytes = (double)d->N * d->K * (kpc == 32 ? 0.5 : 1.0);
    const bool small = wbytes < 64.0 * 1024 * 1024;
    const bool byte_codes = d->format == QGEMV_FMT_U8 || d->format == QGEMV_FMT_FP8;
    return byte_codes || small;
}

int select_plan(const qgemv_desc *d, int M, int cu_count, bool fast_ok, uint32_t extra_flags, bool with_ws,
                LaunchCfg *out) {
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
    c.kparts = 1;
    c.ws_counters = 0;
    c.ws_bytes = 0;

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
    } else if (mfma_ok && M >= 2 && !stream_rows_win(d, M, stream_ok, cu_count, flags)) {
        family = QGEMV_FAMILY_MFMA;
    } else if (mfma_ok && M == 1 && d->format == QGEMV_FMT_NVFP4 && !(flags & QGEMV_FLAG_STREAM_CLASSIC)) {
        // NVFP4 at one row: the matrix family where its plan is the DMA ring and its tile
        // groups outnumber the CUs, else the streaming kernel. Measured (M = 1, one
        // session): NVFP4 248320 x 2048 68.8 -> 53.5 us, 65536 x 2048 19.9 -> 16.2; with
        // fewer groups the streaming kernel holds on longer rows (24576 x 4096: 11.3
        // against 13.0 us on the ring; 28672 x 6144: 17.8 against 19.6); for 4-bit, 8-bit
        // and FP8 codes it stays ahead (4-bit 151936 x 4096 64.4 against 74.5 us, 8-bit
        // 151936 x 2048 61.4 against 65.5, FP8 65536 x 4096 44.1 against 61.7).
        LaunchCfg ring;
        const bool takes_ring = ((d->N + 15) / 16 + 7) / 8 > cu_count &&
                                select_plan(d, 1, cu_count, fast_ok, extra_flags | QGEMV_FAMILY_MFMA, with_ws, &ring) ==
                                    QGEMV_OK &&
                                ring.family == QGEMV_FAMILY_MFMA && (ring.variant & 2);
        if (takes_ring) {
            *out = ring;
            return QGEMV_OK;
        }
        family = stream_ok ? QGEMV_FAMILY_STREAM : QGEMV_FAMILY_GENERIC;
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
        const bool lrows = long_rows(d, M, cu_count, flags, with_ws);
        c.ksplit = lrows ? 1 : mfma_ksplit(d, cu_count, flags);
        // a workgroup holds 8 / ksplit tiles of ksplit waves each
        const int nw = 8;
        c.waves_per_wg = nw;
        const int64_t tiles = (d->N + 15) / 16;
        const int64_t groups = (tiles + (nw / c.ksplit) - 1) / (nw / c.ksplit);
        const int64_t lds_red = c.ksplit > 1 ? (int64_t)nw * rg * 4 * 64 * 4 : 0;
        const int64_t steps = d->K / (4 * k_per_chunk(d->format));
        // Staged layout for kpv K parts: a 64-byte zero block, the rows of the longest
        // K part (stride its k + 8 elements), and for 4-bit codes on bf16 (the zero
        // point's sum(a) term) one 16-byte activation-sum entry per chunk, row group and
        // scale block of the chunk (abytes); then the K-split reduction area, which overlays the staged
        // activations when every workgroup holds a single tile group (always with K
        // parts; without, when one round of them fits at once), as they are dead by
        // then, and else follows them (FP8 8192 x 4096 at M = 16: 131 KB of staged rows
        // and 32 KB of reduction area fit only overlaid); then, with K parts, the
        // 16-byte last-workgroup flag (lds).
        struct Staged { int64_t abytes, lds; };
        auto staged = [&](int kpv) {
            const int64_t ab = staged_act_bytes(d, M, (steps + kpv - 1) / kpv);
            const int64_t fb = kpv > 1 ? 16 : 0;
            const int64_t ovl = (ab > lds_red ? ab : lds_red) + fb;
            int64_t pc = kLdsBytes / ovl;
            if (pc > 32 / nw) pc = 32 / nw;
            const bool overlay = c.ksplit > 1 && (kpv > 1 || groups <= pc * cu_count);
            return Staged{ab, overlay ? ovl : ab + lds_red + fb};
        };
        int kp = with_ws ? mfma_kparts(d, cu_count, flags, c.ksplit, groups) : 1;
        if (lrows) {
            // the most parts (2 to 8) that keep the workgroups to one round over the CUs,
            // then more (up to 8) until this M's rows stage
            kp = 2;
            while (kp < 8 && groups * 2 * kp <= cu_count) kp *= 2;
            while (kp < 8 && staged(kp).lds > kLdsBytes) kp *= 2;
            while (kp > 1 && (steps < 2LL * kp || (int64_t)kp * QGEMV_MAX_M * d->N >= (1LL << 31))) kp /= 2;
        }
        // With a workspace, where the unsplit plan's activations do not fit in LDS at
        // this M, 2 parts: twice the workgroups, each staging half the K range where that
        // fits. The one choice of the K parts that depends on M. Taken where the tile
        // groups fill at most half the CUs, or all of them while each wave of the unsplit
        // plan walks 24 K steps or more (the activations it would carry in the ring cost
        // in proportion). Measured on MI355X, unsplit -> 2 parts: FP8 2048 x 8192 M = 16
        // 36.9 -> 22.1 us; 8-bit 2048 x 8192 M = 16 37.8 -> 26.8; 4-bit 2048 x 16384
        // M = 8 37.1 -> 22.3, M = 16 (unstaged either way) 66.6 -> 44.0; FP8 5120 x 6144
        // M = 16 (160 groups, 24 steps per wave) 49.2 -> 35.1; 4-bit 16384 x 8192 M = 16
        // (256 groups, 32 steps) 123.2 -> 61.7; but 8-bit 4096 x 8192 M = 16 (256
        // groups, 16 steps) 39.5 -> 51.5. Where the rows fit, 2 parts lose (FP8
        // 2048 x 8192 M = 8: 13.8 -> 16.4 us).
        const int64_t spw1 = (steps + c.ksplit - 1) / c.ksplit;
        const bool rows_too_big = (groups * 2 <= cu_count || (groups <= cu_count && spw1 >= 24)) &&
                                  staged(1).lds > kLdsBytes;
        if (with_ws && kp == 1 && !(flags & QGEMV_FLAG_KPARTS_MASK) && rows_too_big && steps >= 4LL * c.ksplit &&
            2LL * QGEMV_MAX_M * d->N < (1LL << 31))
            kp = 2;
        // Otherwise (no workspace, or a forced single part), more than 8 rows whose
        // activations do not stage at this M run as passes of 8 rows, one launch each on
        // the caller's stream, when 8 rows stage (or take the DMA ring): every row's
        // arithmetic is that of the single launch (the K split does not depend on M, and
        // staged and unstaged activations give the same bits), the weight is read once
        // per pass. Unstaged rows travel with the codes in the register ring, 16 rows of
        // activations per 16 columns of codes, which costs more than a second read of
        // the weight. Measured on MI355X, one launch -> passes: FP8 5120 x 6144 M = 16
        // 49.2 -> 32.5 us; FP8 2048 x 8192 M = 16 36.9 -> 27.3, M = 12 28.9 -> 24.5;
        // 4-bit 16384 x 8192 M = 16 122.3 -> 65.0, M = 12 95.3 -> 60.1; 4-bit
        // 24576 x 8192 M = 9 112.6 -> 67.8, M = 16 184.8 -> 77.2; 4-bit 5120 x 6144 M = 16
        // 49.3 -> 29.9; 8-bit 4096 x 8192 M = 16 37.7 -> 30.7, M = 12 30.1 -> 26.9;
        // FP8 24576 x 4096 M = 16 97.0 -> 51.0; 4-bit 151936 x 8192 M = 16 1164.8 ->
        // 478.1; FP8 65536 x 8192 M = 16 475.8 -> 289.5, M = 10 309.6 -> 282.1.
        if (kp == 1 && staged(1).lds > kLdsBytes && M > 8 &&
            !(flags & (QGEMV_FLAG_STAGE_A_OFF | QGEMV_FLAG_STAGE_A_ON))) {
            LaunchCfg half;
            // (the matrix family's plan for 8 rows, whichever family 8 rows alone would
            // take: staged rows in the register ring, or the DMA ring)
            if (select_plan(d, 8, cu_count, fast_ok, extra_flags | QGEMV_FAMILY_MFMA, with_ws, &half) == QGEMV_OK &&
                half.family == QGEMV_FAMILY_MFMA && (half.variant & 3) && half.kparts == 1) {
                half.passes = (M + 7) / 8;
                *out = half;
                return QGEMV_OK;
            }
        }
        const int64_t smax = (steps + kp - 1) / kp;  // K steps of the longest part
        const Staged st = staged(kp);
        const int64_t abytes16 = st.abytes;
        // DMA ring (no K split, one or two row groups, metadata rows in whole dwords):
        // 8 waves per CU, each with R slots of SS K steps; the largest prefetch that
        // fits in LDS next to the staged activations.
        const bool zpp = d->zero_points && (d->format == QGEMV_FMT_U4 || d->format == QGEMV_FMT_U8);
        const bool ring_fits = dma_ring_fits(d, abytes16, zpp, 2, &c.lds_bytes);
        // Ring depth: 2 slots per wave (the next slot loads while the current one
        // computes), 3 for the formats with 16 k per chunk (FP8, 8-bit codes), whose slot
        // holds half the arithmetic of a 4-bit one, where the LDS holds the third. Measured
        // with nontemporal code copies (2 -> 3 slots): FP8 65536 x 4096 M = 3 / 4 56.7 /
        // 57.0 -> 50.2 / 50.4 us, 8-bit 56.4 / 56.7 -> 49.4 / 49.7, 8-bit on bf16 M = 4
        // 57.2 -> 52.2, FP8 151936 x 4096 M = 4 124.2 -> 118.8, but FP8 131072 x 2048
        // (bf16) M = 4 43.4 -> 44.1; 4-bit and NVFP4 lm_heads 2-4% slower with 3. Deeper
        // rings of shorter slots lost everywhere (the per-slot wait and DMA issue). The
        // depth flag forces 2 (value 1) or 3 (value 2) slots where they fit.
        const uint32_t rdep = (flags & QGEMV_FLAG_MFMA_DEPTH_MASK) >> QGEMV_FLAG_MFMA_DEPTH_SHIFT;
        int32_t lds3 = 0;
        const bool three = (rdep == 2 || (rdep == 0 && k_per_chunk(d->format) == 16)) &&
                           dma_ring_fits(d, abytes16, zpp, 3, &lds3);
        bool ring = c.ksplit == 1 && kp == 1 && rg <= 2 && ring_fits && ring_groups_fill(d, groups, cu_count);
        if (flags & QGEMV_FLAG_RING_ON) ring = c.ksplit == 1 && kp == 1 && rg <= 2 && ring_fits;
        if (flags & QGEMV_FLAG_RING_OFF) ring = false;
        if (ring) {
            c.waves_per_wg = 8;
            c.variant = 2 | (three ? 4 : 0);
            if (three) c.lds_bytes = lds3;
            const int64_t wgs = (tiles + 7) / 8;
            c.grid = wgs < cu_count ? wgs : cu_count;
            *out = c;
            return QGEMV_OK;
        }
        c.lds_bytes = 0;
        // Stage the activations in LDS when they fit and every wave has enough K steps
        // per tile (8 or more) to amortize the copy; with fewer, the activations travel
        // with the codes in the register ring instead.
        const int64_t spw = (smax + c.ksplit - 1) / c.ksplit;
        const int64_t flag_b = kp > 1 ? 16 : 0;
        const int64_t lds_staged = st.lds;
        bool stage = lds_staged <= kLdsBytes && spw >= 8;
        if (flags & QGEMV_FLAG_STAGE_A_ON) stage = lds_staged <= kLdsBytes;
        if (flags & QGEMV_FLAG_STAGE_A_OFF) stage = false;
        // register-ring depth: 4 slots unless forced. With the loads coalesced, 8 slots
        // measured no faster anywhere and slower on the staged FP8 and 8-bit rings (FP8
        // 5120 x 6144 M = 8: 16.6 us with 4, 17.4 with 8; 8-bit 4096 x 4096 M = 8: 15.5
        // / 16.2 us; 4-bit lm_head M = 12 and 16: equal)
        const uint32_t fdep = (flags & QGEMV_FLAG_MFMA_DEPTH_MASK) >> QGEMV_FLAG_MFMA_DEPTH_SHIFT;
        // (8 slots only where the kernel takes them: staged rows, one or two row groups,
        // one scale block per chunk, and not one row group of a 32-k chunk format)
        const bool two_blocks = d->format == QGEMV_FMT_NVFP4 || (d->format == QGEMV_FMT_U4 && d->block_size == 16);
        const bool deep8 = fdep == 2 && stage && rg <= 2 && !two_blocks && !(k_per_chunk(d->format) == 32 && rg == 1);
        c.variant = (stage ? 1 : 0) | (deep8 ? 8 : 0);
        // with K parts, 16 bytes more for the last-workgroup flag
        c.lds_bytes = (int)(stage ? lds_staged : lds_red + flag_b);
        // Without K parts, where the rows do not fit in LDS, not even 8 at a time (no row
        // passes above), so the activations would travel in the register ring, and the
        // tile groups fill at most a quarter of the CUs: from M = 6 the streaming family
        // is faster (matrix -> streaming, no workspace: FP8 1024 x 16384 M = 8 36.1 ->
        // 29.7 us, M = 16 66.1 -> 56.0, M = 6 29.4 -> 28.2; 8-bit 1024 x 16384 M = 8
        // 38.8 -> 33.1; 4-bit 1024 x 16384 M = 8 36.6 -> 30.9; FP8 512 x 16384 M = 8
        // 36.0 -> 28.8; at M = 5 the two are even, 26.0 against 26.8). With more tile
        // groups the matrix family stays ahead (4-bit 2048 x 16384, 128 groups: M = 8
        // 37.1 against 43.5 us, M = 16 66.7 against 81.2).
        // FP8 codes at M = 5..8 without K parts, where the tile groups fill at most half the
        // CUs: one pass of eight rows in the persistent streaming kernel, a column per wave,
        // loads every CU (matrix -> streaming: FP8 2048 x 4096 M = 8 9.73 -> 9.35 us; bf16
        // 2048 x 8192 M = 8 13.6 -> 12.1). With more tile groups the matrix family stays
        // ahead (FP8 5120 x 6144, 160 groups: M = 8 16.1 against 20.5 us, M = 5 14.8
        // against 15.2; 8192 x 4096, 256 groups: M = 8 13.1 against 17.9).
        if (forced == 0 && kp == 1 && d->format == QGEMV_FMT_FP8 && M >= 5 && M <= 8 && groups * 2 <= cu_count &&
            stream_ok && !(flags & (QGEMV_FLAG_STAGE_A_OFF | QGEMV_FLAG_STAGE_A_ON | QGEMV_FLAG_STREAM_CLASSIC))) {
            LaunchCfg rows8;
            if (stream1_plan(d, M, cu_count, flags, &rows8))
                return select_plan(d, M, cu_count, fast_ok, extra_flags | QGEMV_FAMILY_STREAM, with_ws, out);
        }
        if (forced == 0 && kp == 1 && !stage && groups * 4 <= cu_count && staged(1).lds > kLdsBytes && M >= 6 &&
            stream_ok && !(flags & (QGEMV_FLAG_STAGE_A_OFF | QGEMV_FLAG_STAGE_A_ON)))
            return select_plan(d, M, cu_count, fast_ok, extra_flags | QGEMV_FAMILY_STREAM, with_ws, out);
        // without K parts, a persistent grid of at most what fits at once; with them,
        // exactly one workgroup per tile group and part
        int64_t grid = groups * kp;
        if (stage && kp == 1) {
            int64_t per_cu = c.lds_bytes > 0 ? kLdsBytes / c.lds_bytes : 8;
            if (per_cu > 32 / nw) per_cu = 32 / nw;
            if (per_cu < 1) per_cu = 1;
            if (grid > per_cu * cu_count) grid = per_cu * cu_count;
        }
        c.grid = grid;
        c.kparts = kp;
        if (kp > 1) {
            // workspace: one 32-bit completion counter per tile group (rounded up to
            // 256 bytes), then the fp32 partial tiles [kp, M, N]
            c.ws_counters = (groups * 4 + 255) / 256 * 256;
            c.ws_bytes = c.ws_counters + ((int64_t)kp * M * d->N * 4 + 255) / 256 * 256;
        }
    } else if (family == QGEMV_FAMILY_GENERIC) {
        c.rows_per_pass = M;
        c.passes = 1;
        c.cols_per_wave = 1;
        const int64_t wgs = (d->N + 3) / 4;
        const int64_t cap = 8LL * cu_count;
        c.grid = wgs < cap ? wgs : cap;
    } else if (!(flags & QGEMV_FLAG_STREAM_CLASSIC) && stream1_plan(d, M, cu_count, flags, &c)) {
        // persistent one-row kernel (plan filled in)
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

bool persistent(const LaunchCfg &c) {
    if (c.family == QGEMV_FAMILY_MFMA) return c.kparts == 1;
    if (c.family == QGEMV_FAMILY_STREAM) return (c.variant & 1) && !(c.variant & 32);
    return c.family == QGEMV_FAMILY_GENERIC;
}

bool same_launch(const LaunchCfg &x, const LaunchCfg &y) {
    return x.family == y.family && x.rows_per_pass == y.rows_per_pass && x.passes == y.passes &&
           x.cols_per_wave == y.cols_per_wave && x.ksplit == y.ksplit && x.waves_per_wg == y.waves_per_wg &&
           x.grid == y.grid && x.lds_bytes == y.lds_bytes && x.variant == y.variant && x.kparts == y.kparts &&
           x.ws_bytes == y.ws_bytes;
}

// The online choice the pages' batched small-M review asks for in place of thresholds
// tuned on one machine ("[CUDA] Batched small-M GEMV for MatMulNBits (4-bit/8-bit)",
// review), limited here to the choices that leave every result bit unchanged: the
// automatic plan's family, K split and K parts fix the order of the fp32 sums, and
// within them the streaming family's columns per wave, batch depth, workgroup size and
// grid, its classic or persistent kernel and its metadata loads, and the matrix
// family's activation staging, weight ring (registers or LDS DMA) and ring depth only
// move work between waves and change how it is fetched. Each dimension takes its
// values in turn (0 = automatic) unless the descriptor's or the environment's flags
// already fix it; the product is cut to the plans that keep family, K split and K
// parts, and to one set of flags per distinct launch (the residency cut, made at
// create, counts as part of the launch for persistent grids).
int tune_candidates(const qgemv_desc *d, int M, int cu_count, bool fast_ok, uint32_t env_flags, bool with_ws,
                    uint32_t *out, int max, int *count) {
    if (!count) return QGEMV_E_NULL;
    *count = 0;
    if (max < 1 || !out) return QGEMV_E_ARG;
    LaunchCfg base;
    int rc = select_plan(d, M, cu_count, fast_ok, env_flags, with_ws, &base);
    if (rc) return rc;
    const uint32_t fixed = d->flags | env_flags;
    struct Dim {
        uint32_t mask;
        uint32_t vals[5];
        int n;
    };
    Dim dims[8];
    int nd = 0;
    auto add = [&](uint32_t mask, std::initializer_list<uint32_t> v) {
        if (fixed & mask) return;
        Dim &x = dims[nd++];
        x.mask = mask;
        x.n = 0;
        for (uint32_t e : v) x.vals[x.n++] = e;
    };
    if (base.family == QGEMV_FAMILY_STREAM) {
        const bool one_row = M == 1;
        // the classic kernel has none of the persistent kernel's shape choices: not
        // offered where the flags fix one of them
        add(QGEMV_FLAG_STREAM_CLASSIC | QGEMV_FLAG_STREAM_CPW_MASK | QGEMV_FLAG_STREAM_UNR_MASK |
                QGEMV_FLAG_STREAM_WPC_MASK | QGEMV_FLAG_STREAM_WIDE_WG | QGEMV_FLAG_STREAM_NWG_MASK |
                QGEMV_FLAG_STREAM_META_CHUNK,
            {0u, QGEMV_FLAG_STREAM_CLASSIC});
        add(QGEMV_FLAG_STREAM_CPW_MASK, {0u, 1u << QGEMV_FLAG_STREAM_CPW_SHIFT, 2u << QGEMV_FLAG_STREAM_CPW_SHIFT,
                                         3u << QGEMV_FLAG_STREAM_CPW_SHIFT});
        if (one_row) {
            add(QGEMV_FLAG_STREAM_UNR_MASK, {0u, 1u << QGEMV_FLAG_STREAM_UNR_SHIFT, 2u << QGEMV_FLAG_STREAM_UNR_SHIFT,
                                             3u << QGEMV_FLAG_STREAM_UNR_SHIFT});
            add(QGEMV_FLAG_STREAM_WIDE_WG, {0u, QGEMV_FLAG_STREAM_WIDE_WG});
        } else {
            add(QGEMV_FLAG_STREAM_NWG_MASK, {0u, 1u << QGEMV_FLAG_STREAM_NWG_SHIFT, 2u << QGEMV_FLAG_STREAM_NWG_SHIFT,
                                             3u << QGEMV_FLAG_STREAM_NWG_SHIFT, 4u << QGEMV_FLAG_STREAM_NWG_SHIFT});
        }
        add(QGEMV_FLAG_STREAM_WPC_MASK, {0u, 2u << QGEMV_FLAG_STREAM_WPC_SHIFT, 4u << QGEMV_FLAG_STREAM_WPC_SHIFT,
                                         6u << QGEMV_FLAG_STREAM_WPC_SHIFT, 7u << QGEMV_FLAG_STREAM_WPC_SHIFT});
        if (d->format == QGEMV_FMT_U8) add(QGEMV_FLAG_STREAM_META_CHUNK, {0u, QGEMV_FLAG_STREAM_META_CHUNK});
    } else if (base.family == QGEMV_FAMILY_MFMA) {
        add(QGEMV_FLAG_STAGE_A_OFF | QGEMV_FLAG_STAGE_A_ON, {0u, QGEMV_FLAG_STAGE_A_OFF, QGEMV_FLAG_STAGE_A_ON});
        add(QGEMV_FLAG_RING_OFF | QGEMV_FLAG_RING_ON, {0u, QGEMV_FLAG_RING_OFF, QGEMV_FLAG_RING_ON});
        add(QGEMV_FLAG_MFMA_DEPTH_MASK, {0u, 1u << QGEMV_FLAG_MFMA_DEPTH_SHIFT, 2u << QGEMV_FLAG_MFMA_DEPTH_SHIFT});
    }
    add(QGEMV_FLAG_NO_RESIDENCY_FIT, {0u, QGEMV_FLAG_NO_RESIDENCY_FIT});
    // the kept launches and the residency bit each was planned with
    LaunchCfg kept[QGEMV_TUNE_MAX_CANDIDATES];
    int n = 0;
    int idx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (;;) {
        uint32_t f = 0;
        for (int i = 0; i < nd; ++i) f |= dims[i].vals[idx[i]];
        LaunchCfg c;
        if (select_plan(d, M, cu_count, fast_ok, env_flags | f, with_ws, &c) == QGEMV_OK && c.family == base.family &&
            c.ksplit == base.ksplit && c.kparts == base.kparts) {
            // the residency cut is part of the launch only for persistent grids
            if (!persistent(c)) f &= ~QGEMV_FLAG_NO_RESIDENCY_FIT;
            bool dup = false;
            for (int j = 0; j < n && !dup; ++j)
                dup = same_launch(kept[j], c) &&
                      ((out[j] ^ f) & QGEMV_FLAG_NO_RESIDENCY_FIT) == 0;
            if (!dup) {
                if (n == max || n == QGEMV_TUNE_MAX_CANDIDATES) break;
                kept[n] = c;
                out[n++] = f;
            }
        }
        int i = nd - 1;
        while (i >= 0 && ++idx[i] == dims[i].n) idx[i--] = 0;
        if (i < 0) break;
    }
    *count = n;
    return QGEMV_OK;
}

}  // namespace qgemv
