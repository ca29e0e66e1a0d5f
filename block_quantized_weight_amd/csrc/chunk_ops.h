// Per-format work on one 16-byte chunk of a column's codes (streaming family).
//
// A chunk holds KPC consecutive k: 32 for U4 and NVFP4, 16 for U8 and FP8. Block
// sizes are powers of two >= 16, so a chunk lies in one scale block, except a U4
// chunk with 16-wide blocks and every NVFP4 chunk, which span two (H = 2 "halves" of
// 16 k, each with its own scale).
//
// Per half the codes are decoded exactly into fp16/bf16 pairs and multiplied into an
// fp32 sum with v_dot2; the block scale then multiplies that sum once:
//     s * sum_k a_k (q_k - z)
// For U8 (both activation types) and for U4 with fp16 activations the decode forms
// (q - z) itself, exactly, so the sum holds only true products ("[CUDA] MatMulNBits
// 8-bit: wide fp16 M=1 kernel", Description: (q - zp) exact, scale applied once per
// chunk to an fp32 partial). U4 with bf16 activations decodes the bare codes q (no
// offset) and takes the zero point as -z * sum(a) over the same k (ASUM): gfx950 has
// no packed bf16 subtract, and the per-element route through fp32 would triple the
// decode's instructions. The rounding of that difference then scales with z <= 15,
// never with an offset added to the codes.
// ("[CUDA] Block-scaled MatMul decode GEMV", FP4 row-tiling paragraph: load, decode
// and scales shared by the rows).
//
// The activation side of a chunk (pairs in the decode's k order, and sum(a) where
// ASUM) is prepared once per row and reused by every column the wave owns.
#pragma once

#include "qgemv_device.h"

namespace qgemv {

// Activations of one chunk for one row: 16 dwords (32 values) at most, in the order
// the format's decode pairs them, plus sum(a) per half (ASUM formats only).
struct ChunkAct {
    uint32_t p[16];
    float asum[2];
};

template <int FMT, int ACT, int H>
struct ChunkOps;

template <int ACT>
__device__ __forceinline__ float sum_pairs(const uint32_t *x, int count) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < count; ++i) s = dot2<ACT>(x[i], ones2<ACT>(), s);
    return s;
}

// ----------------------------------------------------------------------------------
// U4, fp16 activations. Codes become fp16 subnormals: a nibble at bits 0..3 of a half
// is q * 2^-24, a nibble at bits 4..7 is q * 2^-20 (kept in a second sum that weighs
// 1/16 against the first when both return to units of 1). The zero point, placed the
// same way, is subtracted from each pair with one packed fp16 op: (q - z) * 2^-24 and
// (q - z) * 2^-20 are exact subnormals (|q - z| <= 15).
template <int H>
struct ChunkOps<FMT_U4, ACT_F16, H> {
    static constexpr int KPC = 32;
    static constexpr int ND = 16;  // activation dwords per chunk
    static constexpr bool ASUM = false;

    // x: natural pairs (a0,a1),(a2,a3),...; weight dword d (k = 8d..8d+7) decodes to
    // pairs (k0,k4), (k2,k6) [low nibbles] and (k1,k5), (k3,k7) [high nibbles].
    __device__ static void prep(const uint32_t x[16], ChunkAct &h) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t x0 = x[4 * d], x1 = x[4 * d + 1], x2 = x[4 * d + 2], x3 = x[4 * d + 3];
            h.p[4 * d + 0] = perm(x2, x0, 0x05040100u);  // (a0, a4)
            h.p[4 * d + 1] = perm(x3, x1, 0x05040100u);  // (a2, a6)
            h.p[4 * d + 2] = perm(x2, x0, 0x07060302u);  // (a1, a5)
            h.p[4 * d + 3] = perm(x3, x1, 0x07060302u);  // (a3, a7)
        }
    }

    // decoded operand words of a chunk (exact q - z), shared by every row of a tile;
    // z[h]: the integer zero point of half h
    static constexpr int NWD = 16;
    __device__ static void decode(const u4v &w, const uint32_t z[H], uint32_t wd[16]) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int i = (H == 2) ? (d >> 1) : 0;
            const uint32_t zl = z[i] | (z[i] << 16);  // (z, z) * 2^-24
            const uint32_t zh = zl << 4;              // (z, z) * 2^-20
            const uint32_t wv = w[d], w8 = w[d] >> 8;
            wd[4 * d + 0] = sub_h2(wv & 0x000F000Fu, zl);
            wd[4 * d + 1] = sub_h2(w8 & 0x000F000Fu, zl);
            wd[4 * d + 2] = sub_h2(wv & 0x00F000F0u, zh);
            wd[4 * d + 3] = sub_h2(w8 & 0x00F000F0u, zh);
        }
    }

    // sum_k a_k (q_k - z) per half
    __device__ static void dotd(const uint32_t wd[16], const ChunkAct &h, float out[H]) {
        float lo[H], hi[H];
#pragma unroll
        for (int i = 0; i < H; ++i) lo[i] = hi[i] = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int i = (H == 2) ? (d >> 1) : 0;
            lo[i] = dot2<ACT_F16>(wd[4 * d + 0], h.p[4 * d + 0], lo[i]);
            lo[i] = dot2<ACT_F16>(wd[4 * d + 1], h.p[4 * d + 1], lo[i]);
            hi[i] = dot2<ACT_F16>(wd[4 * d + 2], h.p[4 * d + 2], hi[i]);
            hi[i] = dot2<ACT_F16>(wd[4 * d + 3], h.p[4 * d + 3], hi[i]);
        }
#pragma unroll
        for (int i = 0; i < H; ++i) out[i] = __builtin_fmaf(hi[i], 0.0625f, lo[i]) * 16777216.0f;
    }
};

// U4, bf16 activations. The low and the high nibbles of a dword are split into
// bytes (one and, one shift and one and), and the E4M3 converter turns two bytes
// 0..15 into the exact bf16 integers q: dword d gives pairs (k0,k2), (k4,k6) from the
// low nibbles and (k1,k3), (k5,k7) from the high ones. No offset is added to q; the
// zero point enters as -z * sum(a) (ASUM).
template <int H>
struct ChunkOps<FMT_U4, ACT_BF16, H> {
    static constexpr int KPC = 32;
    static constexpr int ND = 16;
    static constexpr bool ASUM = true;

    __device__ static void prep(const uint32_t x[16], ChunkAct &h) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t x0 = x[4 * d], x1 = x[4 * d + 1], x2 = x[4 * d + 2], x3 = x[4 * d + 3];
            h.p[4 * d + 0] = perm(x1, x0, 0x05040100u);  // (a0, a2)
            h.p[4 * d + 1] = perm(x3, x2, 0x05040100u);  // (a4, a6)
            h.p[4 * d + 2] = perm(x1, x0, 0x07060302u);  // (a1, a3)
            h.p[4 * d + 3] = perm(x3, x2, 0x07060302u);  // (a5, a7)
        }
        if constexpr (H == 2) {
            h.asum[0] = sum_pairs<ACT_BF16>(x, 8);
            h.asum[1] = sum_pairs<ACT_BF16>(x + 8, 8);
        } else {
            h.asum[0] = sum_pairs<ACT_BF16>(x, 16);
        }
    }

    static constexpr int NWD = 16;
    __device__ static void decode(const u4v &w, const uint32_t *, uint32_t wd[16]) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t lo = w[d] & 0x0F0F0F0Fu, hi = (w[d] >> 4) & 0x0F0F0F0Fu;
            wd[4 * d + 0] = small_int_bf16_pair<false>(lo);
            wd[4 * d + 1] = small_int_bf16_pair<true>(lo);
            wd[4 * d + 2] = small_int_bf16_pair<false>(hi);
            wd[4 * d + 3] = small_int_bf16_pair<true>(hi);
        }
    }

    // sum_k a_k q_k per half
    __device__ static void dotd(const uint32_t wd[16], const ChunkAct &h, float out[H]) {
        float s[H];
#pragma unroll
        for (int i = 0; i < H; ++i) s[i] = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int i = (H == 2) ? (d >> 1) : 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) s[i] = dot2<ACT_BF16>(wd[4 * d + k], h.p[4 * d + k], s[i]);
        }
#pragma unroll
        for (int i = 0; i < H; ++i) out[i] = s[i];
    }
};

// U8, fp16 activations: bytes become fp16 subnormals q * 2^-24 with one byte permute
// per pair, and the zero point's pair (z, z) * 2^-24 is subtracted with one packed
// fp16 op: (q - z) * 2^-24 is an exact subnormal (|q - z| <= 255). Pairs keep the
// natural k order.
template <int H>
struct ChunkOps<FMT_U8, ACT_F16, H> {
    static constexpr int KPC = 16;
    static constexpr int ND = 8;
    static constexpr bool ASUM = false;

    __device__ static void prep(const uint32_t x[8], ChunkAct &h) {
#pragma unroll
        for (int i = 0; i < 8; ++i) h.p[i] = x[i];
    }

    static constexpr int NWD = 8;
    __device__ static void decode(const u4v &w, const uint32_t z[H], uint32_t wd[8]) {
        const uint32_t zz = z[0] | (z[0] << 16);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            wd[2 * d] = sub_h2(perm(0u, w[d], 0x0C010C00u), zz);
            wd[2 * d + 1] = sub_h2(perm(0u, w[d], 0x0C030C02u), zz);
        }
    }

    __device__ static void dotd(const uint32_t wd[8], const ChunkAct &h, float out[1]) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s = dot2<ACT_F16>(wd[i], h.p[i], s);
        out[0] = s * 16777216.0f;
    }
};

// U8, bf16 activations: each byte q becomes the exact fp32 value q - z, multiplied
// with the widened activation in fp32.
template <int H>
struct ChunkOps<FMT_U8, ACT_BF16, H> {
    static constexpr int KPC = 16;
    static constexpr int ND = 8;
    static constexpr bool ASUM = false;

    __device__ static void prep(const uint32_t x[8], ChunkAct &h) {
#pragma unroll
        for (int i = 0; i < 8; ++i) h.p[i] = x[i];
    }

    // decoded words: the 16 values q - z as float bits
    static constexpr int NWD = 16;
    __device__ static void decode(const u4v &w, const uint32_t z[H], uint32_t wd[16]) {
        const float zf = (float)z[0];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            wd[4 * d + 0] = __builtin_bit_cast(uint32_t, (float)(w[d] & 0xFFu) - zf);
            wd[4 * d + 1] = __builtin_bit_cast(uint32_t, (float)((w[d] >> 8) & 0xFFu) - zf);
            wd[4 * d + 2] = __builtin_bit_cast(uint32_t, (float)((w[d] >> 16) & 0xFFu) - zf);
            wd[4 * d + 3] = __builtin_bit_cast(uint32_t, (float)(w[d] >> 24) - zf);
        }
    }

    __device__ static void dotd(const uint32_t wd[16], const ChunkAct &h, float out[1]) {
        float s = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const float a0 = __builtin_bit_cast(float, h.p[2 * d] << 16);
            const float a1 = __builtin_bit_cast(float, h.p[2 * d] & 0xFFFF0000u);
            const float a2 = __builtin_bit_cast(float, h.p[2 * d + 1] << 16);
            const float a3 = __builtin_bit_cast(float, h.p[2 * d + 1] & 0xFFFF0000u);
            s = __builtin_fmaf(a0, __builtin_bit_cast(float, wd[4 * d + 0]), s);
            s = __builtin_fmaf(a1, __builtin_bit_cast(float, wd[4 * d + 1]), s);
            s = __builtin_fmaf(a2, __builtin_bit_cast(float, wd[4 * d + 2]), s);
            s = __builtin_fmaf(a3, __builtin_bit_cast(float, wd[4 * d + 3]), s);
        }
        out[0] = s;
    }
};

// FP8 (E4M3FN): hardware widening to fp16/bf16, natural pairs.
template <int ACT, int H>
struct ChunkOps<FMT_FP8, ACT, H> {
    static constexpr int KPC = 16;
    static constexpr int ND = 8;
    static constexpr bool ASUM = false;

    __device__ static void prep(const uint32_t x[8], ChunkAct &h) {
#pragma unroll
        for (int i = 0; i < 8; ++i) h.p[i] = x[i];
    }

    static constexpr int NWD = 8;
    __device__ static void decode(const u4v &w, const uint32_t *, uint32_t wd[8]) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            wd[2 * d] = fp8_pair<ACT, false>(w[d]);
            wd[2 * d + 1] = fp8_pair<ACT, true>(w[d]);
        }
    }

    __device__ static void dotd(const uint32_t wd[8], const ChunkAct &h, float out[1]) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s = dot2<ACT>(wd[i], h.p[i], s);
        out[0] = s;
    }
};

// NVFP4: hardware E2M1 widening, natural pairs; two scale blocks per chunk.
template <int ACT, int H>
struct ChunkOps<FMT_NVFP4, ACT, H> {
    static constexpr int KPC = 32;
    static constexpr int ND = 16;
    static constexpr bool ASUM = false;

    __device__ static void prep(const uint32_t x[16], ChunkAct &h) {
#pragma unroll
        for (int i = 0; i < 16; ++i) h.p[i] = x[i];
    }

    static constexpr int NWD = 16;
    __device__ static void decode(const u4v &w, const uint32_t *, uint32_t wd[16]) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            wd[4 * d + 0] = fp4_pair<ACT, 0>(w[d]);
            wd[4 * d + 1] = fp4_pair<ACT, 1>(w[d]);
            wd[4 * d + 2] = fp4_pair<ACT, 2>(w[d]);
            wd[4 * d + 3] = fp4_pair<ACT, 3>(w[d]);
        }
    }

    __device__ static void dotd(const uint32_t wd[16], const ChunkAct &h, float out[2]) {
        float s[2] = {0.0f, 0.0f};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int i = d >> 1;
#pragma unroll
            for (int k = 0; k < 4; ++k) s[i] = dot2<ACT>(wd[4 * d + k], h.p[4 * d + k], s[i]);
        }
        out[0] = s[0];
        out[1] = s[1];
    }
};

// sum over a chunk (per half) of activations times decoded codes: decode, then the
// dot products in the format's fixed order. Splitting the two lets a tile of rows
// share one decode without changing any row's arithmetic.
template <int FMT, int ACT, int H>
__device__ __forceinline__ void chunk_dot(const u4v &w, const uint32_t z[H], const ChunkAct &h, float out[H]) {
    using Ops = ChunkOps<FMT, ACT, H>;
    uint32_t wd[Ops::NWD];
    Ops::decode(w, z, wd);
    Ops::dotd(wd, h, out);
}

// The block sum of half h in the accumulator: acc + s * (part - z * sum(a)) for the
// ASUM format, acc + s * part for the others (whose part already holds q - z).
template <bool ASUM>
__device__ __forceinline__ float block_acc(float acc, float s, float part, uint32_t z, float asum) {
    float v = part;
    if constexpr (ASUM) v = __builtin_fmaf(-(float)z, asum, v);
    return __builtin_fmaf(s, v, acc);
}

// ----------------------------------------------------------------------------------
// Per-column pointers, computed once per wave, and the block metadata of a chunk.

struct ColPtrs {
    const uint8_t *w;   // codes of the column
    const void *s;      // scale row
    const uint8_t *z;   // zero-point row (the scale row when there are no zero points)
};

template <int FMT>
__device__ __forceinline__ ColPtrs col_ptrs(const KArgs &a, int64_t n) {
    ColPtrs p;
    p.w = a.W + n * a.col_bytes;
    if constexpr (FMT == FMT_NVFP4) p.s = (const uint8_t *)a.scales + n * (a.K >> 4);
    else if constexpr (FMT == FMT_FP8) p.s = (const float *)a.scales + n * a.nblk;
    else p.s = (const uint16_t *)a.scales + n * a.nblk;
    // without zero points p.z aliases the scale row (valid memory, at least as long as
    // a zero-point row) so zero-point loads never sit behind a branch; the decode then
    // takes the midpoint
    p.z = a.zp ? a.zp + n * a.zstride : (const uint8_t *)p.s;
    return p;
}

// Raw block metadata of chunk c, loaded ahead of use and decoded by meta_decode_s once
// the loads have landed: per half, the scale bits and the zero-point byte (narrow
// loads), or (DW) the aligned dwords that hold them.
template <int H>
struct MetaS {
    uint32_t s[H];
    uint32_t z[H];
};

template <int FMT>
__device__ __forceinline__ int chunk_block(const KArgs &a, int c, int h) {
    if constexpr (FMT == FMT_U4 || FMT == FMT_NVFP4) return ((c << 5) + 16 * h) >> a.bs_shift;
    else return (c << 4) >> a.bs_shift;
}

// DW: each field comes as the aligned dword that holds it (the host takes this where
// the scale and zero-point rows are whole dwords on 4-byte aligned arrays, so no such
// dword reaches past its row). What a dword load returns is what the decode takes: a
// narrow load's value would need a zero-extension, which the compiler may place where
// the loop hands the next batch's registers over (its latch), and the wait that puts
// there for the batch just issued drains the prefetch.
template <int FMT, int H, bool DW = false>
__device__ __forceinline__ void meta_load_s(const KArgs &a, const ColPtrs &p, int c, MetaS<H> &m) {
    if constexpr (DW && FMT != FMT_FP8) {
        const uint32_t *S = (const uint32_t *)p.s;
        const uint32_t *Z = (const uint32_t *)p.z;
        if constexpr (FMT == FMT_U4) {
#pragma unroll
            for (int h = 0; h < H; ++h) {
                const int b = chunk_block<FMT>(a, c, h);
                m.s[h] = S[b >> 1];  // two fp16 scales per dword
                m.z[h] = Z[b >> 3];  // eight 4-bit zero points per dword
            }
        } else if constexpr (FMT == FMT_U8) {
            const int b = chunk_block<FMT>(a, c, 0);
            m.s[0] = S[b >> 1];
            m.z[0] = Z[b >> 2];  // four 8-bit zero points per dword
        } else {
            m.s[0] = S[c >> 1];  // the chunk's two E4M3 scale bytes: half c & 1 of the dword
            m.z[0] = 0u;
            if constexpr (H == 2) m.s[1] = 0u, m.z[1] = 0u;
        }
        return;
    }
    if constexpr (FMT == FMT_U4) {
#pragma unroll
        for (int h = 0; h < H; ++h) {
            const int b = chunk_block<FMT>(a, c, h);
            m.s[h] = ((const uint16_t *)p.s)[b];
            m.z[h] = p.z[b >> 1];
        }
    } else if constexpr (FMT == FMT_U8) {
        const int b = chunk_block<FMT>(a, c, 0);
        m.s[0] = ((const uint16_t *)p.s)[b];
        m.z[0] = p.z[b];
    } else if constexpr (FMT == FMT_FP8) {
        m.s[0] = ((const uint32_t *)p.s)[chunk_block<FMT>(a, c, 0)];
        m.z[0] = 0u;
    } else {
        const uint8_t *S = (const uint8_t *)p.s + 2 * c;  // the two E4M3 scales of the chunk
        m.s[0] = (uint32_t)S[0] | ((uint32_t)S[1] << 8);
        m.z[0] = 0u;
        if constexpr (H == 2) m.s[1] = 0u, m.z[1] = 0u;
    }
}

// 8-bit codes: the block metadata of one round of a column group (64 * UNR consecutive
// chunks per column) loaded as ONE dword per lane per column instead of two small
// loads per chunk: lane l holds dword l of the round's scale window and dword l of its
// zero-point window (clamped to the row's last dword, so lanes past a short window
// repeat it and nothing is read outside the row). A chunk's scale and zero-point bytes
// are then taken from the lane that holds them with one ds_bpermute each (a lane
// crossbar, no memory traffic): the very bytes meta_load_s reads. The host takes this
// path where a round's windows fit in 64 dwords and the rows are whole dwords on
// 4-byte aligned arrays.
struct MetaW {
    uint32_t s, z;
};

// Blocks of one round (UNR chunks of 16 k per lane), the dword its windows start at.
template <int UNR>
__device__ __forceinline__ int u8_round_blocks(const KArgs &a) {
    return (64 * UNR * 16) >> a.bs_shift;
}

template <int UNR>
__device__ __forceinline__ MetaW meta_window_load_u8(const KArgs &a, const ColPtrs &p, int round, int lane) {
    const int bpr = u8_round_blocks<UNR>(a);
    MetaW m;
    const int sd0 = (round * bpr) >> 1, slast = (a.nblk >> 1) - 1;  // fp16 scales: 2 per dword
    const int sd = sd0 + lane < slast ? sd0 + lane : slast;
    m.s = ((const uint32_t *)p.s)[sd];
    const int zd0 = (round * bpr) >> 2, zlast = (a.zstride >> 2) - 1;  // zero points: 4 per dword
    const int zd = zd0 + lane < zlast ? zd0 + lane : zlast;
    m.z = ((const uint32_t *)p.z)[zd];
    return m;
}

// The raw metadata (what meta_load_s loads) of local chunk lc = 64 u + lane of the
// round, from the round's window dwords.
template <int UNR>
__device__ __forceinline__ void meta_from_window_u8(const KArgs &a, const MetaW &w, int lc, MetaS<1> &m) {
    const int lb = (lc * 16) >> a.bs_shift;  // the chunk's block within the round
    const uint32_t sv = (uint32_t)__builtin_amdgcn_ds_bpermute((lb >> 1) << 2, (int)w.s);
    const uint32_t zv = (uint32_t)__builtin_amdgcn_ds_bpermute((lb >> 2) << 2, (int)w.z);
    m.s[0] = (sv >> ((lb & 1) << 4)) & 0xFFFFu;
    m.z[0] = (zv >> ((lb & 3) << 3)) & 0xFFu;
}

// Scale and integer zero point of each half of chunk c; zs is zsel(a.zp, midpoint
// byte) (0x88 for U4, 128 for U8), so a weight without zero points takes the midpoint.
// With DW, zs.fill holds the midpoint in every field of a dword (0x88888888 for U4,
// 0x80808080 for U8) and the fields are taken at their places in the loaded dwords.
template <int FMT, int H, bool DW = false>
__device__ __forceinline__ void meta_decode_s(const KArgs &a, int c, const MetaS<H> &m, ZSel zs, float sc[H],
                                              uint32_t zr[H]) {
    if constexpr (DW && FMT != FMT_FP8) {
        if constexpr (FMT == FMT_U4) {
#pragma unroll
            for (int h = 0; h < H; ++h) {
                const int b = chunk_block<FMT>(a, c, h);
                sc[h] = half_bits_to_float((uint16_t)(m.s[h] >> ((b & 1) << 4)));
                zr[h] = (((m.z[h] & zs.keep) | zs.fill) >> ((b & 7) << 2)) & 0x0Fu;
            }
        } else if constexpr (FMT == FMT_U8) {
            const int b = chunk_block<FMT>(a, c, 0);
            sc[0] = half_bits_to_float((uint16_t)(m.s[0] >> ((b & 1) << 4)));
            zr[0] = (((m.z[0] & zs.keep) | zs.fill) >> ((b & 3) << 3)) & 0xFFu;
        } else {
            const uint32_t s2 = m.s[0] >> ((c & 1) << 4);
            sc[0] = e4m3_to_float(s2 & 0xFFu);
            sc[1] = e4m3_to_float((s2 >> 8) & 0xFFu);
            zr[0] = zr[1] = 0u;
        }
        return;
    }
    if constexpr (FMT == FMT_U4) {
#pragma unroll
        for (int h = 0; h < H; ++h) {
            const int b = chunk_block<FMT>(a, c, h);
            sc[h] = half_bits_to_float((uint16_t)m.s[h]);
            const uint32_t zb = (m.z[h] & zs.keep) | zs.fill;
            zr[h] = (b & 1) ? ((zb >> 4) & 0x0Fu) : (zb & 0x0Fu);
        }
    } else if constexpr (FMT == FMT_U8) {
        sc[0] = half_bits_to_float((uint16_t)m.s[0]);
        zr[0] = ((m.z[0] & zs.keep) | zs.fill) & 0xFFu;
    } else if constexpr (FMT == FMT_FP8) {
        sc[0] = __builtin_bit_cast(float, m.s[0]);
        zr[0] = 0u;
    } else {
        sc[0] = e4m3_to_float(m.s[0] & 0xFFu);
        sc[1] = e4m3_to_float((m.s[0] >> 8) & 0xFFu);
        zr[0] = zr[1] = 0u;
    }
}

// The dword metadata of one lane's chunks, addressed the way the persistent streaming
// kernel walks them: chunk c = base + lane with base a multiple of 64 (uniform), so a
// block index splits into base * KPC / bs, a multiple of 8 (U4) or 4 (U8) blocks, plus
// the lane's own part, and the dword offsets within a round and the fields' bit
// positions are the lane's alone. Set once per kernel by meta_dw_lane; each load then
// takes the round's uniform offset (meta_dw_round) as its scalar offset.
template <int H>
struct MetaDW {
    uint32_t s_off[H], z_off[H];  // byte offsets of the lane's dwords within a round's window
    uint32_t s_sh[H], z_sh[H];    // bit positions of the fields in them
};

template <int FMT, int H>
__device__ __forceinline__ MetaDW<H> meta_dw_lane(const KArgs &a, int lane) {
    MetaDW<H> d;
#pragma unroll
    for (int h = 0; h < H; ++h) {
        if constexpr (FMT == FMT_NVFP4) {
            d.s_off[h] = (uint32_t)(lane >> 1) * 4u;  // the chunk's two E4M3 scale bytes
            d.s_sh[h] = (uint32_t)(lane & 1) << 4;
            d.z_off[h] = 0u;
            d.z_sh[h] = 0u;
        } else {
            const int bl = chunk_block<FMT>(a, lane, h);
            d.s_off[h] = (uint32_t)(bl >> 1) * 4u;
            d.s_sh[h] = (uint32_t)(bl & 1) << 4;
            d.z_off[h] = (uint32_t)(FMT == FMT_U4 ? (bl >> 3) : (bl >> 2)) * 4u;
            d.z_sh[h] = (uint32_t)(FMT == FMT_U4 ? (bl & 7) << 2 : (bl & 3) << 3);
        }
    }
    return d;
}

// The uniform byte offsets of the scale and zero-point dwords for the chunks base +
// lane (base a multiple of 64).
template <int FMT>
__device__ __forceinline__ void meta_dw_round(const KArgs &a, int base, uint32_t &s_off, uint32_t &z_off) {
    if constexpr (FMT == FMT_NVFP4) {
        s_off = (uint32_t)(base >> 1) * 4u;
        z_off = 0u;
    } else {
        const int bu = chunk_block<FMT>(a, base, 0);
        s_off = (uint32_t)(bu >> 1) * 4u;
        z_off = (uint32_t)(FMT == FMT_U4 ? (bu >> 3) : (bu >> 2)) * 4u;
    }
}

// Decode of dword metadata at the lane's bit positions (what meta_decode_s<.., true>
// takes from the chunk index); zs.fill holds the midpoint in every field.
template <int FMT, int H>
__device__ __forceinline__ void meta_decode_dw(const MetaS<H> &m, const MetaDW<H> &d, ZSel zs, float sc[H],
                                               uint32_t zr[H]) {
    if constexpr (FMT == FMT_NVFP4) {
        const uint32_t s2 = m.s[0] >> d.s_sh[0];
        sc[0] = e4m3_to_float(s2 & 0xFFu);
        sc[1] = e4m3_to_float((s2 >> 8) & 0xFFu);
        zr[0] = zr[1] = 0u;
    } else {
#pragma unroll
        for (int h = 0; h < H; ++h) {
            sc[h] = half_bits_to_float((uint16_t)(m.s[h] >> d.s_sh[h]));
            zr[h] = (((m.z[h] & zs.keep) | zs.fill) >> d.z_sh[h]) & (FMT == FMT_U4 ? 0x0Fu : 0xFFu);
        }
    }
}

// Scale and integer zero point of each of the H halves of chunk c, loaded and decoded.
template <int FMT, int H>
__device__ __forceinline__ void chunk_meta(const KArgs &a, const ColPtrs &p, int c, float sc[H], uint32_t zr[H]) {
    MetaS<H> m;
    meta_load_s<FMT, H>(a, p, c, m);
    meta_decode_s<FMT, H>(a, c, m, zsel(a.zp, FMT == FMT_U4 ? 0x88u : 128u), sc, zr);
}

}  // namespace qgemv
