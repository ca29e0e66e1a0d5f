// Per-format work on one 16-byte chunk of a column's codes (vector family).
//
// A chunk is split into "halves" of 16 consecutive k, each of which lies inside a
// single scale block (block sizes are multiples of 16). U4 and NVFP4 chunks carry
// 32 codes (two halves), U8 and FP8 chunks 16 codes (one half).
//
// Per half the weight codes are decoded exactly into fp16/bf16 pairs and multiplied
// into an fp32 sum with v_dot2; the block scale is applied to that sum, and for the
// integer formats the zero point enters as -z * sum(a) over the same 16 k:
//     s * sum_k a_k (q_k - z) = s * (sum_k a_k q_k - z * sum_k a_k)
// ("[CUDA] MatMulNBits 8-bit: wide fp16 M=1 kernel", Description: the scale is
// applied once per chunk to an fp32 partial; "[CUDA] Block-scaled MatMul decode
// GEMV", FP4 row-tiling paragraph: decode and scales shared across the rows of a tile).
//
// The activation side of a half (permuted pairs and sum(a)) is prepared once per
// row and reused for every column the wave owns.
#pragma once

#include "qgemv_device.h"

namespace qgemv {

// Activation words of one half for one row: 8 dwords (16 values) in the order the
// format's decode pairs them, plus their sum.
struct HalfAct {
    uint32_t p[8];
    float asum;
};

template <int FMT, int ACT>
struct ChunkOps;

// Raw activation load of one half (16 values, 32 bytes) of row m at k = k0.
__device__ __forceinline__ void load_act_half(const KArgs &a, int m, int64_t k0, uint32_t x[8]) {
    const uint16_t *A = (const uint16_t *)a.A + (int64_t)m * a.K + k0;
    u4v v0 = load16(A);
    u4v v1 = load16(A + 8);
    x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
    x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
}

template <int ACT>
__device__ __forceinline__ float sum_pairs(const uint32_t x[8]) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = dot2<ACT>(x[i], ones2<ACT>(), s);
    return s;
}

// ----------------------------------------------------------------------------------
// U4, fp16 activations. Codes become fp16 subnormals: nibble at bits 0..3 of a half
// -> q * 2^-24, nibble at bits 4..7 -> q * 2^-20 (kept in a second sum, weighted 1/16
// against the first before both return to units of 1).
template <>
struct ChunkOps<FMT_U4, ACT_F16> {
    static constexpr int HALVES = 2;
    static constexpr int KPC = 32;

    // x: activations k0..k0+15 of one half as natural pairs (a0,a1),(a2,a3),...
    // For weight dword d (codes k = 8d..8d+7) the decode yields pairs (k0,k4),
    // (k2,k6) [low nibbles] and (k1,k5), (k3,k7) [high nibbles].
    __device__ static void prep(const uint32_t x[8], HalfAct &h) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint32_t x0 = x[4 * d], x1 = x[4 * d + 1], x2 = x[4 * d + 2], x3 = x[4 * d + 3];
            h.p[4 * d + 0] = perm(x2, x0, 0x05040100u);  // (a0, a4)
            h.p[4 * d + 1] = perm(x3, x1, 0x05040100u);  // (a2, a6)
            h.p[4 * d + 2] = perm(x2, x0, 0x07060302u);  // (a1, a5)
            h.p[4 * d + 3] = perm(x3, x1, 0x07060302u);  // (a3, a7)
        }
        h.asum = sum_pairs<ACT_F16>(x);
    }

    // sum_k a_k q_k over the half (2 code dwords).
    __device__ static float dot(const uint32_t w[2], const HalfAct &h) {
        float lo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint32_t wv = w[d], w8 = w[d] >> 8;
            lo = dot2<ACT_F16>(wv & 0x000F000Fu, h.p[4 * d + 0], lo);
            lo = dot2<ACT_F16>(w8 & 0x000F000Fu, h.p[4 * d + 1], lo);
            hi = dot2<ACT_F16>(wv & 0x00F000F0u, h.p[4 * d + 2], hi);
            hi = dot2<ACT_F16>(w8 & 0x00F000F0u, h.p[4 * d + 3], hi);
        }
        return __builtin_fmaf(hi, 0.0625f, lo) * 16777216.0f;  // back from units of 2^-24
    }
};

// U4, bf16 activations. Each nibble is moved into its own byte and widened with the
// E4M3 converter (codes 0..15 of E4M3 are q*2^-9; the converter's 2^9 scale gives q).
template <>
struct ChunkOps<FMT_U4, ACT_BF16> {
    static constexpr int HALVES = 2;
    static constexpr int KPC = 32;

    // decode yields (k0,k2), (k4,k6) from the low nibbles and (k1,k3), (k5,k7) from the high.
    __device__ static void prep(const uint32_t x[8], HalfAct &h) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint32_t x0 = x[4 * d], x1 = x[4 * d + 1], x2 = x[4 * d + 2], x3 = x[4 * d + 3];
            h.p[4 * d + 0] = perm(x1, x0, 0x05040100u);  // (a0, a2)
            h.p[4 * d + 1] = perm(x3, x2, 0x05040100u);  // (a4, a6)
            h.p[4 * d + 2] = perm(x1, x0, 0x07060302u);  // (a1, a3)
            h.p[4 * d + 3] = perm(x3, x2, 0x07060302u);  // (a5, a7)
        }
        h.asum = sum_pairs<ACT_BF16>(x);
    }

    __device__ static float dot(const uint32_t w[2], const HalfAct &h) {
        float s = 0.0f;
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint32_t lo = w[d] & 0x0F0F0F0Fu, hi = (w[d] >> 4) & 0x0F0F0F0Fu;
            s = dot2<ACT_BF16>(small_int_bf16_pair<false>(lo), h.p[4 * d + 0], s);
            s = dot2<ACT_BF16>(small_int_bf16_pair<true>(lo), h.p[4 * d + 1], s);
            s = dot2<ACT_BF16>(small_int_bf16_pair<false>(hi), h.p[4 * d + 2], s);
            s = dot2<ACT_BF16>(small_int_bf16_pair<true>(hi), h.p[4 * d + 3], s);
        }
        return s;
    }
};

// U8, fp16 activations: bytes become fp16 subnormals q*2^-24 with one byte permute
// per pair; pairs keep the natural k order.
template <>
struct ChunkOps<FMT_U8, ACT_F16> {
    static constexpr int HALVES = 1;
    static constexpr int KPC = 16;

    __device__ static void prep(const uint32_t x[8], HalfAct &h) {
#pragma unroll
        for (int i = 0; i < 8; ++i) h.p[i] = x[i];
        h.asum = sum_pairs<ACT_F16>(x);
    }

    __device__ static float dot(const uint32_t w[4], const HalfAct &h) {
        float s = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            s = dot2<ACT_F16>(perm(0u, w[d], 0x0C010C00u), h.p[2 * d], s);
            s = dot2<ACT_F16>(perm(0u, w[d], 0x0C030C02u), h.p[2 * d + 1], s);
        }
        return s * 16777216.0f;
    }
};

// U8, bf16 activations: bytes widened to fp32 and multiplied in fp32.
template <>
struct ChunkOps<FMT_U8, ACT_BF16> {
    static constexpr int HALVES = 1;
    static constexpr int KPC = 16;

    __device__ static void prep(const uint32_t x[8], HalfAct &h) {
#pragma unroll
        for (int i = 0; i < 8; ++i) h.p[i] = x[i];
        h.asum = sum_pairs<ACT_BF16>(x);
    }

    __device__ static float dot(const uint32_t w[4], const HalfAct &h) {
        float s = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const float a0 = __builtin_bit_cast(float, h.p[2 * d] << 16);
            const float a1 = __builtin_bit_cast(float, h.p[2 * d] & 0xFFFF0000u);
            const float a2 = __builtin_bit_cast(float, h.p[2 * d + 1] << 16);
            const float a3 = __builtin_bit_cast(float, h.p[2 * d + 1] & 0xFFFF0000u);
            s = __builtin_fmaf(a0, (float)(w[d] & 0xFFu), s);
            s = __builtin_fmaf(a1, (float)((w[d] >> 8) & 0xFFu), s);
            s = __builtin_fmaf(a2, (float)((w[d] >> 16) & 0xFFu), s);
            s = __builtin_fmaf(a3, (float)(w[d] >> 24), s);
        }
        return s;
    }
};

// FP8 (E4M3FN): hardware widening to fp16/bf16, natural pairs.
template <int ACT>
struct Fp8Ops {
    static constexpr int HALVES = 1;
    static constexpr int KPC = 16;

    __device__ static void prep(const uint32_t x[8], HalfAct &h) {
#pragma unroll
        for (int i = 0; i < 8; ++i) h.p[i] = x[i];
        h.asum = 0.0f;
    }

    __device__ static float dot(const uint32_t w[4], const HalfAct &h) {
        float s = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            s = dot2<ACT>(fp8_pair<ACT, false>(w[d]), h.p[2 * d], s);
            s = dot2<ACT>(fp8_pair<ACT, true>(w[d]), h.p[2 * d + 1], s);
        }
        return s;
    }
};
template <> struct ChunkOps<FMT_FP8, ACT_F16> : Fp8Ops<ACT_F16> {};
template <> struct ChunkOps<FMT_FP8, ACT_BF16> : Fp8Ops<ACT_BF16> {};

// NVFP4: hardware E2M1 widening, natural pairs; the E4M3 block scale multiplies the
// fp32 half sum.
template <int ACT>
struct Fp4Ops {
    static constexpr int HALVES = 2;
    static constexpr int KPC = 32;

    __device__ static void prep(const uint32_t x[8], HalfAct &h) {
#pragma unroll
        for (int i = 0; i < 8; ++i) h.p[i] = x[i];
        h.asum = 0.0f;
    }

    __device__ static float dot(const uint32_t w[2], const HalfAct &h) {
        float s = 0.0f;
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            s = dot2<ACT>(fp4_pair<ACT, 0>(w[d]), h.p[4 * d + 0], s);
            s = dot2<ACT>(fp4_pair<ACT, 1>(w[d]), h.p[4 * d + 1], s);
            s = dot2<ACT>(fp4_pair<ACT, 2>(w[d]), h.p[4 * d + 2], s);
            s = dot2<ACT>(fp4_pair<ACT, 3>(w[d]), h.p[4 * d + 3], s);
        }
        return s;
    }
};
template <> struct ChunkOps<FMT_NVFP4, ACT_F16> : Fp4Ops<ACT_F16> {};
template <> struct ChunkOps<FMT_NVFP4, ACT_BF16> : Fp4Ops<ACT_BF16> {};

// ----------------------------------------------------------------------------------
// Block metadata of one half of one column: scale and zero point.
struct HalfMeta {
    float scale;
    float zero;
};

// Chunk c of column n: halves cover k = c*KPC + 16*h .. +15.
template <int FMT>
__device__ __forceinline__ void load_meta(const KArgs &a, int64_t n, int64_t c, HalfMeta m[2]) {
    if constexpr (FMT == FMT_U4) {
        const uint16_t *S = (const uint16_t *)a.scales + n * a.nblk;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t b = (c * 32 + 16 * h) / a.bs;
            m[h].scale = half_bits_to_float(S[b]);
            int z = 8;
            if (a.zp) {
                const uint8_t zb = a.zp[n * a.zstride + (b >> 1)];
                z = (b & 1) ? (zb >> 4) : (zb & 0x0F);
            }
            m[h].zero = (float)z;
        }
    } else if constexpr (FMT == FMT_U8) {
        const int64_t b = (c * 16) / a.bs;
        m[0].scale = half_bits_to_float(((const uint16_t *)a.scales)[n * a.nblk + b]);
        m[0].zero = a.zp ? (float)a.zp[n * a.nblk + b] : 128.0f;
    } else if constexpr (FMT == FMT_FP8) {
        const int64_t b = (c * 16) / a.bs;
        m[0].scale = ((const float *)a.scales)[n * a.nblk + b];
        m[0].zero = 0.0f;
    } else {
        const uint8_t *S = (const uint8_t *)a.scales + n * (a.K / 16) + 2 * c;
        m[0].scale = e4m3_to_float(S[0]);
        m[1].scale = e4m3_to_float(S[1]);
        m[0].zero = m[1].zero = 0.0f;
    }
}

}  // namespace qgemv
