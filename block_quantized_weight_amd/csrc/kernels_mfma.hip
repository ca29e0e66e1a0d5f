// Matrix-core (MFMA) family of qgemv for gfx950.
//
// The multiply runs on v_mfma_f32_16x16x32_{f16,bf16} with the decoded weight in the
// B operand (16 output columns n) and the activations in the A operand, as the pages
// put the weight in one mma slot and the activation in the other so that both
// fragments keep the tensors' natural layouts ("[CUDA] Block-scaled MatMul decode
// GEMV", FP8 and FP4 mma paragraphs). Differences for CDNA4:
//
//  - Block-diagonal row groups. Lane group g (lanes 16g..16g+15) of a wave loads the
//    16-byte chunk c = 4t + g of each of the 16 columns of a tile. In the A operand,
//    rows 4g..4g+3 of the MFMA carry four rows of activations over exactly the k of
//    chunk 4t + g and are zero elsewhere, so output rows 4g..4g+3 accumulate that one
//    chunk only. The output lands in lane (n, g), the lane that loaded the chunk's
//    block scale, so every per-block epilogue is a few fp32 FMAs in the lane that
//    already holds the scale; no cross-lane traffic, and the MFMA never sums across
//    two scale blocks (the reason the pages fold the NVFP4 scale into the weight).
//  - Rows of A travel in groups of four. M rows take ceil(M/4) groups, each with the
//    same arithmetic, so a row's result never depends on M or on its group.
//  - Zero points: codes enter the MFMA as M0 + q (an exact fp16/bf16 integer built
//    with two bit operations) and sum(a) over the chunk comes from one more MFMA
//    against a ones operand; the epilogue forms s * (D - (M0 + z) * sum(a)).
//  - K split: ksplit waves of a workgroup take strided K steps of the same column
//    tile and reduce through LDS in fixed wave order ("[CUDA] Block-scaled MatMul
//    decode GEMV", FP8 mma paragraph: KSplit warps per block reduce through shared
//    memory; "[CUDA] MatMul: add an opt-in split-K GEMV", deterministic slice order).
//  - Latency: each wave keeps the next P K steps of weights and block metadata in
//    flight in a register ring while it computes the current one; a workgroup of 8-16
//    waves walks tile groups persistently, and when the activations fit they are
//    staged once per workgroup in LDS, already in the MFMA slot order.
#include "launch.h"
#include "qgemv_device.h"

namespace qgemv {

namespace {

// 8 fp16/bf16 operand values of one lane.
typedef uint32_t op4 __attribute__((ext_vector_type(4)));

template <int ACT>
__device__ __forceinline__ f4 mfma(op4 a, op4 b, f4 c) {
    if constexpr (ACT == ACT_F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c, 0, 0, 0);
}

// Integer offset carried by 4-bit codes in the MFMA: fp16 0x6400|q = 1024 + q,
// bf16 0x4300|q = 128 + q.
template <int ACT> struct U4Magic;
template <> struct U4Magic<ACT_F16> { static constexpr uint32_t bits = 0x64006400u; static constexpr float off = 1024.0f; };
template <> struct U4Magic<ACT_BF16> { static constexpr uint32_t bits = 0x43004300u; static constexpr float off = 128.0f; };

// Per-format description of one 16-byte chunk in the MFMA family.
//   MF   : MFMAs per chunk (8 k per lane each)
//   EPI  : epilogues per chunk (one per scale block the chunk touches)
//   PERM : activations need the U4 slot order [0,4,1,5,2,6,3,7] within each 8
template <int FMT> struct MfFmt;
template <> struct MfFmt<FMT_U4> { static constexpr int KPC = 32, MF = 4, PERM = 1, ZP = 1; };
template <> struct MfFmt<FMT_U8> { static constexpr int KPC = 16, MF = 2, PERM = 0, ZP = 1; };
template <> struct MfFmt<FMT_FP8> { static constexpr int KPC = 16, MF = 2, PERM = 0, ZP = 0; };
template <> struct MfFmt<FMT_NVFP4> { static constexpr int KPC = 32, MF = 4, PERM = 0, ZP = 0; };

// B operand (8 weight values) of MFMA j from the chunk's 4 code dwords.
template <int FMT, int ACT, int J>
__device__ __forceinline__ op4 decode_b(const u4v &w) {
    op4 r;
    if constexpr (FMT == FMT_U4) {
        // dword J holds k = 8J..8J+7: slots (k0,k4),(k1,k5),(k2,k6),(k3,k7)
        const uint32_t x = w[J];
        constexpr uint32_t M = U4Magic<ACT>::bits;
        r.x = (x & 0x000F000Fu) | M;
        r.y = ((x >> 4) & 0x000F000Fu) | M;
        r.z = ((x >> 8) & 0x000F000Fu) | M;
        r.w = ((x >> 12) & 0x000F000Fu) | M;
    } else if constexpr (FMT == FMT_U8) {
        // dwords 2J, 2J+1 hold k = 8J..8J+7 in natural order; (1024 + q) as fp16
        constexpr uint32_t MB = 0x64646464u;
        const uint32_t x0 = w[2 * J], x1 = w[2 * J + 1];
        r.x = perm(MB, x0, 0x04010400u);
        r.y = perm(MB, x0, 0x04030402u);
        r.z = perm(MB, x1, 0x04010400u);
        r.w = perm(MB, x1, 0x04030402u);
    } else if constexpr (FMT == FMT_FP8) {
        const uint32_t x0 = w[2 * J], x1 = w[2 * J + 1];
        r.x = fp8_pair<ACT, false>(x0);
        r.y = fp8_pair<ACT, true>(x0);
        r.z = fp8_pair<ACT, false>(x1);
        r.w = fp8_pair<ACT, true>(x1);
    } else {
        const uint32_t x = w[J];
        r.x = fp4_pair<ACT, 0>(x);
        r.y = fp4_pair<ACT, 1>(x);
        r.z = fp4_pair<ACT, 2>(x);
        r.w = fp4_pair<ACT, 3>(x);
    }
    return r;
}

// A operand of MFMA j for row group rg: lane (i, gs) with i>>2 == gs holds row
// 4*rg + (i&3) over the 8 k the weights of chunk 4t+gs use in MFMA j; zero elsewhere.
template <int FMT>
__device__ __forceinline__ op4 load_a(const uint16_t *arow, bool live, uint32_t k0) {
    op4 r = {0u, 0u, 0u, 0u};
    if (live) {
        const u4v v = load16(arow + k0);
        if constexpr (MfFmt<FMT>::PERM) {
            r.x = perm(v.z, v.x, 0x05040100u);  // (a0, a4)
            r.y = perm(v.z, v.x, 0x07060302u);  // (a1, a5)
            r.z = perm(v.w, v.y, 0x05040100u);  // (a2, a6)
            r.w = perm(v.w, v.y, 0x07060302u);  // (a3, a7)
        } else {
            r.x = v.x; r.y = v.y; r.z = v.z; r.w = v.w;
        }
    }
    return r;
}

// Block metadata of one chunk kept raw (one or two dwords) while it waits in the
// prefetch ring, decoded only when the chunk is consumed.
//   U4, one block per chunk : fp16 scale bits | zero-point nibble << 16
//   U4, two blocks per chunk: both fp16 scales | the zero-point byte of the pair
//   U8                      : fp16 scale bits | zero-point byte << 16
//   FP8                     : fp32 scale bits
//   NVFP4                   : the two E4M3 scale bytes
template <int H>
struct MetaRaw {
    uint32_t v[H];
};

struct MfCol {
    const uint8_t *w;
    const void *s;
    const uint8_t *z;
};

template <int FMT>
__device__ __forceinline__ MfCol mf_col(const KArgs &a, int64_t n) {
    MfCol p;
    p.w = a.W + n * a.col_bytes;
    if constexpr (FMT == FMT_NVFP4) p.s = (const uint8_t *)a.scales + n * (a.K >> 4);
    else if constexpr (FMT == FMT_FP8) p.s = (const float *)a.scales + n * a.nblk;
    else p.s = (const uint16_t *)a.scales + n * a.nblk;
    p.z = a.zp ? a.zp + n * a.zstride : nullptr;
    return p;
}

template <int FMT, int H>
__device__ __forceinline__ MetaRaw<H> load_meta_raw(const KArgs &a, const MfCol &p, int c) {
    MetaRaw<H> m;
    if constexpr (FMT == FMT_U4) {
        if constexpr (H == 1) {
            const int b = (c << 5) >> a.bs_shift;
            uint32_t z = 8u;
            if (p.z) {
                const uint32_t zb = p.z[b >> 1];
                z = (b & 1) ? (zb >> 4) : (zb & 0x0Fu);
            }
            m.v[0] = (uint32_t)((const uint16_t *)p.s)[b] | (z << 16);
        } else {
            // 16-wide blocks: blocks 2c and 2c+1, adjacent scales, one zero-point byte
            m.v[0] = *(const uint32_t *)((const uint16_t *)p.s + 2 * c);
            m.v[1] = p.z ? (uint32_t)p.z[c] : 0x88u;
        }
    } else if constexpr (FMT == FMT_U8) {
        const int b = (c << 4) >> a.bs_shift;
        m.v[0] = (uint32_t)((const uint16_t *)p.s)[b] | ((p.z ? (uint32_t)p.z[b] : 128u) << 16);
    } else if constexpr (FMT == FMT_FP8) {
        m.v[0] = ((const uint32_t *)p.s)[(c << 4) >> a.bs_shift];
    } else {
        m.v[0] = (uint32_t)*(const uint16_t *)((const uint8_t *)p.s + 2 * c);
    }
    return m;
}

// Scale and (M0 + zero point) of half h from the raw metadata.
template <int FMT, int ACT, int H>
__device__ __forceinline__ void meta_decode(const MetaRaw<H> &m, int h, float &s, float &zoff) {
    if constexpr (FMT == FMT_U4) {
        if constexpr (H == 1) {
            s = half_bits_to_float((uint16_t)(m.v[0] & 0xFFFFu));
            zoff = U4Magic<ACT>::off + (float)(m.v[0] >> 16);
        } else {
            s = half_bits_to_float((uint16_t)(h ? (m.v[0] >> 16) : (m.v[0] & 0xFFFFu)));
            zoff = U4Magic<ACT>::off + (float)(h ? (m.v[1] >> 4) : (m.v[1] & 0x0Fu));
        }
    } else if constexpr (FMT == FMT_U8) {
        s = half_bits_to_float((uint16_t)(m.v[0] & 0xFFFFu));
        zoff = 1024.0f + (float)(m.v[0] >> 16);
    } else if constexpr (FMT == FMT_FP8) {
        s = __builtin_bit_cast(float, m.v[0]);
        zoff = 0.0f;
    } else {
        s = e4m3_to_float(h ? (m.v[0] >> 8) : (m.v[0] & 0xFFu));
        zoff = 0.0f;
    }
}

// Block metadata through the DMA ring: the aligned dword(s) holding a chunk's scale
// (and zero point) are copied to LDS next to the chunk's codes, then unpacked into
// the same raw form as load_meta_raw. The dispatcher only takes this path when the
// scale and zero-point arrays are 4-byte aligned and whole dwords long, so every
// dword read lies inside them.
template <int FMT, bool ZPP>
struct MetaDma {
    static constexpr int NM = ((FMT == FMT_U4 || FMT == FMT_U8) && ZPP) ? 2 : 1;
};

__device__ __forceinline__ const uint32_t *dword_of(const void *p) {
    return (const uint32_t *)((uintptr_t)p & ~(uintptr_t)3);
}

__device__ __forceinline__ uint32_t byte_shift(const void *p) { return 8u * (uint32_t)((uintptr_t)p & 3); }

template <int FMT, int H, bool ZPP>
__device__ __forceinline__ void meta_dma(const KArgs &a, const MfCol &p, int c, uint32_t *meta0, uint32_t *meta1) {
    const int lane = threadIdx.x & 63;
    if constexpr (FMT == FMT_U4) {
        if constexpr (H == 1) {
            const int b = (c << 5) >> a.bs_shift;
            dma_to_lds<4>(dword_of((const uint16_t *)p.s + b), meta0);
            if constexpr (ZPP) dma_to_lds<4>(dword_of(p.z + (b >> 1)), meta1);
        } else {
            dma_to_lds<4>((const uint16_t *)p.s + 2 * c, meta0);
            if constexpr (ZPP) dma_to_lds<4>(dword_of(p.z + c), meta1);
        }
    } else if constexpr (FMT == FMT_U8) {
        const int b = (c << 4) >> a.bs_shift;
        dma_to_lds<4>(dword_of((const uint16_t *)p.s + b), meta0);
        if constexpr (ZPP) dma_to_lds<4>(dword_of(p.z + b), meta1);
    } else if constexpr (FMT == FMT_FP8) {
        dma_to_lds<4>((const uint32_t *)p.s + ((c << 4) >> a.bs_shift), meta0);
    } else {
        dma_to_lds<4>(dword_of((const uint8_t *)p.s + 2 * c), meta0);
    }
    (void)lane;
}

template <int FMT, int H, bool ZPP>
__device__ __forceinline__ MetaRaw<H> meta_from_lds(const KArgs &a, const MfCol &p, int c, const uint32_t *meta0,
                                                    const uint32_t *meta1) {
    const int lane = threadIdx.x & 63;
    MetaRaw<H> m;
    if constexpr (FMT == FMT_U4) {
        if constexpr (H == 1) {
            const int b = (c << 5) >> a.bs_shift;
            const uint16_t *sp = (const uint16_t *)p.s + b;
            const uint32_t sbits = (meta0[lane] >> byte_shift(sp)) & 0xFFFFu;
            uint32_t z = 8u;
            if constexpr (ZPP) {
                const uint32_t zb = (meta1[lane] >> byte_shift(p.z + (b >> 1))) & 0xFFu;
                z = (b & 1) ? (zb >> 4) : (zb & 0x0Fu);
            }
            m.v[0] = sbits | (z << 16);
        } else {
            m.v[0] = meta0[lane];
            m.v[1] = ZPP ? ((meta1[lane] >> byte_shift(p.z + c)) & 0xFFu) : 0x88u;
        }
    } else if constexpr (FMT == FMT_U8) {
        const int b = (c << 4) >> a.bs_shift;
        const uint32_t sbits = (meta0[lane] >> byte_shift((const uint16_t *)p.s + b)) & 0xFFFFu;
        const uint32_t z = ZPP ? ((meta1[lane] >> byte_shift(p.z + b)) & 0xFFu) : 128u;
        m.v[0] = sbits | (z << 16);
    } else if constexpr (FMT == FMT_FP8) {
        m.v[0] = meta0[lane];
    } else {
        m.v[0] = (meta0[lane] >> byte_shift((const uint8_t *)p.s + 2 * c)) & 0xFFFFu;
    }
    return m;
}

// Sum over the four lane groups (lanes n, n+16, n+32, n+48); every lane gets the
// total, added in the same order in every lane. (ds_bpermute through __shfl_xor: the
// permlane swap builtins given one value for both operands are folded wrongly by this
// compiler, which adds one half to itself.)
__device__ __forceinline__ float sum_groups(float v) {
    const float v2 = v + __shfl_xor(v, 32, 64);
    return v2 + __shfl_xor(v2, 16, 64);
}

}  // namespace

// Padding of a staged activation row in LDS (elements): shifts consecutive rows by
// 16 bytes so the 16 live lanes of an A-operand read hit distinct banks.
constexpr int kAPad = 8;

// One wave owns the 16 columns of a tile for one K slice. A workgroup of nw waves
// holds nw / ksplit tiles; the ksplit waves of a tile take K steps t = kslice,
// kslice + ksplit, ... and reduce in LDS in wave order.
// One K step of one wave: the chunk c = 4t + g of each of the 16 columns (already in
// w, with its raw block metadata m), multiplied by every row group of A. Shared by
// both kernels below so that they compute bit-identical results.
template <int FMT, int ACT, int RG, int H, bool LDSA>
__device__ __forceinline__ void mfma_step(const KArgs &a, const u4v &w, const MetaRaw<H> &m, int c, int ar,
                                          bool a_live_grp, const uint16_t *sA, const uint16_t *sZero, int astride,
                                          f4 acc[RG]) {
    using F = MfFmt<FMT>;
    constexpr uint32_t ONE = (ACT == ACT_F16) ? 0x3C003C00u : 0x3F803F80u;
    const op4 ones = {ONE, ONE, ONE, ONE};
    const uint16_t *A16 = (const uint16_t *)a.A;
    // with one row group the B operands are decoded right before their MFMA; with
    // more they are decoded once and shared by the groups
    op4 bv[RG == 1 ? 1 : F::MF];
    if constexpr (RG > 1) {
        bv[0] = decode_b<FMT, ACT, 0>(w);
        bv[1] = decode_b<FMT, ACT, 1>(w);
        if constexpr (F::MF == 4) {
            bv[2] = decode_b<FMT, ACT, 2>(w);
            bv[3] = decode_b<FMT, ACT, 3>(w);
        }
    }
    const uint32_t kbase = (uint32_t)c * F::KPC;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int row = 4 * rg + ar;
        const bool live = a_live_grp && row < a.M;
        f4 d[H], sa[H];
#pragma unroll
        for (int h = 0; h < H; ++h) d[h] = sa[h] = f4{0.f, 0.f, 0.f, 0.f};
        // staged activations: every lane reads (lanes outside the block diagonal read
        // a 16-byte zero block), so the MF reads issue back to back without predication
        op4 avs[F::MF];
        if constexpr (LDSA) {
            const uint16_t *abase = live ? sA + row * astride + kbase : sZero;
            const int jstride = live ? 8 : 0;
#pragma unroll
            for (int j = 0; j < F::MF; ++j) avs[j] = *(const op4 *)(abase + jstride * j);
        }
#pragma unroll
        for (int j = 0; j < F::MF; ++j) {
            op4 av;
            if constexpr (LDSA) {
                av = avs[j];
            } else {
                av = load_a<FMT>(A16 + (int64_t)(live ? row : 0) * a.K, live, kbase + 8 * j);
            }
            const int h = (H == 2) ? (j / (F::MF / 2)) : 0;
            op4 b;
            if constexpr (RG == 1) {
                if (j == 0) b = decode_b<FMT, ACT, 0>(w);
                else if (j == 1) b = decode_b<FMT, ACT, 1>(w);
                else if (j == 2) b = decode_b<FMT, ACT, (F::MF == 4 ? 2 : 0)>(w);
                else b = decode_b<FMT, ACT, (F::MF == 4 ? 3 : 0)>(w);
            } else {
                b = bv[j];
            }
            d[h] = mfma<ACT>(av, b, d[h]);
            if constexpr (F::ZP) sa[h] = mfma<ACT>(av, ones, sa[h]);
        }
#pragma unroll
        for (int h = 0; h < H; ++h) {
            float sc, zoff;
            meta_decode<FMT, ACT, H>(m, h, sc, zoff);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = d[h][r];
                if constexpr (F::ZP) v = __builtin_fmaf(-zoff, sa[h][r], v);
                acc[rg][r] = __builtin_fmaf(sc, v, acc[rg][r]);
            }
        }
    }
}

// Stage the M activation rows into LDS once per workgroup, permuted into the MFMA
// slot order (row stride K + kAPad elements).
template <int FMT>
__device__ __forceinline__ void stage_a(const KArgs &a, uint16_t *sA, int astride) {
    using F = MfFmt<FMT>;
    const uint16_t *A16 = (const uint16_t *)a.A;
    const int K = (int)a.K;
    const int items = a.M * (K >> 3);
    for (int it = threadIdx.x; it < items; it += blockDim.x) {
        const int m = it / (K >> 3);
        const int k8 = (it - m * (K >> 3)) << 3;
        const u4v v = load16(A16 + (int64_t)m * K + k8);
        u4v o;
        if constexpr (F::PERM) {
            o.x = perm(v.z, v.x, 0x05040100u);  // (a0, a4)
            o.y = perm(v.z, v.x, 0x07060302u);  // (a1, a5)
            o.z = perm(v.w, v.y, 0x05040100u);  // (a2, a6)
            o.w = perm(v.w, v.y, 0x07060302u);  // (a3, a7)
        } else {
            o = v;
        }
        *(u4v *)(sA + m * astride + k8) = o;
    }
}

// K-split reduction over the ksplit waves of a tile (fixed wave order), then the sum
// over the four lane groups and the store of rows 4*rg + g.
template <int ACT, int RG>
__device__ __forceinline__ void finish_tile(const KArgs &a, f4 acc[RG], float *sR, int wave, int lane, int ks,
                                            int kslice, int g, bool tile_ok, int64_t n) {
    if (ks > 1) {
        float *mine = sR + (size_t)wave * (RG * 4 * 64);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int r = 0; r < 4; ++r) mine[(rg * 4 + r) * 64 + lane] = acc[rg][r];
        __syncthreads();
        if (kslice == 0) {
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float sum = mine[(rg * 4 + r) * 64 + lane];
                    for (int w2 = 1; w2 < ks; ++w2) sum += mine[(size_t)w2 * (RG * 4 * 64) + (rg * 4 + r) * 64 + lane];
                    acc[rg][r] = sum;
                }
        }
        __syncthreads();
    }
    if (kslice == 0 && tile_ok) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            float tot[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) tot[r] = sum_groups(acc[rg][r]);
            const float v = (g == 0) ? tot[0] : (g == 1) ? tot[1] : (g == 2) ? tot[2] : tot[3];
            const int row = 4 * rg + g;
            if (n < a.N && row < a.M) store_out<ACT>(a.Y, (int64_t)row * a.N + n, v * a.tscale);
        }
    }
}

// Register budget: four waves per SIMD (<= 128 VGPRs) for one row group, two waves
// per SIMD (<= 256) beyond. A 16-wave workgroup needs four waves per SIMD whatever the
// bound says, so the automatic K split stays at 8 waves or fewer.
template <int FMT, int ACT, int RG, int H, bool LDSA, int P, int NW>
__global__ void __launch_bounds__(64 * NW, (RG == 1 ? 4 : 2)) k_mfma(KArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int ks = a.ksplit;
    const int tpw = NW / ks;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
    const int lane = threadIdx.x & 63;
    const int slot = wave / ks;
    const int kslice = wave - slot * ks;
    const int g = lane >> 4;
    const int ar = lane & 3;
    const bool a_live_grp = ((lane & 15) >> 2) == g;
    const int nsteps = (int)(a.nchunks >> 2);
    const int astride = (int)a.K + kAPad;
    const int64_t ntiles = (a.N + 15) >> 4;
    const int64_t ngroups = (ntiles + tpw - 1) / tpw;
    uint16_t *sZero = (uint16_t *)smem;
    uint16_t *sA = (uint16_t *)(smem + 16);
    float *sR = (float *)(smem + 16 + (LDSA ? (((size_t)a.M * astride * 2 + 15) & ~(size_t)15) : 0));

    if constexpr (LDSA) {
        if (threadIdx.x == 0) *(u4v *)sZero = u4v{0u, 0u, 0u, 0u};
        stage_a<FMT>(a, sA, astride);
        __syncthreads();
    }

    for (int64_t tg = blockIdx.x; tg < ngroups; tg += gridDim.x) {
        const int64_t tile = tg * tpw + slot;
        const bool tile_ok = tile < ntiles;
        const int64_t n = tile * 16 + (lane & 15);
        f4 acc[RG];
#pragma unroll
        for (int r = 0; r < RG; ++r) acc[r] = f4{0.f, 0.f, 0.f, 0.f};
        if (tile_ok) {
            const MfCol col = mf_col<FMT>(a, n < a.N ? n : a.N - 1);
            u4v wb[P];
            MetaRaw<H> mb[P];
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int t = kslice + p * ks;
                if (t < nsteps) {
                    const int c = 4 * t + g;
                    wb[p] = load16_stream(col.w + (uint32_t)c * 16u);
                    mb[p] = load_meta_raw<FMT, H>(a, col, c);
                }
            }
            for (int tb = kslice; tb < nsteps; tb += P * ks) {
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    const int t = tb + p * ks;
                    if (t >= nsteps) break;
                    const u4v w = wb[p];
                    const MetaRaw<H> m = mb[p];
                    const int tn = t + P * ks;
                    if (tn < nsteps) {
                        const int cn = 4 * tn + g;
                        wb[p] = load16_stream(col.w + (uint32_t)cn * 16u);
                        mb[p] = load_meta_raw<FMT, H>(a, col, cn);
                    }
                    mfma_step<FMT, ACT, RG, H, LDSA>(a, w, m, 4 * t + g, ar, a_live_grp, sA, sZero, astride, acc);
                }
            }
        }
        finish_tile<ACT, RG>(a, acc, sR, wave, lane, ks, kslice, g, tile_ok, n);
    }
}

// LDS-ring kernel: each K step's 16-byte code chunk and its block-metadata dword(s)
// travel global -> LDS by DMA (global_load_lds), R slots per wave and R - 1 steps in
// flight, so the prefetch depth costs no VGPRs. The activations are staged in LDS as
// well, which leaves these DMAs as the only vector-memory operations of the K loop;
// they complete in issue order, so the wait before a slot is read is an exact vmcnt.
template <int FMT, int ACT, int RG, int H, bool ZPP, int R, int NW>
__global__ void __launch_bounds__(64 * NW, (RG == 1 ? 4 : 2)) k_mfma_ring(KArgs a) {
    constexpr int P = R - 1;
    constexpr int NM = MetaDma<FMT, ZPP>::NM;
    constexpr int OPS = 1 + NM;                 // DMAs per step
    constexpr int STEADY = (P - 1) * OPS;       // later steps' DMAs still in flight
    constexpr int SLOT = 1024 + 256 * NM;       // bytes per slot
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int ks = a.ksplit;
    const int tpw = NW / ks;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
    const int lane = threadIdx.x & 63;
    const int slot = wave / ks;
    const int kslice = wave - slot * ks;
    const int g = lane >> 4;
    const int ar = lane & 3;
    const bool a_live_grp = ((lane & 15) >> 2) == g;
    const int nsteps = (int)(a.nchunks >> 2);
    const int astride = (int)a.K + kAPad;
    const int64_t ntiles = (a.N + 15) >> 4;
    const int64_t ngroups = (ntiles + tpw - 1) / tpw;
    const size_t abytes = 16 + (((size_t)a.M * astride * 2 + 15) & ~(size_t)15);
    uint16_t *sZero = (uint16_t *)smem;
    uint16_t *sA = (uint16_t *)(smem + 16);
    unsigned char *ring = smem + abytes + (size_t)wave * R * SLOT;
    float *sR = (float *)(smem + abytes + (size_t)NW * R * SLOT);
    // this wave's steps: t = kslice + i * ks, i < nmine
    const int nmine = kslice < nsteps ? (nsteps - kslice + ks - 1) / ks : 0;

    bool staged = false;
    for (int64_t tg = blockIdx.x; tg < ngroups; tg += gridDim.x) {
        const int64_t tile = tg * tpw + slot;
        const bool tile_ok = tile < ntiles;
        const int64_t n = tile * 16 + (lane & 15);
        const MfCol col = mf_col<FMT>(a, n < a.N ? n : a.N - 1);
        f4 acc[RG];
#pragma unroll
        for (int r = 0; r < RG; ++r) acc[r] = f4{0.f, 0.f, 0.f, 0.f};
        // prologue: the first P steps in flight (on the first tile before the
        // activations are staged, so that the copy overlaps the weight fetch)
        if (tile_ok) {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                if (p < nmine) {
                    const int c = 4 * (kslice + p * ks) + g;
                    unsigned char *sl = ring + p * SLOT;
                    dma_to_lds<16>(col.w + (uint32_t)c * 16u, sl);
                    meta_dma<FMT, H, ZPP>(a, col, c, (uint32_t *)(sl + 1024), (uint32_t *)(sl + 1280));
                }
            }
        }
        if (!staged) {
            if (threadIdx.x == 0) *(u4v *)sZero = u4v{0u, 0u, 0u, 0u};
            stage_a<FMT>(a, sA, astride);
            __syncthreads();
            staged = true;
        }
        if (tile_ok) {
            // one step per iteration, slots addressed at run time: nothing from
            // another step is live across the wait
#pragma unroll 1
            for (int i = 0; i < nmine; ++i) {
                if (i + P - 1 < nmine) wait_vmcnt<STEADY>();
                else wait_vmcnt<0>();
                const int c = 4 * (kslice + i * ks) + g;
                const unsigned char *sl = ring + (i % R) * SLOT;
                const u4v w = ((const u4v *)sl)[lane];
                const MetaRaw<H> m = meta_from_lds<FMT, H, ZPP>(a, col, c, (const uint32_t *)(sl + 1024),
                                                                (const uint32_t *)(sl + 1280));
                if (i + P < nmine) {
                    // refill the slot consumed one step ago
                    const int cn = 4 * (kslice + (i + P) * ks) + g;
                    unsigned char *sn = ring + ((i + P) % R) * SLOT;
                    dma_to_lds<16>(col.w + (uint32_t)cn * 16u, sn);
                    meta_dma<FMT, H, ZPP>(a, col, cn, (uint32_t *)(sn + 1024), (uint32_t *)(sn + 1280));
                }
                mfma_step<FMT, ACT, RG, H, true>(a, w, m, c, ar, a_live_grp, sA, sZero, astride, acc);
            }
        }
        finish_tile<ACT, RG>(a, acc, sR, wave, lane, ks, kslice, g, tile_ok, n);
    }
}

namespace {

constexpr int kPrefetch = 2;

template <int FMT, int ACT, int RG, int H, bool LDSA, int NW>
hipError_t go_nw(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    auto kern = k_mfma<FMT, ACT, RG, H, LDSA, kPrefetch, NW>;
    if (cfg.lds_bytes > 65536) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, cfg.lds_bytes);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)cfg.grid), dim3(64u * NW), (size_t)cfg.lds_bytes, s, a);
    return hipGetLastError();
}

template <int FMT, int ACT, int RG, int H, bool LDSA>
hipError_t go(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    return cfg.waves_per_wg == 16 ? go_nw<FMT, ACT, RG, H, LDSA, 16>(cfg, a, s) : go_nw<FMT, ACT, RG, H, LDSA, 8>(cfg, a, s);
}

template <int FMT, int ACT, int RG, int H, bool ZPP, int R, int NW>
hipError_t go_ring_nw(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    auto kern = k_mfma_ring<FMT, ACT, RG, H, ZPP, R, NW>;
    if (cfg.lds_bytes > 65536) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, cfg.lds_bytes);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)cfg.grid), dim3(64u * NW), (size_t)cfg.lds_bytes, s, a);
    return hipGetLastError();
}

// ring depth (bit 2 of the variant: 0 -> 4 slots, 1 -> 8 slots); the ring runs
// without a K split, always with 8-wave workgroups
template <int FMT, int ACT, int RG, int H, bool ZPP>
hipError_t go_ring(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    if (cfg.waves_per_wg != 8 || cfg.ksplit != 1) return hipErrorInvalidValue;
    return ((cfg.variant >> 2) & 1) ? go_ring_nw<FMT, ACT, RG, H, ZPP, 8, 8>(cfg, a, s)
                                    : go_ring_nw<FMT, ACT, RG, H, ZPP, 4, 8>(cfg, a, s);
}

template <int FMT, int ACT, int RG, int H>
hipError_t pick_lds(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    if (cfg.variant & 2) {
        if constexpr (FMT == FMT_U4 || FMT == FMT_U8)
            return a.zp ? go_ring<FMT, ACT, RG, H, true>(cfg, a, s) : go_ring<FMT, ACT, RG, H, false>(cfg, a, s);
        else
            return go_ring<FMT, ACT, RG, H, false>(cfg, a, s);
    }
    return (cfg.variant & 1) ? go<FMT, ACT, RG, H, true>(cfg, a, s) : go<FMT, ACT, RG, H, false>(cfg, a, s);
}

template <int FMT, int ACT, int H>
hipError_t pick_rg(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    switch ((a.M + 3) / 4) {
    case 1: return pick_lds<FMT, ACT, 1, H>(cfg, a, s);
    case 2: return pick_lds<FMT, ACT, 2, H>(cfg, a, s);
    case 3: return pick_lds<FMT, ACT, 3, H>(cfg, a, s);
    case 4: return pick_lds<FMT, ACT, 4, H>(cfg, a, s);
    default: return hipErrorInvalidValue;
    }
}

template <int FMT, int ACT>
hipError_t pick_h(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    // two scale blocks per chunk: every NVFP4 chunk, U4 chunks with 16-wide blocks
    if constexpr (FMT == FMT_NVFP4) return pick_rg<FMT, ACT, 2>(cfg, a, s);
    else if constexpr (FMT == FMT_U4) return a.bs == 16 ? pick_rg<FMT, ACT, 2>(cfg, a, s) : pick_rg<FMT, ACT, 1>(cfg, a, s);
    else return pick_rg<FMT, ACT, 1>(cfg, a, s);
}

template <int FMT>
hipError_t pick_act(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    return cfg.act == ACT_F16 ? pick_h<FMT, ACT_F16>(cfg, a, s) : pick_h<FMT, ACT_BF16>(cfg, a, s);
}

}  // namespace

hipError_t launch_mfma(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    switch (cfg.fmt) {
    case FMT_U4: return pick_act<FMT_U4>(cfg, a, s);
    case FMT_U8:
        if (cfg.act != ACT_F16) return hipErrorInvalidValue;  // 8-bit codes plus an offset exceed bf16's integers
        return pick_h<FMT_U8, ACT_F16>(cfg, a, s);
    case FMT_FP8: return pick_act<FMT_FP8>(cfg, a, s);
    case FMT_NVFP4: return pick_act<FMT_NVFP4>(cfg, a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qgemv
