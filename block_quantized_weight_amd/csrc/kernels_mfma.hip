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

// Block metadata of one chunk kept raw while it waits in the prefetch ring: the
// loaded values as they are (nothing is computed from a load until the chunk is
// consumed, so a prefetch never waits for its own data), decoded by meta_decode.
//   U4, one block per chunk : v0 = fp16 scale bits, v1 = the zero-point byte holding the block
//   U4, two blocks per chunk: v0 = both fp16 scales, v1 = the zero-point byte of the pair
//   U8                      : v0 = fp16 scale bits, v1 = zero-point byte
//   FP8                     : v0 = fp32 scale bits
//   NVFP4                   : v0 = the two E4M3 scale bytes
// (without zero points v1 holds whatever the aliased address held; meta_decode then
// uses the midpoint, 8 for U4 and 128 for U8)
template <int H>
struct MetaRaw {
    uint32_t v[2];
};

struct MfCol {
    const uint8_t *w;
    const void *s;
    const uint8_t *z;
};

// Column pointers. Without zero points p.z aliases the column's scale row (at least
// as many bytes as a zero-point row), so that every zero-point load is issued
// unconditionally from a valid address and the midpoint is selected at decode: no
// branch around a load keeps the compiler's load-counter waits exact in the rings.
template <int FMT>
__device__ __forceinline__ MfCol mf_col(const KArgs &a, int64_t n) {
    MfCol p;
    p.w = a.W + n * a.col_bytes;
    if constexpr (FMT == FMT_NVFP4) p.s = (const uint8_t *)a.scales + n * (a.K >> 4);
    else if constexpr (FMT == FMT_FP8) p.s = (const float *)a.scales + n * a.nblk;
    else p.s = (const uint16_t *)a.scales + n * a.nblk;
    p.z = a.zp ? a.zp + n * a.zstride : (const uint8_t *)p.s;
    return p;
}

template <int FMT, int H>
__device__ __forceinline__ MetaRaw<H> load_meta_raw(const KArgs &a, const MfCol &p, int c) {
    MetaRaw<H> m;
    m.v[1] = 0u;
    if constexpr (FMT == FMT_U4) {
        if constexpr (H == 1) {
            const int b = (c << 5) >> a.bs_shift;
            m.v[0] = ((const uint16_t *)p.s)[b];
            m.v[1] = p.z[b >> 1];
        } else {
            // 16-wide blocks: blocks 2c and 2c+1, adjacent scales, one zero-point byte
            m.v[0] = *(const uint32_t *)((const uint16_t *)p.s + 2 * c);
            m.v[1] = p.z[c];
        }
    } else if constexpr (FMT == FMT_U8) {
        const int b = (c << 4) >> a.bs_shift;
        m.v[0] = ((const uint16_t *)p.s)[b];
        m.v[1] = p.z[b];
    } else if constexpr (FMT == FMT_FP8) {
        m.v[0] = ((const uint32_t *)p.s)[(c << 4) >> a.bs_shift];
    } else {
        m.v[0] = (uint32_t)*(const uint16_t *)((const uint8_t *)p.s + 2 * c);
    }
    return m;
}

// Scale and (M0 + zero point) of half h of chunk c from the raw metadata.
template <int FMT, int ACT, int H>
__device__ __forceinline__ void meta_decode(const KArgs &a, const MetaRaw<H> &m, int c, int h, float &s,
                                            float &zoff) {
    if constexpr (FMT == FMT_U4) {
        const ZSel zs = zsel(a.zp, 0x88u);
        const uint32_t zb = (m.v[1] & zs.keep) | zs.fill;
        if constexpr (H == 1) {
            const int b = (c << 5) >> a.bs_shift;
            s = half_bits_to_float((uint16_t)(m.v[0] & 0xFFFFu));
            zoff = U4Magic<ACT>::off + (float)((b & 1) ? ((zb >> 4) & 0x0Fu) : (zb & 0x0Fu));
        } else {
            s = half_bits_to_float((uint16_t)(h ? (m.v[0] >> 16) : (m.v[0] & 0xFFFFu)));
            zoff = U4Magic<ACT>::off + (float)(h ? ((zb >> 4) & 0x0Fu) : (zb & 0x0Fu));
        }
    } else if constexpr (FMT == FMT_U8) {
        const ZSel zs = zsel(a.zp, 128u);
        s = half_bits_to_float((uint16_t)(m.v[0] & 0xFFFFu));
        zoff = 1024.0f + (float)(((m.v[1] & zs.keep) | zs.fill) & 0xFFu);
    } else if constexpr (FMT == FMT_FP8) {
        s = __builtin_bit_cast(float, m.v[0]);
        zoff = 0.0f;
    } else {
        s = e4m3_to_float(h ? ((m.v[0] >> 8) & 0xFFu) : (m.v[0] & 0xFFu));
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
    m.v[1] = 0u;
    if constexpr (FMT == FMT_U4) {
        if constexpr (H == 1) {
            const int b = (c << 5) >> a.bs_shift;
            m.v[0] = (meta0[lane] >> byte_shift((const uint16_t *)p.s + b)) & 0xFFFFu;
            m.v[1] = ZPP ? ((meta1[lane] >> byte_shift(p.z + (b >> 1))) & 0xFFu) : 0x88u;
        } else {
            m.v[0] = meta0[lane];
            m.v[1] = ZPP ? ((meta1[lane] >> byte_shift(p.z + c)) & 0xFFu) : 0x88u;
        }
    } else if constexpr (FMT == FMT_U8) {
        const int b = (c << 4) >> a.bs_shift;
        m.v[0] = (meta0[lane] >> byte_shift((const uint16_t *)p.s + b)) & 0xFFFFu;
        m.v[1] = ZPP ? ((meta1[lane] >> byte_shift(p.z + b)) & 0xFFu) : 128u;
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
// A operands of one K step for every row group, loaded from global memory (used ahead
// of time by the register-ring kernel when the activations are not staged in LDS).
template <int FMT, int RG>
struct AOps {
    op4 v[RG][MfFmt<FMT>::MF];
};

// Every lane loads (rows past M read row M - 1); lanes off the block diagonal or past
// M are zeroed when the operands are used (mfma_step), so the loads themselves are
// unconditional.
template <int FMT, int RG>
__device__ __forceinline__ void load_a_ops(const KArgs &a, int c, int ar, AOps<FMT, RG> &o) {
    using F = MfFmt<FMT>;
    const uint16_t *A16 = (const uint16_t *)a.A;
    const uint32_t kbase = (uint32_t)c * F::KPC;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int row = 4 * rg + ar;
        const uint16_t *arow = A16 + (int64_t)(row < a.M ? row : a.M - 1) * a.K;
#pragma unroll
        for (int j = 0; j < F::MF; ++j) o.v[rg][j] = load_a<FMT>(arow, true, kbase + 8 * j);
    }
}

template <int FMT, int ACT, int RG, int H, bool LDSA>
__device__ __forceinline__ void mfma_step(const KArgs &a, const u4v &w, const MetaRaw<H> &m, int c, int ar,
                                          bool a_live_grp, const uint16_t *sA, const uint16_t *sZero, int astride,
                                          const AOps<FMT, RG> &areg, bool valid, f4 acc[RG]) {
    using F = MfFmt<FMT>;
    constexpr uint32_t ONE = (ACT == ACT_F16) ? 0x3C003C00u : 0x3F803F80u;
    const op4 ones = {ONE, ONE, ONE, ONE};
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
                const op4 z = {0u, 0u, 0u, 0u};
                av = live ? areg.v[rg][j] : z;
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
            meta_decode<FMT, ACT, H>(a, m, c, h, sc, zoff);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = d[h][r];
                if constexpr (F::ZP) v = __builtin_fmaf(-zoff, sa[h][r], v);
                const float t = __builtin_fmaf(sc, v, acc[rg][r]);
                acc[rg][r] = valid ? t : acc[rg][r];
            }
        }
    }
}

// Compiler fence for the register rings: the accumulators are produced before this
// point and no memory operation moves across it. Emits no instruction.
template <int RG>
__device__ __forceinline__ void pin_accumulators(f4 acc[RG]) {
#pragma unroll
    for (int r = 0; r < RG; ++r) asm volatile("" : "+v"(acc[r])::"memory");
}

// Stage the M activation rows into LDS once per workgroup, permuted into the MFMA
// slot order (row stride K + kAPad elements). Each thread handles 16-byte pieces
// it, it + blockDim, ... in batches of SB whose loads are all issued before the first
// store, so the staging costs about one load latency per batch, not one per piece.
template <int FMT, int SB = 8>
__device__ __forceinline__ void stage_a(const KArgs &a, uint16_t *sA, int astride) {
    using F = MfFmt<FMT>;
    const uint16_t *A16 = (const uint16_t *)a.A;
    const int K = (int)a.K;
    const int k8n = K >> 3;
    const int items = a.M * k8n;
    const int last = items - 1;
    for (int base = threadIdx.x; base < items; base += SB * (int)blockDim.x) {
        u4v v[SB];
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            int it = base + j * (int)blockDim.x;
            it = it < items ? it : last;
            const int m = it / k8n;
            v[j] = load16(A16 + (int64_t)m * K + ((it - m * k8n) << 3));
        }
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int it = base + j * (int)blockDim.x;
            if (it < items) {
                const int m = it / k8n;
                const int k8 = (it - m * k8n) << 3;
                u4v o;
                if constexpr (F::PERM) {
                    o.x = perm(v[j].z, v[j].x, 0x05040100u);  // (a0, a4)
                    o.y = perm(v[j].z, v[j].x, 0x07060302u);  // (a1, a5)
                    o.z = perm(v[j].w, v[j].y, 0x05040100u);  // (a2, a6)
                    o.w = perm(v[j].w, v[j].y, 0x07060302u);  // (a3, a7)
                } else {
                    o = v[j];
                }
                *(u4v *)(sA + m * astride + k8) = o;
            }
        }
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

// Register-ring kernel. A workgroup of 8 waves holds 8 / ksplit tiles of ksplit waves
// each and walks tile groups g = blockIdx.x, + gridDim.x, ...; within a tile, wave
// kslice takes K steps t = kslice, kslice + ksplit, ... Every wave runs the same
// S = ceil(ceil(steps / ksplit) / P) * P slots per tile (a slot past the last step, or
// of a tile past N, computes on a clamped valid address and its accumulator update is
// discarded), so all waves reach the K-split barriers of finish_tile together. The
// (tile, slot) sequence is one pipeline: a register ring of P slots holds the codes and
// raw metadata of the next P - 1 slots in flight, across tile boundaries. Activations
// are either staged once per workgroup in LDS (LDSA) or, when they are not, fetched
// into the same ring with the codes of their slot.
//
// Load-wait discipline: no load and no use of a slot sits behind a branch, a slot is
// consumed before it is refilled (a scheduling barrier keeps the refill below the last
// use), and the slot loop is a whole number of ring turns per tile, so each slot keeps
// its registers and the compiler's wait before a slot leaves the later P - 1 slots in
// flight.
// Register budget: four waves per SIMD (<= 128 VGPRs) for one row group, two waves
// per SIMD (<= 256) beyond.
template <int FMT, int ACT, int RG, int H, bool LDSA, int P>
__global__ void __launch_bounds__(512, (RG == 1 ? 4 : 2)) k_mfma(KArgs a) {
    constexpr int NW = 8;
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
    const int S = ((nsteps + ks - 1) / ks + P - 1) / P * P;
    const int astride = (int)a.K + kAPad;
    const int64_t ntiles = (a.N + 15) >> 4;
    const int64_t ngroups = (ntiles + tpw - 1) / tpw;
    uint16_t *sZero = (uint16_t *)smem;
    uint16_t *sA = (uint16_t *)(smem + 16);
    float *sR = (float *)(smem + 16 + (LDSA ? (((size_t)a.M * astride * 2 + 15) & ~(size_t)15) : 0));

    // issue cursor: tile group, slot within the tile, and the column the lane loads
    int64_t itg = blockIdx.x;
    int is = 0;
    auto icol = [&]() {
        const int64_t n = (itg * tpw + slot) * 16 + (lane & 15);
        return mf_col<FMT>(a, n < a.N ? n : a.N - 1);
    };
    MfCol col = icol();
    u4v wb[P];
    MetaRaw<H> mb[P];
    AOps<FMT, RG> ab[LDSA ? 1 : P];  // activations in the ring when they are not staged
    auto issue = [&](int p) {
        const int t0 = kslice + is * ks;
        const int c = 4 * (t0 < nsteps ? t0 : nsteps - 1) + g;
        wb[p] = load16_stream(col.w + (uint32_t)c * 16u);
        mb[p] = load_meta_raw<FMT, H>(a, col, c);
        if constexpr (!LDSA) load_a_ops<FMT, RG>(a, c, ar, ab[p]);
        if (++is == S) {
            is = 0;
            itg += gridDim.x;
            col = icol();
        }
    };
#pragma unroll
    for (int p = 0; p < P; ++p) issue(p);

    if constexpr (LDSA) {
        if (threadIdx.x == 0) *(u4v *)sZero = u4v{0u, 0u, 0u, 0u};
        stage_a<FMT>(a, sA, astride);
        __syncthreads();
    }

    // One ring turn = P slots. Every turn but the last consumes and refills each slot;
    // the last turn only drains the ring, so nothing is fetched past the wave's work.
    // Tile boundaries fall on turn boundaries (S is a multiple of P).
    const int64_t G = blockIdx.x < ngroups ? (ngroups - blockIdx.x + gridDim.x - 1) / gridDim.x : 0;
    const int64_t turns = G * (S / P);
    const int tpt = S / P;  // turns per tile
    int64_t tg = blockIdx.x;
    int tt = 0;  // turn within the tile
    f4 acc[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) acc[r] = f4{0.f, 0.f, 0.f, 0.f};
    auto turn = [&](bool refill) {
        const int64_t tile = tg * tpw + slot;
        const bool tile_ok = tile < ntiles;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int t = kslice + (tt * P + p) * ks;
            const int tc = t < nsteps ? t : nsteps - 1;
            mfma_step<FMT, ACT, RG, H, LDSA>(a, wb[p], mb[p], 4 * tc + g, ar, a_live_grp, sA, sZero, astride,
                                             ab[LDSA ? 0 : p], tile_ok && t < nsteps, acc);
            if (refill) {
                // the slot's accumulation completes here (nothing of it may sink below
                // the refill), then the refill reuses the slot's registers
                pin_accumulators<RG>(acc);
                __builtin_amdgcn_sched_barrier(0);
                issue(p);
            }
        }
        if (++tt == tpt) {
            finish_tile<ACT, RG>(a, acc, sR, wave, lane, ks, kslice, g, tile_ok, tile * 16 + (lane & 15));
#pragma unroll
            for (int r = 0; r < RG; ++r) acc[r] = f4{0.f, 0.f, 0.f, 0.f};
            tt = 0;
            tg += gridDim.x;
        }
    };
    for (int64_t i = 0; i + 1 < turns; ++i) turn(true);
    if (turns > 0) turn(false);
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
            stage_a<FMT, 4>(a, sA, astride);  // smaller batches: the ring's state is live here
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
                mfma_step<FMT, ACT, RG, H, true>(a, w, m, c, ar, a_live_grp, sA, sZero, astride, AOps<FMT, RG>{}, true,
                                                 acc);
            }
        }
        finish_tile<ACT, RG>(a, acc, sR, wave, lane, ks, kslice, g, tile_ok, n);
    }
}

namespace {

template <int FMT, int ACT, int RG, int H, bool LDSA, int P>
hipError_t go_p(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    auto kern = k_mfma<FMT, ACT, RG, H, LDSA, P>;
    if (cfg.lds_bytes > 65536) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, cfg.lds_bytes);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)cfg.grid), dim3(512), (size_t)cfg.lds_bytes, s, a);
    return hipGetLastError();
}

// Ring depth when the activations travel in the ring too: as deep as the register
// budget allows without spilling (each slot then holds RG * MF activation operands).
template <int FMT, int RG>
constexpr int ring_depth_with_a() {
    return (MfFmt<FMT>::MF == 2 && RG <= 3) ? 4 : ((MfFmt<FMT>::MF == 4 && RG == 4) ? 1 : 2);
}

// Depth with staged activations: variant bit 3 asks for 8 slots, which one row group
// with one scale block per chunk affords; larger tiles take 4 (2 for three or four row
// groups with two scale blocks per chunk), the most that fit without spilling.
template <int RG, int H>
constexpr int ring_depth_staged(bool deep) {
    return (RG <= 2 && H == 1) ? (deep ? 8 : 4) : ((RG <= 2 || H == 1) ? 4 : 2);
}

// register-ring depth (ring_depth_staged / ring_depth_with_a); 8-wave workgroups
template <int FMT, int ACT, int RG, int H, bool LDSA>
hipError_t go(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    if (cfg.waves_per_wg != 8) return hipErrorInvalidValue;
    if constexpr (LDSA) {
        constexpr int PD = ring_depth_staged<RG, H>(true), PS = ring_depth_staged<RG, H>(false);
        return ((cfg.variant >> 3) & 1) ? go_p<FMT, ACT, RG, H, LDSA, PD>(cfg, a, s)
                                        : go_p<FMT, ACT, RG, H, LDSA, PS>(cfg, a, s);
    } else {
        return go_p<FMT, ACT, RG, H, LDSA, ring_depth_with_a<FMT, RG>()>(cfg, a, s);
    }
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
    // two scale blocks per chunk (and zero points) do not fit an 8-slot ring's registers
    constexpr int RD = (H == 2 && ZPP) ? 4 : 8;
    return ((cfg.variant >> 2) & 1) ? go_ring_nw<FMT, ACT, RG, H, ZPP, RD, 8>(cfg, a, s)
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
