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

// Block scale(s) and zero point of chunk c of a column: up to two blocks per chunk.
struct ChunkMeta {
    float s[2];
    float zoff[2];  // (M0 + z) for the integer formats
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

template <int FMT, int ACT>
__device__ __forceinline__ void load_chunk_meta(const KArgs &a, const MfCol &p, int c, ChunkMeta &m) {
    if constexpr (FMT == FMT_U4) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int b = ((c << 5) + 16 * h) >> a.bs_shift;
            m.s[h] = half_bits_to_float(((const uint16_t *)p.s)[b]);
            int z = 8;
            if (p.z) {
                const uint32_t zb = p.z[b >> 1];
                z = (b & 1) ? (int)(zb >> 4) : (int)(zb & 0x0Fu);
            }
            m.zoff[h] = U4Magic<ACT>::off + (float)z;
        }
    } else if constexpr (FMT == FMT_U8) {
        const int b = (c << 4) >> a.bs_shift;
        m.s[0] = m.s[1] = half_bits_to_float(((const uint16_t *)p.s)[b]);
        m.zoff[0] = m.zoff[1] = 1024.0f + (p.z ? (float)p.z[b] : 128.0f);
    } else if constexpr (FMT == FMT_FP8) {
        m.s[0] = m.s[1] = ((const float *)p.s)[(c << 4) >> a.bs_shift];
        m.zoff[0] = m.zoff[1] = 0.0f;
    } else {
        const uint8_t *S = (const uint8_t *)p.s + 2 * c;
        m.s[0] = e4m3_to_float(S[0]);
        m.s[1] = e4m3_to_float(S[1]);
        m.zoff[0] = m.zoff[1] = 0.0f;
    }
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

// One wave owns the 16 columns of a tile for one K slice; `ksplit` waves of a
// workgroup cover the tile's K steps (step t goes to wave t % ksplit).
template <int FMT, int ACT, int RG>
__global__ void __launch_bounds__(1024) k_mfma(KArgs a) {
    using F = MfFmt<FMT>;
    extern __shared__ float red[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int ks = a.ksplit;
    const int ni = lane & 15;        // column within the tile
    const int g = lane >> 4;         // lane group: chunk 4t+g, output rows 4g..4g+3
    const int ai = lane & 15;        // A-operand row index i
    const bool a_live_grp = (ai >> 2) == g;
    const int64_t tile = blockIdx.x;
    const int64_t n = tile * 16 + ni;
    const int64_t nl = n < a.N ? n : a.N - 1;
    const int nsteps = (int)(a.nchunks >> 2);
    const MfCol col = mf_col<FMT>(a, nl);

    f4 acc[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) acc[r] = f4{0.f, 0.f, 0.f, 0.f};

    constexpr uint32_t ONE = (ACT == ACT_F16) ? 0x3C003C00u : 0x3F803F80u;
    const op4 ones = {ONE, ONE, ONE, ONE};
    const uint16_t *A16 = (const uint16_t *)a.A;

    for (int t = wave; t < nsteps; t += ks) {
        const int c = 4 * t + g;
        const u4v w = load16_stream(col.w + (uint32_t)c * 16u);
        ChunkMeta meta;
        load_chunk_meta<FMT, ACT>(a, col, c, meta);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            const int row = 4 * rg + (ai & 3);
            const bool live = a_live_grp && row < a.M;
            const uint16_t *arow = A16 + (int64_t)(live ? row : 0) * a.K;
            // a live A lane of group g feeds rows 4g..4g+3 over the k of chunk 4t+g
            const uint32_t kbase = (uint32_t)c * F::KPC;
            f4 d[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
            f4 sa[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int j = 0; j < F::MF; ++j) {
                const op4 av = load_a<FMT>(arow, live, kbase + 8 * j);
                op4 bv;
                if constexpr (F::MF == 4) {
                    if (j == 0) bv = decode_b<FMT, ACT, 0>(w);
                    else if (j == 1) bv = decode_b<FMT, ACT, 1>(w);
                    else if (j == 2) bv = decode_b<FMT, ACT, 2>(w);
                    else bv = decode_b<FMT, ACT, 3>(w);
                } else {
                    if (j == 0) bv = decode_b<FMT, ACT, 0>(w);
                    else bv = decode_b<FMT, ACT, 1>(w);
                }
                const int h = (F::MF == 4) ? (j >> 1) : 0;  // half of the chunk (16 k)
                d[h] = mfma<ACT>(av, bv, d[h]);
                if constexpr (F::ZP) sa[h] = mfma<ACT>(av, ones, sa[h]);
            }
#pragma unroll
            for (int h = 0; h < (F::MF == 4 ? 2 : 1); ++h) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = d[h][r];
                    if constexpr (F::ZP) v = __builtin_fmaf(-meta.zoff[h], sa[h][r], v);
                    acc[rg][r] = __builtin_fmaf(meta.s[h], v, acc[rg][r]);
                }
            }
        }
    }

    // cross-wave reduction in fixed wave order
    if (ks > 1) {
        float *mine = red + (size_t)wave * (RG * 4 * 64);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int r = 0; r < 4; ++r) mine[(rg * 4 + r) * 64 + lane] = acc[rg][r];
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float s = red[(rg * 4 + r) * 64 + lane];
                for (int w2 = 1; w2 < ks; ++w2) s += red[(size_t)w2 * (RG * 4 * 64) + (rg * 4 + r) * 64 + lane];
                acc[rg][r] = s;
            }
    }

    // sum the four lane groups; lane (n, g) then stores row 4*rg + g
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

namespace {

template <int FMT, int ACT, int RG>
hipError_t go(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    const unsigned threads = 64u * (unsigned)cfg.ksplit;
    hipLaunchKernelGGL((k_mfma<FMT, ACT, RG>), dim3((unsigned)cfg.grid), dim3(threads), (size_t)cfg.lds_bytes, s, a);
    return hipGetLastError();
}

template <int FMT, int ACT>
hipError_t pick_rg(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    switch ((a.M + 3) / 4) {
    case 1: return go<FMT, ACT, 1>(cfg, a, s);
    case 2: return go<FMT, ACT, 2>(cfg, a, s);
    case 3: return go<FMT, ACT, 3>(cfg, a, s);
    case 4: return go<FMT, ACT, 4>(cfg, a, s);
    default: return hipErrorInvalidValue;
    }
}

template <int FMT>
hipError_t pick_act(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    return cfg.act == ACT_F16 ? pick_rg<FMT, ACT_F16>(cfg, a, s) : pick_rg<FMT, ACT_BF16>(cfg, a, s);
}

}  // namespace

hipError_t launch_mfma(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    switch (cfg.fmt) {
    case FMT_U4: return pick_act<FMT_U4>(cfg, a, s);
    case FMT_U8:
        if (cfg.act != ACT_F16) return hipErrorInvalidValue;  // 8-bit codes exceed bf16's integer range with an offset
        return pick_rg<FMT_U8, ACT_F16>(cfg, a, s);
    case FMT_FP8: return pick_act<FMT_FP8>(cfg, a, s);
    case FMT_NVFP4: return pick_act<FMT_NVFP4>(cfg, a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qgemv
