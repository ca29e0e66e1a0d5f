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
//  - Zero points: with fp16 activations the codes enter the MFMA as the exact fp16
//    integers q - z (1024 + q and 1024 + z built with bit operations, subtracted with
//    one packed fp16 op), as the pages form (q - zp) exactly before the mma ("[CUDA]
//    MatMulNBits 8-bit: wide fp16 M=1 kernel", Description). With bf16 activations,
//    8-bit codes form q - z exactly in fp32 and round the pair to bf16 (exact); 4-bit
//    codes enter as the bare bf16 integers q (E4M3 converter, no offset) and sum(a)
//    over the chunk comes from one more MFMA against a ones operand, the epilogue
//    forming s * (D - z * sum(a)) (gfx950 has no packed bf16 subtract).
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

// Per-format description of one 16-byte chunk in the MFMA family.
//   MF   : MFMAs per chunk (8 k per lane each)
template <int FMT> struct MfFmt;
template <> struct MfFmt<FMT_U4> { static constexpr int KPC = 32, MF = 4; };
template <> struct MfFmt<FMT_U8> { static constexpr int KPC = 16, MF = 2; };
template <> struct MfFmt<FMT_FP8> { static constexpr int KPC = 16, MF = 2; };
template <> struct MfFmt<FMT_NVFP4> { static constexpr int KPC = 32, MF = 4; };

// Per (format, activation type):
//   ASUM : the zero point enters as -z * sum(a) (4-bit codes on bf16); the other
//          formats with zero points form q - z in the decode
//   PERM : slot order of the 8 activations of one MFMA: 0 natural; 1 = [0,4,1,5,2,6,3,7]
//          (4-bit codes on fp16); 2 = [0,2,4,6,1,3,5,7] (4-bit codes on bf16)
template <int FMT, int ACT> struct MfAct {
    static constexpr bool ASUM = FMT == FMT_U4 && ACT == ACT_BF16;
    static constexpr int PERM = FMT == FMT_U4 ? (ACT == ACT_F16 ? 1 : 2) : 0;
};

// The zero-point operand of a chunk half the decode subtracts, from the integer z:
// fp16 (1024 + z, 1024 + z) for codes on fp16, fp32 z for 8-bit codes on bf16.
template <int FMT, int ACT>
__device__ __forceinline__ uint32_t zero_word(uint32_t z) {
    if constexpr (ACT == ACT_F16) return (0x6400u | z) * 0x00010001u;
    else return __builtin_bit_cast(uint32_t, (float)z);
}

// B operand (8 weight values) of MFMA j from the chunk's 4 code dwords; zw: the
// zero-point operand (zero_word) of the chunk half MFMA j lies in.
template <int FMT, int ACT, int J>
__device__ __forceinline__ op4 decode_b(const u4v &w, uint32_t zw) {
    op4 r;
    if constexpr (FMT == FMT_U4 && ACT == ACT_F16) {
        // dword J holds k = 8J..8J+7: slots (k0,k4),(k1,k5),(k2,k6),(k3,k7) as the
        // fp16 integers 1024 + q, minus (1024 + z): exactly q - z
        const uint32_t x = w[J];
        r.x = sub_h2(and_or(x, 0x000F000Fu, 0x64006400u), zw);
        r.y = sub_h2(and_or(x >> 4, 0x000F000Fu, 0x64006400u), zw);
        r.z = sub_h2(and_or(x >> 8, 0x000F000Fu, 0x64006400u), zw);
        r.w = sub_h2(and_or(x >> 12, 0x000F000Fu, 0x64006400u), zw);
    } else if constexpr (FMT == FMT_U4) {
        // bf16: the bare integers q from the E4M3 converter, slots (k0,k2),(k4,k6) from
        // the low nibbles and (k1,k3),(k5,k7) from the high ones
        const uint32_t lo = w[J] & 0x0F0F0F0Fu, hi = (w[J] >> 4) & 0x0F0F0F0Fu;
        r.x = small_int_bf16_pair<false>(lo);
        r.y = small_int_bf16_pair<true>(lo);
        r.z = small_int_bf16_pair<false>(hi);
        r.w = small_int_bf16_pair<true>(hi);
    } else if constexpr (FMT == FMT_U8 && ACT == ACT_F16) {
        // dwords 2J, 2J+1 hold k = 8J..8J+7 in natural order; (1024 + q) - (1024 + z)
        constexpr uint32_t MB = 0x64646464u;
        const uint32_t x0 = w[2 * J], x1 = w[2 * J + 1];
        r.x = sub_h2(perm(MB, x0, 0x04010400u), zw);
        r.y = sub_h2(perm(MB, x0, 0x04030402u), zw);
        r.z = sub_h2(perm(MB, x1, 0x04010400u), zw);
        r.w = sub_h2(perm(MB, x1, 0x04030402u), zw);
    } else if constexpr (FMT == FMT_U8) {
        // bf16: q - z formed in fp32 (exact), rounded to bf16 pairs (exact)
        const float z = __builtin_bit_cast(float, zw);
        const uint32_t x0 = w[2 * J], x1 = w[2 * J + 1];
        r.x = u8_diff_bf16_pair<0>(x0, z);
        r.y = u8_diff_bf16_pair<2>(x0, z);
        r.z = u8_diff_bf16_pair<0>(x1, z);
        r.w = u8_diff_bf16_pair<2>(x1, z);
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

// 8 activations (4 natural pairs) in the MFMA slot order PERM of MfAct.
template <int PERM>
__device__ __forceinline__ u4v slot_order(const u4v &v) {
    u4v o;
    if constexpr (PERM == 1) {
        o.x = perm(v.z, v.x, 0x05040100u);  // (a0, a4)
        o.y = perm(v.z, v.x, 0x07060302u);  // (a1, a5)
        o.z = perm(v.w, v.y, 0x05040100u);  // (a2, a6)
        o.w = perm(v.w, v.y, 0x07060302u);  // (a3, a7)
    } else if constexpr (PERM == 2) {
        o.x = perm(v.y, v.x, 0x05040100u);  // (a0, a2)
        o.y = perm(v.w, v.z, 0x05040100u);  // (a4, a6)
        o.z = perm(v.y, v.x, 0x07060302u);  // (a1, a3)
        o.w = perm(v.w, v.z, 0x07060302u);  // (a5, a7)
    } else {
        o = v;
    }
    return o;
}

// A operand of MFMA j for row group rg: lane (i, gs) with i>>2 == gs holds row
// 4*rg + (i&3) over the 8 k the weights of chunk 4t+gs use in MFMA j; zero elsewhere.
template <int FMT, int ACT>
__device__ __forceinline__ op4 load_a(const uint16_t *arow, bool live, uint32_t k0) {
    op4 r = {0u, 0u, 0u, 0u};
    if (live) {
        const u4v v = slot_order<MfAct<FMT, ACT>::PERM>(load16(arow + k0));
        r.x = v.x; r.y = v.y; r.z = v.z; r.w = v.w;
    }
    return r;
}

// Block metadata of one chunk kept raw while it waits in the prefetch ring: the
// loaded values as they are (nothing is computed from a load until the chunk is
// consumed, so a prefetch never waits for its own data), decoded by meta_scale and
// meta_zero.
//   U4, one block per chunk : v0 = fp16 scale bits, v1 = the zero-point byte holding the block
//   U4, two blocks per chunk: v0 = both fp16 scales, v1 = the zero-point byte of the pair
//   U8                      : v0 = fp16 scale bits, v1 = zero-point byte
//   FP8                     : v0 = fp32 scale bits
//   NVFP4                   : v0 = the two E4M3 scale bytes
// (without zero points v1 holds whatever the aliased address held; meta_zero then
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

// Scale of half h of a chunk from its raw metadata word v0 (as MetaRaw holds it).
template <int FMT, int H>
__device__ __forceinline__ float meta_scale(uint32_t v0, int h) {
    if constexpr (FMT == FMT_U4) {
        if constexpr (H == 1) return half_bits_to_float((uint16_t)(v0 & 0xFFFFu));
        else return half_bits_to_float((uint16_t)(h ? (v0 >> 16) : (v0 & 0xFFFFu)));
    } else if constexpr (FMT == FMT_U8) {
        return half_bits_to_float((uint16_t)(v0 & 0xFFFFu));
    } else if constexpr (FMT == FMT_FP8) {
        return __builtin_bit_cast(float, v0);
    } else {
        return e4m3_to_float(h ? ((v0 >> 8) & 0xFFu) : (v0 & 0xFFu));
    }
}

// Integer zero point of half h of a chunk from its raw zero-point word v1 (the
// midpoint when the weight has none; 0 for the formats without). zsh is the bit
// position of the chunk's zero-point nibble in v1 for 4-bit codes with one block per
// chunk (4 for an odd block index, else 0).
template <int FMT, int H>
__device__ __forceinline__ uint32_t meta_zero(const KArgs &a, uint32_t v1, int zsh, int h) {
    if constexpr (FMT == FMT_U4) {
        const ZSel zs = zsel(a.zp, 0x88u);
        const uint32_t zb = (v1 & zs.keep) | zs.fill;
        if constexpr (H == 1) return (zb >> zsh) & 0x0Fu;
        else return h ? ((zb >> 4) & 0x0Fu) : (zb & 0x0Fu);
    } else if constexpr (FMT == FMT_U8) {
        const ZSel zs = zsel(a.zp, 128u);
        return ((v1 & zs.keep) | zs.fill) & 0xFFu;
    } else {
        return 0u;
    }
}

// The B operands of every MFMA of a chunk, decoded with their half's zero point.
template <int FMT, int ACT, int H>
__device__ __forceinline__ void decode_chunk(const u4v &w, const uint32_t (&z)[H], op4 (&bv)[MfFmt<FMT>::MF]) {
    // MFMAs 0 .. MF/2 - 1 lie in half 0, the rest in half H - 1
    const uint32_t z0 = zero_word<FMT, ACT>(z[0]);
    const uint32_t z1 = H == 2 ? zero_word<FMT, ACT>(z[H - 1]) : z0;
    bv[0] = decode_b<FMT, ACT, 0>(w, z0);
    bv[1] = decode_b<FMT, ACT, 1>(w, MfFmt<FMT>::MF == 4 ? z0 : z1);
    if constexpr (MfFmt<FMT>::MF == 4) {
        bv[2] = decode_b<FMT, ACT, 2>(w, z1);
        bv[3] = decode_b<FMT, ACT, 3>(w, z1);
    }
}

// Zero-point nibble position of chunk c (4-bit codes, one block per chunk).
__device__ __forceinline__ int u4_zshift(const KArgs &a, int c) {
    return (((c << 5) >> a.bs_shift) & 1) << 2;
}

// One output group's epilogue: acc += s * (d - z * sa) (the zero-point term only for
// the ASUM format; the others hold q - z in d already). Shared by every
// matrix-family kernel.
template <bool ASUM>
__device__ __forceinline__ void epilogue(const f4 &d, const f4 &sa, float sc, uint32_t z, f4 &acc) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float v = d[r];
        if constexpr (ASUM) v = __builtin_fmaf(-(float)z, sa[r], v);
        acc[r] = __builtin_fmaf(sc, v, acc[r]);
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

// Padding of a staged activation row in LDS (elements): shifts consecutive rows by
// 16 bytes so the 16 live lanes of an A-operand read hit distinct banks.
constexpr int kAPad = 8;

// LDS layout of the kernels that stage the activations: a 64-byte zero block (the A
// operand of lanes off the block diagonal, MF reads of 16 bytes), the staged rows,
// then for the ASUM format (4-bit codes on bf16) the per-chunk activation sums (f4
// entries indexed (chunk * RG + row group) * H + half), then the kernel's own area.
constexpr int kZeroBytes = 64;

__device__ __forceinline__ size_t staged_rows_bytes(const KArgs &a, int astride) {
    return ((size_t)a.M * astride * 2 + 15) & ~(size_t)15;
}

template <int FMT, int ACT, int RG, int H>
__device__ __forceinline__ size_t sums_bytes(size_t nch) {
    return MfAct<FMT, ACT>::ASUM ? nch * RG * H * 16 : 0;
}

// One wave owns the 16 columns of a tile for one K slice. A workgroup of nw waves
// holds nw / ksplit tiles; the ksplit waves of a tile take K steps t = kslice,
// kslice + ksplit, ... and reduce in LDS in wave order.
// One K step of one wave: the chunk c = 4t + g of each of the 16 columns (already in
// w, with its raw block metadata m), multiplied by every row group of A. Staged
// activations (and their sums) start at chunk cbase of the row. Shared by both
// kernels below so that they compute bit-identical results.
// A operands of one K step for every row group, loaded from global memory (used ahead
// of time by the register-ring kernel when the activations are not staged in LDS).
template <int FMT, int RG>
struct AOps {
    op4 v[RG][MfFmt<FMT>::MF];
};

// Every lane loads (rows past M read row M - 1); lanes off the block diagonal or past
// M are zeroed when the operands are used (mfma_step), so the loads themselves are
// unconditional.
template <int FMT, int ACT, int RG>
__device__ __forceinline__ void load_a_ops(const KArgs &a, int c, int ar, AOps<FMT, RG> &o) {
    using F = MfFmt<FMT>;
    const uint16_t *A16 = (const uint16_t *)a.A;
    const uint32_t kbase = (uint32_t)c * F::KPC;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int row = 4 * rg + ar;
        const uint16_t *arow = A16 + (int64_t)(row < a.M ? row : a.M - 1) * a.K;
#pragma unroll
        for (int j = 0; j < F::MF; ++j) o.v[rg][j] = load_a<FMT, ACT>(arow, true, kbase + 8 * j);
    }
}

// The ones-operand MFMA chain that sums the activations of one row group over a
// chunk (per half h with two scale blocks per chunk): element r of lane (n, g) gets
// row 4 * rg + r of chunk 4t + g. Run per K step by the kernels that load the
// activations into registers, and once per chunk into the LDS sum table by the ones
// that stage them, so both see the same bits.
template <int FMT, int ACT, int H>
__device__ __forceinline__ void chunk_sums(const op4 (&av)[MfFmt<FMT>::MF], f4 (&sa)[H]) {
    using F = MfFmt<FMT>;
    constexpr uint32_t ONE = (ACT == ACT_F16) ? 0x3C003C00u : 0x3F803F80u;
    const op4 ones = {ONE, ONE, ONE, ONE};
#pragma unroll
    for (int h = 0; h < H; ++h) sa[h] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < F::MF; ++j) {
        const int h = (H == 2) ? (j / (F::MF / 2)) : 0;
        sa[h] = mfma<ACT>(av[j], ones, sa[h]);
    }
}

template <int FMT, int ACT, int RG, int H, bool LDSA>
__device__ __forceinline__ void mfma_step(const KArgs &a, const u4v &w, const MetaRaw<H> &m, int c, int ar,
                                          bool a_live_grp, const uint16_t *sA, const uint16_t *sZero,
                                          const f4 *sSum, int astride, int cbase, const AOps<FMT, RG> &areg,
                                          bool valid, f4 acc[RG]) {
    using F = MfFmt<FMT>;
    constexpr bool ASUM = MfAct<FMT, ACT>::ASUM;
    // A discarded step (past K, or a tile past N, both on clamped valid addresses)
    // gets a zero scale: it adds 0 * (a finite value) to the accumulators, which
    // leaves them as they are, with one select per step instead of one per element.
    const uint32_t v0 = valid ? m.v[0] : 0u;
    const int zsh = (FMT == FMT_U4 && H == 1) ? u4_zshift(a, c) : 0;
    uint32_t zq[H];
#pragma unroll
    for (int h = 0; h < H; ++h) zq[h] = meta_zero<FMT, H>(a, m.v[1], zsh, h);
    // with one row group the B operands are decoded right before their MFMA; with
    // more they are decoded once and shared by the groups
    op4 bv[F::MF];
    if constexpr (RG > 1) decode_chunk<FMT, ACT, H>(w, zq, bv);
    const uint32_t kbase = (uint32_t)(c - cbase) * F::KPC;  // within the staged K range
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int row = 4 * rg + ar;
        const bool live = a_live_grp && row < a.M;
        f4 d[H], sa[H];
#pragma unroll
        for (int h = 0; h < H; ++h) d[h] = f4{0.f, 0.f, 0.f, 0.f};
        // staged activations: every lane reads (lanes outside the block diagonal read
        // the zero block), so the MF reads issue back to back without predication
        op4 avs[F::MF];
        if constexpr (LDSA) {
            const uint16_t *abase = live ? sA + row * astride + kbase : sZero;
#pragma unroll
            for (int j = 0; j < F::MF; ++j) avs[j] = *(const op4 *)(abase + 8 * j);
            if constexpr (ASUM) {
#pragma unroll
                for (int h = 0; h < H; ++h) sa[h] = sSum[((size_t)(c - cbase) * RG + rg) * H + h];
            }
        } else {
            const op4 z = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < F::MF; ++j) avs[j] = live ? areg.v[rg][j] : z;
            if constexpr (ASUM) chunk_sums<FMT, ACT, H>(avs, sa);
        }
#pragma unroll
        for (int j = 0; j < F::MF; ++j) {
            const int h = (H == 2) ? (j / (F::MF / 2)) : 0;
            op4 b;
            if constexpr (RG == 1) {
                const uint32_t zw = zero_word<FMT, ACT>(zq[h]);
                if (j == 0) b = decode_b<FMT, ACT, 0>(w, zw);
                else if (j == 1) b = decode_b<FMT, ACT, 1>(w, zw);
                else if (j == 2) b = decode_b<FMT, ACT, (F::MF == 4 ? 2 : 0)>(w, zw);
                else b = decode_b<FMT, ACT, (F::MF == 4 ? 3 : 0)>(w, zw);
            } else {
                b = bv[j];
            }
            d[h] = mfma<ACT>(avs[j], b, d[h]);
        }
#pragma unroll
        for (int h = 0; h < H; ++h) epilogue<ASUM>(d[h], sa[h], meta_scale<FMT, H>(v0, h), zq[h], acc[rg]);
    }
}

// Fill the per-chunk activation-sum table (formats with zero points) from the staged
// rows: the waves of the workgroup take the nsteps staged K steps in turn and run
// chunk_sums on the same A operands mfma_step reads; lane (0, g) of each lane group
// stores its chunk's entry. The caller synchronizes the workgroup before and after.
template <int FMT, int ACT, int RG, int H>
__device__ __forceinline__ void stage_sums(const KArgs &a, const uint16_t *sA, const uint16_t *sZero, int astride,
                                           f4 *sSum, int nsteps) {
    using F = MfFmt<FMT>;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwv = (int)(blockDim.x >> 6);
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int ar = lane & 3;
    const bool a_live_grp = ((lane & 15) >> 2) == g;
    for (int t = wave; t < nsteps; t += nwv) {
        const int c = 4 * t + g;
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            const int row = 4 * rg + ar;
            const bool live = a_live_grp && row < a.M;
            const uint16_t *abase = live ? sA + row * astride + (uint32_t)c * F::KPC : sZero;
            op4 avs[F::MF];
#pragma unroll
            for (int j = 0; j < F::MF; ++j) avs[j] = *(const op4 *)(abase + 8 * j);
            f4 sa[H];
            chunk_sums<FMT, ACT, H>(avs, sa);
            if ((lane & 15) == 0) {
#pragma unroll
                for (int h = 0; h < H; ++h) sSum[((size_t)c * RG + rg) * H + h] = sa[h];
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

// The register ring loads codes in a coalesced lane order: lane l reads chunk
// 4t + (l & 3) of the tile's column l >> 2, so four neighbouring lanes read 64
// contiguous bytes of one column (in the MFMA order, lane n + 16g holding column n's
// chunk 4t + g, neighbouring lanes sit in different columns and every lane's load
// becomes its own cache and translation request). This moves a loaded chunk to its
// MFMA lane: lane m takes the chunk of load lane 4 (m & 15) + (m >> 4), one
// ds_bpermute per dword (a lane crossbar, no memory traffic).
__device__ __forceinline__ u4v to_mfma_lanes(const u4v &v, int src_byte) {
    u4v o;
    o.x = (uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)v.x);
    o.y = (uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)v.y);
    o.z = (uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)v.z);
    o.w = (uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)v.w);
    return o;
}

// The same move for a chunk's raw block metadata (the zero-point word only for the
// formats that have zero points).
template <int FMT, int H>
__device__ __forceinline__ MetaRaw<H> meta_to_mfma_lanes(const MetaRaw<H> &m, int src_byte) {
    MetaRaw<H> o;
    o.v[0] = (uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)m.v[0]);
    o.v[1] = (FMT == FMT_U4 || FMT == FMT_U8) ? (uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)m.v[1]) : 0u;
    return o;
}

// Stage k = k0 .. k0 + klen - 1 of the M activation rows into LDS once per
// workgroup, permuted into the MFMA slot order (row stride astride elements). Each
// thread handles 16-byte pieces it, it + blockDim, ... in batches of SB whose loads
// are all issued before the first store, so the staging costs about one load latency
// per batch, not one per piece.
template <int FMT, int ACT, int SB = 8>
__device__ __forceinline__ void stage_a(const KArgs &a, uint16_t *sA, int astride, int k0, int klen) {
    using F = MfFmt<FMT>;
    const uint16_t *A16 = (const uint16_t *)a.A + k0;
    const int K = (int)a.K;
    const int k8n = klen >> 3;
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
                *(u4v *)(sA + m * astride + k8) = slot_order<MfAct<FMT, ACT>::PERM>(v[j]);
            }
        }
    }
}

// K-split reduction over the ksplit waves of a tile (fixed wave order), then the sum
// over the four lane groups and the store of rows 4*rg + g.
//
// With K parts (XWG and a.kparts > 1; every wave of the workgroup calls this at the
// same point, for tile group tg, of which this workgroup holds part `part`), the
// K-part split across workgroups of "[CUDA] MatMul: add an opt-in split-K GEMV"
// (Cross-block reduction; review: cache-safe publication, one counter contract with
// an explicitly atomic reset):
//  1. publish: each row's fp32 partial goes to the workspace ([kparts, M, N]) by
//     agent-scope atomic stores (coherent for every compute unit), each wave waits
//     until its stores have completed, then a workgroup barrier;
//  2. count: one thread adds 1 to the tile group's counter with an agent-scope
//     release RMW (the one cache write-back of the workgroup); the workgroup that
//     brings it to kparts is the last: that thread takes the agent-scope acquire
//     fence, resets the counter with an atomic store and tells the waves through
//     LDS (a barrier orders their loads after the acquire);
//  3. reduce: the last workgroup's waves load the kparts partials with agent-scope
//     atomic loads and add them in part order
//     0, 1, ..., so the result does not depend on which workgroup finished last,
//     then store zeros over the partials they read. A completed run thus leaves the
//     whole workspace as it found it, all zero, whatever handle or M used it before.
// No workgroup waits for another: the last to arrive does the work.
//
// red_alias: the reduction area sR overlays the staged activations, so every wave
// waits at a barrier until all have finished their K steps before writing to it.
template <int ACT, int RG, bool XWG = true>
__device__ __forceinline__ void finish_tile(const KArgs &a, f4 acc[RG], float *sR, int wave, int lane, int ks,
                                            int kslice, int g, bool tile_ok, int64_t n, int part = 0,
                                            int64_t tg = 0, uint32_t *sFlag = nullptr, bool red_alias = false) {
    if (ks > 1) {
        if (red_alias) __syncthreads();
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
    const bool xwg = XWG && a.kparts > 1;
    // partial tiles [kparts, M, N]: 32-bit offsets (the dispatcher keeps
    // kparts * M * N below 2^31)
    const uint32_t pstride = (uint32_t)a.M * (uint32_t)a.N;
    uint32_t *part_u = (uint32_t *)a.part;
    if (kslice == 0 && tile_ok) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            float tot[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) tot[r] = sum_groups(acc[rg][r]);
            const float v = (g == 0) ? tot[0] : (g == 1) ? tot[1] : (g == 2) ? tot[2] : tot[3];
            const int row = 4 * rg + g;
            if (n < a.N && row < a.M) {
                if (!xwg)
                    store_out<ACT>(a.Y, (int64_t)row * a.N + n, add_bias<ACT>(a.bias, n, v * a.tscale));
                else
                    __hip_atomic_store(part_u + ((uint32_t)part * pstride + (uint32_t)row * (uint32_t)a.N + (uint32_t)n),
                                       __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    if (!xwg) return;
    // every wave's partial stores complete before the barrier; one release per
    // workgroup, on the counter
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t done = __hip_atomic_fetch_add(a.cnt + tg, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) + 1u;
        const bool last = done == (uint32_t)a.kparts;
        if (last) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            __hip_atomic_store(a.cnt + tg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        *sFlag = last ? 1u : 0u;
    }
    __syncthreads();
    if (*sFlag) {  // uniform over the workgroup
        if (kslice == 0 && tile_ok) {
            const uint32_t kpm1 = (uint32_t)a.kparts - 1u;
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                const int row = 4 * rg + g;
                if (n < a.N && row < a.M) {
                    // all eight loads issue unconditionally (parts past kparts - 1 re-read
                    // the last), then the first kparts are added in part order
                    const uint32_t base = (uint32_t)row * (uint32_t)a.N + (uint32_t)n;
                    uint32_t pv[8];
#pragma unroll
                    for (int p = 0; p < 8; ++p) {
                        const uint32_t pp = (uint32_t)p < kpm1 ? (uint32_t)p : kpm1;
                        pv[p] = __hip_atomic_load(part_u + (base + pp * pstride), __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
                    }
                    float v = __uint_as_float(pv[0]);
#pragma unroll
                    for (int p = 1; p < 8; ++p) {
                        const float w = v + __uint_as_float(pv[p]);
                        v = (uint32_t)p <= kpm1 ? w : v;
                    }
                    store_out<ACT>(a.Y, (int64_t)row * a.N + n, add_bias<ACT>(a.bias, n, v * a.tscale));
                    // each lane clears what it read (after its loads, same addresses)
#pragma unroll
                    for (int p = 0; p < 8; ++p) {
                        const uint32_t pp = (uint32_t)p < kpm1 ? (uint32_t)p : kpm1;
                        __hip_atomic_store(part_u + (base + pp * pstride), 0u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
        }
    }
    __syncthreads();  // the flag is written again at the next tile group
}

// Register-ring kernel. A workgroup of 8 waves holds 8 / ksplit tiles of ksplit waves
// each. Without K parts (KP 0) it walks tile groups blockIdx.x, + gridDim.x, ...
// over all of K. With K parts (KP 1 with a K split inside the workgroup, 2 without;
// a.kparts > 1; the grid is one workgroup per tile
// group and part), workgroup b takes tile group b / kparts and part b mod kparts of
// its K steps (a contiguous range, parts as even as whole steps allow), and the
// cross-workgroup finish runs once, after the ring has drained. Within a tile,
// wave kslice takes the part's K steps t = kslice, kslice + ksplit, ... Every wave
// of a workgroup runs the same S = ceil(ceil(part steps / ksplit) / P) * P slots per
// tile (a slot past the last step, or of a tile past N, computes on a clamped valid
// address and its accumulator update is discarded), so all waves reach the barriers
// of finish_tile together. The
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
template <int FMT, int ACT, int RG, int H, bool LDSA, int P, int KP>
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
    // K part of this workgroup: steps pbeg .. pbeg + nsteps - 1 (nsteps >= 1, as the
    // dispatcher takes at most one part per step); the tile-group walk of the part
    const uint32_t kp = KP != 0 ? (uint32_t)a.kparts : 1u;
    const uint32_t part = blockIdx.x % kp;
    const int64_t gx = blockIdx.x / kp;
    const int64_t gdim = gridDim.x / kp;
    const uint32_t steps_all = (uint32_t)(a.nchunks >> 2);
    const int pbeg = (int)(steps_all * part / kp);
    const int nsteps = (int)(steps_all * (part + 1) / kp) - pbeg;
    const int smax = (int)((steps_all + kp - 1) / kp);  // the longest part: the LDS layout
    const int cbase = 4 * pbeg;
    const int S = ((nsteps + ks - 1) / ks + P - 1) / P * P;
    const int astride = smax * 4 * MfFmt<FMT>::KPC + kAPad;
    const int64_t ntiles = (a.N + 15) >> 4;
    const int64_t ngroups = (ntiles + tpw - 1) / tpw;
    // LDS: [zero block | staged rows | activation sums] when staged, then the K-split
    // reduction area, then (with K parts) the last-workgroup flag. When the workgroup
    // holds a single tile group (always with K parts), the staged activations are dead
    // once its K steps are done, and the reduction area overlays them from byte 0.
    uint16_t *sZero = (uint16_t *)smem;
    uint16_t *sA = (uint16_t *)(smem + kZeroBytes);
    const size_t rows_b = LDSA ? staged_rows_bytes(a, astride) : 0;
    f4 *sSum = (f4 *)(smem + kZeroBytes + rows_b);
    const size_t abytes = LDSA ? kZeroBytes + rows_b + sums_bytes<FMT, ACT, RG, H>((size_t)4 * smax) : 0;
    const size_t red_b = ks > 1 ? (size_t)NW * RG * 4 * 64 * 4 : 0;
    const bool red_alias = LDSA && ks > 1 && (KP != 0 || gdim >= ngroups);
    float *sR = (float *)(red_alias ? smem : smem + abytes);
    uint32_t *sFlag = (uint32_t *)(smem + (red_alias ? (abytes > red_b ? abytes : red_b) : abytes + red_b));

    // issue cursor: tile group, slot within the tile, and the column the lane loads
    // codes and block metadata of, in the coalesced order of to_mfma_lanes (column
    // lane >> 2, chunk 4t + (lane & 3) of the step)
    int64_t itg = gx;
    int is = 0;
    auto icol = [&]() {
        const int64_t n = (itg * tpw + slot) * 16 + (lane >> 2);
        return mf_col<FMT>(a, n < a.N ? n : a.N - 1);
    };
    const int perm_src = ((lane & 15) * 4 + (lane >> 4)) * 4;  // ds_bpermute source byte
    MfCol col = icol();
    u4v wb[P];
    MetaRaw<H> mb[P];
    AOps<FMT, RG> ab[LDSA ? 1 : P];  // activations in the ring when they are not staged
    auto issue = [&](int p) {
        const int t0 = kslice + is * ks;
        const int c4 = 4 * (pbeg + (t0 < nsteps ? t0 : nsteps - 1));
        const int c = c4 + g;
        // A step reads 64 bytes of each column, half of a 128-byte line whose other half
        // the next step reads. Ordinary loads keep the line in the L2 for it; with
        // nontemporal ones about a third of the pairs both went to HBM (4-bit lm_head,
        // M = 16: 1.32x the weight bytes fetched, 1.008x with ordinary loads; 137.9 ->
        // 132.4 us; FP8 5120 x 6144 M = 8 16.0 -> 14.3 us). With K parts, nontemporal
        // loads measured faster where K is also split inside the workgroup (KP = 1: FP8
        // 1024 x 16384 M = 8: 14.5 against 15.1 us), whose waves walk strided steps;
        // without that split (KP = 2) a wave reads both halves itself and the ordinary
        // loads win again (FP8 8192 x 28672 M = 4 / 8: 69.6 / 80.1 -> 63.3 / 74.5 us;
        // 4-bit 8192 x 28672 M = 8 57.6 -> 53.9; 8-bit 8192 x 8192 M = 16 34.0 -> 31.7).
        const u4v *wp = (const u4v *)(col.w + (uint32_t)(c4 + (lane & 3)) * 16u);
        wb[p] = KP == 1 ? load16_stream(wp) : load16(wp);
        mb[p] = load_meta_raw<FMT, H>(a, col, c4 + (lane & 3));
        if constexpr (!LDSA) load_a_ops<FMT, ACT, RG>(a, c, ar, ab[p]);
        if (++is == S) {
            is = 0;
            itg += gdim;
            col = icol();
        }
    };
#pragma unroll
    for (int p = 0; p < P; ++p) issue(p);

    if constexpr (LDSA) {
        if (threadIdx.x < kZeroBytes / 16) ((u4v *)sZero)[threadIdx.x] = u4v{0u, 0u, 0u, 0u};
        stage_a<FMT, ACT>(a, sA, astride, cbase * MfFmt<FMT>::KPC, nsteps * 4 * MfFmt<FMT>::KPC);
        __syncthreads();
        if constexpr (MfAct<FMT, ACT>::ASUM) {
            stage_sums<FMT, ACT, RG, H>(a, sA, sZero, astride, sSum, nsteps);
            __syncthreads();
        }
    }

    // One ring turn = P slots. Every turn but the last consumes and refills each slot;
    // the last turn only drains the ring, so nothing is fetched past the wave's work.
    // Tile boundaries fall on turn boundaries (S is a multiple of P).
    const int64_t G = KP != 0 ? (gx < ngroups ? 1 : 0) : (gx < ngroups ? (ngroups - gx + gdim - 1) / gdim : 0);
    const int64_t turns = G * (S / P);
    const int tpt = S / P;  // turns per tile
    int64_t tg = gx;
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
            mfma_step<FMT, ACT, RG, H, LDSA>(a, to_mfma_lanes(wb[p], perm_src), meta_to_mfma_lanes<FMT, H>(mb[p], perm_src),
                                             4 * (pbeg + tc) + g, ar,
                                             a_live_grp, sA, sZero, sSum, astride, cbase, ab[LDSA ? 0 : p],
                                             tile_ok && t < nsteps, acc);
            if (refill) {
                // the slot's accumulation completes here (nothing of it may sink below
                // the refill), then the refill reuses the slot's registers
                pin_accumulators<RG>(acc);
                __builtin_amdgcn_sched_barrier(0);
                issue(p);
            }
        }
        if constexpr (KP == 0) {
            if (++tt == tpt) {
                finish_tile<ACT, RG, false>(a, acc, sR, wave, lane, ks, kslice, g, tile_ok, tile * 16 + (lane & 15), 0,
                                            0, nullptr, red_alias);
#pragma unroll
                for (int r = 0; r < RG; ++r) acc[r] = f4{0.f, 0.f, 0.f, 0.f};
                tt = 0;
                tg += gdim;
            }
        } else {
            ++tt;
        }
    };
    for (int64_t i = 0; i + 1 < turns; ++i) turn(true);
    if (turns > 0) turn(false);
    if constexpr (KP != 0) {
        // one tile group per workgroup: its finish, with nothing left in flight
        const int64_t tile = gx * tpw + slot;
        finish_tile<ACT, RG, true>(a, acc, sR, wave, lane, ks, kslice, g, tile < ntiles, tile * 16 + (lane & 15),
                                   (int)part, gx, sFlag, red_alias);
    }
}

// DMA-ring kernel for wide N without a K split. Each wave owns 16-column tiles
// (tiles gw, gw + nwaves, ...) over the whole of K. Codes and block metadata travel
// global -> LDS by DMA (global_load_lds) in slots of SS K steps (CS = 4 * SS chunks
// of each of the 16 columns), R slots per wave and R - 1 in flight, so the prefetch
// depth costs no VGPRs and the waits are exact load counts. The launcher takes SS = 4
// and R = 2 (the next slot loads while the current one computes) or 3.
//  - Coalescing: one code DMA instruction moves 64 / CS whole columns' CS chunks
//    (CS * 16 contiguous bytes each, whole cache lines), not 16 columns' 64-byte
//    pieces. Which lane fetches which chunk is permuted (chunk j of column n lands
//    at position j ^ (n mod CS)), so that the MFMA-order reads of a step, where the
//    16 columns ask for the same chunk, fall in 16 distinct LDS bank groups.
//  - Metadata: each column's scale bytes of the slot (and zero-point bytes) are one
//    contiguous window of the row, copied as whole dwords; a chunk's raw metadata is
//    then cut from LDS in the form load_meta_raw gives.
//  - Every K step keeps the chunk -> (step, lane group) assignment of k_mfma (step t,
//    lane group g: chunk 4t + g) and calls the same mfma_step, so results are
//    bit-identical to k_mfma with no K split.
template <int FMT, int SS, int H>
struct DmaGeom {
    static constexpr int CS = 4 * SS;                      // chunks per column per slot
    static constexpr int CPD = 64 / CS;                    // columns per code DMA
    static constexpr int DSTRIDE = SS == 4 ? 1024 : 1152;  // bytes per code DMA block (+pad)
    static constexpr int CODEB = (16 / CPD) * DSTRIDE;     // code bytes per slot
    // scale-window DMAs per slot: the most the format's block sizes need (16 columns
    // x the slot's scale bytes, 256 bytes per DMA); FP8 takes 16-wide blocks, 4-bit
    // codes with one block per chunk at most 16 per 512 k
    static constexpr int NSD = (FMT == FMT_FP8 || (FMT == FMT_U4 && H == 2)) ? (SS == 4 ? 4 : 2) : (SS == 4 ? 2 : 1);
};

template <int FMT, int ACT, int RG, int H, bool ZPP, int R, int SS>
__global__ void __launch_bounds__(512, 1) k_mfma_dma(KArgs a) {
    using Gm = DmaGeom<FMT, SS, H>;
    using F = MfFmt<FMT>;
    constexpr int NW = 8;
    constexpr int CS = Gm::CS;
    constexpr int SLOT = Gm::CODEB + 256 * Gm::NSD + (ZPP ? 256 : 0);
    constexpr int SB = (FMT == FMT_FP8) ? 4 : ((FMT == FMT_NVFP4) ? 1 : 2);  // scale bytes
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int ar = lane & 3;
    const bool a_live_grp = (n >> 2) == g;
    const int nch = (int)a.nchunks;
    const int nslots = (nch + CS - 1) / CS;
    const int astride = (int)a.K + kAPad;
    const int64_t ntiles = (a.N + 15) >> 4;
    const int64_t nw = (int64_t)gridDim.x * NW;
    const int64_t gw = (int64_t)blockIdx.x * NW + wave;
    const int64_t mytiles = gw < ntiles ? (ntiles - gw + nw - 1) / nw : 0;
    const int64_t total = mytiles * nslots;
    constexpr bool ASUM = MfAct<FMT, ACT>::ASUM;
    const size_t abytes = kZeroBytes + staged_rows_bytes(a, astride) + sums_bytes<FMT, ACT, RG, H>((size_t)a.nchunks);
    uint16_t *sZero = (uint16_t *)smem;
    uint16_t *sA = (uint16_t *)(smem + kZeroBytes);
    f4 *sSum = (f4 *)(smem + kZeroBytes + staged_rows_bytes(a, astride));
    unsigned char *ring = smem + abytes + (size_t)wave * R * SLOT;

    // per-slot metadata windows (uniform): blocks per slot (slots hold whole blocks:
    // the dispatcher ensures CS * KPC >= block size), bytes per column, dwords
    const int bps = (H == 2) ? 2 * CS : ((CS * F::KPC) >> a.bs_shift);
    const int sbc = bps * SB;
    const int mds = sbc >= 4 ? sbc / 4 : 1;
    const int nsd = (16 * mds + 63) / 64;
    const int zbc = (FMT == FMT_U4) ? (bps >> 1) : bps;
    const int mdz = zbc >= 4 ? zbc / 4 : 1;
    const int srow = a.nblk * SB;                                     // scale row bytes
    const int zrow = a.zstride;                                       // zero-point row bytes
    constexpr int OPS = SS + Gm::NSD + (ZPP ? 1 : 0);                  // DMAs per slot

    // Lane constants of the DMA sources, relative to a uniform per-slot base address
    // (the tile's first column at the slot's first chunk or metadata dword): the
    // column part and the chunk (or dword) part, each clamped per slot with one min
    // against a uniform limit, so that a ragged tile re-reads column N - 1 and a
    // ragged slot the column's last chunk, as every load here stays in bounds.
    uint32_t ccol[16 / Gm::CPD], cchk[16 / Gm::CPD];
#pragma unroll
    for (int d = 0; d < 16 / Gm::CPD; ++d) {
        const int cn = d * Gm::CPD + lane / CS;
        ccol[d] = (uint32_t)cn * (uint32_t)a.col_bytes;
        cchk[d] = (uint32_t)((lane % CS) ^ (cn % CS)) * 16u;
    }
    // every slot issues all NSD scale DMAs (a DMA past the window's nsd repeats the
    // last one into an unused part of the area), so the DMA count per slot is a
    // compile-time constant and the waits are immediates
    uint32_t scol[Gm::NSD], sq4[Gm::NSD];
#pragma unroll
    for (int e = 0; e < Gm::NSD; ++e) {
        const int idx = (e < nsd ? e : nsd - 1) * 64 + lane;
        int cn = idx / mds, q = idx - (idx / mds) * mds;
        if (cn > 15) cn = 15, q = mds - 1;
        scol[e] = (uint32_t)(cn * srow);
        sq4[e] = (uint32_t)(4 * q);
    }
    uint32_t zcol = 0, zq4 = 0;
    if constexpr (ZPP) {
        int cn = lane / mdz, q = lane - (lane / mdz) * mdz;
        if (cn > 15) cn = 15, q = mdz - 1;
        zcol = (uint32_t)(cn * zrow);
        zq4 = (uint32_t)(4 * q);
    }

    // issue cursor: tile, slot within the column, ring buffer, and the tile's
    // first-column addresses and column clamps (uniform; advanced per tile)
    int64_t itile = gw;
    int isl = 0, iring = 0;
    const uint8_t *wt = a.W + gw * 16 * a.col_bytes;
    const uint8_t *st = (const uint8_t *)a.scales + gw * 16 * srow;
    const uint8_t *zt = ZPP ? a.zp + gw * 16 * zrow : nullptr;
    uint32_t limcw = 0, limcs = 0, limcz = 0;
    auto tile_limits = [&]() {
        const int64_t lastc = a.N - 1 - itile * 16;
        const uint32_t limc = (uint32_t)(lastc < 15 ? lastc : 15);  // last column in the tile
        limcw = limc * (uint32_t)a.col_bytes;
        limcs = limc * (uint32_t)srow;
        limcz = limc * (uint32_t)zrow;
    };
    tile_limits();
    auto issue = [&]() {
        unsigned char *slot = ring + iring * SLOT;
        // codes: DMA d moves columns d*CPD .. d*CPD + CPD - 1, nontemporal (read once;
        // measured against cached copies: 4-bit lm_head M = 2 65.9 -> 61.1 us, M = 8 84.1
        // -> 81.4; NVFP4 lm_head M = 1 50.2 -> 45.5, M = 4 54.2 -> 48.5). The metadata
        // copies below stay cached: a column's consecutive slots read neighbouring
        // windows of the same lines.
        const uint8_t *wbase = wt + isl * (CS * 16);
        const uint32_t limj = (uint32_t)(nch - 1 - isl * CS) * 16u;
#pragma unroll
        for (int d = 0; d < 16 / Gm::CPD; ++d) {
            const uint32_t off = (ccol[d] < limcw ? ccol[d] : limcw) + (cchk[d] < limj ? cchk[d] : limj);
            dma_to_lds<16, true>(wbase + off, slot + d * Gm::DSTRIDE);
        }
        // scale windows: dword q of column cn's window
        const int wbs = (isl * sbc) & ~3;
        const uint8_t *sbase = st + wbs;
        const uint32_t limq = (uint32_t)(srow - wbs - 4);
#pragma unroll
        for (int e = 0; e < Gm::NSD; ++e) {
            const uint32_t off = (scol[e] < limcs ? scol[e] : limcs) + (sq4[e] < limq ? sq4[e] : limq);
            dma_to_lds<4>(sbase + off, slot + Gm::CODEB + e * 256);
        }
        if constexpr (ZPP) {
            const int zb0 = (FMT == FMT_U4) ? ((isl * bps) >> 1) : isl * bps;
            const int wbz = zb0 & ~3;
            const uint8_t *zbase = zt + wbz;
            const uint32_t limqz = (uint32_t)(zrow - wbz - 4);
            const uint32_t off = (zcol < limcz ? zcol : limcz) + (zq4 < limqz ? zq4 : limqz);
            dma_to_lds<4>(zbase + off, slot + Gm::CODEB + Gm::NSD * 256);
        }
        if (++iring == R) iring = 0;
        if (++isl == nslots) {
            isl = 0;
            itile += nw;
            wt += nw * 16 * a.col_bytes;
            st += nw * 16 * srow;
            if constexpr (ZPP) zt += nw * 16 * zrow;
            tile_limits();
        }
    };

    // the first R - 1 slots in flight, then the activations staged (the copy overlaps
    // the weight fetch)
    // (the zero block is stored first: an LDS store after the DMAs waits for them, as
    // the compiler cannot tell the DMAs' LDS writes from the store's address)
    if (threadIdx.x < kZeroBytes / 16) ((u4v *)sZero)[threadIdx.x] = u4v{0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < R - 1; ++r)
        if (r < total) issue();
    stage_a<FMT, ACT, 4>(a, sA, astride, 0, (int)a.K);
    __syncthreads();
    if constexpr (ASUM) {
        stage_sums<FMT, ACT, RG, H>(a, sA, sZero, astride, sSum, nch >> 2);
        __syncthreads();
    }

    // Consumer lane constants. Step s of a slot is the lane's chunk j = 4s + g of the
    // slot's CS: its code bytes at cofs[s] in the slot, its scale (zero-point) bytes at
    // sofs[s] (zofs[s]) from the start of the slot plus the window's sub-dword start,
    // the bit of its zero-point nibble zsh[s]; the A operands of row group rg at
    // abase[rg] plus the step's K offset (kept at the zero block off the block diagonal
    // by amask), the activation sums at sumb plus the step's chunk.
    uint32_t cofs[SS], sofs[SS], zofs[SS];
    int zsh[SS];
#pragma unroll
    for (int st = 0; st < SS; ++st) {
        const int j = 4 * st + g;
        const int lb = (H == 2) ? 2 * j : ((j * F::KPC) >> a.bs_shift);  // first block of the chunk
        cofs[st] = (uint32_t)((n / Gm::CPD) * Gm::DSTRIDE + ((n % Gm::CPD) * CS + (j ^ (n % CS))) * 16);
        sofs[st] = (uint32_t)(Gm::CODEB + n * mds * 4 + lb * SB);
        zofs[st] = (uint32_t)(Gm::CODEB + Gm::NSD * 256 + n * mdz * 4 + ((FMT == FMT_U4) ? (lb >> 1) : lb));
        zsh[st] = (FMT == FMT_U4 && H == 1) ? ((lb & 1) << 2) : 0;
    }
    const unsigned char *abase[RG];
    uint32_t amask[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int row = 4 * rg + ar;
        const bool live = a_live_grp && row < a.M;
        abase[rg] = live ? (const unsigned char *)(sA + row * astride + g * F::KPC) : (const unsigned char *)sZero;
        amask[rg] = live ? 0xFFFFFFFFu : 0u;
    }
    const f4 *sumb = sSum + g * (RG * H);

    // Operands of one K step, read from LDS one step ahead of their use (the A
    // operands too, except with two row groups and two scale blocks per chunk, where
    // a second set would not fit in the registers: those are read at their use).
    constexpr bool PREA = !(RG == 2 && H == 2);
    struct In {
        u4v w;
        uint32_t sv, zv;
        int kc;
        op4 av[PREA ? RG : 1][F::MF];
        f4 sa[RG][H];
    };
    auto read_a = [&](int kc, int rg, op4 (&av)[F::MF]) {
        const unsigned char *ap = abase[rg] + (((uint32_t)kc * (F::KPC * 2)) & amask[rg]);
#pragma unroll
        for (int j = 0; j < F::MF; ++j) av[j] = *(const op4 *)(ap + 16 * j);
    };
    // st: step within the slot; kc: the step's first chunk in the column (uniform)
    auto read_step = [&](const unsigned char *slot, int st, int kc, int ssub, int zsub, In &o) {
        o.w = *(const u4v *)(slot + cofs[st]);
        if constexpr (SB == 4 || (FMT == FMT_U4 && H == 2)) o.sv = *(const uint32_t *)(slot + sofs[st] + ssub);
        else o.sv = *(const uint16_t *)(slot + sofs[st] + ssub);
        o.zv = 0u;
        if constexpr (ZPP) o.zv = *(const uint8_t *)(slot + zofs[st] + zsub);
        // a step past K (ragged last slot) reads the last step's activations and sums:
        // finite values, discarded by the zero scale (nch is a multiple of 4)
        kc = kc < nch - 4 ? kc : nch - 4;
        o.kc = kc;
        if constexpr (PREA) {
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) read_a(kc, rg, o.av[rg]);
        }
        if constexpr (ASUM) {
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                for (int h = 0; h < H; ++h) o.sa[rg][h] = sumb[(size_t)kc * (RG * H) + rg * H + h];
        }
    };
    // The arithmetic of mfma_step on the operands read (valid: the step lies within K)
    f4 acc[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) acc[r] = f4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const In &o, int st, bool valid) {
        const uint32_t v0 = valid ? o.sv : 0u;
        float sc[H];
        uint32_t zq[H];
#pragma unroll
        for (int h = 0; h < H; ++h) {
            sc[h] = meta_scale<FMT, H>(v0, h);
            zq[h] = meta_zero<FMT, H>(a, o.zv, zsh[st], h);
        }
        op4 bv[F::MF];
        decode_chunk<FMT, ACT, H>(o.w, zq, bv);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            f4 d[H];
#pragma unroll
            for (int h = 0; h < H; ++h) d[h] = f4{0.f, 0.f, 0.f, 0.f};
            op4 avl[F::MF];
            if constexpr (!PREA) read_a(o.kc, rg, avl);
#pragma unroll
            for (int j = 0; j < F::MF; ++j) {
                const int h = (H == 2) ? (j / (F::MF / 2)) : 0;
                d[h] = mfma<ACT>(PREA ? o.av[PREA ? rg : 0][j] : avl[j], bv[j], d[h]);
            }
#pragma unroll
            for (int h = 0; h < H; ++h) {
                const f4 z4 = {0.f, 0.f, 0.f, 0.f};
                epilogue<ASUM>(d[h], ASUM ? o.sa[rg][h] : z4, sc[h], zq[h], acc[rg]);
            }
        }
    };

    // slot i's DMAs are done once at most the later issued slots' remain
    auto wait_slot = [&](int64_t i) { wait_slots<R - 2, OPS>(total - 1 - i); };
    auto win_ssub = [&](int sl) { return (sl * sbc) & 3; };  // nonzero only for windows under a dword
    auto win_zsub = [&](int sl) { return ((FMT == FMT_U4) ? ((sl * bps) >> 1) : sl * bps) & 3; };

    int64_t ctile = gw;
    int csl = 0, cring = 0;
    // two operand sets, by step parity: step st computes on opd[st & 1] while the next
    // step is read into the other; a slot has an even number of steps, so the next
    // slot's first step lands in opd[0], where the loop expects it (no copy of the
    // operands across the loop's back edge)
    static_assert(SS % 2 == 0, "the operand sets alternate by step parity");
    In opd[2];
    if (total > 0) {
        wait_slot(0);
        read_step(ring, 0, 0, win_ssub(0), win_zsub(0), opd[0]);
    }
#pragma unroll 1
    for (int64_t i = 0; i < total; ++i) {
        const unsigned char *slot = ring + cring * SLOT;
        const int nring = cring + 1 == R ? 0 : cring + 1;
        // refill the slot consumed in the previous iteration (all its reads have
        // returned: the last was waited for by that iteration's last step)
        if (i + R - 1 < total) issue();
        const int ssub = win_ssub(csl), zsub = win_zsub(csl);
#pragma unroll
        for (int st = 0; st < SS; ++st) {
            In &nxt = opd[(st + 1) & 1];
            if (st + 1 < SS) {
                read_step(slot, st + 1, csl * CS + 4 * (st + 1), ssub, zsub, nxt);
            } else if (i + 1 < total) {
                // the next slot's first step: wait for its DMAs, then read it
                const int nsl = csl + 1 == nslots ? 0 : csl + 1;
                wait_slot(i + 1);
                read_step(ring + nring * SLOT, 0, nsl * CS, win_ssub(nsl), win_zsub(nsl), nxt);
            }
            compute(opd[st & 1], st, csl * CS + 4 * st < nch);
        }
        cring = nring;
        if (++csl == nslots) {
            finish_tile<ACT, RG, false>(a, acc, nullptr, wave, lane, 1, 0, g, true, ctile * 16 + n);
#pragma unroll
            for (int r = 0; r < RG; ++r) acc[r] = f4{0.f, 0.f, 0.f, 0.f};
            csl = 0;
            ctile += nw;
        }
    }
}

namespace {

template <int FMT, int ACT, int RG, int H, bool LDSA, int P>
hipError_t go_p(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    // K parts: with a K split inside the workgroup (1) or without (2)
    const int kp = a.kparts > 1 ? (a.ksplit > 1 ? 1 : 2) : 0;
    auto kern = kp == 1   ? k_mfma<FMT, ACT, RG, H, LDSA, P, 1>
                : kp == 2 ? k_mfma<FMT, ACT, RG, H, LDSA, P, 2>
                          : k_mfma<FMT, ACT, RG, H, LDSA, P, 0>;
    static std::atomic<uint64_t> lds_set[3] = {{0}, {0}, {0}};  // per kernel
    hipError_t e = lds_limit_once((const void *)kern, cfg.device, cfg.lds_bytes, lds_set[kp]);
    if (e != hipSuccess) return e;
    return launch_or_report(cfg, kern, 512, a, s);
}

// Ring depth when the activations travel in the ring too: as deep as the register
// budget allows without spilling (each slot then holds RG * MF activation operands).
template <int FMT, int RG>
constexpr int ring_depth_with_a() {
    return (MfFmt<FMT>::MF == 2 && RG <= 3) ? 4 : ((MfFmt<FMT>::MF == 4 && RG == 4) ? 1 : 2);
}

// Depth with staged activations: variant bit 3 asks for 8 slots, which tiles of one or
// two row groups with one scale block per chunk afford (not one row group of a 32-k
// chunk format, whose decode constants take the room); the rest take 4 (2 for three or
// four row groups with two scale blocks per chunk), the most that fit without spilling.
template <int FMT, int RG, int H>
constexpr int ring_depth_staged(bool deep) {
    return (RG <= 2 && H == 1 && !(MfFmt<FMT>::MF == 4 && RG == 1)) ? (deep ? 8 : 4)
                                                                     : ((RG <= 2 || H == 1) ? 4 : 2);
}

// register-ring depth (ring_depth_staged / ring_depth_with_a); 8-wave workgroups
template <int FMT, int ACT, int RG, int H, bool LDSA>
hipError_t go(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    if (cfg.waves_per_wg != 8) return hipErrorInvalidValue;
    if constexpr (LDSA) {
        constexpr int PD = ring_depth_staged<FMT, RG, H>(true), PS = ring_depth_staged<FMT, RG, H>(false);
        return ((cfg.variant >> 3) & 1) ? go_p<FMT, ACT, RG, H, LDSA, PD>(cfg, a, s)
                                        : go_p<FMT, ACT, RG, H, LDSA, PS>(cfg, a, s);
    } else {
        return go_p<FMT, ACT, RG, H, LDSA, ring_depth_with_a<FMT, RG>()>(cfg, a, s);
    }
}

template <int FMT, int ACT, int RG, int H, bool ZPP, int R, int SS>
hipError_t go_dma_rs(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    auto kern = k_mfma_dma<FMT, ACT, RG, H, ZPP, R, SS>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = lds_limit_once((const void *)kern, cfg.device, cfg.lds_bytes, lds_set);
    if (e != hipSuccess) return e;
    return launch_or_report(cfg, kern, 512, a, s);
}

// DMA ring: 4-step slots, two or three per wave; one or two row groups only
template <int FMT, int ACT, int RG, int H, bool ZPP>
hipError_t go_dma(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    if (cfg.waves_per_wg != 8 || cfg.ksplit != 1) return hipErrorInvalidValue;
    if constexpr (RG <= 2) {
        // variant bit 2: three slots per wave (the dispatcher's depth rule), else two
        return (cfg.variant & 4) ? go_dma_rs<FMT, ACT, RG, H, ZPP, 3, 4>(cfg, a, s)
                                 : go_dma_rs<FMT, ACT, RG, H, ZPP, 2, 4>(cfg, a, s);
    } else {
        return hipErrorInvalidValue;
    }
}

template <int FMT, int ACT, int RG, int H>
hipError_t pick_lds(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    if (cfg.variant & 2) {
        if constexpr (FMT == FMT_U4 || FMT == FMT_U8)
            return a.zp ? go_dma<FMT, ACT, RG, H, true>(cfg, a, s) : go_dma<FMT, ACT, RG, H, false>(cfg, a, s);
        else
            return go_dma<FMT, ACT, RG, H, false>(cfg, a, s);
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
    case FMT_U8: return pick_act<FMT_U8>(cfg, a, s);
    case FMT_FP8: return pick_act<FMT_FP8>(cfg, a, s);
    case FMT_NVFP4: return pick_act<FMT_NVFP4>(cfg, a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qgemv
