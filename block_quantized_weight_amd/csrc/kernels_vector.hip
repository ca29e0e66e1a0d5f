// Vector kernels of qgemv for gfx950: the streaming family and the generic fallback.
//
// Streaming family ("[CUDA] MatMulNBits 8-bit: wide fp16 M=1 kernel", Description;
// "[CUDA] Block-scaled MatMul decode GEMV", FP4 row-tiling paragraph):
//  - a wave owns CPW output columns; each lane takes 16-byte chunks of every column
//    (chunk c = lane + 64*j), so a wave-wide load moves 1 KiB of contiguous codes;
//  - UNR chunks per lane are issued before any is consumed, and the block scales and
//    zero points are read straight from global memory (no LDS staging, no barrier);
//  - MT rows of A share every weight load, decode and scale (row tiling), and the
//    whole M range is covered in ceil(M/MT) passes, so each weight byte is read once
//    per pass, never once per row; the classic kernel's code loads are ordinary
//    (cached) loads, so a later pass finds the weight in the caches (the weights it
//    takes are small: 5-18% faster than nontemporal loads on every shape measured,
//    e.g. 4-bit 1024 x 2048 M = 8 6.54 -> 6.21 us, FP8 1024 x 4096 M = 16 15.2 -> 12.4);
//  - per-row arithmetic (decode, dot order, scale application, wave reduction) does
//    not depend on MT, CPW or the row's position, so a row's result is bit-identical
//    whatever tile carries it;
//  - the 64 lane partials of a column are summed with a fixed DPP tree.
//
// Generic family: one wave per column, one element per lane step, any alignment and
// any K that is a multiple of the block size. Correct and slow; used only when the
// streaming family's preconditions do not hold.
#include "chunk_ops.h"
#include "launch.h"

namespace qgemv {

template <int FMT, int ACT, int MT, int CPW, int UNR, int H>
__global__ void __launch_bounds__(256) k_stream(KArgs a) {
    using Ops = ChunkOps<FMT, ACT, H>;
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t nbase = wave * CPW;
    if (nbase >= a.N) return;  // uniform per wave

    ColPtrs cp[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) cp[i] = col_ptrs<FMT>(a, (nbase + i < a.N) ? nbase + i : a.N - 1);
    const int nch = (int)a.nchunks;

    for (int m0 = 0; m0 < a.M; m0 += MT) {
        const uint16_t *arow[MT];
        bool rlive[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            rlive[m] = m0 + m < a.M;
            arow[m] = (const uint16_t *)a.A + (int64_t)(rlive[m] ? m0 + m : 0) * a.K;
        }
        float acc[CPW][MT];
#pragma unroll
        for (int i = 0; i < CPW; ++i)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[i][m] = 0.0f;

        for (int base = 0; base < nch; base += 64 * UNR) {
            u4v w[UNR][CPW];
            float sc[UNR][CPW][H];
            uint32_t zr[UNR][CPW][H];
            bool valid[UNR];
            // all weight loads of this round first, then the block metadata
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int c = base + 64 * u + lane;
                valid[u] = c < nch;
                if (valid[u]) {
#pragma unroll
                    for (int i = 0; i < CPW; ++i) w[u][i] = load16(cp[i].w + (uint32_t)c * 16u);
                }
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int c = base + 64 * u + lane;
                if (valid[u]) {
#pragma unroll
                    for (int i = 0; i < CPW; ++i) chunk_meta<FMT, H>(a, cp[i], c, sc[u][i], zr[u][i]);
                }
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                if (!valid[u]) continue;
                const int c = base + 64 * u + lane;
                ChunkAct act[MT];
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    uint32_t x[Ops::ND];
                    if (rlive[m]) {
                        const uint16_t *ap = arow[m] + (uint32_t)c * (uint32_t)Ops::KPC;
#pragma unroll
                        for (int q = 0; q < Ops::ND / 4; ++q) {
                            const u4v v = load16(ap + 8 * q);
                            x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
                        }
                    } else {
#pragma unroll
                        for (int q = 0; q < Ops::ND; ++q) x[q] = 0u;
                    }
                    Ops::prep(x, act[m]);
                }
#pragma unroll
                for (int i = 0; i < CPW; ++i) {
                    uint32_t wd[Ops::NWD];
                    Ops::decode(w[u][i], zr[u][i], wd);  // once per chunk, shared by the rows
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        float part[H];
                        Ops::dotd(wd, act[m], part);
#pragma unroll
                        for (int h = 0; h < H; ++h)
                            acc[i][m] = block_acc<Ops::ASUM>(acc[i][m], sc[u][i][h], part[h], zr[u][i][h],
                                                             act[m].asum[h]);
                    }
                }
            }
        }

#pragma unroll
        for (int i = 0; i < CPW; ++i) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float s = wave_sum(acc[i][m]) * a.tscale;
                if (lane == 0 && nbase + i < a.N && rlive[m])
                    store_out<ACT>(a.Y, (int64_t)(m0 + m) * a.N + nbase + i, add_bias<ACT>(a.bias, nbase + i, s));
            }
        }
    }
}

// ----------------------------------------------------------------------------------
// Persistent streaming kernel for MT = 1, 2 or 4 rows in one pass.
//
// The same per-row arithmetic as k_stream (same lanes per chunk, same chunk order per
// lane, same decode, zero-point and scale steps, same wave reduction), so results are
// bit-identical to it; what differs is how the latency is covered:
//  - the activation rows are staged once per workgroup in LDS, already in the
//    decode's pair order and laid out so that the 64 lanes of a wave read consecutive
//    16-byte pieces, together with sum(a) of every chunk (half);
//  - each wave walks column groups g = wave, wave + nwaves, ... and the batches of one
//    group (UNR chunks per lane of each of its CPW columns); the codes and raw block
//    metadata of the next batch are in flight while the current one is computed
//    (two register buffers); a chunk's codes are decoded once for all rows;
//  - no load and no use sits behind a branch (clamped indexes, selected updates), so
//    the compiler's wait before a batch leaves the other batch in flight.

template <int FMT, int H, int UNR, int CPW>
struct SBatch {
    u4v w[UNR][CPW];
    MetaS<H> m[UNR][CPW];  // per-chunk metadata loads (narrow, or the dwords that hold them)
    MetaW mw[CPW];         // or the round's metadata windows (8-bit codes)
};

// Keep a chunk's metadata decode at its use: an empty asm that takes the loaded values
// and hands them back, so the compiler cannot hoist the decode (a zero-point mask, a
// shift) up to the refill of the other buffer, where it would wait for these loads
// while that refill is being issued. It emits no instruction; the wait it implies is
// the one the chunk's use needs anyway.
template <int H>
__device__ __forceinline__ void pin_meta(MetaS<H> &m) {
#pragma unroll
    for (int h = 0; h < H; ++h) asm volatile("" : "+v"(m.s[h]), "+v"(m.z[h]));
}

// Index (in 16-byte pieces) of piece q of chunk c of a staged activation row.
template <int NQ>
__device__ __forceinline__ int stage_index(int c, int q) {
    return (((c >> 6) * NQ + q) << 6) + (c & 63);
}

// Stage the M activation rows: each thread prepares chunks c, c + blockDim, ... of
// every row, two at a time, with both chunks' loads issued before either is used.
// Row m's pieces start at sP + m * rowq, its chunk sums at sS + m * rows.
template <int FMT, int ACT, int H>
__device__ __forceinline__ void stage_rows(const KArgs &a, u4v *sP, float *sS, int rowq, int rows) {
    using Ops = ChunkOps<FMT, ACT, H>;
    constexpr int NQ = Ops::ND / 4;
    constexpr int SB = 2;
    const uint16_t *A16 = (const uint16_t *)a.A;
    const int nch = (int)a.nchunks;
    const int items = a.M * nch;
    for (int i0 = threadIdx.x; i0 < items; i0 += SB * (int)blockDim.x) {
        uint32_t x[SB][Ops::ND];
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            int it = i0 + j * (int)blockDim.x;
            it = it < items ? it : items - 1;
            const int m = it / nch, c = it - (it / nch) * nch;
            const uint16_t *ap = A16 + (int64_t)m * a.K + (uint32_t)c * (uint32_t)Ops::KPC;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const u4v v = load16(ap + 8 * q);
                x[j][4 * q] = v.x; x[j][4 * q + 1] = v.y; x[j][4 * q + 2] = v.z; x[j][4 * q + 3] = v.w;
            }
        }
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int it = i0 + j * (int)blockDim.x;
            if (it < items) {
                const int m = it / nch, c = it - (it / nch) * nch;
                ChunkAct act;
                Ops::prep(x[j], act);
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    sP[m * rowq + stage_index<NQ>(c, q)] =
                        u4v{act.p[4 * q], act.p[4 * q + 1], act.p[4 * q + 2], act.p[4 * q + 3]};
                if constexpr (Ops::ASUM) {
#pragma unroll
                    for (int h = 0; h < H; ++h) sS[m * rows + c * H + h] = act.asum[h];
                }
            }
        }
    }
}

// MD, how the block metadata is loaded (the values, and so the results, are the same):
// 0 per chunk with narrow loads; 1 (8-bit codes) one window dword per lane per column
// and round (meta_window_load_u8); 2 per chunk as the aligned dwords that hold it.
template <int FMT, int ACT, int MT, int CPW, int UNR, int H, int NWG, int MD>
__global__ void __launch_bounds__(64 * NWG) k_stream1(KArgs a) {
    constexpr bool WM = MD == 1, DW = MD == 2;
    // one row and up to two columns per wave: loads through buffer resources (below);
    // the other shapes keep clamped global addresses (their accumulators, or four
    // columns' resources, would not leave the scalar registers for them)
    constexpr bool BUF = MT == 1 && CPW <= 2;
    using Ops = ChunkOps<FMT, ACT, H>;
    using B = SBatch<FMT, H, UNR, CPW>;
    constexpr int NQ = Ops::ND / 4;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t gw = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nch = (int)a.nchunks;
    const int nch64 = (nch + 63) & ~63;
    const int rowq = nch64 * NQ;          // 16-byte pieces per staged row
    const int rows = nch64 * H;           // chunk sums per staged row
    u4v *sP = (u4v *)smem;
    float *sS = (float *)(smem + (size_t)MT * rowq * 16);
    const int64_t ngroups = (a.N + CPW - 1) / CPW;
    const int rounds = (nch + 64 * UNR - 1) / (64 * UNR);
    const int mine = gw < ngroups ? (int)((ngroups - gw + nw - 1) / nw) : 0;
    const int total = mine * rounds;
    const ZSel zs = zsel(a.zp, FMT == FMT_U4 ? (DW ? 0x88888888u : 0x88u) : (DW ? 0x80808080u : 128u));
    // Addressing (BUF): chunk c = base + lane of a column, base = round * 64 * UNR + 64 u
    // (uniform). The codes, and with DW the metadata dwords, are loaded through a buffer
    // resource per column with the lane's part as the vector offset and the base's as
    // the scalar one: a chunk past the column reads zeros, which the select below
    // discards, so no index needs clamping, and the per-chunk address arithmetic is a
    // scalar one per round.
    const uint32_t col_bytes = (uint32_t)a.col_bytes;
    const uint32_t lane16 = (uint32_t)lane * 16u;
    const MetaDW<H> mdw = meta_dw_lane<FMT, H>(a, lane);
    // bytes of a column's scale row and zero-point row (the scale row again without
    // zero points, as col_ptrs aliases it)
    const uint32_t srow = (uint32_t)(FMT == FMT_NVFP4 ? (a.K >> 4) : (int64_t)a.nblk * (FMT == FMT_FP8 ? 4 : 2));
    const uint32_t zrow = a.zp ? (uint32_t)a.zstride : srow;

    // issue cursor (group, round)
    int64_t ig = gw;
    int ir = 0;
    auto issue = [&](B &b) {
        ColPtrs cp[CPW];
        __amdgpu_buffer_rsrc_t rw[CPW], rs[CPW], rz[CPW];
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int64_t n = ig * CPW + i;
            cp[i] = col_ptrs<FMT>(a, n < a.N ? n : a.N - 1);
            if constexpr (BUF) {
                rw[i] = buf_rsrc(cp[i].w, col_bytes);
                if constexpr (DW) {
                    rs[i] = buf_rsrc(cp[i].s, srow);
                    rz[i] = buf_rsrc(cp[i].z, zrow);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int base = ir * (64 * UNR) + 64 * u;
            const int cc = base + lane < nch ? base + lane : nch - 1;
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                if constexpr (BUF) b.w[u][i] = buf_load16_stream(rw[i], lane16, (uint32_t)base * 16u);
                else b.w[u][i] = load16_stream(cp[i].w + (uint32_t)cc * 16u);
            }
        }
        if constexpr (WM) {
#pragma unroll
            for (int i = 0; i < CPW; ++i) b.mw[i] = meta_window_load_u8<UNR>(a, cp[i], ir, lane);
        } else if constexpr (DW && BUF) {
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                uint32_t so, zo;
                meta_dw_round<FMT>(a, ir * (64 * UNR) + 64 * u, so, zo);
#pragma unroll
                for (int i = 0; i < CPW; ++i) {
#pragma unroll
                    for (int h = 0; h < H; ++h) {
                        b.m[u][i].s[h] = buf_load4(rs[i], mdw.s_off[h], so);
                        b.m[u][i].z[h] = FMT == FMT_NVFP4 ? 0u : buf_load4(rz[i], mdw.z_off[h], zo);
                    }
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int c = ir * (64 * UNR) + 64 * u + lane;
                const int cc = c < nch ? c : nch - 1;
#pragma unroll
                for (int i = 0; i < CPW; ++i) meta_load_s<FMT, H, DW>(a, cp[i], cc, b.m[u][i]);
            }
        }
        if (++ir == rounds) {
            ir = 0;
            ig += nw;
        }
    };

    // consume cursor and the accumulators of the group being computed
    int64_t cg = gw;
    int cr = 0;
    float acc[CPW][MT];
#pragma unroll
    for (int i = 0; i < CPW; ++i)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[i][m] = 0.0f;
    // branch-free: a chunk past the end is computed on the clamped chunk and its
    // update of the accumulator is discarded by a select (acc keeps its bits)
    auto consume = [&](const B &b) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int c = cr * (64 * UNR) + 64 * u + lane;
            const bool valid = c < nch;
            const int cc = valid ? c : nch - 1;
            // BUF: the staged pieces of the chunk are those of block blk = c / 64, clamped
            // (uniformly) to the staged rows, which never clamps a valid chunk, and the
            // lane (piece q at pbase + 64 q, sums at sbase); else those of the clamped chunk
            const int blk = min(cr * UNR + u, (nch64 >> 6) - 1);
            const int pbase = blk * (NQ * 64) + lane;
            const int sbase = (blk * 64 + lane) * H;
            if constexpr (MT == 1) {
                // one row: the activations are read once and each column's codes are
                // decoded right before their dot products
                ChunkAct act;
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const u4v v = BUF ? sP[pbase + 64 * q] : sP[stage_index<NQ>(cc, q)];
                    act.p[4 * q] = v.x; act.p[4 * q + 1] = v.y; act.p[4 * q + 2] = v.z; act.p[4 * q + 3] = v.w;
                }
                if constexpr (Ops::ASUM) {
#pragma unroll
                    for (int h = 0; h < H; ++h) act.asum[h] = BUF ? sS[sbase + h] : sS[cc * H + h];
                }
#pragma unroll
                for (int i = 0; i < CPW; ++i) {
                    float sc[H], part[H];
                    uint32_t zr[H];
                    MetaS<H> mu;
                    if constexpr (WM) meta_from_window_u8<UNR>(a, b.mw[i], 64 * u + lane, mu);
                    else mu = b.m[u][i];
                    pin_meta(mu);
                    if constexpr (DW && BUF) meta_decode_dw<FMT, H>(mu, mdw, zs, sc, zr);
                    else meta_decode_s<FMT, H, DW>(a, cc, mu, zs, sc, zr);
                    chunk_dot<FMT, ACT, H>(b.w[u][i], zr, act, part);
                    float t = acc[i][0];
#pragma unroll
                    for (int h = 0; h < H; ++h) t = block_acc<Ops::ASUM>(t, sc[h], part[h], zr[h], act.asum[h]);
                    acc[i][0] = valid ? t : acc[i][0];
                }
            } else {
                // several rows: every column's codes are decoded once and shared
                uint32_t wd[CPW][Ops::NWD];
                float sc[CPW][H];
                uint32_t zr[CPW][H];
#pragma unroll
                for (int i = 0; i < CPW; ++i) {
                    MetaS<H> mu;
                    if constexpr (WM) meta_from_window_u8<UNR>(a, b.mw[i], 64 * u + lane, mu);
                    else mu = b.m[u][i];
                    pin_meta(mu);
                    if constexpr (DW && BUF) meta_decode_dw<FMT, H>(mu, mdw, zs, sc[i], zr[i]);
                    else meta_decode_s<FMT, H, DW>(a, cc, mu, zs, sc[i], zr[i]);
                    Ops::decode(b.w[u][i], zr[i], wd[i]);
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m >= a.M) break;  // uniform; no memory operation is skipped
                    ChunkAct act;
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        const u4v v = sP[m * rowq + stage_index<NQ>(cc, q)];
                        act.p[4 * q] = v.x; act.p[4 * q + 1] = v.y; act.p[4 * q + 2] = v.z; act.p[4 * q + 3] = v.w;
                    }
                    if constexpr (Ops::ASUM) {
#pragma unroll
                        for (int h = 0; h < H; ++h) act.asum[h] = sS[m * rows + cc * H + h];
                    }
#pragma unroll
                    for (int i = 0; i < CPW; ++i) {
                        float part[H];
                        Ops::dotd(wd[i], act, part);
                        float t = acc[i][m];
#pragma unroll
                        for (int h = 0; h < H; ++h) t = block_acc<Ops::ASUM>(t, sc[i][h], part[h], zr[i][h], act.asum[h]);
                        acc[i][m] = valid ? t : acc[i][m];
                    }
                }
            }
        }
        // the batch's accumulation completes here (nothing of it may sink below the
        // next refill of this buffer); emits no instruction
#pragma unroll
        for (int i = 0; i < CPW; ++i)
#pragma unroll
            for (int m = 0; m < MT; ++m) asm volatile("" : "+v"(acc[i][m])::"memory");
        if (++cr == rounds) {
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                const int64_t n = cg * CPW + i;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (MT == 1 || m < a.M) {
                        const float v = wave_sum(acc[i][m]) * a.tscale;
                        if (lane == 0 && n < a.N) store_out<ACT>(a.Y, (int64_t)m * a.N + n, add_bias<ACT>(a.bias, n, v));
                    }
                    acc[i][m] = 0.0f;
                }
            }
            cr = 0;
            cg += nw;
        }
    };

    // Two buffers, refilled in turn; the steady-state loop has no branch around a load
    // or a use, so the compiler's wait before a batch is consumed leaves the other
    // batch in flight. The last one or two batches are drained without refills, so
    // nothing is fetched past the wave's work. (Scheduling barriers keep each refill
    // below the last use of the buffer's old contents.) A third buffer (two batches in
    // flight) measured slower: the registers it takes cost more resident waves than
    // the extra depth brings.
    B b0, b1;
    if (total > 0) issue(b0);  // the first batch's fetch overlaps the staging below
    stage_rows<FMT, ACT, H>(a, sP, sS, rowq, rows);
    __syncthreads();
    int i = 0;
    for (; i + 2 < total; i += 2) {
        issue(b1);
        consume(b0);
        __builtin_amdgcn_sched_barrier(0);
        issue(b0);
        consume(b1);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (total - i == 2) {
        issue(b1);
        consume(b0);
        consume(b1);
    } else if (total - i == 1) {
        consume(b0);
    }
}

// ----------------------------------------------------------------------------------
// generic element-wise kernel

template <int ACT>
__device__ __forceinline__ float act_at(const KArgs &a, int m, int64_t k) {
    const uint16_t bits = ((const uint16_t *)a.A)[(int64_t)m * a.K + k];
    if constexpr (ACT == ACT_F16) return (float)__builtin_bit_cast(_Float16, bits);
    else return __builtin_bit_cast(float, (uint32_t)bits << 16);
}

template <int FMT>
__device__ __forceinline__ float weight_at(const KArgs &a, int64_t n, int64_t k) {
    const int64_t b = k >> a.bs_shift;
    if constexpr (FMT == FMT_U4) {
        const uint8_t byte = a.W[n * a.col_bytes + (k >> 1)];
        const int q = (k & 1) ? (byte >> 4) : (byte & 0x0F);
        int z = 8;
        if (a.zp) {
            const uint8_t zb = a.zp[n * a.zstride + (b >> 1)];
            z = (b & 1) ? (zb >> 4) : (zb & 0x0F);
        }
        return half_bits_to_float(((const uint16_t *)a.scales)[n * a.nblk + b]) * (float)(q - z);
    } else if constexpr (FMT == FMT_U8) {
        const int q = a.W[n * a.col_bytes + k];
        const int z = a.zp ? a.zp[n * a.nblk + b] : 128;
        return half_bits_to_float(((const uint16_t *)a.scales)[n * a.nblk + b]) * (float)(q - z);
    } else if constexpr (FMT == FMT_FP8) {
        return ((const float *)a.scales)[n * a.nblk + b] * e4m3_to_float(a.W[n * a.col_bytes + k]);
    } else {
        const uint8_t byte = a.W[n * a.col_bytes + (k >> 1)];
        const uint32_t code = (k & 1) ? (byte >> 4) : (byte & 0x0F);
        const uint32_t pair = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, 1.0f, 0));
        const float e2 = (float)__builtin_bit_cast(_Float16, (uint16_t)(pair & 0xFFFFu));
        return e4m3_to_float(((const uint8_t *)a.scales)[n * (a.K / 16) + k / 16]) * e2;
    }
}

template <int FMT, int ACT>
__global__ void __launch_bounds__(256) k_generic(KArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    for (int64_t n = wave; n < a.N; n += nwaves) {
        float acc[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) acc[m] = 0.0f;
        for (int64_t k = lane; k < a.K; k += 64) {
            const float w = weight_at<FMT>(a, n, k);
#pragma unroll
            for (int m = 0; m < 16; ++m)
                if (m < a.M) acc[m] = __builtin_fmaf(act_at<ACT>(a, m, k), w, acc[m]);
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            if (m < a.M) {
                const float s = wave_sum(acc[m]) * a.tscale;
                if (lane == 0) store_out<ACT>(a.Y, (int64_t)m * a.N + n, add_bias<ACT>(a.bias, n, s));
            }
        }
    }
}

// ----------------------------------------------------------------------------------
// launchers

namespace {

template <int FMT, int ACT, int MT, int CPW>
hipError_t go_stream(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    // two scale blocks per chunk: every NVFP4 chunk, and U4 chunks with 16-wide blocks
    if constexpr (FMT == FMT_NVFP4) {
        return launch_or_report(cfg, k_stream<FMT, ACT, MT, CPW, 2, 2>, 256, a, s);
    } else if constexpr (FMT == FMT_U4) {
        if (a.bs == 16) return launch_or_report(cfg, k_stream<FMT, ACT, MT, CPW, 2, 2>, 256, a, s);
        return launch_or_report(cfg, k_stream<FMT, ACT, MT, CPW, 2, 1>, 256, a, s);
    } else {
        return launch_or_report(cfg, k_stream<FMT, ACT, MT, CPW, 2, 1>, 256, a, s);
    }
}

template <int FMT, int ACT, int MT>
hipError_t pick_cpw(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    switch (cfg.cols_per_wave) {
    case 1: return go_stream<FMT, ACT, MT, 1>(cfg, a, s);
    case 2: return go_stream<FMT, ACT, MT, 2>(cfg, a, s);
    case 4: return go_stream<FMT, ACT, MT, 4>(cfg, a, s);
    default: return hipErrorInvalidValue;
    }
}

template <int FMT, int ACT>
hipError_t pick_mt(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    switch (cfg.rows_per_pass) {
    case 1: return pick_cpw<FMT, ACT, 1>(cfg, a, s);
    case 2: return pick_cpw<FMT, ACT, 2>(cfg, a, s);
    case 4: return pick_cpw<FMT, ACT, 4>(cfg, a, s);
    default: return hipErrorInvalidValue;
    }
}

// One-row persistent kernel: cols_per_wave 1/2/4; unroll 2/3/4 from variant bits 1..2
// (2 -> 2, 3 -> 3, 0 -> 4).
template <int FMT, int ACT, int MT, int CPW, int UNR, int H, int NWG>
hipError_t go_stream1_w(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    // variant bit 3: the round's metadata windows (8-bit codes); bit 4: metadata as
    // the dwords that hold it (4-bit, 8-bit and NVFP4 codes; FP8 scales are dwords)
    // (8-bit windows next to eight rows would spill scalar registers: not built)
    constexpr bool can_wm = FMT == FMT_U8 && MT < 8, can_dw = FMT != FMT_FP8;
    const bool wm = (cfg.variant >> 3) & 1, dw = (cfg.variant >> 4) & 1;
    if ((wm && !can_wm) || (dw && !can_dw) || (wm && dw)) return hipErrorInvalidValue;
    void (*kern)(KArgs) = k_stream1<FMT, ACT, MT, CPW, UNR, H, NWG, 0>;
    if constexpr (can_wm) {
        if (wm) kern = k_stream1<FMT, ACT, MT, CPW, UNR, H, NWG, 1>;
    }
    if constexpr (can_dw) {
        if (dw) kern = k_stream1<FMT, ACT, MT, CPW, UNR, H, NWG, 2>;
    }
    const int md = wm ? 1 : (dw ? 2 : 0);
    static std::atomic<uint64_t> lds_set[3] = {{0}, {0}, {0}};
    hipError_t e = lds_limit_once((const void *)kern, cfg.device, cfg.lds_bytes, lds_set[md]);
    if (e != hipSuccess) return e;
    return launch_or_report(cfg, kern, 64 * NWG, a, s);
}

// Workgroups of 4 waves; of 16 for one row with one column per wave; of 4, 8, 12 or
// 16 for several rows, as far as the kernel fits the register share that many waves
// per CU leave without spilling (the dispatcher picks within the same limits): 8 with
// two columns per wave, 12 for four rows of 4-bit codes with two blocks per chunk.
template <int FMT, int MT, int CPW, int H>
constexpr int stream_rows_max_wg() {
    return (CPW == 2 || (MT == 8 && (FMT == FMT_U4 || FMT == FMT_NVFP4))) ? 8
                                                                         : ((FMT == FMT_U4 && H == 2 && MT == 4) ? 12 : 16);
}

template <int FMT, int ACT, int MT, int CPW, int UNR, int H>
hipError_t go_stream1_k(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    if constexpr (MT == 1) {
        if constexpr (CPW == 1) {
            if (cfg.waves_per_wg == 16) return go_stream1_w<FMT, ACT, MT, CPW, UNR, H, 16>(cfg, a, s);
        }
    } else {
        constexpr int MX = stream_rows_max_wg<FMT, MT, CPW, H>();
        if (cfg.waves_per_wg > MX) return hipErrorInvalidValue;
        switch (cfg.waves_per_wg) {
        case 8: return go_stream1_w<FMT, ACT, MT, CPW, UNR, H, 8>(cfg, a, s);
        case 12:
            if constexpr (MX >= 12) return go_stream1_w<FMT, ACT, MT, CPW, UNR, H, 12>(cfg, a, s);
            break;
        case 16:
            if constexpr (MX >= 16) return go_stream1_w<FMT, ACT, MT, CPW, UNR, H, 16>(cfg, a, s);
            break;
        default: break;
        }
    }
    if (cfg.waves_per_wg != 4) return hipErrorInvalidValue;
    return go_stream1_w<FMT, ACT, MT, CPW, UNR, H, 4>(cfg, a, s);
}

template <int FMT, int ACT, int MT, int CPW, int UNR>
hipError_t go_stream1_h(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    if constexpr (FMT == FMT_NVFP4) return go_stream1_k<FMT, ACT, MT, CPW, UNR, 2>(cfg, a, s);
    else if constexpr (FMT == FMT_U4)
        return a.bs == 16 ? go_stream1_k<FMT, ACT, MT, CPW, UNR, 2>(cfg, a, s)
                          : go_stream1_k<FMT, ACT, MT, CPW, UNR, 1>(cfg, a, s);
    else return go_stream1_k<FMT, ACT, MT, CPW, UNR, 1>(cfg, a, s);
}

// unroll 2/3/4 from variant bits 1..2 (2 -> 2, 3 -> 3, 0 -> 4) for one row; two or
// four rows take 2 chunks per lane and 1 or 2 columns per wave
template <int FMT, int ACT, int MT, int CPW>
hipError_t go_stream1_u(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    if constexpr (MT > 1) {
        if (((cfg.variant >> 1) & 3) != 2) return hipErrorInvalidValue;
        return go_stream1_h<FMT, ACT, MT, CPW, 2>(cfg, a, s);
    } else {
        switch ((cfg.variant >> 1) & 3) {
        case 2: return go_stream1_h<FMT, ACT, MT, CPW, 2>(cfg, a, s);
        case 3: return go_stream1_h<FMT, ACT, MT, CPW, 3>(cfg, a, s);
        case 0: return go_stream1_h<FMT, ACT, MT, CPW, 4>(cfg, a, s);
        default: return hipErrorInvalidValue;
        }
    }
}

template <int FMT, int ACT, int MT>
hipError_t go_stream1_c(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    switch (cfg.cols_per_wave) {
    case 1: return go_stream1_u<FMT, ACT, MT, 1>(cfg, a, s);
    case 2:
        if constexpr (MT <= 4) return go_stream1_u<FMT, ACT, MT, 2>(cfg, a, s);
        else return hipErrorInvalidValue;
    case 4:
        if constexpr (MT == 1) return go_stream1_u<FMT, ACT, MT, 4>(cfg, a, s);
        else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <int FMT, int ACT>
hipError_t go_stream1(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    switch (cfg.rows_per_pass) {
    case 1: return go_stream1_c<FMT, ACT, 1>(cfg, a, s);
    case 2: return go_stream1_c<FMT, ACT, 2>(cfg, a, s);
    case 4: return go_stream1_c<FMT, ACT, 4>(cfg, a, s);
    case 8:
        // eight rows, one column per wave: every format but 4-bit codes on bf16 (whose
        // per-row activation sums would spill scalar registers next to eight rows)
        if constexpr (!(FMT == FMT_U4 && ACT == ACT_BF16)) return go_stream1_c<FMT, ACT, 8>(cfg, a, s);
        else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <int FMT>
hipError_t pick_act(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    if (cfg.variant & 1)
        return cfg.act == ACT_F16 ? go_stream1<FMT, ACT_F16>(cfg, a, s) : go_stream1<FMT, ACT_BF16>(cfg, a, s);
    return cfg.act == ACT_F16 ? pick_mt<FMT, ACT_F16>(cfg, a, s) : pick_mt<FMT, ACT_BF16>(cfg, a, s);
}

template <int FMT>
hipError_t generic_act(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    if (cfg.act == ACT_F16) return launch_or_report(cfg, k_generic<FMT, ACT_F16>, 256, a, s);
    return launch_or_report(cfg, k_generic<FMT, ACT_BF16>, 256, a, s);
}

}  // namespace

hipError_t launch_stream(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    switch (cfg.fmt) {
    case FMT_U4: return pick_act<FMT_U4>(cfg, a, s);
    case FMT_U8: return pick_act<FMT_U8>(cfg, a, s);
    case FMT_FP8: return pick_act<FMT_FP8>(cfg, a, s);
    case FMT_NVFP4: return pick_act<FMT_NVFP4>(cfg, a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_generic(const LaunchCfg &cfg, const KArgs &a, hipStream_t s) {
    switch (cfg.fmt) {
    case FMT_U4: return generic_act<FMT_U4>(cfg, a, s);
    case FMT_U8: return generic_act<FMT_U8>(cfg, a, s);
    case FMT_FP8: return generic_act<FMT_FP8>(cfg, a, s);
    case FMT_NVFP4: return generic_act<FMT_NVFP4>(cfg, a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qgemv
