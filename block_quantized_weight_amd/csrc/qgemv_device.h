// Device-side building blocks shared by the qgemv kernels (gfx950 / CDNA4 only).
//
// Decoders turn 16-byte chunks of packed codes into fp16/bf16 operand pairs that
// feed v_dot2_f32_{f16,bf16} (vector family) or v_mfma_f32_16x16x32_{f16,bf16}
// (matrix family). Every decode here is exact:
//  - With fp16 activations, 4-/8-bit codes q and the block's zero point z are both
//    placed in fp16 bit patterns (subnormals q*2^-24, or the integers 1024 + q) and
//    subtracted with one packed fp16 op, which forms (q - z) exactly ("[CUDA]
//    MatMulNBits 8-bit: wide fp16 M=1 kernel", Description: (q - zp) formed exactly
//    in fp16 before the multiply).
//  - With bf16 activations gfx950 has no packed bf16 subtract. 8-bit codes form
//    q - z exactly in fp32 and round the pair to bf16 (exact: |q - z| <= 255 needs 8
//    significant bits). 4-bit codes become the bf16 integers q through the E4M3
//    converter (codes 0..15 of E4M3 are exactly q*2^-9; the converter's power-of-two
//    scale 2^9 restores q), and the zero point enters the fp32 block sum as
//    z * sum(a), with no offset added to q.
//  - E4M3 and E2M1 use the hardware converters, which decode OCP E4M3FN and
//    E2M1 exactly (E4M3 to fp16/bf16 widening is lossless: "[CUDA] Block-scaled
//    MatMul decode GEMV", FP8 mma paragraph).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace qgemv {

enum Fmt : int { FMT_U4 = 1, FMT_U8 = 2, FMT_FP8 = 3, FMT_NVFP4 = 4 };
enum Act : int { ACT_F16 = 1, ACT_BF16 = 2 };

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));


// ---------------------------------------------------------------------------------
// small helpers

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    // v_perm_b32: selector bytes 0..3 pick bytes of `lo`, 4..7 bytes of `hi`, 0x0c gives 0.
    return __builtin_amdgcn_perm(hi, lo, sel);
}

template <int ACT>
__device__ __forceinline__ float dot2(uint32_t x, uint32_t y, float c) {
    if constexpr (ACT == ACT_F16) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, x), __builtin_bit_cast(h2, y), c, false);
    } else {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, x), __builtin_bit_cast(b2, y), c, false);
    }
}

// Pair (1, 1) in the activation type, for sums of activations through dot2.
template <int ACT>
__device__ __forceinline__ constexpr uint32_t ones2() {
    return ACT == ACT_F16 ? 0x3C003C00u : 0x3F803F80u;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float e4m3_to_float(uint32_t byte) {
    return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// E4M3 -> fp16/bf16 pairs: bytes (2*word, 2*word+1) of w.
template <int ACT, bool WORD>
__device__ __forceinline__ uint32_t fp8_pair(uint32_t w) {
    if constexpr (ACT == ACT_F16)
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, WORD));
    else
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, WORD));
}

// E2M1 -> fp16/bf16 pair from byte `sel` of w (low nibble -> element 0).
template <int ACT, int SEL>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t w) {
    if constexpr (ACT == ACT_F16)
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL));
    else
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
}

// bf16 pair of integers (q_a, q_b) from bytes (2*word, 2*word+1) of w holding 0..15.
template <bool WORD>
__device__ __forceinline__ uint32_t small_int_bf16_pair(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 512.0f, WORD));
}

// Packed fp16 difference x - y of two fp16 pairs (one v_pk_add_f16 with negated
// second operand); exact whenever the differences are representable, as they are for
// the integer codes and zero points here.
__device__ __forceinline__ uint32_t sub_h2(uint32_t x, uint32_t y) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, x) - __builtin_bit_cast(h2, y));
}

// bf16 pair (x, y) rounded from fp32 (v_cvt_pk_bf16_f32, nearest-even; exact for the
// small integers it is given here).
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
    typedef float f2v __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){x, y}, b2));
}

// bf16 pair (q[sel] - z, q[sel + 1] - z) from bytes sel, sel + 1 of w (8-bit codes):
// formed in fp32, where the difference is exact, then packed.
template <int SEL>
__device__ __forceinline__ uint32_t u8_diff_bf16_pair(uint32_t w, float z) {
    const float a = (float)((w >> (8 * SEL)) & 0xFFu) - z;
    const float b = (float)((w >> (8 * SEL + 8)) & 0xFFu) - z;
    return pack_bf16(a, b);
}

// (x & mask) | bits in one v_bitop3 (truth table 0xEA: bit i is the result for
// inputs x = i>>2 & 1, mask = i>>1 & 1, bits = i & 1).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) {
    return __builtin_amdgcn_bitop3_b32(x, mask, bits, 0xEA);
}

template <int ACT>
__device__ __forceinline__ void store_out(void *Y, int64_t idx, float v) {
    if constexpr (ACT == ACT_F16) {
        ((_Float16 *)Y)[idx] = (_Float16)v;
    } else {
        ((__bf16 *)Y)[idx] = (__bf16)v;
    }
}

// v + bias[n] in fp32 (the bias in the activation dtype), or v as it is without a
// bias: added once, after every scale, right before the rounding to the output type.
// The bias pointer is uniform, so the test is a scalar branch.
template <int ACT>
__device__ __forceinline__ float add_bias(const void *bias, int64_t n, float v) {
    if (!bias) return v;
    const uint16_t bits = ((const uint16_t *)bias)[n];
    if constexpr (ACT == ACT_F16) return v + (float)__builtin_bit_cast(_Float16, bits);
    else return v + __builtin_bit_cast(float, (uint32_t)bits << 16);
}

// Sum over the 64 lanes of a wave with DPP; the total lands in lane 63 and is
// returned to every lane through readlane. Fixed order: the result depends only on
// the 64 inputs.
__device__ __forceinline__ float wave_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));  // row_half_mirror
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));  // row_mirror
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false)); // row_bcast:15
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false)); // row_bcast:31
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Wait until at most N vector-memory operations of this wave are outstanding. Written
// as volatile asm with a memory clobber so that it is also a compiler barrier: no LDS
// read of a DMA destination may be hoisted above it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Zero-point presence as bit masks: byte = (loaded & keep) | fill gives the loaded
// zero point, or the midpoint when the weight has none. The mask is laundered through
// an empty asm so the optimizer cannot turn the selection back into a branch on the
// (uniform) kernel argument, which would move zero-point decodes next to their loads
// and make a prefetch wait for its own data.
struct ZSel {
    uint32_t keep, fill;
};

__device__ __forceinline__ ZSel zsel(const void *zp, uint32_t midpoint) {
    uint32_t keep = zp ? 0xFFFFFFFFu : 0u;
    asm volatile("" : "+v"(keep));
    return ZSel{keep, ~keep & midpoint};
}

// Wait until at most min(left, K) groups of OPS loads remain in flight (uniform
// left >= 0): a compile-time count in each branch.
template <int K, int OPS>
__device__ __forceinline__ void wait_slots(int64_t left) {
    static_assert(K * OPS <= 63, "vmcnt holds at most 63");
    if constexpr (K <= 0) {
        wait_vmcnt<0>();
    } else {
        if (left >= K) wait_vmcnt<K * OPS>();
        else wait_slots<K - 1, OPS>(left);
    }
}

typedef __attribute__((address_space(3))) void lds_void;

// Asynchronous global -> LDS copy of BYTES (4 or 16) per lane: lane l's bytes land at
// lds + l * BYTES (global_load_lds_dword / _dwordx4). Counted by vmcnt. NT: cache
// policy nontemporal, for bytes read once (aux bit 1, as for the streaming buffer loads).
template <int BYTES, bool NT = false>
__device__ __forceinline__ void dma_to_lds(const void *src, void *lds) {
    static_assert(BYTES == 4 || BYTES == 16, "dword or dwordx4 copies");
    if constexpr (BYTES == 4) __builtin_amdgcn_global_load_lds(src, (lds_void *)lds, 4, 0, NT ? 2 : 0);
    else __builtin_amdgcn_global_load_lds(src, (lds_void *)lds, 16, 0, NT ? 2 : 0);
}

__device__ __forceinline__ u4v load16(const void *p) {
    return *(const u4v *)p;
}

// Streaming load of weight bytes: read once, so keep them out of the caches' way.
__device__ __forceinline__ u4v load16_stream(const void *p) {
    return __builtin_nontemporal_load((const u4v *)p);
}

// A raw buffer resource over the n bytes at p (gfx9 descriptor word 3: no swizzle,
// stride 0). Loads through it are range-checked against n: one that reaches past n
// returns zeros instead of touching memory. The base is uniform (a column's start), so
// the resource lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, uint32_t n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)n, 0x00020000);
}

// 16 bytes at voff + soff of r, nontemporal (the weight stream; cache policy NT).
__device__ __forceinline__ u4v buf_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2));
}

// The dword at voff + soff of r (zero past the range).
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}

}  // namespace qgemv
