// Plain streaming read of a device buffer: the control the GEMV's weight stream is
// measured against. The pages compare their M = 1 kernel with "a plain streaming
// read of the same bytes" ("[CUDA] MatMulNBits 8-bit: wide fp16 M=1 kernel for decode
// GEMVs", Motivation). Built into its own library (libreadctl.so), which only the
// benchmark loads; the GEMV library does not contain it.
//
// Each lane reads 16-byte pieces with nontemporal loads, U in flight before the
// first is used, over a grid-stride walk (the streaming kernel's load shape), and
// folds them with xor; a lane writes its fold only if it equals a value the caller
// passes and the data never produces (so the reads cannot be removed, and nothing
// is written in practice). The caller picks U and the grid; the benchmark takes the
// fastest of a few, as the control is a ceiling.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u4v __attribute__((ext_vector_type(4)));

template <int U>
__global__ void __launch_bounds__(256) k_read_control(const u4v *src, int64_t n16, uint32_t never, uint32_t *sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t x = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u4v v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
        u4v e = v[0];
#pragma unroll
        for (int u = 1; u < U; ++u) e ^= v[u];
        x ^= e.x ^ e.y ^ e.z ^ e.w;
    }
    for (; i < n16; i += stride) {
        const u4v a = __builtin_nontemporal_load(src + i);
        x ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (x == never) sink[0] = x;
}

extern "C" {

// Read bytes / 16 pieces of src (16-byte aligned) on hip_stream with `blocks`
// workgroups of 256 threads and `unroll` (4, 8 or 16) loads in flight per lane.
// Returns 0, or the HIP error of the launch.
int read_control(const void *src, int64_t bytes, int blocks, int unroll, uint32_t never, void *sink,
                 void *hip_stream) {
    if (!src || !sink || bytes < 16 || blocks < 1 || (uintptr_t)src % 16) return (int)hipErrorInvalidValue;
    const u4v *p = (const u4v *)src;
    hipStream_t s = (hipStream_t)hip_stream;
    switch (unroll) {
    case 4: hipLaunchKernelGGL(k_read_control<4>, dim3((unsigned)blocks), dim3(256), 0, s, p, bytes / 16, never,
                               (uint32_t *)sink); break;
    case 8: hipLaunchKernelGGL(k_read_control<8>, dim3((unsigned)blocks), dim3(256), 0, s, p, bytes / 16, never,
                               (uint32_t *)sink); break;
    case 16: hipLaunchKernelGGL(k_read_control<16>, dim3((unsigned)blocks), dim3(256), 0, s, p, bytes / 16, never,
                                (uint32_t *)sink); break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

}  // extern "C"
