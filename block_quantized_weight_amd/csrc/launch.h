// Host-side launch description shared by the dispatcher and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace qgemv {

// Arguments every kernel receives (by value).
struct KArgs {
    const uint8_t *W;        // packed codes
    const void *scales;      // block scales
    const uint8_t *zp;       // zero points or nullptr
    const void *A;           // [M, K] activations
    void *Y;                 // [M, N] output
    int64_t N;
    int64_t K;
    int64_t col_bytes;       // bytes of codes per column
    int64_t nchunks;         // 16-byte chunks per column
    int32_t bs;              // block size along K (a power of two)
    int32_t bs_shift;        // log2(bs)
    int32_t nblk;            // K / bs
    int32_t zstride;         // bytes of zero points per column
    int32_t M;
    int32_t ksplit;          // waves sharing one column tile's K range
    float tscale;            // nvfp4 tensor scale (1 otherwise)
    const void *bias;        // [N] bias in the activation dtype, or nullptr
    // K parts split across workgroups (MFMA register ring only): 1 = none; else the
    // fp32 partial tiles [kparts, M, N] and one completion counter per tile group,
    // both in the caller's workspace
    int32_t kparts;
    float *part;
    uint32_t *cnt;
};

// The kernel a launcher would launch: reported instead of launching when a plan's
// `query` points here (used to ask the runtime how many of its workgroups stay
// resident on one CU).
struct KernelRef {
    const void *fn;
    int threads;    // per workgroup
    int lds_bytes;  // dynamic LDS per workgroup
};

struct LaunchCfg {
    KernelRef *query;   // when set, the launcher fills *query and launches nothing
    int device;         // device the launch goes to (set by the caller of a launcher)
    int fmt;            // Fmt
    int act;            // Act
    int family;         // qgemv_family
    int rows_per_pass;  // MT
    int passes;
    int cols_per_wave;
    int ksplit;
    int waves_per_wg;
    int64_t grid;
    int lds_bytes;
    int variant;
    int kparts;               // K parts split across workgroups (1 = none)
    int64_t ws_counters;      // workspace bytes of completion counters (256-byte multiple)
    int64_t ws_bytes;         // workspace bytes in all (0 without K parts)
};

// Dynamic LDS of one gfx950 compute unit (bytes).
constexpr int kMaxLdsBytes = 160 * 1024;

// Report (query set) or launch kernel `kern` with the plan's grid, `threads` per
// workgroup and the plan's dynamic LDS.
template <typename Kern>
inline hipError_t launch_or_report(const LaunchCfg &cfg, Kern kern, int threads, const KArgs &a, hipStream_t s) {
    if (cfg.query) {
        *cfg.query = KernelRef{(const void *)kern, threads, cfg.lds_bytes};
        return hipSuccess;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)cfg.grid), dim3(threads), (size_t)cfg.lds_bytes, s, a);
    return hipGetLastError();
}

// Raise kern's dynamic-LDS limit to the whole CU once per device (bit d of `done`):
// the limit is a property of the function on a device, so a launch that needs more
// than the default 64 KB pays the call once, not per launch. `done` is a static of the
// launcher instantiation that owns kern.
inline hipError_t lds_limit_once(const void *kern, int device, int lds_bytes, std::atomic<uint64_t> &done) {
    if (lds_bytes <= 65536) return hipSuccess;
    const uint64_t bit = 1ull << (device & 63);
    if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsBytes);
    if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
    return e;
}

hipError_t launch_stream(const LaunchCfg &cfg, const KArgs &a, hipStream_t s);
hipError_t launch_generic(const LaunchCfg &cfg, const KArgs &a, hipStream_t s);
hipError_t launch_mfma(const LaunchCfg &cfg, const KArgs &a, hipStream_t s);
hipError_t launch_sweep(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s);  // sweep.hip

}  // namespace qgemv
