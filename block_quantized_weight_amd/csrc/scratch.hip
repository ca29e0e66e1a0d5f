// The library's own device scratch for qgemv_run_noalloc: a fixed array in device
// memory that takes the place of the caller's workspace (K-part completion counters
// and fp32 partial tiles), for callers that cannot allocate.
//
// The array's name is a host-side stand-in in host code, not a device address, so the
// address is looked up once per device with hipGetSymbolAddress, with that device
// current, and only that address is handed to kernels. Each device holds its own copy
// of the array, at its own address, until the process ends.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/qgemv.h"

namespace qgemv {

static __device__ __align__(256) unsigned char scratch[QGEMV_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_mu;
void *g_ptr[64];
}  // namespace

// The scratch array's device address on `device` (0..63), looked up and zeroed the
// first time a handle is created for that device; later calls return the recorded
// address. The zeroing is what the K-part kernels need at their first use (their
// completion counters must start at zero); every completed run leaves the area it
// used zero again. Returns a qgemv_status.
int scratch_address(int device, void **out) {
    if (device < 0 || device >= 64) return QGEMV_E_DEVICE;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[device]) {
        int prev = -1;
        if (hipGetDevice(&prev) != hipSuccess) return QGEMV_E_DEVICE;
        if (prev != device && hipSetDevice(device) != hipSuccess) return QGEMV_E_DEVICE;
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e == hipSuccess) e = hipMemset(p, 0, QGEMV_NOALLOC_SCRATCH_BYTES);
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (prev != device) hipSetDevice(prev);
        if (e != hipSuccess || !p || (uintptr_t)p % 256) return QGEMV_E_DEVICE;
        g_ptr[device] = p;
    }
    *out = g_ptr[device];
    return QGEMV_OK;
}

}  // namespace qgemv
