// Matrix-core (MFMA) family of qgemv for gfx950.
#include "qgemv_device.h"

namespace qgemv {

hipError_t launch_mfma(const LaunchCfg &, const KArgs &, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace qgemv
