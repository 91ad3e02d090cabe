// Backward KPage attention for gfx950 (placeholder until the kernels land).
#include <hip/hip_runtime.h>

#include "device.hpp"

namespace kpage {

hipError_t launch_bwd(const BwdArgs &, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kpage
