// Backward kernels (placeholder until the dQ and dK/dV kernels land).
#include "launch.h"

namespace skv {
hipError_t launch_bwd(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace skv
