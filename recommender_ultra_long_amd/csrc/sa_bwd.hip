// sa_bwd.hip — Sketch Attention backward (placeholder until implemented).
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {
hipError_t launch_bwd(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace sa
