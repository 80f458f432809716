// Backward kernels of chunkwise gated linear attention on gfx950 (in progress).
#include "gla_device.hpp"
#include "gla_launch.hpp"

namespace gla {

hipError_t launch_bwd(const BwdLaunch& a) {
    (void)a;
    return hipErrorNotSupported;
}

}  // namespace gla
