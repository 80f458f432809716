// Host-only stand-ins for the kernel launchers, linked into the sanitizer
// build of the ABI layer (gla_api.cpp, gla_timing.cpp compiled by the host
// compiler with AddressSanitizer and UndefinedBehaviorSanitizer).  That build
// checks argument validation, launch planning and workspace arithmetic on a
// machine without a GPU; any call that gets as far as a launch reports
// hipErrorNoDevice instead, so it returns GLA_ERR_HIP.
#include <hip/hip_runtime.h>

#include "gla_gate.hpp"
#include "gla_launch.hpp"

namespace gla {

hipError_t noalloc_scratch(void**) { return hipErrorNoDevice; }
hipError_t launch_fwd(const FwdLaunch&) { return hipErrorNoDevice; }
hipError_t launch_fwd_general(const FwdLaunch&) { return hipErrorNoDevice; }
hipError_t launch_bwd(const BwdLaunch&) { return hipErrorNoDevice; }
hipError_t launch_bwd_general(const BwdGeneralLaunch&) { return hipErrorNoDevice; }
hipError_t launch_decode(const DecodeLaunch&) { return hipErrorNoDevice; }
// the real launchers return success without launching when there is nothing to do
hipError_t launch_out_gate(const GateLaunch& a) {
    return a.R <= 0 && !(a.backward && (a.dw || a.db)) ? hipSuccess : hipErrorNoDevice;
}
hipError_t launch_state_copy(const float*, float*, long n, hipStream_t) {
    return n <= 0 ? hipSuccess : hipErrorNoDevice;
}

hipError_t launch_copy_cols(bool, const void*, long, long, void*, long, long, long W, long rows, hipStream_t) {
    return rows <= 0 || W <= 0 ? hipSuccess : hipErrorNoDevice;
}
hipError_t launch_add_into(bool, void*, const void*, long n, hipStream_t) { return n <= 0 ? hipSuccess : hipErrorNoDevice; }
hipError_t launch_pad_cols(bool, const void*, long, long, void*, long, long W_dst, long rows, hipStream_t) {
    return rows <= 0 || W_dst <= 0 ? hipSuccess : hipErrorNoDevice;
}
hipError_t launch_bcast_cols(const float*, float*, long W, long rows, hipStream_t) {
    return rows <= 0 || W <= 0 ? hipSuccess : hipErrorNoDevice;
}
hipError_t launch_row_sums(const float*, long, float*, long rows, hipStream_t) {
    return rows <= 0 ? hipSuccess : hipErrorNoDevice;
}

}  // namespace gla
