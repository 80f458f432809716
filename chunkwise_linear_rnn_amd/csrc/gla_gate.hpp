// Internal interface between the ABI layer (gla_api.cpp) and the output
// epilogue's launcher (gla_gate.hip): per-head LayerNorm, per-channel scale
// and shift, Swish output gate.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

namespace gla {

// Backward: `ws` holds 2 * kGateMaxBlocks * V floats of per-workgroup column sums.
constexpr int kGateMaxBlocks = 256;

struct GateLaunch {
    bool bf16, backward;
    int V;
    long R;             // rows = B * T * H
    const void *o, *z;  // [R][V] dtype
    const float *w, *b; // [V] (b may be null)
    float eps;
    void* y;            // forward output [R][V]
    const void* dy;     // backward input [R][V]
    void *dx, *dz;      // backward outputs [R][V]
    float *dw, *db;     // backward column sums [V] (either may be null)
    float* ws;
    hipStream_t stream;
};

hipError_t launch_out_gate(const GateLaunch& a);

}  // namespace gla
