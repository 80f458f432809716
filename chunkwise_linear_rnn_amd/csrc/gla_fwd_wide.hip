// Forward pass of 16-bit heads with 256 key columns: the chunk-record kernels
// of gla_fwd_wide.hpp and their launcher.  Built as its own translation unit
// with MFMA accumulators in VGPRs (the decay of the state between chunks is a
// vector multiply, which would otherwise copy the state out of and back into
// AGPRs every chunk).
//
// Source of the method: "Gated Linear Attention Transformers with
// Hardware-Efficient Training", Sections 4.2 and 4.3.
#include "gla_fwd_wide.hpp"
#include "gla_launch.hpp"
#include "gla_plan.hpp"
#include "gla_timing.hpp"

namespace gla {

template <typename T>
void launch_combine_fwd(const FwdLaunch& a, int KD);  // gla_fwd.hip

// Wide heads (16-bit, dk = 256): chunk records, then the state pass over
// segments 0..P-2, the combine, and the output walk over every segment.
template <int KD, int BV, bool SG>
static hipError_t launch_fwd_wide_bv(const FwdLaunch& a) {
    using T = bf16;
    static_assert(sizeof(WidePrepSmem<T, KD>) <= 80 * 1024, "two prep workgroups per CU");
    static_assert(sizeof(WideSmem<T, KD, BV, true>) <= 160 * 1024, "LDS budget");
    static_assert(WideRec<KD>::bytes == (long)wide_record_bytes(KD), "record size as the workspace plans it");
    const int nvb = a.V / BV;
    unsigned char* rec = static_cast<unsigned char*>(a.ws_rec);
    GLA_LAUNCH("fwd_prep", (gla_fwd_wide_prep<T, KD, SG>), dim3((unsigned)(a.BH * a.N)), dim3(256), a.stream,
               (const T*)a.q, (const T*)a.k, (const T*)a.g, rec, a.T, a.H, a.N);
    if (a.P > 1) {
        const int nseg = a.P - 1;
        GLA_LAUNCH("fwd_seg_state", (gla_fwd_wide_walk<T, KD, BV, false>), dim3((unsigned)xcd_grid(nseg * a.BH, nvb)),
                   dim3(512), a.stream, (const unsigned char*)rec, (const T*)a.v, (const T*)nullptr,
                   (const float*)nullptr, (T*)nullptr, (float*)nullptr, (T*)a.ws_state, a.ws_gate, a.T, a.H, a.V,
                   a.N, a.P, a.seg_len, nseg, (int)a.BH);
        launch_combine_fwd<T>(a, KD);
    }
    GLA_LAUNCH("fwd_walk", (gla_fwd_wide_walk<T, KD, BV, true>), dim3((unsigned)xcd_grid(a.P * a.BH, nvb)),
               dim3(512), a.stream, (const unsigned char*)rec, (const T*)a.v, (const T*)a.ws_state, a.s0, (T*)a.o,
               a.s_final, (T*)nullptr, (float*)nullptr, a.T, a.H, a.V, a.N, a.P, a.seg_len, a.P, (int)a.BH);
    return hipGetLastError();
}

template <int KD, int BV>
static hipError_t launch_fwd_wide_t(const FwdLaunch& a) {
    return a.sg ? launch_fwd_wide_bv<KD, BV, true>(a) : launch_fwd_wide_bv<KD, BV, false>(a);
}

hipError_t launch_fwd_wide(const FwdLaunch& a) {
    if (a.K != 256) return hipErrorInvalidValue;
    if (a.BV == 64) return launch_fwd_wide_t<256, 64>(a);
    if (a.BV == 128) return launch_fwd_wide_t<256, 128>(a);
    return hipErrorInvalidValue;
}

}  // namespace gla
