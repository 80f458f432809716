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
void launch_combine_fwd(const FwdLaunch& a, int KD, bool ck_out, bool st_out);  // gla_fwd.hip

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
               (const T*)a.q, (const T*)a.k, (const T*)a.g, rec, a.T, a.H, a.N, (long)WideRec<KD>::bytes);
    if (a.P > 1) {
        const int nseg = a.P - 1;
        GLA_LAUNCH("fwd_seg_state", (gla_fwd_wide_walk<T, KD, BV, false>), dim3((unsigned)xcd_grid(nseg * a.BH, nvb)),
                   dim3(512), a.stream, (const unsigned char*)rec, (const T*)a.v, (const T*)nullptr,
                   (const float*)nullptr, (T*)nullptr, (float*)nullptr, (T*)a.ws_state, a.ws_gate, a.T, a.H, a.V,
                   a.N, a.P, a.seg_len, nseg, (int)a.BH);
        launch_combine_fwd<T>(a, KD, false, false);
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

// Segment combine under general gates: out[0] = S_0, out[p+1] = exp2(GA_p[i] +
// GB_p[j]) out[p] + in[p], with GA/GB the segment's log2 decays of key row i
// and value column j.  One thread per 4 adjacent elements of a state row.  The
// outputs overwrite the inputs in place, so the loop form (any P) reads each
// segment only after storing the one before; for P <= NMAX every input is read
// first (NMAX loads per thread, the ones past P - 1 repeating segment 0), then
// the chain runs from registers.
template <int NMAX>
__global__ void __launch_bounds__(256)
gla_seg_combine_fwd_general(const float* __restrict__ s0, bf16* __restrict__ ws_state,
                            const float* __restrict__ ws_gate, const float* __restrict__ ws_gateb, int K, int V,
                            int P) {
    using VT = bf16 __attribute__((ext_vector_type(4)));
    const long KV = (long)K * V;
    const long e = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
    const long bh = blockIdx.y;
    if (e >= KV) return;
    const int i = (int)(e / V), j = (int)(e % V);
    bf16* st = ws_state + bh * P * KV + e;
    const float* ga = ws_gate + bh * P * (long)K + i;
    const float* gbv = ws_gateb + bh * P * (long)V + j;
    f32x4 cur = s0 ? *reinterpret_cast<const f32x4*>(s0 + bh * KV + e) : f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (NMAX > 0) {
        VT in[NMAX];
        float gr[NMAX];
        f32x4 gcol[NMAX];
#pragma unroll
        for (int u = 0; u < NMAX; ++u) {
            const int p = u + 1 < P ? u : 0;  // segment P-1 has no state of its own
            in[u] = *reinterpret_cast<const VT*>(st + p * KV);
            gr[u] = ga[(long)p * K];
            gcol[u] = *reinterpret_cast<const f32x4*>(gbv + (long)p * V);
        }
#pragma unroll
        for (int u = 0; u < NMAX; ++u) {
            if (u < P) {
                VT o;
#pragma unroll
                for (int c = 0; c < 4; ++c) o[c] = Elem<bf16>::from_f(cur[c]);
                *reinterpret_cast<VT*>(st + u * KV) = o;
                if (u + 1 < P) {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        cur[c] = exp2f(gr[u] + gcol[u][c]) * cur[c] + Elem<bf16>::to_f(in[u][c]);
                }
            }
        }
        return;
    }
    for (int p = 0; p < P; ++p) {
        // segment P-1 has no state of its own: only its initial state is written
        const bool feeds = p + 1 < P;
        VT in{};
        float gr = 0.f;
        f32x4 gcol{0.f, 0.f, 0.f, 0.f};
        if (feeds) {
            in = *reinterpret_cast<const VT*>(st + p * KV);
            gr = ga[(long)p * K];
            gcol = *reinterpret_cast<const f32x4*>(gbv + (long)p * V);
        }
        VT o;
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] = Elem<bf16>::from_f(cur[c]);
        *reinterpret_cast<VT*>(st + p * KV) = o;
        if (feeds) {
#pragma unroll
            for (int c = 0; c < 4; ++c) cur[c] = exp2f(gr + gcol[c]) * cur[c] + Elem<bf16>::to_f(in[c]);
        }
    }
}

// General gates (16-bit): records, the state pass over segments 0..P-2, the
// combine, and the output walk, at BV value columns per workgroup.
template <int KD, int VP, int BV>
static hipError_t launch_fwd_general_kv(const FwdLaunch& a) {
    using T = bf16;
    static_assert(sizeof(GenPrepSmem<T, VP>) <= 80 * 1024, "two value-side workgroups per CU");
    static_assert(sizeof(WideSmem<T, KD, BV, true, true>) <= 160 * 1024, "LDS budget");
    static_assert(GenRec<KD>::bytes(512) == (long)gen_record_bytes(KD, 512), "record size as the workspace plans it");
    static_assert(GenRec<KD>::bytes(64) % 256 == 0 && GenRec<KD>::bytes(128) % 256 == 0, "records stay 256-byte aligned");
    if ((long)GenRec<KD>::bytes(a.V) != (long)gen_record_bytes(KD, a.V)) return hipErrorInvalidValue;
    const int nvb = a.V / BV;
    unsigned char* rec = static_cast<unsigned char*>(a.ws_rec);
    GLA_LAUNCH("fwd_prep", (gla_fwd_wide_prep<T, KD, false>), dim3((unsigned)(a.BH * a.N)), dim3(256), a.stream,
               (const T*)a.q, (const T*)a.k, (const T*)a.g, rec, a.T, a.H, a.N, (long)GenRec<KD>::bytes(a.V), a.rev);
    GLA_LAUNCH("fwd_general_vprep", (gla_fwd_general_vprep<T, KD, VP, WideSmem<T, KD, BV, true, true>::WI>),
               dim3((unsigned)(a.BH * a.N), (unsigned)(a.V / VP)), dim3(256), a.stream, (const T*)a.v,
               (const T*)a.h, rec, a.T, a.H, a.V, a.N, a.rev);
    const dim3 gw((unsigned)xcd_grid(a.P * a.BH, nvb));
    if (a.init_t) {
        // every segment starts from the transpose of a known state: no state pass, no combine
        if (a.ws_hs) return hipErrorInvalidValue;
        if (a.rev)
            GLA_LAUNCH("fwd_general_walk", (gla_fwd_wide_walk<T, KD, BV, true, true, false, true, true>), gw,
                       dim3(512), a.stream, (const unsigned char*)rec, (const T*)a.v, (const T*)a.init_t, a.s0,
                       (T*)a.o, a.s_final, (T*)nullptr, (float*)nullptr, a.T, a.H, a.V, a.N, a.P, a.seg_len, a.P,
                       (int)a.BH, (float*)nullptr, (T*)nullptr);
        else
            GLA_LAUNCH("fwd_general_walk", (gla_fwd_wide_walk<T, KD, BV, true, true, false, false, true>), gw,
                       dim3(512), a.stream, (const unsigned char*)rec, (const T*)a.v, (const T*)a.init_t, a.s0,
                       (T*)a.o, a.s_final, (T*)nullptr, (float*)nullptr, a.T, a.H, a.V, a.N, a.P, a.seg_len, a.P,
                       (int)a.BH, (float*)nullptr, (T*)nullptr);
        return hipGetLastError();
    }
    if (a.P > 1) {
        const int nseg = a.P - 1;
        GLA_LAUNCH("fwd_general_seg_state", (gla_fwd_wide_walk<T, KD, BV, false, true>),
                   dim3((unsigned)xcd_grid(nseg * a.BH, nvb)), dim3(512), a.stream, (const unsigned char*)rec,
                   (const T*)a.v, (const T*)nullptr, (const float*)nullptr, (T*)nullptr, (float*)nullptr,
                   (T*)a.ws_state, a.ws_gate, a.T, a.H, a.V, a.N, a.P, a.seg_len, nseg, (int)a.BH, a.ws_gateb);
        const long KV = (long)KD * a.V;
        const dim3 gc((unsigned)((KV / 4 + 255) / 256), (unsigned)a.BH);
        if (a.P <= 8)
            GLA_LAUNCH("combine_fwd_general", gla_seg_combine_fwd_general<8>, gc, dim3(256), a.stream, a.s0,
                       (T*)a.ws_state, (const float*)a.ws_gate, (const float*)a.ws_gateb, KD, a.V, a.P);
        else if (a.P <= 16)
            GLA_LAUNCH("combine_fwd_general", gla_seg_combine_fwd_general<16>, gc, dim3(256), a.stream, a.s0,
                       (T*)a.ws_state, (const float*)a.ws_gate, (const float*)a.ws_gateb, KD, a.V, a.P);
        else if (a.P <= 32)
            GLA_LAUNCH("combine_fwd_general", gla_seg_combine_fwd_general<32>, gc, dim3(256), a.stream, a.s0,
                       (T*)a.ws_state, (const float*)a.ws_gate, (const float*)a.ws_gateb, KD, a.V, a.P);
        else
            GLA_LAUNCH("combine_fwd_general", gla_seg_combine_fwd_general<0>, gc, dim3(256), a.stream, a.s0,
                       (T*)a.ws_state, (const float*)a.ws_gate, (const float*)a.ws_gateb, KD, a.V, a.P);
    }
    if (a.ws_hs && a.rev)
        GLA_LAUNCH("fwd_general_walk_hs", (gla_fwd_wide_walk<T, KD, BV, true, true, true, true>), gw, dim3(512),
                   a.stream, (const unsigned char*)rec, (const T*)a.v, (const T*)a.ws_state, a.s0, (T*)a.o,
                   a.s_final, (T*)nullptr, (float*)nullptr, a.T, a.H, a.V, a.N, a.P, a.seg_len, a.P, (int)a.BH,
                   (float*)nullptr, (T*)a.ws_hs);
    else if (a.ws_hs)
        GLA_LAUNCH("fwd_general_walk_hs", (gla_fwd_wide_walk<T, KD, BV, true, true, true>), gw, dim3(512), a.stream,
                   (const unsigned char*)rec, (const T*)a.v, (const T*)a.ws_state, a.s0, (T*)a.o, a.s_final,
                   (T*)nullptr, (float*)nullptr, a.T, a.H, a.V, a.N, a.P, a.seg_len, a.P, (int)a.BH, (float*)nullptr,
                   (T*)a.ws_hs, a.s_final2);
    else if (a.rev)
        GLA_LAUNCH("fwd_general_walk", (gla_fwd_wide_walk<T, KD, BV, true, true, false, true>), gw, dim3(512),
                   a.stream, (const unsigned char*)rec, (const T*)a.v, (const T*)a.ws_state, a.s0, (T*)a.o,
                   a.s_final, (T*)nullptr, (float*)nullptr, a.T, a.H, a.V, a.N, a.P, a.seg_len, a.P, (int)a.BH,
                   (float*)nullptr, (T*)nullptr);
    else
        GLA_LAUNCH("fwd_general_walk", (gla_fwd_wide_walk<T, KD, BV, true, true>), gw, dim3(512), a.stream,
                   (const unsigned char*)rec, (const T*)a.v, (const T*)a.ws_state, a.s0, (T*)a.o, a.s_final,
                   (T*)nullptr, (float*)nullptr, a.T, a.H, a.V, a.N, a.P, a.seg_len, a.P, (int)a.BH, (float*)nullptr,
                   (T*)nullptr);
    return hipGetLastError();
}

template <int KD>
static hipError_t launch_fwd_general_k(const FwdLaunch& a) {
    if (a.BV == 128 && a.V % 128 == 0) return launch_fwd_general_kv<KD, 128, 128>(a);
    if (a.BV == 64 && a.V == 64) return launch_fwd_general_kv<KD, 64, 64>(a);
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_general(const FwdLaunch& a) {
    if (!a.bf16 || a.V % 64 != 0) return hipErrorInvalidValue;
    if (a.K == 128) return launch_fwd_general_k<128>(a);
    if (a.K == 256) return launch_fwd_general_k<256>(a);
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_wide(const FwdLaunch& a) {
    if (a.K != 256) return hipErrorInvalidValue;
    if (a.BV == 64) return launch_fwd_wide_t<256, 64>(a);
    if (a.BV == 128) return launch_fwd_wide_t<256, 128>(a);
    return hipErrorInvalidValue;
}

}  // namespace gla
