// Recurrent form of gated linear attention for token-by-token inference on
// gfx950.
//
// Source of the method: "Gated Linear Attention Transformers with
// Hardware-Efficient Training", Section 4.1, Eq. 3 (the recurrence
// S_t = Diag(alpha_t) S_{t-1} + k_t^T v_t, o_t = q_t S_t) in its recurrent,
// one-token-at-a-time form (Section 3.1), which costs O(K V) per token and
// needs no chunking.  Used when tokens arrive one (or a few) at a time and the
// state is carried between calls.
//
// One workgroup per (head, 64 value columns).  Thread t owns columns
// v0 + 4*(t%16) .. +3 of the key rows i = t/16 + 16m, so the K x 64 slice of
// the fp32 state stays in registers across the call's tokens and every state
// row is read and written as 256 contiguous bytes.  Per token the gate decay,
// k, q and the 64 v values are staged in LDS; the q S column sums of the 16
// row groups are reduced through LDS.
//
// Gate forms (GM): 0, the key-side gate alpha_t = exp(g_t) per key column; 1,
// one gate per token and head (alpha_t = exp(g_t) times the all-ones row); 2,
// the outer product alpha_t^T beta_t with a value-side gate beta_t = exp(h_t)
// per value column (the general form, the chapter summary's Knowl 12), which
// scales column j of the state by beta_t[j] as well.
#include <hip/hip_runtime.h>

#include "gla_device.hpp"
#include "gla_launch.hpp"
#include "gla_timing.hpp"

namespace gla {

namespace {

constexpr int kDecCols = 64;   // value columns per workgroup
constexpr int kDecThreads = 256;

template <typename T, int K, int GM>
__global__ void __launch_bounds__(kDecThreads)
gla_decode_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                  const T* __restrict__ g, const T* __restrict__ hg, float* __restrict__ state, T* __restrict__ o,
                  int T_, int H, int V) {
    constexpr int R = K / 16;  // state rows per thread
    __shared__ float s_dec[2][K], s_k[2][K], s_q[2][K], s_v[2][kDecCols], s_beta[2][kDecCols];
    __shared__ f32x4 s_part[16][16];
    const int tid = threadIdx.x;
    const int cg = tid & 15, rp = tid >> 4;
    const int nvb = V / kDecCols;
    const int bh = blockIdx.x / nvb, v0 = (blockIdx.x % nvb) * kDecCols;
    const int b = bh / H, h = bh % H;
    float* st = state + (long)bh * K * V + v0 + 4 * cg;

    f32x4 S[R];
#pragma unroll
    for (int m = 0; m < R; ++m) S[m] = *reinterpret_cast<const f32x4*>(st + (long)(rp + 16 * m) * V);

    // token t's operands into LDS buffer t&1 (a barrier separates a buffer's
    // reads for token t from its refill for token t+2)
    auto stage = [&](int t) {
        const long rk = ((long)b * T_ + t) * H + h;
        const int buf = t & 1;
        for (int i = tid; i < K; i += kDecThreads) {
            s_dec[buf][i] = exp2_fast(Elem<T>::to_f(g[GM == 1 ? rk : rk * K + i]) * kLog2e);
            s_k[buf][i] = Elem<T>::to_f(k[rk * K + i]);
            s_q[buf][i] = Elem<T>::to_f(q[rk * K + i]);
        }
        if (tid < kDecCols) s_v[buf][tid] = Elem<T>::to_f(v[rk * V + v0 + tid]);
        if (GM == 2 && tid < kDecCols) s_beta[buf][tid] = exp2_fast(Elem<T>::to_f(hg[rk * V + v0 + tid]) * kLog2e);
    };
    if (T_ > 0) stage(0);
    __syncthreads();
    for (int t = 0; t < T_; ++t) {
        const int buf = t & 1;
        const f32x4 vv = *reinterpret_cast<const f32x4*>(&s_v[buf][4 * cg]);
        const f32x4 bb = GM == 2 ? *reinterpret_cast<const f32x4*>(&s_beta[buf][4 * cg]) : f32x4{1.f, 1.f, 1.f, 1.f};
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const int i = rp + 16 * m;
            const float dec = s_dec[buf][i], ki = s_k[buf][i], qi = s_q[buf][i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                S[m][e] = (GM == 2 ? dec * bb[e] : dec) * S[m][e] + ki * vv[e];
                acc[e] += qi * S[m][e];
            }
        }
        s_part[rp][cg] = acc;
        if (t + 1 < T_) stage(t + 1);
        __syncthreads();
        // o_t for this workgroup's 64 columns: sum of the 16 row groups
        if (tid < kDecCols) {
            const int c = tid >> 2, e = tid & 3;
            float sum = 0.f;
#pragma unroll
            for (int p = 0; p < 16; ++p) sum += s_part[p][c][e];
            o[(((long)b * T_ + t) * H + h) * V + v0 + tid] = Elem<T>::from_f(sum);
        }
        __syncthreads();
    }
#pragma unroll
    for (int m = 0; m < R; ++m) *reinterpret_cast<f32x4*>(st + (long)(rp + 16 * m) * V) = S[m];
}

template <typename T, int K, int GM>
hipError_t launch_decode_kg(const DecodeLaunch& a) {
    const long grid = a.BH * (a.V / kDecCols);
    GLA_LAUNCH("decode", (gla_decode_kernel<T, K, GM>), dim3((unsigned)grid), dim3(kDecThreads), a.stream,
               (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.g, (const T*)a.h, a.state, (T*)a.o, a.T,
               a.H, a.V);
    return hipGetLastError();
}
template <typename T, int K>
hipError_t launch_decode_k(const DecodeLaunch& a) {
    switch (a.gate) {
        case 0: return launch_decode_kg<T, K, 0>(a);
        case 1: return launch_decode_kg<T, K, 1>(a);
        case 2: return launch_decode_kg<T, K, 2>(a);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_decode_t(const DecodeLaunch& a) {
    switch (a.K) {
        case 64: return launch_decode_k<T, 64>(a);
        case 128: return launch_decode_k<T, 128>(a);
        case 256: return launch_decode_k<T, 256>(a);
        case 512: return launch_decode_k<T, 512>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeLaunch& a) {
    return a.bf16 ? launch_decode_t<bf16>(a) : launch_decode_t<float>(a);
}

}  // namespace gla
