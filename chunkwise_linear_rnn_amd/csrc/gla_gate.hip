// Output epilogue of the multi-head GLA layer on gfx950: per-head LayerNorm,
// per-channel scale and shift, and the Swish output gate, fused in one pass.
//
// Source of the method: "Gated Linear Attention Transformers with
// Hardware-Efficient Training", Section 4.4 (GLA Transformer): each head's
// output o_t^h is normalised by LayerNorm on its own, the normalised heads are
// concatenated and multiplied elementwise by r_t = Swish(x_t W_r + b_r).  Here
// z = x W_r + b_r (a plain projection, outside this call) comes in as an input:
//     y = Swish(z) * (LN(o) * w + b),   Swish(z) = z * sigmoid(z),
//     LN(x) = (x - mean(x)) / sqrt(var(x) + eps)   over each head's V channels,
// with w, b in R^V shared by the heads.  The backward returns do, dz and the
// sums of the scale and shift gradients over all rows.
//
// Both passes are HBM-bound (a few flops per byte): a lane group of LPR lanes
// owns one row (b, t, h) with EPL contiguous channels per lane, so every row is
// read and written as whole cache lines; the row's mean and variance are
// butterfly sums inside the group.  The backward's per-channel sums of the
// scale and shift gradients are reduced per workgroup (lane groups, then waves
// through LDS) into per-workgroup partial rows, which a second small kernel
// adds in block order, so the result does not depend on scheduling.
#include <hip/hip_runtime.h>

#include "gla_device.hpp"
#include "gla_gate.hpp"
#include "gla_timing.hpp"

namespace gla {

namespace {

constexpr int kGateThreads = 256;      // forward workgroup
constexpr int kGateBwdThreads = 1024;  // backward workgroup (one per CU, kGateMaxBlocks of them)
constexpr int kGateRowsPerGroup = 2;   // rows a lane group has in flight (2 measured best of 1, 2, 4, 8)
constexpr int kGateFwdBlocks = 2048;   // forward workgroups (each loops over row passes)
constexpr int kColsumWaves = 16;       // waves per column group in the column-sum kernel

template <int V, int NT>
struct GateGeom {
    static constexpr int EPL = V >= 512 ? V / 64 : 4;  // channels per lane
    static constexpr int LPR = V / EPL;                // lanes per row
    static constexpr int RPW = 64 / LPR;               // rows per wave
    static constexpr int ROWS = (NT / 64) * RPW * kGateRowsPerGroup;  // rows per workgroup pass
    static_assert(LPR * EPL == V && LPR <= 64 && 64 % LPR == 0, "row tiling");
};

// n contiguous elements of T (16-byte aligned run of 8 or a multiple of 16 bytes)
template <typename T, int N>
__device__ __forceinline__ void load_run(const T* __restrict__ p, float* x) {
    constexpr int BYTES = N * (int)sizeof(T);
    if constexpr (BYTES % 16 == 0) {
        constexpr int E = 16 / (int)sizeof(T);
#pragma unroll
        for (int i = 0; i < BYTES / 16; ++i) {
            const u32x4 u = reinterpret_cast<const u32x4*>(p)[i];
            const T* e = reinterpret_cast<const T*>(&u);
#pragma unroll
            for (int j = 0; j < E; ++j) x[i * E + j] = Elem<T>::to_f(e[j]);
        }
    } else {
        static_assert(BYTES == 8, "8-byte run");
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 u = *reinterpret_cast<const u32x2*>(p);
        const T* e = reinterpret_cast<const T*>(&u);
#pragma unroll
        for (int j = 0; j < N; ++j) x[j] = Elem<T>::to_f(e[j]);
    }
}

template <typename T, int N>
__device__ __forceinline__ void store_run(T* __restrict__ p, const float* x) {
    constexpr int BYTES = N * (int)sizeof(T);
    if constexpr (BYTES % 16 == 0) {
        constexpr int E = 16 / (int)sizeof(T);
#pragma unroll
        for (int i = 0; i < BYTES / 16; ++i) {
            u32x4 u;
            T* e = reinterpret_cast<T*>(&u);
#pragma unroll
            for (int j = 0; j < E; ++j) e[j] = Elem<T>::from_f(x[i * E + j]);
            reinterpret_cast<u32x4*>(p)[i] = u;
        }
    } else {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        u32x2 u;
        T* e = reinterpret_cast<T*>(&u);
#pragma unroll
        for (int j = 0; j < N; ++j) e[j] = Elem<T>::from_f(x[j]);
        *reinterpret_cast<u32x2*>(p) = u;
    }
}

// sum over the LPR lanes of an aligned lane group
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = LPR / 2; m > 0; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

__device__ __forceinline__ float sigmoid(float z) { return 1.f / (1.f + __expf(-z)); }

// Row mean and reciprocal standard deviation (two passes over registers).
template <int V, int EPL, int LPR>
__device__ __forceinline__ void row_stats(const float* x, float eps, float& mean, float& rstd) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) s += x[j];
    mean = group_sum<LPR>(s) * (1.f / V);
    float q = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) q += (x[j] - mean) * (x[j] - mean);
    rstd = rsqrtf(group_sum<LPR>(q) * (1.f / V) + eps);
}

// Workgroup g covers row passes g, g + gridDim.x, ... of G::ROWS rows each.
template <typename T, int V>
__global__ void __launch_bounds__(kGateThreads)
gla_out_gate_fwd(const T* __restrict__ o, const T* __restrict__ z, const float* __restrict__ w,
                 const float* __restrict__ b, float eps, T* __restrict__ y, long R) {
    using G = GateGeom<V, kGateThreads>;
    constexpr int EPL = G::EPL;
    constexpr int NWV = kGateThreads / 64;
    const int l = lane_id();
    const int c0 = (l % G::LPR) * EPL;
    float wv[EPL], bv[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        wv[j] = w[c0 + j];
        bv[j] = b ? b[c0 + j] : 0.f;
    }
    const long npass = (R + G::ROWS - 1) / G::ROWS;
    for (long pass = blockIdx.x; pass < npass; pass += gridDim.x) {
        const long row0 = pass * G::ROWS + wave_id() * G::RPW + l / G::LPR;
        float x[kGateRowsPerGroup][EPL], zz[kGateRowsPerGroup][EPL];
#pragma unroll
        for (int u = 0; u < kGateRowsPerGroup; ++u) {
            const long row = row0 + (long)u * NWV * G::RPW;
            if (row < R) {
                load_run<T, EPL>(o + row * V + c0, x[u]);
                load_run<T, EPL>(z + row * V + c0, zz[u]);
            } else {
#pragma unroll
                for (int j = 0; j < EPL; ++j) x[u][j] = zz[u][j] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < kGateRowsPerGroup; ++u) {
            const long row = row0 + (long)u * NWV * G::RPW;
            float mean, rstd;
            row_stats<V, EPL, G::LPR>(x[u], eps, mean, rstd);
            float out[EPL];
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                const float a = (x[u][j] - mean) * rstd * wv[j] + bv[j];
                out[j] = a * zz[u][j] * sigmoid(zz[u][j]);
            }
            if (row < R) store_run<T, EPL>(y + row * V + c0, out);
        }
    }
}

// Backward of y = Swish(z) * (n * w + b), n = (x - mean) * rstd, per row:
//   da = dy * Swish(z),  dz = dy * a * sigmoid(z) * (1 + z * (1 - sigmoid(z))),
//   dn = da * w,  dx = rstd * (dn - mean(dn) - n * mean(dn * n)),
// and, summed over rows, dw = da * n, db = da.  Workgroup g covers row passes
// g, g + gridDim.x, ...; its column sums go to part_w[g][V], part_b[g][V].
template <typename T, int V>
__global__ void __launch_bounds__(kGateBwdThreads)
gla_out_gate_bwd(const T* __restrict__ o, const T* __restrict__ z, const float* __restrict__ w,
                 const float* __restrict__ b, float eps, const T* __restrict__ dy, T* __restrict__ dx,
                 T* __restrict__ dz, float* __restrict__ part_w, float* __restrict__ part_b, long R) {
    using G = GateGeom<V, kGateBwdThreads>;
    constexpr int EPL = G::EPL;
    constexpr int NWV = kGateBwdThreads / 64;
    __shared__ float s_red[2][NWV][V];
    const int l = lane_id(), wv_id = wave_id();
    const int c0 = (l % G::LPR) * EPL;
    float wv[EPL], bv[EPL], acc_w[EPL], acc_b[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        wv[j] = w[c0 + j];
        bv[j] = b ? b[c0 + j] : 0.f;
        acc_w[j] = acc_b[j] = 0.f;
    }
    const long npass = (R + G::ROWS - 1) / G::ROWS;
    for (long pass = blockIdx.x; pass < npass; pass += gridDim.x) {
        const long row0 = pass * G::ROWS + wv_id * G::RPW + l / G::LPR;
        float x[kGateRowsPerGroup][EPL], zz[kGateRowsPerGroup][EPL], g[kGateRowsPerGroup][EPL];
#pragma unroll
        for (int u = 0; u < kGateRowsPerGroup; ++u) {
            const long row = row0 + (long)u * NWV * G::RPW;
            if (row < R) {
                load_run<T, EPL>(o + row * V + c0, x[u]);
                load_run<T, EPL>(z + row * V + c0, zz[u]);
                load_run<T, EPL>(dy + row * V + c0, g[u]);
            } else {
#pragma unroll
                for (int j = 0; j < EPL; ++j) x[u][j] = zz[u][j] = g[u][j] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < kGateRowsPerGroup; ++u) {
            const long row = row0 + (long)u * NWV * G::RPW;
            float mean, rstd;
            row_stats<V, EPL, G::LPR>(x[u], eps, mean, rstd);
            float n[EPL], dn[EPL], dzo[EPL];
            float s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                n[j] = (x[u][j] - mean) * rstd;
                const float a = n[j] * wv[j] + bv[j];
                const float sg = sigmoid(zz[u][j]);
                const float da = g[u][j] * zz[u][j] * sg;  // dy (padded rows: 0) times Swish(z)
                dzo[j] = g[u][j] * a * sg * (1.f + zz[u][j] * (1.f - sg));
                dn[j] = da * wv[j];
                acc_w[j] += da * n[j];
                acc_b[j] += da;
                s1 += dn[j];
                s2 += dn[j] * n[j];
            }
            const float m1 = group_sum<G::LPR>(s1) * (1.f / V);
            const float m2 = group_sum<G::LPR>(s2) * (1.f / V);
            float dxo[EPL];
#pragma unroll
            for (int j = 0; j < EPL; ++j) dxo[j] = rstd * (dn[j] - m1 - n[j] * m2);
            if (row < R) {
                store_run<T, EPL>(dx + row * V + c0, dxo);
                store_run<T, EPL>(dz + row * V + c0, dzo);
            }
        }
    }
    // column sums: the wave's row groups (lanes LPR apart hold the same channels), then the waves
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
#pragma unroll
        for (int m = G::LPR; m < 64; m <<= 1) {
            acc_w[j] += __shfl_xor(acc_w[j], m);
            acc_b[j] += __shfl_xor(acc_b[j], m);
        }
    }
    if (l < G::LPR) {
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            s_red[0][wv_id][c0 + j] = acc_w[j];
            s_red[1][wv_id][c0 + j] = acc_b[j];
        }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < V; c += kGateBwdThreads) {
        float sw = 0.f, sb = 0.f;
#pragma unroll
        for (int q = 0; q < NWV; ++q) {
            sw += s_red[0][q][c];
            sb += s_red[1][q][c];
        }
        part_w[(long)blockIdx.x * V + c] = sw;
        part_b[(long)blockIdx.x * V + c] = sb;
    }
}

// dw[c] = sum_g part_w[g][c], db likewise.  One workgroup per 64 columns of
// [dw | db] (V is a multiple of 64, so a group never straddles the two):
// wave q adds the rows g = q (mod kColsumWaves) in four interleaved running
// sums (64 lanes read 256 contiguous bytes per row), then wave 0 adds the
// waves' sums in order.  The order is fixed, so the result is reproducible.
__global__ void __launch_bounds__(64 * kColsumWaves)
gla_out_gate_colsum(const float* __restrict__ part_w, const float* __restrict__ part_b, int nblk, int V,
                    float* __restrict__ dw, float* __restrict__ db) {
    __shared__ float s_sum[kColsumWaves][64];
    const int l = lane_id(), q = wave_id();
    const int c = blockIdx.x * 64 + l;
    const bool live = c < 2 * V;
    const bool is_w = c < V;
    const int col = is_w ? c : c - V;
    const float* src = is_w ? part_w : part_b;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    if (live && nblk > 0) {
        constexpr int S = kColsumWaves;
        int g = q;
        for (; g + 3 * S < nblk; g += 4 * S) {
            a0 += src[(long)g * V + col];
            a1 += src[(long)(g + S) * V + col];
            a2 += src[(long)(g + 2 * S) * V + col];
            a3 += src[(long)(g + 3 * S) * V + col];
        }
        for (; g < nblk; g += S) a0 += src[(long)g * V + col];
    }
    s_sum[q][l] = (a0 + a1) + (a2 + a3);
    __syncthreads();
    if (q == 0 && live) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < kColsumWaves; ++i) t += s_sum[i][l];
        float* dst = is_w ? dw : db;
        if (dst) dst[col] = t;
    }
}

template <typename T, int V>
hipError_t launch_gate_v(const GateLaunch& a) {
    if (!a.backward) {
        using G = GateGeom<V, kGateThreads>;
        const long npass = (a.R + G::ROWS - 1) / G::ROWS;
        const unsigned nfwd = (unsigned)(npass < kGateFwdBlocks ? npass : kGateFwdBlocks);
        GLA_LAUNCH("out_gate_fwd", (gla_out_gate_fwd<T, V>), dim3(nfwd), dim3(kGateThreads), a.stream,
                   (const T*)a.o, (const T*)a.z, a.w, a.b, a.eps, (T*)a.y, a.R);
        return hipGetLastError();
    }
    using G = GateGeom<V, kGateBwdThreads>;
    const long npass = (a.R + G::ROWS - 1) / G::ROWS;
    const int nblk = (int)(npass < kGateMaxBlocks ? npass : kGateMaxBlocks);
    float* part_w = a.ws;
    float* part_b = a.ws + (long)kGateMaxBlocks * V;
    GLA_LAUNCH("out_gate_bwd", (gla_out_gate_bwd<T, V>), dim3((unsigned)nblk), dim3(kGateBwdThreads), a.stream,
               (const T*)a.o, (const T*)a.z, a.w, a.b, a.eps, (const T*)a.dy, (T*)a.dx, (T*)a.dz, part_w, part_b,
               a.R);
    if (a.dw || a.db) {
        GLA_LAUNCH("out_gate_colsum", gla_out_gate_colsum, dim3((unsigned)(2 * V / 64)), dim3(64 * kColsumWaves),
                   a.stream, (const float*)part_w, (const float*)part_b, nblk, V, a.dw, a.db);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_gate_t(const GateLaunch& a) {
    switch (a.V) {
        case 64: return launch_gate_v<T, 64>(a);
        case 128: return launch_gate_v<T, 128>(a);
        case 256: return launch_gate_v<T, 256>(a);
        case 512: return launch_gate_v<T, 512>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_out_gate(const GateLaunch& a) {
    if (a.R <= 0) {
        // no rows: the backward's column sums are zero
        if (a.backward && (a.dw || a.db)) {
            GLA_LAUNCH("out_gate_colsum", gla_out_gate_colsum, dim3((unsigned)(2 * a.V / 64)),
                       dim3(64 * kColsumWaves), a.stream, (const float*)nullptr, (const float*)nullptr, 0, a.V, a.dw,
                       a.db);
            return hipGetLastError();
        }
        return hipSuccess;
    }
    return a.bf16 ? launch_gate_t<bf16>(a) : launch_gate_t<float>(a);
}

}  // namespace gla
