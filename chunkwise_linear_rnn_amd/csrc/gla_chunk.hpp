// Chunk-level pieces shared by the forward and backward kernels: the LDS
// layout of one chunk for the column-split kernels, the per-wave state tiles,
// the decayed state update, and the segment-local state kernel.
#pragma once

#include "gla_device.hpp"

namespace gla {

// ---------------------------------------------------------------------------
// Shared-memory layout of one chunk for the column-split kernels.
template <typename T, int KD, int BV, int NT>
struct ChunkSmem {
    static constexpr int PT = Elem<T>::pad;
    static constexpr int pB = KD + 4;      // fp32 cumulative log gate
    static constexpr int pQ = KD + PT;     // q-side operand, row-major [t][i]
    static constexpr int pK = KD + PT;     // k-side operand, row-major [s][i]
    static constexpr int pV = BV + PT;     // value (or d_o) tile, row-major [s][j]
    static constexpr int pA = kChunk + PT; // intra-chunk attention A[t][s]
    float B[kChunk * pB];
    T Q[kChunk * pQ];
    T K[kChunk * pK];
    T V[kChunk * pV];
    T A[kChunk * pA];
    float tot[NT];
    float last[KD];
    float gam[KD];
    int flag;
};

// One wave's share of the state: rows 0..KD-1, columns col0 .. col0+16*CB-1,
// as KD/16 x CB accumulator tiles.
template <int KD, int CB>
struct StateRegs {
    f32x4 s[KD / 16][CB];
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int a = 0; a < KD / 16; ++a)
#pragma unroll
            for (int c = 0; c < CB; ++c) s[a][c] = zero4();
    }
    // element (i, j) of tile (a, c) for accumulator slot r: i = 16a + 4*(l/16) + r, j = col0 + 16c + l%16
    __device__ __forceinline__ void load(const float* __restrict__ src, long ld, int col0) {
        const int l = lane_id();
#pragma unroll
        for (int a = 0; a < KD / 16; ++a)
#pragma unroll
            for (int c = 0; c < CB; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s[a][c][r] = src[(long)(16 * a + 4 * (l >> 4) + r) * ld + col0 + 16 * c + (l & 15)];
    }
    __device__ __forceinline__ void store(float* __restrict__ dst, long ld, int col0) const {
        const int l = lane_id();
#pragma unroll
        for (int a = 0; a < KD / 16; ++a)
#pragma unroll
            for (int c = 0; c < CB; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(long)(16 * a + 4 * (l >> 4) + r) * ld + col0 + 16 * c + (l & 15)] = s[a][c][r];
    }
};

// S <- Diag(gamma) S + X^T Y over the 64 rows of the chunk (Section 4.2:
// S_[i+1] = (gamma^T 1) * S_[i] + (K*Gamma)^T V).  X (row-major [t][i], the
// already-decayed key/query tile) and Y (row-major [t][j]) are in LDS, and so
// is gamma.  Columns of this wave: col0 .. col0 + 16*CB - 1.
template <typename T, int KD, int CB>
__device__ __forceinline__ void state_update(StateRegs<KD, CB>& S, const T* X, int pX, const T* Y, int pY,
                                             const float* gamma, int col0) {
    const int l = lane_id();
#pragma unroll
    for (int a = 0; a < KD / 16; ++a) {
        const f32x4 gam = *reinterpret_cast<const f32x4*>(gamma + 16 * a + 4 * (l >> 4));
#pragma unroll
        for (int c = 0; c < CB; ++c) S.s[a][c] *= gam;
    }
    vec4_t<T> yf[4][CB];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
        for (int c = 0; c < CB; ++c) yf[sb][c] = frag_cm<T>(Y, pY, 16 * sb, col0 + 16 * c);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int a = 0; a < KD / 16; ++a) {
            vec4_t<T> xlo = frag_cm<T>(X, pX, 32 * ks, 16 * a);
            vec4_t<T> xhi = frag_cm<T>(X, pX, 32 * ks + 16, 16 * a);
#pragma unroll
            for (int c = 0; c < CB; ++c) S.s[a][c] = mma32(S.s[a][c], xlo, xhi, yf[2 * ks][c], yf[2 * ks + 1][c]);
        }
    }
}

__device__ __forceinline__ void decode_tile(int tile, int& is, int& js) {
    // lower-triangular 16x16 tiles of the 64x64 chunk, row by row
    constexpr int tis[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
    constexpr int tjs[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
    is = tis[tile];
    js = tjs[tile];
}

// ---------------------------------------------------------------------------
// Step 2: the linear recurrence across segments for one state element.
//   forwards  (REV = false): out[0] = init, out[p+1] = exp2(G_p) out[p] + in[p]
//   backwards (REV = true):  out[P-1] = init, out[p-1] = exp2(G_p) out[p] + in[p]
// `st` holds in[] on entry and out[] on exit (stride KV), `gt` the segment gate
// totals G_p in log2 units (stride K).  The loads of U segments are issued
// before any of their results is needed, so one thread keeps U independent
// requests in flight rather than one per step.
template <bool REV>
__device__ __forceinline__ void combine_element(float* st, const float* gt, long KV, long K, int P, float cur) {
    constexpr int U = 8;
    for (int b0 = 0; b0 < P; b0 += U) {
        float a[U], gm[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = REV ? P - 1 - (b0 + u) : b0 + u;
            const bool feeds = b0 + u < P && (REV ? p >= 1 : p + 1 < P);
            a[u] = feeds ? st[p * KV] : 0.f;
            gm[u] = feeds ? exp2_fast(gt[p * K]) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = REV ? P - 1 - (b0 + u) : b0 + u;
            if (b0 + u < P) {
                st[p * KV] = cur;
                cur = gm[u] * cur + a[u];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Step 1: segment-local states.  REV = false: S*_p from the keys and values of
// the segment walked forwards (decay Gamma = exp2(B_63 - B_t) on the keys).
// REV = true: the backward pass's dS*_p from queries and d_o walked backwards
// (decay Lambda = exp2(B_t) on the queries; dS_[n-1] = gamma dS_[n] + (Q*Lambda)^T dO).
template <typename T, int KD, int BV, int NW, bool REV>
__global__ void __launch_bounds__(NW * 64)
gla_seg_state(const T* __restrict__ x, const T* __restrict__ g, const T* __restrict__ y,
              float* __restrict__ ws_state, float* __restrict__ ws_gate,
              int T_, int H, int V, int N, int P, int seg_len, int seg_first, int nseg) {
    constexpr int NT = NW * 64;
    constexpr int CB = BV / NW / 16;
    using Sm = ChunkSmem<T, KD, BV, NT>;
    __shared__ Sm sm;
    const int tid = threadIdx.x, w = wave_id();
    const int nvb = V / BV;
    int bid = blockIdx.x;
    const int vb = bid % nvb; bid /= nvb;
    const int seg = seg_first + bid % nseg; bid /= nseg;
    const int bh = bid;
    const int b = bh / H, h = bh % H;
    const int v0 = vb * BV;
    const int c_begin = seg * seg_len;
    const int c_end = min(N, c_begin + seg_len);
    const int nchunks = c_end - c_begin;
    const int rsK = H * KD, rsV = H * V;
    const int col0 = w * (BV / NW);

    StateRegs<KD, CB> S;
    S.zero();
    float gate_total = 0.f;

    TileRegs<T, KD, NT> rx, rg;
    TileRegs<T, BV, NT> ry;
    auto issue = [&](int c) {
        const long tok0 = (long)b * T_ + (long)c * kChunk;
        rx.load(x + (tok0 * H + h) * KD, rsK, tid);
        rg.load(g + (tok0 * H + h) * KD, rsK, tid);
        ry.load(y + (tok0 * H + h) * V + v0, rsV, tid);
    };
    issue(REV ? c_end - 1 : c_begin);
    for (int it = 0; it < nchunks; ++it) {
        if (tid == 0) sm.flag = 0;
        chunk_log_cumsum<T, KD, NT>(rg, sm.B, Sm::pB, sm.tot, sm.last, sm.gam, &sm.flag, tid);
        if (tid < KD) gate_total += sm.last[tid];
        // decayed operand: K*Gamma (forward) or Q*Lambda (reverse)
        using TR = TileRegs<T, KD, NT>;
#pragma unroll
        for (int p = 0; p < TR::PER; ++p) {
            if (!TR::owns(p, tid)) continue;
            const int row = TR::row_of(p, tid), c0 = TR::col_of(p, tid);
            float vals[TR::VEC];
#pragma unroll
            for (int e = 0; e < TR::VEC; ++e) {
                const float bt = sm.B[row * Sm::pB + c0 + e];
                const float ex = REV ? bt : (sm.last[c0 + e] - bt);
                vals[e] = rx.get(p, e) * exp2_fast(ex);
            }
            store_vec_lds<T>(sm.K + row * Sm::pK + c0, vals);
        }
        ry.store_lds(sm.V, Sm::pV, tid);
        if (it + 1 < nchunks) issue(REV ? c_end - 2 - it : c_begin + it + 1);
        __syncthreads();
        state_update<T, KD, CB>(S, sm.K, Sm::pK, sm.V, Sm::pV, sm.gam, col0);
        __syncthreads();
    }
    float* dst = ws_state + ((long)bh * P + seg) * (long)KD * V + v0;
    S.store(dst, V, col0);
    if (vb == 0 && tid < KD) ws_gate[((long)bh * P + seg) * KD + tid] = gate_total;
}

}  // namespace gla
