// Forward kernels of chunkwise gated linear attention on gfx950.
//
// Source of the method: "Gated Linear Attention Transformers with
// Hardware-Efficient Training", Section 4.2 (chunkwise form: Lambda, Gamma,
// gamma, the inter-chunk state recurrence and O_inter = (Q*Lambda) S) and
// Section 4.3 (secondary chunking of the intra-chunk attention).  Section 3.3
// describes the two ways of exposing parallelism over the sequence; here the
// sequence of each head is cut into P segments:
//
//   1. gla_seg_state   (parallel over head x segment x column block)
//        S*_p = sum over the segment's chunks of the decayed K^T V products,
//        starting from zero, plus the segment's total log decay.
//   2. gla_seg_combine (parallel over head x state element; serial over P)
//        S_init(p+1) = Diag(decay_p) S_init(p) + S*_p,  S_init(0) = S_0.
//   3. gla_fwd_walk    (parallel over head x segment x column block)
//        walks the segment's chunks from S_init(p) with the state resident in
//        VGPRs, producing O = (Q*Lambda) S + P V chunk by chunk, and the
//        final state for the last segment.
// With P = 1 only step 3 runs (the non-materialised form of Section 3.3).
#include "gla_chunk.hpp"
#include "gla_launch.hpp"
#include "gla_timing.hpp"

namespace gla {

// ---------------------------------------------------------------------------
// Step 2 (forward): S_init(0) = S_0 (or 0); S_init(p+1) = Diag(exp2 G_p) S_init(p) + S*_p.
// ws_state[p] holds S*_p on entry and S_init(p) on exit.  One thread per
// kCombineVec adjacent elements of a state row (V is a multiple of 64).
// CKO: S_init(p) for p = m * ck_r (m >= 1) goes to ck[bh][m] ([BH][ck_P][K][V])
// instead of ws_state[p]: the starting states of a backward whose segments are
// ck_r forward segments long, which the walk then reads from there.
// STO: ws_state also holds the last segment's S*, and the final state S_T goes
// to s_final ([BH][K][V] fp32), so the walk need not store it.
template <typename ST, bool CKO = false, bool STO = false>
__global__ void __launch_bounds__(256)
gla_seg_combine_fwd(const float* __restrict__ s0, ST* __restrict__ ws_state, const float* __restrict__ ws_gate,
                    int K, int V, int P, ST* __restrict__ ck = nullptr, int ck_r = 1, int ck_P = 1,
                    float* __restrict__ s_final = nullptr) {
    const long KV = (long)K * V;
    const long e = ((long)blockIdx.x * 256 + threadIdx.x) * kCombineVec;
    const long bh = blockIdx.y;
    if (e >= KV) return;
    const int i = (int)(e / V);
    combine_row<false, ST, CKO, STO>(ws_state + bh * P * KV + e, ws_gate + bh * P * (long)K + i, KV, K, P,
                                     s0 ? s0 + bh * KV + e : nullptr, CKO ? ck + bh * ck_P * KV + e : nullptr, ck_r,
                                     STO ? s_final + bh * KV + e : nullptr);
}

// The same with each element group's segments split between two threads
// (P <= 2 * NMAX): threads t and t + 128 of a workgroup share 4 elements.
// The grid covers K*V exactly (K*V / (128 * kCombineVec) workgroups per head):
// no thread may leave before the exchange barrier.
template <int NMAX, typename ST, bool CKO = false, bool STO = false>
__global__ void __launch_bounds__(256)
gla_seg_combine_fwd_split(const float* __restrict__ s0, ST* __restrict__ ws_state, const float* __restrict__ ws_gate,
                          int K, int V, int P, ST* __restrict__ ck = nullptr, int ck_r = 1, int ck_P = 1,
                          float* __restrict__ s_final = nullptr) {
    __shared__ f32x4 carry[128];
    const long KV = (long)K * V;
    const int slot = threadIdx.x & 127, part = threadIdx.x >> 7;
    const long e = ((long)blockIdx.x * 128 + slot) * kCombineVec;
    const long bh = blockIdx.y;
    const int i = (int)(e / V);
    combine_row_split<NMAX, false, ST, CKO, STO>(ws_state + bh * P * KV + e, ws_gate + bh * P * (long)K + i, KV, K, P,
                                           s0 ? s0 + bh * KV + e : nullptr, part, &carry[slot],
                                           CKO ? ck + bh * ck_P * KV + e : nullptr, ck_r,
                                           STO ? s_final + bh * KV + e : nullptr);
}

// Copy (or zero) a [BH][K][V] fp32 state: final state of an empty sequence.
__global__ void __launch_bounds__(256) gla_state_copy(const float* __restrict__ src, float* __restrict__ dst, long n) {
    long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e < n) dst[e] = src ? src[e] : 0.f;
}

// ---------------------------------------------------------------------------
// Step 3: walk the chunks of one segment for one block of BV value columns.
//
// Per chunk (64 tokens, B = intra-chunk cumulative log2 gate, reference row
// 63; Section 4.2 with the sub-chunk tiling of Section 4.3 at c = 16):
//   Qh = q * exp2(B_t - B_63)   Kt = k * exp2(B_63 - B_s)   Ql = q * exp2(B_t)
//   A[t][s] = sum_i Qh[t][i] Kt[s][i]  for s <= t: ten 16x16 MFMA tiles
//   O  = Ql S + A V                                         (inter + intra)
//   S  = Diag(exp2 B_63) S + Kt^T V                          (state passing)
// The operands are prepared without LDS round trips: each wave owns KD/NW key
// columns with one token row per lane, scans the gate down the 64 lanes with
// DPP, and writes Qh, Kt and Ql straight to LDS.  O is accumulated transposed
// (O^T = S^T Ql^T + V^T A^T) so each lane stores four consecutive columns.
// Chunks whose gate range exceeds kRangeLimit rebuild A element by element
// (Eq. 4, fp32, exp2 of the log-gate difference).
template <typename T, int KD, int BV>
struct WalkSmem {
    static constexpr int PT = Elem<T>::pad;
    static constexpr int pB = KD + 4;       // fp32 gate cumsum (exact-path chunks only)
    static constexpr int pQ = KD + PT;
    static constexpr int pV = BV + PT;
    static constexpr int pA = kChunk + PT;
    union {
        float B[kChunk * pB];
        T Ql[kChunk * pQ];                  // q * Lambda
    };
    T Q[kChunk * pQ];                       // q * exp2(B_t - B_63), raw q on exact-path chunks
    T K[kChunk * pQ];                       // k * exp2(B_63 - B_s), raw k while A is rebuilt exactly
    T V[kChunk * pV];
    T A[kChunk * pA];
    float last[KD];
    float gam[KD];
    int flag[2];
};

template <typename T, int KD, int BV, int NW>
__global__ void __launch_bounds__(NW * 64)
gla_fwd_walk(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ g,
             const float* __restrict__ s_init, long s_init_seg_stride, long s_init_bh_stride,
             T* __restrict__ o, float* __restrict__ s_final,
             int T_, int H, int V, int N, int P, int seg_len, int BH) {
    constexpr int NT = NW * 64;
    constexpr int CB = BV / NW / 16;
    constexpr int CPK = KD / NW;            // key columns per wave in the row-slab preparation
    using Sm = WalkSmem<T, KD, BV>;
    __shared__ Sm sm;
    const int tid = threadIdx.x, w = wave_id(), l = lane_id();
    const int nvb = V / BV;
    int unit, vb;
    xcd_decode(nvb, unit, vb);
    if (unit >= BH * P) return;
    const int seg = unit % P;
    const int bh = unit / P;
    const int b = bh / H, h = bh % H;
    const int v0 = vb * BV;
    const int c_begin = seg * seg_len;
    const int c_end = min(N, c_begin + seg_len);
    const int rsK = H * KD, rsV = H * V;
    const int col0 = w * (BV / NW);
    const int kc0 = w * CPK;

    // zero the strictly-upper 16x16 tiles of A once; they are never written
    for (int e = tid; e < kChunk * kChunk; e += NT) {
        const int t = e / kChunk, s = e % kChunk;
        if ((s >> 4) > (t >> 4)) sm.A[t * Sm::pA + s] = Elem<T>::from_f(0.f);
    }
    if (tid < 2) sm.flag[tid] = 0;

    StateRegs<KD, CB> S;
    if (s_init) S.load(s_init + (long)bh * s_init_bh_stride + (long)seg * s_init_seg_stride + v0, V, col0);
    else S.zero();

    RowSlab<T, CPK> rq, rk, rg;
    TileRegs<T, BV, NT> rv;
    auto kbase = [&](const T* p, int c) { return p + ((long)b * T_ + (long)c * kChunk) * rsK + (long)h * KD; };
    auto vbase = [&](const T* p, int c) { return p + ((long)b * T_ + (long)c * kChunk) * rsV + (long)h * V + v0; };
    auto obase_of = [&](int c) { return o + ((long)b * T_ + (long)c * kChunk) * rsV + (long)h * V + v0; };
    rq.load(kbase(q, c_begin), rsK, kc0);
    rk.load(kbase(k, c_begin), rsK, kc0);
    rg.load(kbase(g, c_begin), rsK, kc0);
    rv.load(vbase(v, c_begin), rsV, tid);
    __syncthreads();
    for (int c = c_begin; c < c_end; ++c) {
        const bool more = c + 1 < c_end;
        // (a) gate cumsum down the lanes, decays, operands
        {
            float bt[CPK], bl[CPK];
            float rng = -3.0e38f;
#pragma unroll
            for (int j = 0; j < CPK; ++j) {
                bt[j] = wave_incl_scan(rg.get(j) * kLog2e);
                bl[j] = lane_bcast(bt[j], 63);
                rng = fmaxf(rng, lane_bcast(bt[j], 0) - bl[j]);
            }
            if (l == 0) {
                if (rng > kRangeLimit) sm.flag[c & 1] = 1;
#pragma unroll
                for (int j = 0; j < CPK; ++j) {
                    sm.last[kc0 + j] = bl[j];
                    sm.gam[kc0 + j] = exp2_fast(bl[j]);
                }
            }
            constexpr int VEC = 16 / (int)sizeof(T);
#pragma unroll
            for (int j0 = 0; j0 < CPK; j0 += VEC) {
                float qh[VEC], kt[VEC], ql[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const int j = j0 + e;
                    const float qq = rq.get(j), kk = rk.get(j);
                    qh[e] = qq * exp2_fast(bt[j] - bl[j]);
                    kt[e] = kk * exp2_fast(bl[j] - bt[j]);
                    ql[e] = qq * exp2_fast(bt[j]);
                }
                store_vec_lds<T>(sm.Q + l * Sm::pQ + kc0 + j0, qh);
                store_vec_lds<T>(sm.K + l * Sm::pQ + kc0 + j0, kt);
                store_vec_lds<T>(sm.Ql + l * Sm::pQ + kc0 + j0, ql);
            }
        }
        rv.store_lds(sm.V, Sm::pV, tid);
        if (more) {
            rq.load(kbase(q, c + 1), rsK, kc0);
            rk.load(kbase(k, c + 1), rsK, kc0);
            rg.load(kbase(g, c + 1), rsK, kc0);
            rv.load(vbase(v, c + 1), rsV, tid);
        }
        __syncthreads();
        const bool exact = sm.flag[c & 1] != 0;
        if (tid == 0) sm.flag[(c + 1) & 1] = 0;
        if (exact) {
            // rebuild A from raw q, k and the fp32 cumsum (element-wise Eq. 4)
            RowSlab<T, CPK> xq, xk, xg;
            xq.load(kbase(q, c), rsK, kc0);
            xk.load(kbase(k, c), rsK, kc0);
            xg.load(kbase(g, c), rsK, kc0);
            float bt[CPK], bl[CPK];
#pragma unroll
            for (int j = 0; j < CPK; ++j) {
                bt[j] = wave_incl_scan(xg.get(j) * kLog2e);
                bl[j] = lane_bcast(bt[j], 63);
            }
            __syncthreads();
            constexpr int VEC = 16 / (int)sizeof(T);
#pragma unroll
            for (int j0 = 0; j0 < CPK; j0 += VEC) {
                float qq[VEC], kk[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    qq[e] = xq.get(j0 + e);
                    kk[e] = xk.get(j0 + e);
                    sm.B[l * Sm::pB + kc0 + j0 + e] = bt[j0 + e];
                }
                store_vec_lds<T>(sm.Q + l * Sm::pQ + kc0 + j0, qq);
                store_vec_lds<T>(sm.K + l * Sm::pQ + kc0 + j0, kk);
            }
            __syncthreads();
            for (int tile = w; tile < 10; tile += NW) {
                int is, js;
                decode_tile(tile, is, js);
                const int t = 16 * is + (l & 15);
                f32x4 acc;
                for (int r = 0; r < 4; ++r) {
                    const int s = 16 * js + 4 * (l >> 4) + r;
                    float sum = 0.f;
                    if (s <= t)
                        for (int i = 0; i < KD; ++i)
                            sum += Elem<T>::to_f(sm.Q[t * Sm::pQ + i]) * Elem<T>::to_f(sm.K[s * Sm::pQ + i]) *
                                   exp2_fast(sm.B[t * Sm::pB + i] - sm.B[s * Sm::pB + i]);
                    acc[r] = sum;
                }
                *reinterpret_cast<vec4_t<T>*>(sm.A + (16 * is + (l & 15)) * Sm::pA + 16 * js + 4 * (l >> 4)) =
                    to_vec4<T>(acc);
            }
            __syncthreads();
#pragma unroll
            for (int j0 = 0; j0 < CPK; j0 += VEC) {
                float kt[VEC], ql[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const int j = j0 + e;
                    kt[e] = xk.get(j) * exp2_fast(bl[j] - bt[j]);
                    ql[e] = xq.get(j) * exp2_fast(bt[j]);
                }
                store_vec_lds<T>(sm.K + l * Sm::pQ + kc0 + j0, kt);
                store_vec_lds<T>(sm.Ql + l * Sm::pQ + kc0 + j0, ql);
            }
        } else {
            // (b) A tiles from Qh and Kt
            for (int tile = w; tile < 10; tile += NW) {
                int is, js;
                decode_tile(tile, is, js);
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < KD / 32; ++ks) {
                    vec4_t<T> alo = frag_rm<T>(sm.K, Sm::pQ, 16 * js, 32 * ks);
                    vec4_t<T> ahi = frag_rm<T>(sm.K, Sm::pQ, 16 * js, 32 * ks + 16);
                    vec4_t<T> blo = frag_rm<T>(sm.Q, Sm::pQ, 16 * is, 32 * ks);
                    vec4_t<T> bhi = frag_rm<T>(sm.Q, Sm::pQ, 16 * is, 32 * ks + 16);
                    acc = mma32(acc, alo, ahi, blo, bhi);
                }
                // acc holds A^T[s][t] for s = 16js + 4(l/16) + r, t = 16is + l%16
                if (is == js) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (4 * (l >> 4) + r > (l & 15)) acc[r] = 0.f;
                }
                *reinterpret_cast<vec4_t<T>*>(sm.A + (16 * is + (l & 15)) * Sm::pA + 16 * js + 4 * (l >> 4)) =
                    to_vec4<T>(acc);
            }
        }
        __syncthreads();
        // (c) outputs from the state before this chunk, then the state update
        {
            vec4_t<T> sf[KD / 32][CB][2];
#pragma unroll
            for (int ks = 0; ks < KD / 32; ++ks)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    sf[ks][cb][0] = to_vec4<T>(S.s[2 * ks][cb]);
                    sf[ks][cb][1] = to_vec4<T>(S.s[2 * ks + 1][cb]);
                }
            vec4_t<T> vf[4][CB];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) vf[sb][cb] = frag_cm<T>(sm.V, Sm::pV, 16 * sb, col0 + 16 * cb);
            T* obase = obase_of(c);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                f32x4 acc[CB];
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) acc[cb] = zero4();
                // O^T[j][t] = sum_i S[i][j] Ql[t][i] + sum_s V[s][j] A[t][s]
#pragma unroll
                for (int ks = 0; ks < KD / 32; ++ks) {
                    vec4_t<T> blo = frag_rm<T>(sm.Ql, Sm::pQ, 16 * rb, 32 * ks);
                    vec4_t<T> bhi = frag_rm<T>(sm.Ql, Sm::pQ, 16 * rb, 32 * ks + 16);
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) acc[cb] = mma32(acc[cb], sf[ks][cb][0], sf[ks][cb][1], blo, bhi);
                }
#pragma unroll
                for (int ks2 = 0; ks2 <= rb / 2; ++ks2) {
                    vec4_t<T> blo = frag_rm<T>(sm.A, Sm::pA, 16 * rb, 32 * ks2);
                    vec4_t<T> bhi = frag_rm<T>(sm.A, Sm::pA, 16 * rb, 32 * ks2 + 16);
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        acc[cb] = mma32(acc[cb], vf[2 * ks2][cb], vf[2 * ks2 + 1][cb], blo, bhi);
                }
                // slot r: column j = col0 + 16cb + 4(l/16) + r, token t = 16rb + l%16
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
                    *reinterpret_cast<vec4_t<T>*>(obase + (16 * rb + (l & 15)) * rsV + col0 + 16 * cb +
                                                  4 * (l >> 4)) = to_vec4<T>(acc[cb]);
            }
        }
        state_update<T, KD, CB>(S, sm.K, Sm::pQ, sm.V, Sm::pV, sm.gam, col0);
        __syncthreads();
    }
    if (s_final && seg == P - 1) S.store(s_final + (long)bh * KD * V + v0, V, col0);
}

// ---------------------------------------------------------------------------
// Step 3, software-pipelined (16-bit operands).  Same mathematics as
// gla_fwd_walk, with the operands in the chunk-start basis
//   Ql = q * exp2(B_t)   Kt = k * exp2(-B_s)   A[t][s] = sum_i Ql[t][i] Kt[s][i]
//   S  <- Diag(gamma) (S + Kt^T V)
// so two exp2 per element build both the intra and the inter operands.  A
// column whose chunk decay exceeds kBasisLimit (log2 units) keeps the
// reference-row key factor instead, Kt = k * exp2(B_63 - B_s), with the
// state update S <- Diag(gamma) S + Kt^T V; such a chunk builds A element by
// element (Eq. 4).  The state update is written as S <- post * (pre * S +
// Kt^T V) with per-column (pre, post) = (1, gamma) or (gamma, 1).
//
// Two phases per chunk, one barrier after each:
//   phase 1: A(c) from Ql(c), Kt(c);  preparation of chunk c+1 into the other
//            buffer (DPP cumsum down the lanes, exp2, bf16 packing)
//   phase 2: O(c) = Ql(c) S + A(c) V(c);  state update;  V(c+1) into the
//            wave's own LDS slice
// so the vector-ALU preparation of the next chunk overlaps the matrix work of
// this one.  Each wave owns BV/NW value columns: its slice of V never needs a
// workgroup barrier.
//
// CK (checkpointing forward): after the update of every chunk c with c + 1 a
// multiple of ck_len (and c + 1 < N), the state before chunk c + 1 is also
// written to ck[bh][(c + 1) / ck_len] ([BH][ck_P][K][V], input dtype): the
// segment-start states of a backward whose segments are ck_len chunks long.
// CKI (the combine wrote that checkpoint): segments seg with seg % ck_len == 0
// (ck_len counted in segments here) start from ck[bh][seg / ck_len].
template <typename T, int KD, int BV, int NW, bool SG = false, bool CK = false, bool CKI = false>
__global__ void __launch_bounds__(NW * 64)
gla_fwd_walk_pipe(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                  const T* __restrict__ g, const T* __restrict__ ws_init, const float* __restrict__ s0,
                  T* __restrict__ o, float* __restrict__ s_final, int T_, int H, int V, int N, int P, int seg_len,
                  int BH, T* __restrict__ ck = nullptr, int ck_len = 1, int ck_P = 1) {
    constexpr int NT = NW * 64;
    using Sm = PipeSmem<T, KD, BV, NW, false>;
    constexpr int CW = Sm::CW, CB = CW / 16, CPK = KD / NW;
    static_assert(CW % 16 == 0 && CPK % (16 / (int)sizeof(T)) == 0, "wave tiling");
    __shared__ Sm sm;
    const int tid = threadIdx.x, w = wave_id(), l = lane_id();
    const int nvb = V / BV;
    int unit, vb;
    xcd_decode(nvb, unit, vb);
    if (unit >= BH * P) return;
    const int seg = unit % P;
    const int bh = unit / P;
    const int b = bh / H, h = bh % H;
    const int c_begin = seg * seg_len;
    const int c_end = min(N, c_begin + seg_len);
    const int rsK = H * KD, rsV = H * V;
    const int col0 = vb * BV + w * CW;      // first value column of this wave
    const int kc0 = w * CPK;                // first key column this wave prepares
    auto vslice = [&](int c) { return sm.Vw + ((Sm::VB == 2 ? (c & 1) : 0) * NW + w) * kChunk * Sm::pW; };

    for (int e = tid; e < kChunk * kChunk; e += NT) {
        const int t = e / kChunk, s = e % kChunk;
        if ((s >> 4) > (t >> 4)) sm.A[t * Sm::pA + s] = Elem<T>::from_f(0.f);
    }
    if (tid < 2) sm.buf[tid].flag[0] = 0;

    // segment 0 starts from the caller's fp32 S_0, later ones from the combined
    // segment states ([BH][P][K][V], input dtype)
    StateRegs<KD, CB> S;
    if (seg > 0) {
        const T* st = ws_init + ((long)bh * P + seg) * KD * V;
        if constexpr (CKI) {
            if (seg % ck_len == 0) st = ck + ((long)bh * ck_P + seg / ck_len) * KD * V;
        }
        S.load(st, V, col0);
    } else if (s0) {
        S.load(s0 + (long)bh * KD * V, V, col0);
    } else {
        S.zero();
    }

    RowSlab<T, CPK> rq, rk;
    GateSlab<T, CPK, SG> rg;
    TileRegs<T, CW, 64> rv;
    auto kbase = [&](const T* p, int c) { return p + ((long)b * T_ + (long)c * kChunk) * rsK + (long)h * KD; };
    // g: per key column [B,T,H,K], or (SG) one value per token and head [B,T,H]
    auto gbase = [&](int c) { return SG ? g + ((long)b * T_ + (long)c * kChunk) * H + h : kbase(g, c); };
    const int rsG = SG ? H : rsK;
    auto vrow = [&](const T* p, int c) { return p + ((long)b * T_ + (long)c * kChunk) * rsV + (long)h * V + col0; };
    auto load_slabs = [&](int c) {
        rq.load(kbase(q, c), rsK, kc0);
        rk.load(kbase(k, c), rsK, kc0);
        rg.load(gbase(c), rsG, kc0);
    };
    // column groups of the preparation done in phase 1 (m < MG) and phase 2
    constexpr int NG = CPK / (16 / (int)sizeof(T)), MG = (NG + 1) / 2;
    auto load_groups = [&](int c, int m0, int m1) {
        rq.load_part(kbase(q, c), rsK, kc0, m0, m1);
        rk.load_part(kbase(k, c), rsK, kc0, m0, m1);
        rg.load_part(gbase(c), rsG, kc0, m0, m1);
    };
    load_slabs(c_begin);
    rv.load(vrow(v, c_begin), rsV, l);
    __syncthreads();
    pipe_prep<T, CPK>(sm.buf[c_begin & 1], Sm::pQl, Sm::pKt, rq, rk, rg, kc0, 0, NG);
    rv.store_lds(vslice(c_begin), Sm::pW, l);
    if (c_begin + 1 < c_end) {
        load_slabs(c_begin + 1);
        if (Sm::VB == 1) rv.load(vrow(v, c_begin + 1), rsV, l);
    }
    __syncthreads();
    for (int c = c_begin; c < c_end; ++c) {
        auto& cur = sm.buf[c & 1];
        auto& nxt = sm.buf[(c + 1) & 1];
        const bool more = c + 1 < c_end;
        const bool exact = cur.flag[0] != 0;
        if (Sm::VB == 2 && more) rv.load(vrow(v, c + 1), rsV, l);
        // ---- phase 1: A(c), preparation of chunk c+1
        if (!exact) {
            for (int tile = w; tile < 10; tile += NW) {
                int is, js;
                decode_tile(tile, is, js);
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < KD / 32; ++ks)
                    acc = mma32_rr<T>(acc, cur.Kt, Sm::pKt, 16 * js, cur.Ql, Sm::pQl, 16 * is, 32 * ks);
                // acc holds A^T[s][t] for s = 16js + 4(l/16) + r, t = 16is + l%16
                if (is == js) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (4 * (l >> 4) + r > (l & 15)) acc[r] = 0.f;
                }
                *reinterpret_cast<vec4_t<T>*>(sm.A + (16 * is + (l & 15)) * Sm::pA + 16 * js + 4 * (l >> 4)) =
                    to_vec4<T>(acc);
            }
        } else {
            // Eq. 4 element by element: A[t][s] = sum_i q_ti k_si exp2(B_ti - B_si)
            // into an fp32 tile (the spare buffer, refilled below once A is final),
            // each wave summing every key column for its own key tokens s.
            float* Af = reinterpret_cast<float*>(nxt.Ql);
            for (int e = tid; e < kChunk * Sm::pF; e += NT) Af[e] = 0.f;
            __syncthreads();
            exact_intra_tile<T, KD, NW, SG>(Af, Sm::pF, kbase(q, c), kbase(k, c), gbase(c), rsK, rsG, w);
            __syncthreads();
            for (int e = tid; e < kChunk * kChunk; e += NT) {
                const int t = e / kChunk, s = e % kChunk;
                if ((s >> 4) == (t >> 4) || s < t)
                    sm.A[t * Sm::pA + s] = Elem<T>::from_f(s <= t ? Af[t * Sm::pF + s] : 0.f);
            }
            __syncthreads();
        }
        // Inter-chunk outputs O^T[j][t] = sum_i S[i][j] Ql[t][i] need no A, so they
        // share phase 1 with the next chunk's preparation.  Waves w and w + NW/2
        // run on the same SIMD and take the two pieces in opposite order, so
        // one's matrix work overlaps the other's vector work.  On the last chunk
        // the preparation runs on stale registers into the unused buffer.
        f32x4 acc[4][CB];
        auto inter = [&]() {
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = zero4();
#pragma unroll
            for (int ks = 0; ks < KD / 32; ++ks) {
                vec4_t<T> sf[CB][2];
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    sf[cb][0] = to_vec4<T>(S.s[2 * ks][cb]);
                    sf[cb][1] = to_vec4<T>(S.s[2 * ks + 1][cb]);
                }
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const vec4_t<T> blo = frag_rm<T>(cur.Ql, Sm::pQl, 16 * rb, 32 * ks);
                    const vec4_t<T> bhi = frag_rm<T>(cur.Ql, Sm::pQl, 16 * rb, 32 * ks + 16);
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        acc[rb][cb] = mma32(acc[rb][cb], sf[cb][0], sf[cb][1], blo, bhi);
                }
            }
        };
        if (w < NW / 2) {
            inter();
            __builtin_amdgcn_sched_barrier(0);
            pipe_prep<T, CPK>(nxt, Sm::pQl, Sm::pKt, rq, rk, rg, kc0, 0, MG);
        } else {
            pipe_prep<T, CPK>(nxt, Sm::pQl, Sm::pKt, rq, rk, rg, kc0, 0, MG);
            __builtin_amdgcn_sched_barrier(0);
            inter();
        }
        if (c + 2 < c_end) load_groups(c + 2, 0, MG);
        if (Sm::VB == 2 && more) rv.store_lds(vslice(c + 1), Sm::pW, l);
        __syncthreads();
        // ---- phase 2: intra-chunk outputs, then the state update
        {
            const T* Vw = vslice(c);
            vec4_t<T> vf[4][CB];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) vf[sb][cb] = frag_cm<T>(Vw, Sm::pW, 16 * sb, 16 * cb);
            T* obase = o + ((long)b * T_ + (long)c * kChunk) * rsV + (long)h * V + col0;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                // O^T[j][t] += sum_s V[s][j] A[t][s]
#pragma unroll
                for (int ks2 = 0; ks2 <= rb / 2; ++ks2) {
                    const vec4_t<T> blo = frag_rm<T>(sm.A, Sm::pA, 16 * rb, 32 * ks2);
                    const vec4_t<T> bhi = frag_rm<T>(sm.A, Sm::pA, 16 * rb, 32 * ks2 + 16);
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        acc[rb][cb] = mma32(acc[rb][cb], vf[2 * ks2][cb], vf[2 * ks2 + 1][cb], blo, bhi);
                }
                // slot r: column j = col0 + 16cb + 4(l/16) + r, token t = 16rb + l%16
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
                    *reinterpret_cast<vec4_t<T>*>(obase + (16 * rb + (l & 15)) * rsV + 16 * cb + 4 * (l >> 4)) =
                        to_vec4<T>(acc[rb][cb]);
            }
            // S <- post * (pre * S + Kt^T V); slot r of tile (a, cb) is key row 16a + 4(l/16) + r
            auto update = [&]() {
                // pre is 1 in every column of a chunk inside the basis range
                if (exact)
#pragma unroll
                    for (int a = 0; a < KD / 16; ++a) {
                        const f32x4 pre = *reinterpret_cast<const f32x4*>(cur.pre + 16 * a + 4 * (l >> 4));
#pragma unroll
                        for (int cb = 0; cb < CB; ++cb) S.s[a][cb] *= pre;
                    }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                    for (int a = 0; a < KD / 16; ++a) {
                        const vec4_t<T> xlo = frag_cm<T>(cur.Kt, Sm::pKt, 32 * ks, 16 * a);
                        const vec4_t<T> xhi = frag_cm<T>(cur.Kt, Sm::pKt, 32 * ks + 16, 16 * a);
#pragma unroll
                        for (int cb = 0; cb < CB; ++cb)
                            S.s[a][cb] = mma32(S.s[a][cb], xlo, xhi, vf[2 * ks][cb], vf[2 * ks + 1][cb]);
                    }
                }
#pragma unroll
                for (int a = 0; a < KD / 16; ++a) {
                    const f32x4 post = *reinterpret_cast<const f32x4*>(cur.post + 16 * a + 4 * (l >> 4));
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) S.s[a][cb] *= post;
                }
            };
            if (w < NW / 2) {
                update();
                __builtin_amdgcn_sched_barrier(0);
                pipe_prep<T, CPK>(nxt, Sm::pQl, Sm::pKt, rq, rk, rg, kc0, MG, NG);
            } else {
                pipe_prep<T, CPK>(nxt, Sm::pQl, Sm::pKt, rq, rk, rg, kc0, MG, NG);
                __builtin_amdgcn_sched_barrier(0);
                update();
            }
            if (c + 2 < c_end) load_groups(c + 2, MG, NG);
            if constexpr (CK) {
                if ((c + 1) % ck_len == 0 && c + 1 < N) {
                    // the lane's offset is formed here, behind an empty asm: hoisted
                    // out of the chunk loop, the store's 64 addresses would stay
                    // live across every chunk and spill
                    int lo = 4 * (l >> 4) * V + col0 + (l & 15);
                    int vs = V;
                    asm volatile("" : "+v"(lo), "+s"(vs));
                    T* dst = ck + ((long)bh * ck_P + (c + 1) / ck_len) * KD * V + lo;
#pragma unroll
                    for (int a = 0; a < KD / 16; ++a)
#pragma unroll
                        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                dst[(16 * a + r) * vs + 16 * cb] = Elem<T>::from_f(S.s[a][cb][r]);
                }
            }
        }
        if (tid == 0) cur.flag[0] = 0;  // read by every thread before the phase-1 barrier
        if (Sm::VB == 1 && more) {
            rv.store_lds(vslice(c + 1), Sm::pW, l);
            if (c + 2 < c_end) rv.load(vrow(v, c + 2), rsV, l);
        }
        __syncthreads();
    }
    if (s_final && seg == P - 1) S.store(s_final + (long)bh * KD * V, V, col0);
}

// ---------------------------------------------------------------------------
// Host launchers.
// ck_out: the combine writes every a.ck_len / a.seg_len-th segment start into
// the checkpoint a.ckpt instead of the workspace (the caller checks that this
// ratio is whole), so the walk stores none and reads those from there.
// st_out: the segment pass has formed every segment's S*, and the combine
// writes S_T to a.s_final (the walk's last segments then store nothing).
template <typename T, bool CKO, bool STO>
static void launch_combine_fwd_v(const FwdLaunch& a, int KD) {
    const long KV = (long)KD * a.V;
    const int r = CKO ? a.ck_len / a.seg_len : 1;
    if (a.P <= 2 * kSplitMax && KV % (128 * kCombineVec) == 0) {
        dim3 g2((unsigned)(KV / (128 * kCombineVec)), (unsigned)a.BH);
        const int nm = split_nmax(a.P);
        if (nm == 4)
            GLA_LAUNCH("combine_fwd", (gla_seg_combine_fwd_split<4, T, CKO, STO>), g2, dim3(256), a.stream, a.s0,
                       (T*)a.ws_state, a.ws_gate, KD, a.V, a.P, (T*)a.ckpt, r, a.ck_P, a.s_final);
        else if (nm == 8)
            GLA_LAUNCH("combine_fwd", (gla_seg_combine_fwd_split<8, T, CKO, STO>), g2, dim3(256), a.stream, a.s0,
                       (T*)a.ws_state, a.ws_gate, KD, a.V, a.P, (T*)a.ckpt, r, a.ck_P, a.s_final);
        else
            GLA_LAUNCH("combine_fwd", (gla_seg_combine_fwd_split<16, T, CKO, STO>), g2, dim3(256), a.stream, a.s0,
                       (T*)a.ws_state, a.ws_gate, KD, a.V, a.P, (T*)a.ckpt, r, a.ck_P, a.s_final);
    } else {
        dim3 g2((unsigned)((KV / kCombineVec + 255) / 256), (unsigned)a.BH);
        GLA_LAUNCH("combine_fwd", (gla_seg_combine_fwd<T, CKO, STO>), g2, dim3(256), a.stream, a.s0,
                   (T*)a.ws_state, a.ws_gate, KD, a.V, a.P, (T*)a.ckpt, r, a.ck_P, a.s_final);
    }
}
template <typename T>
void launch_combine_fwd(const FwdLaunch& a, int KD, bool ck_out, bool st_out) {
    if (ck_out && st_out) launch_combine_fwd_v<T, true, true>(a, KD);
    else if (ck_out) launch_combine_fwd_v<T, true, false>(a, KD);
    else if (st_out) launch_combine_fwd_v<T, false, true>(a, KD);
    else launch_combine_fwd_v<T, false, false>(a, KD);
}

template <typename T, int KD, int BV, bool SG>
static hipError_t launch_fwd_sg(const FwdLaunch& a) {
    constexpr int NW = (BV / 16 < 8) ? BV / 16 : 8;
    constexpr int NT = NW * 64;
    static_assert(sizeof(ChunkSmem<T, KD, BV, NT>) <= 160 * 1024, "LDS budget");
    const int nvb = a.V / BV;
    const long KV = (long)KD * a.V;
    // a checkpoint whose states are all segment starts comes from the combine;
    // so does S_T (16-bit inputs): the segment pass then also forms the last
    // segment's S* (its workgroups fill CUs that would otherwise stay idle),
    // and the walk's last segments need not store S_T at their end
    const bool ck_comb = sizeof(T) == 2 && a.ckpt && a.P > 1 && a.ck_len % a.seg_len == 0;
    const bool st_comb = sizeof(T) == 2 && a.s_final && a.P > 1;
    if (a.P > 1) {
        // segments 0..P-2 feed the combine, and the last one too for S_T
        const int nseg = st_comb ? a.P : a.P - 1;
        dim3 grid((unsigned)xcd_grid(nseg * a.BH, nvb));
        GLA_LAUNCH("fwd_seg_state", (gla_seg_state<T, KD, BV, NW, false, SG>), grid, dim3(NT), a.stream,
                           (const T*)a.k, (const T*)a.g, (const T*)a.v, (T*)a.ws_state, a.ws_gate,
                           a.T, a.H, a.V, a.N, a.P, a.seg_len, 0, nseg, (int)a.BH);
        launch_combine_fwd<T>(a, KD, ck_comb, st_comb);
    }
    float* walk_sfinal = st_comb ? nullptr : a.s_final;
    dim3 grid((unsigned)xcd_grid(a.P * a.BH, nvb));
    if constexpr (sizeof(T) == 2) {
        static_assert(sizeof(PipeSmem<T, KD, BV, NW, false>) <= 160 * 1024, "LDS budget");
        if (a.ckpt) {
            if (ck_comb)
                GLA_LAUNCH("fwd_walk", (gla_fwd_walk_pipe<T, KD, BV, NW, SG, false, true>), grid, dim3(NT),
                           a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.g,
                           (const T*)a.ws_state, a.s0, (T*)a.o, walk_sfinal, a.T, a.H, a.V, a.N, a.P, a.seg_len,
                           (int)a.BH, (T*)a.ckpt, a.ck_len / a.seg_len, a.ck_P);
            else
                GLA_LAUNCH("fwd_walk", (gla_fwd_walk_pipe<T, KD, BV, NW, SG, true>), grid, dim3(NT), a.stream,
                           (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.g, (const T*)a.ws_state, a.s0,
                           (T*)a.o, walk_sfinal, a.T, a.H, a.V, a.N, a.P, a.seg_len, (int)a.BH, (T*)a.ckpt,
                           a.ck_len, a.ck_P);
        } else {
            GLA_LAUNCH("fwd_walk", (gla_fwd_walk_pipe<T, KD, BV, NW, SG>), grid, dim3(NT), a.stream,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.g, (const T*)a.ws_state, a.s0,
                       (T*)a.o, walk_sfinal, a.T, a.H, a.V, a.N, a.P, a.seg_len, (int)a.BH);
        }
    } else {
        static_assert(!SG, "scalar gates take the 16-bit path");
        // fp32: the workspace states are fp32 and hold S_init(0) = S_0 after the combine
        const float* sinit = a.P > 1 ? (const float*)a.ws_state : a.s0;
        const long seg_stride = a.P > 1 ? KV : 0;
        const long bh_stride = a.P > 1 ? (long)a.P * KV : KV;
        static_assert(sizeof(WalkSmem<T, KD, BV>) <= 160 * 1024, "LDS budget");
        GLA_LAUNCH("fwd_walk", (gla_fwd_walk<T, KD, BV, NW>), grid, dim3(NT), a.stream,
                           (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.g, sinit, seg_stride, bh_stride,
                           (T*)a.o, a.s_final, a.T, a.H, a.V, a.N, a.P, a.seg_len, (int)a.BH);
    }
    return hipGetLastError();
}

// per-column gates, or (16-bit inputs) a scalar gate per token and head
template <typename T, int KD, int BV>
static hipError_t launch_fwd_t(const FwdLaunch& a) {
    if constexpr (sizeof(T) == 2) {
        if (a.sg) return launch_fwd_sg<T, KD, BV, true>(a);
    } else {
        if (a.sg) return hipErrorInvalidValue;
    }
    return launch_fwd_sg<T, KD, BV, false>(a);
}

template void launch_combine_fwd<bf16>(const FwdLaunch& a, int KD, bool ck_out, bool st_out);

hipError_t launch_state_copy(const float* src, float* dst, long n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    GLA_LAUNCH("state_copy", gla_state_copy, dim3((unsigned)((n + 255) / 256)), dim3(256), stream, src, dst, n);
    return hipGetLastError();
}

hipError_t launch_fwd(const FwdLaunch& a) {
    if (a.bf16) {
        if (a.K == 64) {
            if (a.BV == 64) return launch_fwd_t<bf16, 64, 64>(a);
            if (a.BV == 128) return launch_fwd_t<bf16, 64, 128>(a);
            if (a.BV == 256) return launch_fwd_t<bf16, 64, 256>(a);
        } else if (a.K == 128) {
            if (a.BV == 64) return launch_fwd_t<bf16, 128, 64>(a);
            if (a.BV == 128) return launch_fwd_t<bf16, 128, 128>(a);
            if (a.BV == 256) return launch_fwd_t<bf16, 128, 256>(a);
        } else if (a.K == 256) {
            return launch_fwd_wide(a);
        }
    } else {
        if (a.K == 64) {
            if (a.BV == 64) return launch_fwd_t<float, 64, 64>(a);
            if (a.BV == 128) return launch_fwd_t<float, 64, 128>(a);
        } else if (a.K == 128) {
            if (a.BV == 64) return launch_fwd_t<float, 128, 64>(a);
            if (a.BV == 128) return launch_fwd_t<float, 128, 128>(a);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace gla
