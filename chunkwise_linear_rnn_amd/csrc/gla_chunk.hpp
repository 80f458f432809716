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
    // (U: fp32 caller states or the workspace's segment states in the input dtype)
    template <typename U>
    __device__ __forceinline__ void load(const U* __restrict__ src, long ld, int col0) {
        const int l = lane_id();
#pragma unroll
        for (int a = 0; a < KD / 16; ++a)
#pragma unroll
            for (int c = 0; c < CB; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s[a][c][r] = Elem<U>::to_f(src[(long)(16 * a + 4 * (l >> 4) + r) * ld + col0 + 16 * c + (l & 15)]);
    }
    // the transpose of a [cols][ld] array: element (i, j) from src[j * ld + i]
    template <typename U>
    __device__ __forceinline__ void load_t(const U* __restrict__ src, long ld, int col0) {
        const int l = lane_id();
#pragma unroll
        for (int a = 0; a < KD / 16; ++a)
#pragma unroll
            for (int c = 0; c < CB; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s[a][c][r] = Elem<U>::to_f(src[(long)(col0 + 16 * c + (l & 15)) * ld + 16 * a + 4 * (l >> 4) + r]);
    }
    template <typename U>
    __device__ __forceinline__ void store(U* __restrict__ dst, long ld, int col0) const {
        const int l = lane_id();
#pragma unroll
        for (int a = 0; a < KD / 16; ++a)
#pragma unroll
            for (int c = 0; c < CB; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(long)(16 * a + 4 * (l >> 4) + r) * ld + col0 + 16 * c + (l & 15)] = Elem<U>::from_f(s[a][c][r]);
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
    // lower-triangular 16x16 tiles of the 64x64 chunk, row by row.  Computed, not
    // looked up: a table indexed at run time becomes a global load, and waiting
    // for it would also wait for every prefetch issued before it.
    is = (tile >= 1) + (tile >= 3) + (tile >= 6);
    js = tile - (is * (is + 1)) / 2;
}

// ---------------------------------------------------------------------------
// Pieces of the software-pipelined walks (forward output walk, backward dv
// walk): operands in the chunk-start basis Ql = q * exp2(B_t), Kt = k *
// exp2(-B_s) (reference-row key factor k * exp2(B_63 - B_s) for columns beyond
// kBasisLimit), double-buffered per chunk, plus wave-private value slices.
constexpr float kBasisLimit = 96.0f;

// Pitch (elements) of a 64-row tile with KD columns.  Two-byte tiles read with
// row fragments (8 bytes per lane down 16 rows) are conflict-free at 4 mod 64
// dwords; tiles also read with transposed column fragments (ds_read_b64_tr_b16:
// 4 rows x 4 pieces per 16 lanes) need 36 mod 64 dwords for both patterns.
// The wider pitch is used for KD <= 128 only.
template <typename T, int KD, bool COLS>
constexpr int tile_pitch() {
    if (sizeof(T) != 2) return KD + Elem<T>::pad;
    if (!COLS || KD > 128) return KD + 8;
    const int dw = KD / 2;
    return 2 * (dw + ((36 - dw % 64) % 64 + 64) % 64);
}

// QL_COLS: the Ql tile is also read with column fragments (the backward's dS update).
template <typename T, int KD, int BV, int NW, bool QL_COLS>
struct PipeSmem {
    static constexpr int PT = Elem<T>::pad;
    static constexpr int CW = BV / NW;      // value columns per wave
    static constexpr int pQl = tile_pitch<T, KD, QL_COLS>();
    // the forward walk reads Kt transposed in its state update: 8 mod 64 dwords
    // keeps those reads' four rows apart at 2 KB of LDS more
    static constexpr int pKt =
        (!QL_COLS && sizeof(T) == 2 && KD <= 128) ? KD + 16 : tile_pitch<T, KD, false>();
    static constexpr int pA = kChunk + PT;
    static constexpr int pF = kChunk + 4;   // fp32 A of exact-path chunks
    // wave-private V slices, read with ds_read_b64_tr_b16: the four rows a
    // 16-lane group reads fall on disjoint banks at a pitch of 8 or 16 dwords
    // (CW = 16 or 32 two-byte columns), and rows stay 16-byte aligned.  Two
    // slices per wave when they fit, so the next chunk's V is written during
    // phase 1 instead of being held in registers through phase 2.
    static constexpr int pW = (sizeof(T) == 2 && (CW == 16 || CW == 32)) ? CW : CW + PT;
    static constexpr int VB =
        (2 * (sizeof(T) * kChunk * (pQl + pKt) + 2 * sizeof(float) * KD + 16) + sizeof(T) * kChunk * pA +
             2 * sizeof(T) * NW * kChunk * pW <= 160 * 1024) ? 2 : 1;
    struct alignas(16) Buf {
        T Ql[kChunk * pQl];
        T Kt[kChunk * pKt];
        float pre[KD];
        float post[KD];
        int flag[4];
    };
    static_assert(sizeof(T) * kChunk * (pQl + pKt) >= sizeof(float) * kChunk * pF, "exact-path scratch");
    Buf buf[2];
    alignas(16) T A[kChunk * pA];
    alignas(16) T Vw[VB * NW * kChunk * pW];
};

// One wave prepares 16-byte column groups m0 .. m1-1 of its key columns
// kc0 .. kc0+NC-1 (lane = token row) from its register slabs of q, k and the
// raw log gate.  Lane j collects B_63 of column kc0 + j and the factors are
// formed once per lane at the end, so the column loop has no branches and the
// scans of a group's VEC columns interleave.  A scalar gate (GS::scalar) has
// one cumulative gate per token: one scan and two exp2 per lane serve every
// column, and the chunk needs the exact path only if that one decay leaves the
// basis range.  KP (16-bit only): Kt is written in the paired column layout.
template <typename T, int NC, bool KP = false, typename Buf, typename GS>
__device__ __forceinline__ void pipe_prep(Buf& bf, int pQl, int pKt, const RowSlab<T, NC>& rq,
                                          const RowSlab<T, NC>& rk, const GS& rg, int kc0, int m0, int m1) {
    constexpr int VEC = 16 / (int)sizeof(T);
    static_assert(NC <= 64, "one lane per prepared column");
    const int l = lane_id();
    if constexpr (GS::scalar) {
        if (m0 >= m1) return;  // no group: the slab may already hold a later chunk's gate
        const float bt = wave_incl_scan(rg.get(0) * kLog2e);
        const float bl = lane_bcast(bt, 63);
        const bool in = -bl <= kBasisLimit;
        const float fq = exp2_fast(bt), fk = exp2_fast((in ? 0.f : bl) - bt);
#pragma unroll
        for (int m = 0; m < NC / VEC; ++m) {
            if (m < m0 || m >= m1) continue;
            const int j0 = m * VEC;
            float ql[VEC], kt[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                ql[e] = rq.get(j0 + e) * fq;
                kt[e] = rk.get(j0 + e) * fk;
            }
            store_vec_lds<T>(bf.Ql + l * pQl + kc0 + j0, ql);
            if constexpr (KP) store_paired8(bf.Kt + l * pKt, kc0 + j0, kt);
            else store_vec_lds<T>(bf.Kt + l * pKt + kc0 + j0, kt);
        }
        if (l >= m0 * VEC && l < m1 * VEC) {
            const float gm = exp2_fast(bl);
            bf.pre[kc0 + l] = in ? 1.f : gm;
            bf.post[kc0 + l] = in ? gm : 1.f;
        }
        if (!in && l == 0) bf.flag[0] = 1;
    } else {
        float last_l = 0.f;
        bool wide = false;
#pragma unroll
        for (int m = 0; m < NC / VEC; ++m) {
            if (m < m0 || m >= m1) continue;
            const int j0 = m * VEC;
            float bt[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) bt[e] = rg.get(j0 + e) * kLog2e;
            wave_incl_scan_n<VEC>(bt);
            float ql[VEC], kt[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float bl = lane_bcast(bt[e], 63);
                const bool in = -bl <= kBasisLimit;
                wide |= !in;
                last_l = (l == j0 + e) ? bl : last_l;
                ql[e] = rq.get(j0 + e) * exp2_fast(bt[e]);
                kt[e] = rk.get(j0 + e) * exp2_fast((in ? 0.f : bl) - bt[e]);
            }
            store_vec_lds<T>(bf.Ql + l * pQl + kc0 + j0, ql);
            if constexpr (KP) store_paired8(bf.Kt + l * pKt, kc0 + j0, kt);
            else store_vec_lds<T>(bf.Kt + l * pKt + kc0 + j0, kt);
        }
        if (l >= m0 * VEC && l < m1 * VEC) {
            const float gm = exp2_fast(last_l);
            const bool in = -last_l <= kBasisLimit;
            bf.pre[kc0 + l] = in ? 1.f : gm;
            bf.post[kc0 + l] = in ? gm : 1.f;
        }
        if (wide && l == 0) bf.flag[0] = 1;
    }
}

// Exact path of a chunk whose decay leaves the basis range (Eq. 4 element by
// element): Af[t][s] (fp32, pitch pF) = sum over all KD key columns i of
// q_ti k_si exp2(B_ti - B_si) for s <= t (entries s > t are left as they are).
// Wave w owns the key tokens s = w, w + NW, ... and sums every column for them
// in a fixed order, so each entry is written once by one lane and the result
// does not depend on timing.  q, k rows at qrow/krow (row stride rs, column 0 of
// the head), the log gate at grow: per column with stride rs, or SG one value
// per token with stride rsG (strides may be negative: rows taken in reverse
// time order).  zero_g0: token 0's gate is zero and not read (a time-reversed
// sequence whose first step has no decay).  Token s's values reach the lanes
// by shuffle.
// Not inlined: this rarely taken branch would otherwise change the register
// allocation and schedule of the walk's main loop (2-3 us per launch).
template <typename T, int KD, int NW, bool SG>
__device__ __attribute__((noinline)) void exact_intra_tile(float* Af, int pF, const T* __restrict__ qrow,
                                                 const T* __restrict__ krow, const T* __restrict__ grow, int rs,
                                                 int rsG, int w, bool zero_g0 = false) {
    constexpr int VEC = 16 / (int)sizeof(T);
    constexpr int NS = kChunk / NW;  // key tokens per wave
    const int l = lane_id();
    float part[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) part[u] = 0.f;
    float b0 = 0.f;
    const bool z0 = zero_g0 && l == 0;  // token 0's gate is zero and lies outside the tensor
    if constexpr (SG) b0 = wave_incl_scan(z0 ? 0.f : Elem<T>::to_f(grow[l * rsG]) * kLog2e);
    for (int j0 = 0; j0 < KD; j0 += VEC) {
        RowSlab<T, VEC> xq, xk;
        xq.load(qrow, rs, j0);
        xk.load(krow, rs, j0);
        float bt[VEC];
        if constexpr (SG) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) bt[j] = b0;
        } else {
            RowSlab<T, VEC> xg;
            xg.load_unless(grow, rs, j0, z0);
#pragma unroll
            for (int j = 0; j < VEC; ++j) bt[j] = xg.get(j) * kLog2e;
            wave_incl_scan_n<VEC>(bt);
        }
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int s = w + NW * u;
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                part[u] += xq.get(j) * __shfl(xk.get(j), s) * exp2_fast(bt[j] - __shfl(bt[j], s));
        }
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int s = w + NW * u;
        if (l >= s) Af[l * pF + s] = part[u];
    }
}

// ---------------------------------------------------------------------------
// Step 2: the linear recurrence across segments for CE adjacent elements of
// one state row.
//   forwards  (REV = false): out[0] = init, out[p+1] = exp2(G_p) out[p] + in[p]
//   backwards (REV = true):  out[P-1] = init, out[p-1] = exp2(G_p) out[p] + in[p]
// `st` holds in[] on entry and out[] on exit (stride KV, input dtype or fp32),
// `gt` the row's segment gate totals G_p in log2 units (stride K), `init` the
// CE fp32 starting values (null: zero).  The loads of up to CU segments are
// issued before any of their results is needed, and each is CE elements wide,
// so a thread keeps CU * CE * sizeof(ST) bytes in flight.  The running value
// stays fp32; only the stored states are rounded.
constexpr int kCombineVec = 4;  // elements per thread
template <typename ST> using combine_vec_t = ST __attribute__((ext_vector_type(kCombineVec)));

//
// CKO (forward only): every output S_init(p) with p > 0 and p % ck_r == 0 is
// stored to ck[(p / ck_r) * KV] instead of st[p * KV] (a checkpoint of the
// states at every ck_r-th segment start, read from there by the walk).
// STO (forward only): the last segment's S* is present too, and the state
// after it, S_T = Diag(exp2 G_{P-1}) S_init(P-1) + S*_{P-1}, goes to sT (fp32).
template <bool REV, typename ST, bool CKO = false, bool STO = false>
__device__ __forceinline__ void combine_row(ST* st, const float* gt, long KV, long K, int P, const float* init,
                                            ST* ck = nullptr, int ck_r = 1, float* sT = nullptr) {
    static_assert(!((CKO || STO) && REV), "the checkpoint and S_T are written by the forward combine");
    constexpr int CE = kCombineVec;
    constexpr int CU = 32;
    using VT = combine_vec_t<ST>;
    f32x4 cur = init ? *reinterpret_cast<const f32x4*>(init) : f32x4{0.f, 0.f, 0.f, 0.f};
    for (int b0 = 0; b0 < P; b0 += CU) {
        VT a[CU];
        float gm[CU];
        // unconditional loads from a clamped (always valid) segment, then a
        // select: a conditional load becomes a branch with its own wait
#pragma unroll
        for (int u = 0; u < CU; ++u) {
            const int j = b0 + u < P ? b0 + u : P - 1;
            const int p = REV ? P - 1 - j : j;
            a[u] = *reinterpret_cast<const VT*>(st + p * KV);
            gm[u] = gt[p * K];
        }
#pragma unroll
        for (int u = 0; u < CU; ++u) {
            const int p = REV ? P - 1 - (b0 + u) : b0 + u;
            const bool feeds = b0 + u < P && (REV ? p >= 1 : (STO || p + 1 < P));
            gm[u] = feeds ? exp2_fast(gm[u]) : 0.f;
            if (!feeds) a[u] = VT{};
        }
        // CKO: segment b0 + u is checkpoint entry m when rem == 0 (one division per block)
        int m = CKO ? b0 / ck_r : 0, rem = CKO ? b0 % ck_r : 0;
#pragma unroll
        for (int u = 0; u < CU; ++u) {
            const int p = REV ? P - 1 - (b0 + u) : b0 + u;
            if (b0 + u < P) {
                VT o;
#pragma unroll
                for (int c = 0; c < CE; ++c) o[c] = Elem<ST>::from_f(cur[c]);
                ST* dst = st + p * KV;
                if constexpr (CKO) {
                    if (p > 0 && rem == 0) dst = ck + (long)m * KV;
                    if (++rem == ck_r) rem = 0, ++m;
                }
                *reinterpret_cast<VT*>(dst) = o;
#pragma unroll
                for (int c = 0; c < CE; ++c) cur[c] = gm[u] * cur[c] + Elem<ST>::to_f(a[u][c]);
            }
        }
    }
    if constexpr (STO) *reinterpret_cast<f32x4*>(sT) = cur;
}

// The same recurrence split between two threads, for P <= 2 * NMAX: part
// 0 walks the first ceil(P/2) segments (in walking order) from `init`, part 1
// the rest from zero, keeping its outputs and the running product of its gates
// in registers.  Part 0's value after its last segment (the input of part 1's
// first) goes through `carry` (LDS, one slot per element group), and part 1
// adds it, decayed by its gate product, to each of its outputs.  Both parts of
// a slot must be in the same workgroup; every thread must call this (barrier).
// NMAX (4, 8 or 16, the launcher picks the smallest that holds ceil(P/2))
// bounds the segments per thread: each thread issues NMAX loads, the ones past
// its n repeating its last segment's address.
constexpr int kSplitMax = 16;
__host__ __device__ constexpr int split_nmax(int P) { return (P + 1) / 2 <= 4 ? 4 : ((P + 1) / 2 <= 8 ? 8 : 16); }
template <int NMAX, bool REV, typename ST, bool CKO = false, bool STO = false>
__device__ __forceinline__ void combine_row_split(ST* st, const float* gt, long KV, long K, int P, const float* init,
                                                  int part, f32x4* carry, ST* ck = nullptr, int ck_r = 1,
                                                  float* sT = nullptr) {
    static_assert(NMAX <= kSplitMax, "segments per thread");
    static_assert(!((CKO || STO) && REV), "the checkpoint and S_T are written by the forward combine");
    constexpr int CE = kCombineVec;
    using VT = combine_vec_t<ST>;
    const int h = (P + 1) / 2;
    const int j0 = part ? h : 0, n = part ? P - h : h;  // 1 <= n <= NMAX
    VT a[NMAX];
    float gm[NMAX];
#pragma unroll
    for (int u = 0; u < NMAX; ++u) {
        const int j = j0 + (u < n ? u : n - 1);
        const int p = REV ? P - 1 - j : j;
        a[u] = *reinterpret_cast<const VT*>(st + p * KV);
        gm[u] = gt[p * K];
    }
    f32x4 cur = (part == 0 && init) ? *reinterpret_cast<const f32x4*>(init) : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 loc[NMAX], fin = cur;
    float mul[NMAX];
    float m = 1.f, mfin = 1.f;
#pragma unroll
    for (int u = 0; u < NMAX; ++u) {
        const int j = j0 + u;
        const int p = REV ? P - 1 - j : j;
        const bool feeds = u < n && (REV ? p >= 1 : (STO || p + 1 < P));
        const float gu = feeds ? exp2_fast(gm[u]) : 0.f;
        loc[u] = cur;
        mul[u] = m;
#pragma unroll
        for (int c = 0; c < CE; ++c) cur[c] = gu * cur[c] + (feeds ? Elem<ST>::to_f(a[u][c]) : 0.f);
        m *= gu;
        fin = (u == n - 1) ? cur : fin;
        if constexpr (STO) mfin = (u == n - 1) ? m : mfin;
    }
    if (part == 0) *carry = fin;
    __syncthreads();
    const f32x4 cin = part ? *carry : f32x4{0.f, 0.f, 0.f, 0.f};
    int ckm = CKO ? j0 / ck_r : 0, rem = CKO ? j0 % ck_r : 0;  // as in combine_row (CKO: REV is false)
#pragma unroll
    for (int u = 0; u < NMAX; ++u) {
        if (u < n) {
            const int j = j0 + u;
            const int p = REV ? P - 1 - j : j;
            VT o;
#pragma unroll
            for (int c = 0; c < CE; ++c) o[c] = Elem<ST>::from_f(loc[u][c] + mul[u] * cin[c]);
            ST* dst = st + p * KV;
            if constexpr (CKO) {
                if (p > 0 && rem == 0) dst = ck + (long)ckm * KV;
                if (++rem == ck_r) rem = 0, ++ckm;
            }
            *reinterpret_cast<VT*>(dst) = o;
        }
    }
    // S_T: part 1 holds the last segment (P >= 2); its chain from zero plus part 0's carry
    if constexpr (STO) {
        if (part == 1) {
            f32x4 t;
#pragma unroll
            for (int c = 0; c < CE; ++c) t[c] = fin[c] + mfin * cin[c];
            *reinterpret_cast<f32x4*>(sT) = t;
        }
    }
}

// ---------------------------------------------------------------------------
// Step 1: segment-local states.  REV = false: S*_p from the keys and values of
// the segment walked forwards, S <- Diag(gamma) S + (K*Gamma)^T V with
// Gamma_s = exp2(B_63 - B_s).  REV = true: the backward pass's dS*_p from
// queries and d_o walked backwards, dS <- Diag(gamma) dS + (Q*Lambda)^T dO with
// Lambda_t = exp2(B_t).  Both decay factors are at most 1, so no chunk needs
// an exact path.
//
// One barrier per chunk: while a wave applies chunk c to its state columns it
// also prepares its key columns of chunk c+1 (register slabs, lane = token,
// DPP scan of the log gate) into the other buffer.  Waves w and w + NW/2 share
// a SIMD and take the two pieces in opposite order.  Each wave's value (or
// d_o) slice is private and double-buffered.
template <typename T, int KD, int BV, int NW>
struct SegSmem {
    static constexpr int PT = Elem<T>::pad;
    static constexpr int CW = BV / NW;  // value columns per wave
    // decayed operand, read only with column fragments: a pitch of 8 mod 64
    // dwords (bf16) keeps the four rows of a transposed read on separate banks
    static constexpr int pX = sizeof(T) == 2 ? KD + 16 : KD + 4;
    static constexpr int pW = (sizeof(T) == 2 && (CW == 16 || CW == 32)) ? CW : CW + PT;
    struct alignas(16) Buf {
        T X[kChunk * pX];
        float gam[KD];
    };
    Buf buf[2];
    alignas(16) T Yw[2 * NW * kChunk * pW];
};

// One workgroup's segment; `bid` is its block index within its own grid.  SG:
// g is a scalar per token and head ([B, T, H]), shared by every key column.
template <typename T, int KD, int BV, int NW, bool REV, bool SG = false>
__device__ __forceinline__ void seg_state_body(SegSmem<T, KD, BV, NW>& sm, int bid, const T* __restrict__ x,
                                               const T* __restrict__ g, const T* __restrict__ y,
                                               T* __restrict__ ws_state, float* __restrict__ ws_gate, int T_,
                                               int H, int V, int N, int P, int seg_len, int seg_first, int nseg,
                                               int BH, int gate_first, T* __restrict__ ws_mid = nullptr,
                                               float* __restrict__ ws_gmid = nullptr, int split = 0) {
    using Sm = SegSmem<T, KD, BV, NW>;
    constexpr int CW = Sm::CW, CB = CW / 16, CPK = KD / NW;
    constexpr int VEC = 16 / (int)sizeof(T);
    static_assert(CW % 16 == 0 && CPK % VEC == 0 && CPK <= 64, "wave tiling");
    static_assert(sizeof(Sm) <= 160 * 1024, "LDS budget");
    const int w = wave_id(), l = lane_id();
    const int nvb = V / BV;
    int unit, vb;
    xcd_decode(nvb, unit, vb, bid);
    if (unit >= BH * nseg) return;
    const int seg = seg_first + unit % nseg;
    const int bh = unit / nseg;
    const int b = bh / H, h = bh % H;
    const int c_begin = seg * seg_len;
    const int c_end = min(N, c_begin + seg_len);
    const int nchunks = c_end - c_begin;
    const int rsK = H * KD, rsV = H * V;
    const int col0 = vb * BV + w * CW;  // first value column of this wave
    const int kc0 = w * CPK;            // first key column this wave prepares

    StateRegs<KD, CB> S;
    S.zero();
    float gtot = 0.f;  // lane j: sum of B_63 over the segment for key column kc0 + j

    RowSlab<T, CPK> rx;
    GateSlab<T, CPK, SG> rg;
    TileRegs<T, CW, 64> ry;
    auto chunk_of = [&](int it) { return REV ? c_end - 1 - it : c_begin + it; };
    auto krow = [&](const T* p, int c) { return p + ((long)b * T_ + (long)c * kChunk) * rsK + (long)h * KD; };
    auto grow = [&](int c) { return SG ? g + ((long)b * T_ + (long)c * kChunk) * H + h : krow(g, c); };
    const int rsG = SG ? H : rsK;
    auto vrow = [&](const T* p, int c) { return p + ((long)b * T_ + (long)c * kChunk) * rsV + (long)h * V + col0; };
    auto yslice = [&](int it) { return sm.Yw + ((it & 1) * NW + w) * kChunk * Sm::pW; };
    auto prep = [&](typename Sm::Buf& bf) {
        if constexpr (SG) {
            const float bt = wave_incl_scan(rg.get(0) * kLog2e);
            const float bl = lane_bcast(bt, 63);
            const float f = exp2_fast(REV ? bt : bl - bt);
#pragma unroll
            for (int j0 = 0; j0 < CPK; j0 += VEC) {
                float xv[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) xv[e] = rx.get(j0 + e) * f;
                store_vec_lds<T>(bf.X + l * Sm::pX + kc0 + j0, xv);
            }
            if (l < CPK) {
                bf.gam[kc0 + l] = exp2_fast(bl);
                gtot += bl;
            }
            return;
        }
        float last_l = 0.f;
#pragma unroll
        for (int j0 = 0; j0 < CPK; j0 += VEC) {
            float bt[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) bt[e] = rg.get(j0 + e) * kLog2e;
            wave_incl_scan_n<VEC>(bt);
            float xv[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float bl = lane_bcast(bt[e], 63);
                last_l = (l == j0 + e) ? bl : last_l;
                xv[e] = rx.get(j0 + e) * exp2_fast(REV ? bt[e] : bl - bt[e]);
            }
            store_vec_lds<T>(bf.X + l * Sm::pX + kc0 + j0, xv);
        }
        if (l < CPK) {
            bf.gam[kc0 + l] = exp2_fast(last_l);
            gtot += last_l;
        }
    };
    auto update = [&](const typename Sm::Buf& bf, const T* Yw) {
        vec4_t<T> yf[4][CB];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) yf[sb][cb] = frag_cm<T>(Yw, Sm::pW, 16 * sb, 16 * cb);
#pragma unroll
        for (int a = 0; a < KD / 16; ++a) {
            const f32x4 gm = *reinterpret_cast<const f32x4*>(bf.gam + 16 * a + 4 * (l >> 4));
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) S.s[a][cb] *= gm;
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int a = 0; a < KD / 16; ++a) {
                const vec4_t<T> xlo = frag_cm<T>(bf.X, Sm::pX, 32 * ks, 16 * a);
                const vec4_t<T> xhi = frag_cm<T>(bf.X, Sm::pX, 32 * ks + 16, 16 * a);
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) S.s[a][cb] = mma32(S.s[a][cb], xlo, xhi, yf[2 * ks][cb], yf[2 * ks + 1][cb]);
            }
    };

    // Optional midpoint output (ws_mid != null): the state after the first m2
    // chunks walked (for REV, the local dS* of the segment's chunks from
    // c_begin + split on) and the gate total of those chunks.  The prep of
    // walk step j runs in step j-1, so the gate total is taken right after it.
    const int m2 = ws_mid ? max(0, nchunks - split) : -1;
    float gmid = 0.f;
    auto store_mid = [&]() {
        S.store(ws_mid + ((long)bh * P + seg) * (long)KD * V, V, col0);
        if (vb == 0 && l < CPK) ws_gmid[((long)bh * P + seg) * KD + kc0 + l] = gmid;
    };
    if (m2 == 0) store_mid();
    if (nchunks > 0) {
        rx.load(krow(x, chunk_of(0)), rsK, kc0);
        rg.load(grow(chunk_of(0)), rsG, kc0);
        ry.load(vrow(y, chunk_of(0)), rsV, l);
        prep(sm.buf[0]);
        if (m2 == 1) gmid = gtot;
        ry.store_lds(yslice(0), Sm::pW, l);
        if (nchunks > 1) {
            rx.load(krow(x, chunk_of(1)), rsK, kc0);
            rg.load(grow(chunk_of(1)), rsG, kc0);
            ry.load(vrow(y, chunk_of(1)), rsV, l);
        }
    }
    __syncthreads();
    auto step = [&](int it) {
        const bool more = it + 1 < nchunks;
        const auto& cur = sm.buf[it & 1];
        auto& nxt = sm.buf[(it + 1) & 1];
        if (w < NW / 2) {
            update(cur, yslice(it));
            __builtin_amdgcn_sched_barrier(0);
            if (more) prep(nxt);
        } else {
            if (more) prep(nxt);
            __builtin_amdgcn_sched_barrier(0);
            update(cur, yslice(it));
        }
        if (it + 2 == m2) gmid = gtot;
        if (more) {
            ry.store_lds(yslice(it + 1), Sm::pW, l);
            if (it + 2 < nchunks) {
                rx.load(krow(x, chunk_of(it + 2)), rsK, kc0);
                rg.load(grow(chunk_of(it + 2)), rsG, kc0);
                ry.load(vrow(y, chunk_of(it + 2)), rsV, l);
            }
        }
        __syncthreads();
    };
    // the midpoint store sits between two loops: inside one, the compiler would
    // keep its per-element addresses live across every step
    int it = 0;
    if (m2 > 0) {
        for (; it < m2; ++it) step(it);
        store_mid();
    }
    for (; it < nchunks; ++it) step(it);
    S.store(ws_state + ((long)bh * P + seg) * (long)KD * V, V, col0);
    // each segment's gate total is written by one workgroup only (segments >= gate_first)
    if (vb == 0 && seg >= gate_first && l < CPK) ws_gate[((long)bh * P + seg) * KD + kc0 + l] = gtot;
}

template <typename T, int KD, int BV, int NW, bool REV, bool SG = false>
__global__ void __launch_bounds__(NW * 64)
gla_seg_state(const T* __restrict__ x, const T* __restrict__ g, const T* __restrict__ y,
              T* __restrict__ ws_state, float* __restrict__ ws_gate,
              int T_, int H, int V, int N, int P, int seg_len, int seg_first, int nseg, int BH) {
    __shared__ SegSmem<T, KD, BV, NW> sm;
    seg_state_body<T, KD, BV, NW, REV, SG>(sm, blockIdx.x, x, g, y, ws_state, ws_gate, T_, H, V, N, P, seg_len,
                                           seg_first, nseg, BH, 0);
}

// Both directions of the backward's segment states in one grid (they are
// independent): blocks [0, nfwd) take S*_p of segments 0 .. P-2 from k, v; the
// rest take dS*_p of segments 1 .. P-1 from q, d_o, or, with ws_dmid, of every
// segment together with its midpoint state (the local dS* of the chunks from
// c_begin + split on) and that half's gate total, from which the dv walk
// starts a segment's first half.  Each segment's gate total G_p is written by
// the forward direction, except from rev_gate_first on, where the backward
// direction writes it (P - 1 when both directions run; 0 when nfwd = 0 because
// the states come from a checkpointing forward).
template <typename T, int KD, int BV, int NW, bool SG = false>
__global__ void __launch_bounds__(NW * 64)
gla_seg_state_pair(const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ q,
                   const T* __restrict__ d_o, const T* __restrict__ g, T* __restrict__ ws_state,
                   T* __restrict__ ws_dstate, float* __restrict__ ws_gate, int T_, int H, int V, int N, int P,
                   int seg_len, int nseg, int BH, int nfwd, T* __restrict__ ws_dmid, float* __restrict__ ws_gmid,
                   int split, int rev_gate_first) {
    __shared__ SegSmem<T, KD, BV, NW> sm;
    const int bid = blockIdx.x;
    if (bid < nfwd)
        seg_state_body<T, KD, BV, NW, false, SG>(sm, bid, k, g, v, ws_state, ws_gate, T_, H, V, N, P, seg_len, 0,
                                                 nseg, BH, 0);
    else if (!ws_dmid)  // only segment P-1 is not covered by the forward direction
        seg_state_body<T, KD, BV, NW, true, SG>(sm, bid - nfwd, q, g, d_o, ws_dstate, ws_gate, T_, H, V, N, P,
                                                seg_len, 1, nseg, BH, rev_gate_first);
    else  // every segment, for its midpoint state (segment 0's total is not needed)
        seg_state_body<T, KD, BV, NW, true, SG>(sm, bid - nfwd, q, g, d_o, ws_dstate, ws_gate, T_, H, V, N, P,
                                                seg_len, 0, nseg + 1, BH, rev_gate_first, ws_dmid, ws_gmid, split);
}

}  // namespace gla
