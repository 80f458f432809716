// Forward kernels for 16-bit heads with 256 key columns.
//
// Method: "Gated Linear Attention Transformers with Hardware-Efficient
// Training", Section 4.2 (chunkwise form) and Section 4.3 (intra-chunk
// attention in log-gate space).  The mathematics is that of the column-split
// walk in gla_fwd.hip: per chunk, with B_t the cumulative log2 gate from the
// chunk start,
//   Ql = q * exp2(B_t),  Kt = k * exp2(-B_s)   (k * exp2(B_63 - B_s) for a key
//   column whose chunk decay leaves the basis range),  A = causal(Ql Kt^T)
//   (element by element when some column leaves the range),
//   O = Ql S + A V,      S <- post * (pre * S + Kt^T V).
//
// At dk = 256 the state of one value column block is 256 rows deep, so a
// workgroup holds few value columns and each head's value width is split over
// several workgroups.  Forming Ql, Kt, the gate factors and A inside every one
// of them repeats the vector work (cumulative sums, two exponentials per key
// element) and the 64 x 64 x 256 product once per value block and pass.  Here
// they are formed once per chunk and head by gla_fwd_wide_prep and stored as a
// record in the workspace; the state pass and the output walk then stream the
// records, and their inner loops are matrix products only.
#pragma once

#include "gla_chunk.hpp"

namespace gla {

// Byte layout of one chunk's record (KD key columns, 16-bit operands).  The
// contraction index of a 16x16x32 MFMA step is laid out as the two halves its
// operand fragments use: lane group g (lanes 16g .. 16g+15) holds indices
// 4g .. 4g+3 and 16+4g .. 16+4g+3 of the step.  Ql's key columns and Kt^T's
// tokens are stored in that order within each block of 32 (position 8g + e
// holds index 4g + e for e < 4 and 12 + 4g + e otherwise), so each lane reads a
// whole 32-deep fragment as one 16-byte LDS row read.

// A whole 32-deep row fragment of a tile stored in that order: lane l reads row
// r0 + l%16, positions c0 + 8(l/16) .. +7, in one 16-byte LDS read; elements
// 0-3 are the fragment's first half, 4-7 its second.
template <typename T>
__device__ __forceinline__ void frag_rm32(const T* base, int pitch, int r0, int c0, vec4_t<T> (&x)[2]) {
    static_assert(sizeof(T) == 2, "16-bit tiles");
    typedef unsigned int __attribute__((ext_vector_type(2))) u32x2;
    const int l = lane_id();
    const u32x4 v = *reinterpret_cast<const u32x4*>(base + (r0 + (l & 15)) * pitch + c0 + 8 * (l >> 4));
    x[0] = __builtin_bit_cast(vec4_t<T>, u32x2{v[0], v[1]});
    x[1] = __builtin_bit_cast(vec4_t<T>, u32x2{v[2], v[3]});
}

template <int KD>
struct WideRec {
    static constexpr long oQl = 0;                          // [64][KD]  Ql, key columns in MFMA order
    static constexpr long oKtT = oQl + 2L * kChunk * KD;    // [KD][64]  Kt transposed, tokens in MFMA order
    static constexpr long oA = oKtT + 2L * kChunk * KD;     // [64][64]  A, zero for s > t
    static constexpr long oPP = oA + 2L * kChunk * kChunk;  // fp32 [3][KD]: pre, post, B_63
    static constexpr long oFlag = oPP + 12L * KD;           // int: some column left the basis range
    static constexpr long bytes = oFlag + 256;
    static_assert(bytes % 256 == 0, "records stay 256-byte aligned");
};

// The record of one chunk and head under general gates G_t = alpha_t^T beta_t
// ("Gated Linear Attention Transformers with Hardware-Efficient Training", the
// chapter summary's Knowl 12 and Appendix C): the key-side record above, then
// the value side, with C_t the intra-chunk cumulative log2 of beta per column.
template <int KD>
struct GenRec {
    static constexpr long oQl = WideRec<KD>::oQl, oKtT = WideRec<KD>::oKtT, oA = WideRec<KD>::oA;
    static constexpr long oPP = WideRec<KD>::oPP, oFlag = WideRec<KD>::oFlag;
    static constexpr long oVp = WideRec<KD>::bytes;                           // [64][V]  v * exp2(C_63 - C_t)
    static constexpr long oCs(int V) { return oVp + 2L * kChunk * V; }      // [64][V]  exp2(C_t)
    static constexpr long oOi(int V) { return oCs(V) + 2L * kChunk * V; }   // [64][V]  intra-chunk output
    static constexpr long oPB(int V) { return oOi(V) + 2L * kChunk * V; }   // fp32 [2][V]: exp2(C_63), C_63
    static constexpr long oVF(int V) { return oPB(V) + 8L * V; }            // int [16]: value pass out of range
    // 256 bytes for the flags keep every record 256-byte aligned (as the record
    // without them is): an unaligned record splits each row across one more line
    static constexpr long bytes(int V) { return oVF(V) + 256; }
};

template <typename T, int KD>
struct WidePrepSmem {
    static constexpr int pQl = tile_pitch<T, KD, false>();
    static constexpr int pKt = tile_pitch<T, KD, false>();
    static constexpr int pF = kChunk + 4;  // fp32 A of an exact-path chunk, laid over Ql
    struct alignas(16) Buf {
        T Ql[kChunk * pQl];
        T Kt[kChunk * pKt];
        float pre[KD];
        float post[KD];
        int flag[4];
    };
    static_assert(sizeof(T) * kChunk * pQl >= sizeof(float) * kChunk * pF, "exact-path scratch");
    Buf buf;
};

// One workgroup (four waves, 64 key columns each) per chunk and head.
// rev (general gates, per-column g): the records of the time-reversed
// sequence, whose token t is the input's token T-1-t and whose gate at t is the
// input's gate of token T-t (none at t = 0): chunk c reads the input's rows
// T-1-64c down to T-64-64c, its gates one token later, in place.
template <typename T, int KD, bool SG>
__global__ void __launch_bounds__(256)
gla_fwd_wide_prep(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ g,
                  unsigned char* __restrict__ rec, int T_, int H, int N, long rstride, int rev = 0) {
    constexpr int NW = 4, NT = NW * 64, CPK = KD / NW, VEC = 16 / (int)sizeof(T), VPR = KD / VEC;
    static_assert(CPK <= 64 && (kChunk * VPR) % NT == 0, "prep tiling");
    using Sm = WidePrepSmem<T, KD>;
    using R = WideRec<KD>;
    __shared__ Sm sm;
    const int tid = threadIdx.x, w = wave_id(), l = lane_id();
    const long unit = blockIdx.x;  // bh * N + chunk; the grid has exactly BH * N blocks
    const int bh = (int)(unit / N), c = (int)(unit % N);
    const int b = bh / H, h = bh % H;
    const bool rv = !SG && rev;
    const int rsK = rv ? -H * KD : H * KD, rsG = SG ? H : rsK;
    // input rows of the chunk's token 0 (q, k) and of its gate
    const long row0 = rv ? (long)b * T_ + T_ - 1 - (long)c * kChunk : (long)b * T_ + (long)c * kChunk;
    const long rowg = rv ? row0 + 1 : row0;
    const bool zg0 = rv && c == 0;  // the reversed sequence's token 0 has no gate
    const T* qb = q + row0 * (H * KD) + (long)h * KD;
    const T* kb = k + row0 * (H * KD) + (long)h * KD;
    // g: per key column [B,T,H,K], or (SG) one value per token and head [B,T,H]
    const T* gb = SG ? g + rowg * H + h : g + rowg * (H * KD) + (long)h * KD;
    const int kc0 = w * CPK;

    RowSlab<T, CPK> rq, rk;
    GateSlab<T, CPK, SG> rg;
    rq.load(qb, rsK, kc0);
    rk.load(kb, rsK, kc0);
    if constexpr (SG)
        rg.load(gb, rsG, kc0);
    else
        rg.load_unless(gb, rsG, kc0, zg0 && l == 0);
    if (tid == 0) sm.buf.flag[0] = 0;
    __syncthreads();
    pipe_prep<T, CPK>(sm.buf, Sm::pQl, Sm::pKt, rq, rk, rg, kc0, 0, CPK / VEC);
    __syncthreads();

    unsigned char* r = rec + unit * rstride;  // records of WideRec or GenRec layout
    T* oQl = reinterpret_cast<T*>(r + R::oQl);
    T* oKtT = reinterpret_cast<T*>(r + R::oKtT);
    T* oA = reinterpret_cast<T*>(r + R::oA);
    float* opp = reinterpret_cast<float*>(r + R::oPP);
    // Ql rows: the 16-byte vector at positions 8g .. 8g+7 of a 32-column block
    // takes columns 4g .. 4g+3 and 16+4g .. 16+4g+3
    typedef unsigned int __attribute__((ext_vector_type(2))) u32x2;
#pragma unroll
    for (int i = 0; i < kChunk * VPR / NT; ++i) {
        const int p = tid + i * NT, row = p / VPR, col = (p % VPR) * VEC;
        const int src = (col & ~31) + 4 * ((col & 31) >> 3);
        const u32x2 lo = *reinterpret_cast<const u32x2*>(sm.buf.Ql + row * Sm::pQl + src);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(sm.buf.Ql + row * Sm::pQl + src + 16);
        *reinterpret_cast<u32x4*>(oQl + row * KD + col) = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    // Kt^T rows (one per key column): two LDS transpose reads give lane l key
    // column c0 + l%16 at tokens 32ks + 4(l/16) + e and 32ks + 16 + 4(l/16) + e,
    // the eight positions 8(l/16) .. +7 of that row's token block ks
#pragma unroll
    for (int u = w; u < (KD / 16) * (kChunk / 32); u += NW) {
        const int c0 = 16 * (u % (KD / 16)), ks = u / (KD / 16);
        const vec4_t<T> lo = frag_cm<T>(sm.buf.Kt, Sm::pKt, 32 * ks, c0);
        const vec4_t<T> hi = frag_cm<T>(sm.buf.Kt, Sm::pKt, 32 * ks + 16, c0);
        const u32x2 a = __builtin_bit_cast(u32x2, lo), bq = __builtin_bit_cast(u32x2, hi);
        *reinterpret_cast<u32x4*>(oKtT + (c0 + (l & 15)) * kChunk + 32 * ks + 8 * (l >> 4)) = u32x4{a[0], a[1], bq[0], bq[1]};
    }
    for (int i = tid; i < KD; i += NT) {
        const float pre = sm.buf.pre[i], post = sm.buf.post[i];
        opp[i] = pre;
        opp[KD + i] = post;
        opp[2 * KD + i] = log2f(pre * post);  // one factor is 1: the chunk's log2 decay B_63
    }
    const bool exact = sm.buf.flag[0] != 0;
    if (tid == 0) *reinterpret_cast<int*>(r + R::oFlag) = exact ? 1 : 0;
    if (!exact) {
        // the ten lower-triangular 16 x 16 tiles
        for (int tile = w; tile < 10; tile += NW) {
            int is, js;
            decode_tile(tile, is, js);
            f32x4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < KD / 32; ++ks)
                acc = mma32_rr<T>(acc, sm.buf.Kt, Sm::pKt, 16 * js, sm.buf.Ql, Sm::pQl, 16 * is, 32 * ks);
            // acc holds A^T[s][t] for s = 16js + 4(l/16) + r, t = 16is + l%16
            if (is == js) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * (l >> 4) + e > (l & 15)) acc[e] = 0.f;
            }
            *reinterpret_cast<vec4_t<T>*>(oA + (16 * is + (l & 15)) * kChunk + 16 * js + 4 * (l >> 4)) =
                to_vec4<T>(acc);
        }
        // the six tiles above the diagonal: (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
        for (int z = w; z < 6; z += NW) {
            const int is = (z >= 3) + (z >= 5);
            const int js = z + 1 - (is == 1 ? 2 : (is == 2 ? 3 : 0));
            *reinterpret_cast<vec4_t<T>*>(oA + (16 * is + (l & 15)) * kChunk + 16 * js + 4 * (l >> 4)) =
                to_vec4<T>(zero4());
        }
    } else {
        // Eq. 4 element by element into an fp32 tile laid over Ql, whose copy
        // to the record every thread has finished at this barrier
        __syncthreads();
        float* Af = reinterpret_cast<float*>(sm.buf.Ql);
        exact_intra_tile<T, KD, NW, SG>(Af, Sm::pF, qb, kb, gb, rsK, rsG, w, zg0);
        __syncthreads();
        for (int e = tid; e < kChunk * kChunk; e += NT) {
            const int t = e / kChunk, s = e % kChunk;
            oA[e] = Elem<T>::from_f(s <= t ? Af[t * Sm::pF + s] : 0.f);
        }
    }
}

template <typename T, int VP>
struct GenPrepSmem {
    static constexpr int NT = 256;
    static constexpr int pA = kChunk + 8;  // A, read as row fragments
    static constexpr int pV = VP + 8;      // scaled (or raw) values, read as column fragments
    static constexpr int pC = VP + 4;      // C_t, fp32
    alignas(16) T A[kChunk * pA];
    alignas(16) T Vt[kChunk * pV];
    alignas(16) float Cl[kChunk * pC];
    alignas(16) float tot[NT / (VP / 8)][VP];
    int flagb;
};

// The value side of a general-gate record: one workgroup (four waves) per
// chunk, head and VP value columns, after the key side (gla_fwd_wide_prep,
// which leaves A in the record):
//   C_t = cumulative sum of h * log2(e) within the chunk (exp(h) = beta)
//   Vp = v * exp2(C_63 - C_t), Cs = exp2(C_t), and the intra-chunk output
//   Oi[t][j] = sum_{s <= t} A[t][s] v[s][j] exp2(C_t[j] - C_s[j])
// formed as exp2(C_t) * (A (v * exp2(-C))) on the matrix cores, or element by
// element when some column's C_63 leaves the basis range (exp2(-C) would not
// stay a well-scaled fp32/bf16 value).  rev: the time-reversed sequence, read in
// place as gla_fwd_wide_prep reads it (values at token T-1-t, gates at T-t).
// The pass's range flag goes to the record; WI (the walk forms the intra-chunk
// output itself from A and Vp): the output is stored for flagged passes only.
template <typename T, int KD, int VP, bool WI>
__global__ void __launch_bounds__(256)
gla_fwd_general_vprep(const T* __restrict__ v, const T* __restrict__ hg, unsigned char* __restrict__ rec, int T_,
                      int H, int V, int N, int rev = 0) {
    constexpr int NW = 4, NT = NW * 64;
    constexpr int CV = VP / 8, NPART = NT / CV, TPP = kChunk / NPART;  // column vectors, token parts, tokens per part
    constexpr int CB2 = VP / NW / 16;                                  // 16-column blocks per wave in the output product
    static_assert((VP == 64 || VP == 128) && CB2 >= 1 && NPART * TPP == kChunk, "value pass width");
    using Sm = GenPrepSmem<T, VP>;
    using G = GenRec<KD>;
    __shared__ Sm sm;
    const int tid = threadIdx.x, w = wave_id(), l = lane_id();
    const long unit = blockIdx.x;  // bh * N + chunk; the grid has exactly BH * N x V / VP blocks
    const int j0 = blockIdx.y * VP;
    const int bh = (int)(unit / N), c = (int)(unit % N);
    const int b = bh / H, h = bh % H;
    const int rsV = H * V;
    // input rows of the chunk's token 0 (v) and of its gate, and the row step
    const long row0 = rev ? (long)b * T_ + T_ - 1 - (long)c * kChunk : (long)b * T_ + (long)c * kChunk;
    const long rowh = rev ? row0 + 1 : row0;
    const long rstep = rev ? -(long)rsV : (long)rsV;
    unsigned char* r = rec + unit * G::bytes(V);
    // A of the chunk (from the key side), for the intra-chunk output
    auto load_a = [&]() {
        const T* a = reinterpret_cast<const T*>(r + G::oA);
#pragma unroll
        for (int i = 0; i < kChunk * kChunk / 8 / NT; ++i) {
            const int p = tid + i * NT, row = p / (kChunk / 8), col = (p % (kChunk / 8)) * 8;
            *reinterpret_cast<u32x4*>(sm.A + row * Sm::pA + col) = *reinterpret_cast<const u32x4*>(a + row * kChunk + col);
        }
    };
    if constexpr (!WI) load_a();
    // ---- value side, VP columns per pass; thread (part, cv) scans columns
    // 8cv .. 8cv+7 over tokens part*TPP .. +TPP-1 with 16-byte loads and stores
    T* oVp = reinterpret_cast<T*>(r + G::oVp);
    T* oCs = reinterpret_cast<T*>(r + G::oCs(V));
    T* oOi = reinterpret_cast<T*>(r + G::oOi(V));
    float* opb = reinterpret_cast<float*>(r + G::oPB(V));
    const int cv = tid % CV, part = tid / CV, t0 = part * TPP, jv = 8 * cv;
    const int jj = tid % VP, epart = tid / VP;  // element-wise path: column jj, tokens epart + k * (NT / VP)
    {
        const long cofs = (long)h * V + j0 + jv;
        u32x4 hraw[TPP], vraw[TPP];
#pragma unroll
        for (int i = 0; i < TPP; ++i) {
            // the reversed sequence's token 0 has no gate (its row lies past the input)
            const bool nog = rev && c == 0 && t0 + i == 0;
            hraw[i] = nog ? u32x4{0u, 0u, 0u, 0u}
                          : *reinterpret_cast<const u32x4*>(hg + rowh * rsV + cofs + (long)(t0 + i) * rstep);
            vraw[i] = *reinterpret_cast<const u32x4*>(v + row0 * rsV + cofs + (long)(t0 + i) * rstep);
        }
        float cl[TPP][8];
#pragma unroll
        for (int i = 0; i < TPP; ++i) {
            const T* hx = reinterpret_cast<const T*>(&hraw[i]);
#pragma unroll
            for (int e = 0; e < 8; ++e) cl[i][e] = Elem<T>::to_f(hx[e]) * kLog2e + (i > 0 ? cl[i - 1][e] : 0.f);
        }
        if (tid == 0) sm.flagb = 0;
        *reinterpret_cast<f32x4*>(&sm.tot[part][jv]) = f32x4{cl[TPP - 1][0], cl[TPP - 1][1], cl[TPP - 1][2], cl[TPP - 1][3]};
        *reinterpret_cast<f32x4*>(&sm.tot[part][jv + 4]) = f32x4{cl[TPP - 1][4], cl[TPP - 1][5], cl[TPP - 1][6], cl[TPP - 1][7]};
        __syncthreads();  // B1: part totals (and A) visible, flag cleared
        float off[8], c63[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) off[e] = c63[e] = 0.f;
        for (int pp = 0; pp < NPART; ++pp) {
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(&sm.tot[pp][jv]);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(&sm.tot[pp][jv + 4]);
            const float m = pp < part ? 1.f : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                off[e] += m * x0[e];
                off[4 + e] += m * x1[e];
                c63[e] += x0[e];
                c63[4 + e] += x1[e];
            }
        }
        bool out_of_range = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) out_of_range |= -c63[e] > kBasisLimit;
        if (out_of_range) sm.flagb = 1;
        if (part == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                opb[j0 + jv + e] = exp2f(c63[e]);
                opb[V + j0 + jv + e] = c63[e];
            }
        }
        __syncthreads();  // B2: the pass's flag
        const bool fl = sm.flagb != 0;
        if (tid == 0) reinterpret_cast<int*>(r + G::oVF(V))[blockIdx.y] = fl ? 1 : 0;
        if (WI && fl) load_a();  // visible after B3
#pragma unroll
        for (int i = 0; i < TPP; ++i) {
            const int t = t0 + i;
            const T* vx = reinterpret_cast<const T*>(&vraw[i]);
            alignas(16) T vp8[8], cs8[8], vt8[8];
            alignas(16) float ct8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float ct = off[e] + cl[i][e], vv = Elem<T>::to_f(vx[e]);
                ct8[e] = ct;
                vp8[e] = Elem<T>::from_f(vv * exp2f(c63[e] - ct));
                cs8[e] = Elem<T>::from_f(exp2f(ct));
                vt8[e] = Elem<T>::from_f(fl ? vv : vv * exp2f(-ct));
            }
            *reinterpret_cast<u32x4*>(oVp + t * V + j0 + jv) = *reinterpret_cast<const u32x4*>(vp8);
            *reinterpret_cast<u32x4*>(oCs + t * V + j0 + jv) = *reinterpret_cast<const u32x4*>(cs8);
            *reinterpret_cast<u32x4*>(sm.Vt + t * Sm::pV + jv) = *reinterpret_cast<const u32x4*>(vt8);
            *reinterpret_cast<f32x4*>(sm.Cl + t * Sm::pC + jv) = *reinterpret_cast<const f32x4*>(ct8);
            *reinterpret_cast<f32x4*>(sm.Cl + t * Sm::pC + jv + 4) = *reinterpret_cast<const f32x4*>(ct8 + 4);
        }
        __syncthreads();  // B3: Vt and Cl complete
        if (!fl && !WI) {
            const int c0 = w * (VP / NW);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                f32x4 acc[CB2];
#pragma unroll
                for (int cb = 0; cb < CB2; ++cb) acc[cb] = zero4();
#pragma unroll
                for (int ks2 = 0; ks2 <= rb / 2; ++ks2) {
                    const vec4_t<T> blo = frag_rm<T>(sm.A, Sm::pA, 16 * rb, 32 * ks2);
                    const vec4_t<T> bhi = frag_rm<T>(sm.A, Sm::pA, 16 * rb, 32 * ks2 + 16);
#pragma unroll
                    for (int cb = 0; cb < CB2; ++cb)
                        acc[cb] = mma32(acc[cb], frag_cm<T>(sm.Vt, Sm::pV, 32 * ks2, c0 + 16 * cb),
                                        frag_cm<T>(sm.Vt, Sm::pV, 32 * ks2 + 16, c0 + 16 * cb), blo, bhi);
                }
                // slot e: column c0 + 16cb + 4(l/16) + e of the pass, token 16rb + l%16
                const int t = 16 * rb + (l & 15);
#pragma unroll
                for (int cb = 0; cb < CB2; ++cb) {
                    const int jc = c0 + 16 * cb + 4 * (l >> 4);
                    const f32x4 ct = *reinterpret_cast<const f32x4*>(sm.Cl + t * Sm::pC + jc);
                    f32x4 o4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o4[e] = acc[cb][e] * exp2f(ct[e]);
                    *reinterpret_cast<vec4_t<T>*>(oOi + t * V + j0 + jc) = to_vec4<T>(o4);
                }
            }
        } else if (fl) {
            for (int t = epart; t < kChunk; t += NT / VP) {
                const float ct = sm.Cl[t * Sm::pC + jj];
                float acc = 0.f;
                for (int s2 = 0; s2 <= t; ++s2)
                    acc += Elem<T>::to_f(sm.A[t * Sm::pA + s2]) * Elem<T>::to_f(sm.Vt[s2 * Sm::pV + jj]) *
                           exp2f(ct - sm.Cl[s2 * Sm::pC + jj]);
                oOi[t * V + j0 + jj] = Elem<T>::from_f(acc);
            }
        }
    }
}

template <typename T, int KD, int BV, bool OUT, bool GEN = false>
struct WideSmem {
    static constexpr int NC = 4;        // consumer (matrix) waves
    static constexpr int CW = BV / NC;  // value columns per consumer wave
    static constexpr int pQl = tile_pitch<T, KD, false>();
    // Kt^T rows (one per key column, tokens in MFMA order) read as 16-byte row
    // fragments: a pitch of 36 (mod 64) dwords keeps sixteen rows on disjoint banks
    static constexpr int pKtT = kChunk + 8;
    static constexpr int pA = kChunk + Elem<T>::pad;
    // wave-private V slices read with ds_read_b64_tr_b16: a pitch of 16 or 32
    // two-byte columns keeps the four rows of a 16-lane group on disjoint banks
    static constexpr int pW = CW;
    static_assert(CW == 16 || CW == 32, "value slice width");
    // general output walk at KD <= 128: the intra-chunk output is formed here
    // from A and the record's v * exp2(C_63 - C_t), unless the value pass is
    // out of range (then the record holds it)
    static constexpr bool WI = GEN && OUT && KD <= 128;
    // two buffers of everything but Ql, which the output walk refills between
    // the inter-chunk product and the rest of the chunk
    alignas(16) T KtT[2][KD * pKtT];
    alignas(16) T Vw[2][NC * kChunk * pW];
    alignas(16) float pp[2][2 * KD];  // pre, post
    alignas(16) T A[OUT && (!GEN || WI) ? 2 : 1][OUT && (!GEN || WI) ? kChunk * pA : 8];
    alignas(16) T Ql[OUT ? kChunk * pQl : 8];
    // general gates: exp2(C_63) of the block's value columns
    alignas(16) float pb[GEN ? 2 : 1][GEN ? BV : 4];
    int flag[2];
    int vflag[2];  // WI: the value pass of the chunk is out of range
};

// The state pass (OUT = false: segments 0 .. nseg-1 from a zero state, the
// local state S*_p in the input dtype and the segment's log2 decay for the
// combine) and the output walk (OUT = true: every segment from S_init(p),
// writing O and, for the last segment, the final state).
//
// Eight waves: waves 0-3 hold the state (wave w: value columns col0 .. col0 +
// BV/4 - 1, all 256 rows, in VGPRs) and run the matrix products; waves 4-7 move
// the records from memory into LDS.  A SIMD runs one wave of each kind, so the
// loads and LDS writes overlap the MFMAs.  Per chunk c (buffer c&1):
//   consumers: O_inter = Ql S  | barrier X | O += A V, store O; S update | barrier E
//   producers: Kt, A, V, gate factors of c+1 into buffer (c+1)&1 | barrier X |
//              Ql of c+1 into the single Ql buffer | barrier E
// Each producer wave keeps the records of two chunks in registers: at chunk c
// it fetches chunk c+2 into the set that chunk c came in.
//
// GEN: general gates (value-side gate beta = exp(h) as well, records of
// GenRec): the value slices come from the records (v * exp2(C_63 - C_t)), the
// output is (Ql S) * exp2(C_t) plus the record's intra-chunk output, and the
// state's columns decay by exp2(C_63) as its rows do by the key-side gate; the
// state pass also writes the segment's column log2 decays to ws_gateb, and the
// output walk with HS the state before every chunk to hs_out (and S_T to
// s_final2 as well as s_final, when given).  REV (GEN output
// walk): the records are those of the time-reversed sequence, and the output
// of its token t goes to row T-1-t.  TI (GEN output walk): each segment's
// initial state is the transpose of a known state of the transposed recurrence,
// ws_init[bh][chunk][V][KD] at the segment's first chunk (segment 0: s0 given as
// [V][KD]), so no state pass or combine precedes the walk.
template <typename T, int KD, int BV, bool OUT, bool GEN = false, bool HS = false, bool REV = false,
          bool TI = false>
__global__ void __launch_bounds__(512)
gla_fwd_wide_walk(const unsigned char* __restrict__ rec, const T* __restrict__ v, const T* __restrict__ ws_init,
                  const float* __restrict__ s0, T* __restrict__ o, float* __restrict__ s_final,
                  T* __restrict__ ws_state, float* __restrict__ ws_gate, int T_, int H, int V, int N, int P,
                  int seg_len, int nseg, int BH, float* __restrict__ ws_gateb = nullptr,
                  T* __restrict__ hs_out = nullptr, float* __restrict__ s_final2 = nullptr) {
    constexpr int NC = 4, NP = 64 * NC;  // consumer waves; producer threads
    using Sm = WideSmem<T, KD, BV, OUT, GEN>;
    using R = WideRec<KD>;
    using G = GenRec<KD>;
    const long rbytes = GEN ? G::bytes(V) : R::bytes;
    const long oQl = GEN ? G::oQl : R::oQl, oKtT = GEN ? G::oKtT : R::oKtT;
    const long oPP = GEN ? G::oPP : R::oPP, oFlag = GEN ? G::oFlag : R::oFlag;
    constexpr int CW = Sm::CW, CB = CW / 16;
    static_assert(2 * KD / 4 <= NP && KD <= NP && BV <= NP, "gate factors: one vector or value per producer thread");
    __shared__ Sm sm;
    const int tid = threadIdx.x, l = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const bool producer = w >= NC;
    const int nvb = V / BV;
    int unit, vb;
    xcd_decode(nvb, unit, vb);
    if (unit >= BH * nseg) return;
    const int seg = unit % nseg;
    const int bh = unit / nseg;
    const int b = bh / H, h = bh % H;
    const int c_begin = seg * seg_len;
    const int c_end = min(N, c_begin + seg_len);
    const int rsV = H * V;
    const int cw = producer ? w - NC : w;  // the consumer wave a value slice belongs to
    const int col0 = vb * BV + cw * CW;

    if (producer) {
        // ---------------- producers: records -> LDS
        const int ptid = tid - NP;
        float gtot = 0.f;   // state pass: thread ptid sums B_63 of key column ptid
        float gtotb = 0.f;  // GEN state pass: thread ptid sums C_63 of value column vb*BV + ptid
        struct Regs {
            TileRegs<T, KD, NP> Ql, Kt;  // Kt: the [KD][64] Kt^T block as 64 rows of KD (linear)
            TileRegs<T, kChunk, NP> A;
            TileRegs<T, CW, 64> v;
            f32x4 pp;
            float bl, gb, cb;
            int flag, vflag;
        };
        Regs ra, rb;
        auto fetch = [&](Regs& x, int c) {
            const unsigned char* r = rec + ((long)bh * N + c) * rbytes;
            x.Kt.load(reinterpret_cast<const T*>(r + oKtT), KD, ptid);
            if constexpr (OUT) {
                x.Ql.load(reinterpret_cast<const T*>(r + oQl), KD, ptid);
                if constexpr (!GEN || Sm::WI) x.A.load(reinterpret_cast<const T*>(r + R::oA), kChunk, ptid);
            }
            const float* pp = reinterpret_cast<const float*>(r + oPP);
            if (ptid < KD / 2) x.pp = *reinterpret_cast<const f32x4*>(pp + 4 * ptid);
            if (!OUT && ptid < KD) x.bl = pp[2 * KD + ptid];
            if (ptid == 0) x.flag = *reinterpret_cast<const int*>(r + oFlag);
            if constexpr (GEN) {
                x.v.load(reinterpret_cast<const T*>(r + G::oVp) + col0, V, l);
                const float* pbg = reinterpret_cast<const float*>(r + G::oPB(V));
                if (ptid < BV) {
                    x.gb = pbg[vb * BV + ptid];
                    if (!OUT) x.cb = pbg[V + vb * BV + ptid];
                }
                if (Sm::WI && ptid == 0) x.vflag = reinterpret_cast<const int*>(r + G::oVF(V))[vb];
            } else {
                x.v.load(v + ((long)b * T_ + (long)c * kChunk) * rsV + (long)h * V + col0, rsV, l);
            }
        };
        // everything but Ql into buffer bf
        auto stash = [&](const Regs& x, int bf) {
            // linear vector q of the record is row q / 8, tokens 8 (q % 8) .. of Kt^T
#pragma unroll
            for (int i = 0; i < TileRegs<T, KD, NP>::PER; ++i) {
                const int q = ptid + i * NP;
                *reinterpret_cast<u32x4*>(sm.KtT[bf] + (q / (kChunk / 8)) * Sm::pKtT + (q % (kChunk / 8)) * 8) = x.Kt.r[i];
            }
            if constexpr (OUT && (!GEN || Sm::WI)) x.A.store_lds(sm.A[bf], Sm::pA, ptid);
            if (Sm::WI && ptid == 0) sm.vflag[bf] = x.vflag;
            if (ptid < KD / 2) *reinterpret_cast<f32x4*>(sm.pp[bf] + 4 * ptid) = x.pp;
            if (!OUT && ptid < KD) gtot += x.bl;
            if (ptid == 0) sm.flag[bf] = x.flag;
            x.v.store_lds(sm.Vw[bf] + cw * kChunk * Sm::pW, Sm::pW, l);
            if constexpr (GEN) {
                if (ptid < BV) {
                    sm.pb[bf][ptid] = x.gb;
                    if (!OUT) gtotb += x.cb;
                }
            }
        };
        // chunk c+1 (in x) into LDS during chunk c, then chunk c+3 into x
        auto step = [&](Regs& x, int c) {
            const bool more = c + 1 < c_end;
            if (more) stash(x, (c + 1) & 1);
            if constexpr (OUT) {
                __syncthreads();  // X: the consumers are done with Ql(c)
                if (more) x.Ql.store_lds(sm.Ql, Sm::pQl, ptid);
            }
            if (c + 3 < c_end) fetch(x, c + 3);
            __syncthreads();  // E
        };
        if (c_begin < c_end) {
            fetch(ra, c_begin);
            stash(ra, c_begin & 1);  // chunk c is read from buffer c & 1
            if constexpr (OUT) ra.Ql.store_lds(sm.Ql, Sm::pQl, ptid);
            if (c_begin + 1 < c_end) fetch(rb, c_begin + 1);
            if (c_begin + 2 < c_end) fetch(ra, c_begin + 2);
        }
        __syncthreads();  // E of the prologue
        for (int c = c_begin; c < c_end; c += 2) {
            step(rb, c);
            if (c + 1 < c_end) step(ra, c + 1);
        }
        if (!OUT && vb == 0 && ptid < KD) ws_gate[((long)bh * P + seg) * KD + ptid] = gtot;
        if (GEN && !OUT && ptid < BV) ws_gateb[((long)bh * P + seg) * V + vb * BV + ptid] = gtotb;
        return;
    }

    // ---------------- consumers: the state and the matrix products
    StateRegs<KD, CB> S;
    if constexpr (TI) {
        if (seg > 0) S.load_t(ws_init + ((long)bh * N + (long)seg * seg_len) * KD * V, KD, col0);
        else if (s0) S.load_t(s0 + (long)bh * KD * V, KD, col0);
        else S.zero();
    } else {
        if (OUT && seg > 0) S.load(ws_init + ((long)bh * P + seg) * KD * V, V, col0);
        else if (OUT && s0) S.load(s0 + (long)bh * KD * V, V, col0);
        else S.zero();
    }
    // HS (general mode): the state before every chunk to hs_out, [BH][N][KD][V];
    // each is written after the previous chunk's update, when little else is live
    if constexpr (OUT && GEN && HS) {
        if (c_begin < c_end) S.store(hs_out + ((long)bh * N + c_begin) * KD * V, V, col0);
    }
    __syncthreads();  // E of the prologue
    for (int c = c_begin; c < c_end; ++c) {
        const int bf = c & 1;
        const T* Vw = sm.Vw[bf] + w * kChunk * Sm::pW;
        vec4_t<T> vf[4][CB];
        f32x4 acc[4][CB];
        // general gates: this lane's exp2(C_t) and intra-chunk output values,
        // loaded from the record now and used after the matrix products
        vec4_t<T> csr[GEN && OUT ? 4 : 1][CB], oir[GEN && OUT ? 4 : 1][CB];
        // WI: the record's intra-chunk output is read only for a value pass out of range
        const bool vfl = Sm::WI ? sm.vflag[bf] != 0 : true;
        if constexpr (GEN && OUT) {
            const unsigned char* r = rec + ((long)bh * N + c) * rbytes;
            const T* csg = reinterpret_cast<const T*>(r + G::oCs(V)) + col0;
            const T* oig = reinterpret_cast<const T*>(r + G::oOi(V)) + col0;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const int off = (16 * rb + (l & 15)) * V + 16 * cb + 4 * (l >> 4);
                    csr[rb][cb] = *reinterpret_cast<const vec4_t<T>*>(csg + off);
                    oir[rb][cb] = vfl ? *reinterpret_cast<const vec4_t<T>*>(oig + off) : vec4_t<T>{};
                }
        }
        if constexpr (OUT) {
            // O^T[j][t] = sum_i S[i][j] Ql[t][i]; the Ql fragments of step ks + 1
            // are read while the MFMAs of step ks run
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = zero4();
            vec4_t<T> qf[2][4][2];
            auto rd = [&](int ks, vec4_t<T> (&x)[4][2]) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) frag_rm32<T>(sm.Ql, Sm::pQl, 16 * rb, 32 * ks, x[rb]);
            };
            __builtin_amdgcn_sched_barrier(0);
            rd(0, qf[0]);
#pragma unroll
            for (int ks = 0; ks < KD / 32; ++ks) {
                if (ks + 1 < KD / 32) rd(ks + 1, qf[(ks + 1) & 1]);
                vec4_t<T> sf[CB][2];
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    sf[cb][0] = to_vec4<T>(S.s[2 * ks][cb]);
                    sf[cb][1] = to_vec4<T>(S.s[2 * ks + 1][cb]);
                }
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        acc[rb][cb] = mma32(acc[rb][cb], sf[cb][0], sf[cb][1], qf[ks & 1][rb][0], qf[ks & 1][rb][1]);
            }
            // four reads ahead, then one read per MFMA (CB = 1) or per two (CB = 2)
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < (KD / 32 - 1) * 4 * CB; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (CB == 1 || (i & 1)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4 * CB, 0);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();  // X: Ql may be refilled
        }
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) vf[sb][cb] = frag_cm<T>(Vw, Sm::pW, 16 * sb, 16 * cb);
        if constexpr (Sm::WI) {
            // in range: O^T += (A Vp) / exp2(C_63), i.e. A (v * exp2(-C_t)), per column
            if (!vfl) {
                float ig[CB][4];
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        ig[cb][e] = __builtin_amdgcn_rcpf(sm.pb[bf][w * CW + 16 * cb + 4 * (l >> 4) + e]);
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    f32x4 t4[CB];
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) t4[cb] = zero4();
#pragma unroll
                    for (int ks2 = 0; ks2 <= rb / 2; ++ks2) {
                        const vec4_t<T> blo = frag_rm<T>(sm.A[bf], Sm::pA, 16 * rb, 32 * ks2);
                        const vec4_t<T> bhi = frag_rm<T>(sm.A[bf], Sm::pA, 16 * rb, 32 * ks2 + 16);
#pragma unroll
                        for (int cb = 0; cb < CB; ++cb)
                            t4[cb] = mma32(t4[cb], vf[2 * ks2][cb], vf[2 * ks2 + 1][cb], blo, bhi);
                    }
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[rb][cb][e] += t4[cb][e] * ig[cb][e];
                }
            }
        }
        if constexpr (OUT && GEN) {
            // O = (Ql S + intra) * exp2(C_t) + the record's intra-chunk output; slot e:
            // column 16cb + 4(l/16) + e of the slice, token 16rb + l%16 (REV:
            // the time-reversed sequence's token, written to row T-1-t)
            const long orow = REV ? (long)b * T_ + T_ - 1 - (long)c * kChunk : (long)b * T_ + (long)c * kChunk;
            const int ostep = REV ? -rsV : rsV;
            T* obase = o + orow * rsV + (long)h * V + col0;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const int t = 16 * rb + (l & 15), jc = 16 * cb + 4 * (l >> 4);
                    f32x4 o4;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o4[e] = acc[rb][cb][e] * Elem<T>::to_f(csr[rb][cb][e]) + Elem<T>::to_f(oir[rb][cb][e]);
                    *reinterpret_cast<vec4_t<T>*>(obase + t * ostep + jc) = to_vec4<T>(o4);
                }
        } else if constexpr (OUT) {
            // O^T[j][t] += sum_s V[s][j] A[t][s]
            T* obase = o + ((long)b * T_ + (long)c * kChunk) * rsV + (long)h * V + col0;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
                for (int ks2 = 0; ks2 <= rb / 2; ++ks2) {
                    const vec4_t<T> blo = frag_rm<T>(sm.A[bf], Sm::pA, 16 * rb, 32 * ks2);
                    const vec4_t<T> bhi = frag_rm<T>(sm.A[bf], Sm::pA, 16 * rb, 32 * ks2 + 16);
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        acc[rb][cb] = mma32(acc[rb][cb], vf[2 * ks2][cb], vf[2 * ks2 + 1][cb], blo, bhi);
                }
                // slot e: column j = col0 + 16cb + 4(l/16) + e, token t = 16rb + l%16
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
                    *reinterpret_cast<vec4_t<T>*>(obase + (16 * rb + (l & 15)) * rsV + 16 * cb + 4 * (l >> 4)) =
                        to_vec4<T>(acc[rb][cb]);
            }
        }
        // S <- post * (pre * S + Kt^T V); pre is 1 in every column unless some
        // column of the chunk left the basis range (the flag)
        const float* pre = sm.pp[bf];
        const float* post = sm.pp[bf] + KD;
        if constexpr (GEN) {
            // rows by pre (when flagged), columns by exp2(C_63): slot e of S.s[a][cb]
            // is key row 16a + 4(l/16) + e, column 16cb + l%16 of the slice
            float gc[CB];
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) gc[cb] = sm.pb[bf][w * CW + 16 * cb + (l & 15)];
            const bool fl = sm.flag[bf] != 0;
#pragma unroll
            for (int a = 0; a < KD / 16; ++a) {
                const f32x4 f = fl ? *reinterpret_cast<const f32x4*>(pre + 16 * a + 4 * (l >> 4))
                                   : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) S.s[a][cb] *= f * gc[cb];
            }
        } else if (sm.flag[bf]) {
#pragma unroll
            for (int a = 0; a < KD / 16; ++a) {
                const f32x4 f = *reinterpret_cast<const f32x4*>(pre + 16 * a + 4 * (l >> 4));
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) S.s[a][cb] *= f;
            }
        }
        // 2 x KD/16 steps (ks, a); the Kt fragments run LA steps ahead of the MFMAs
        {
            constexpr int NA = KD / 16, NS = 2 * NA, LA = 4;
            const T* KtT = sm.KtT[bf];
            vec4_t<T> xf[LA][2];
            auto rd = [&](int n, vec4_t<T> (&x)[2]) { frag_rm32<T>(KtT, Sm::pKtT, 16 * (n % NA), 32 * (n / NA), x); };
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int n = 0; n < LA; ++n) rd(n, xf[n]);
#pragma unroll
            for (int n = 0; n < NS; ++n) {
                const int ks = n / NA, a = n % NA;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
                    S.s[a][cb] = mma32(S.s[a][cb], xf[n % LA][0], xf[n % LA][1], vf[2 * ks][cb], vf[2 * ks + 1][cb]);
                if (n + LA < NS) rd(n + LA, xf[n % LA]);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
            for (int n = 0; n < NS - LA; ++n) {
                __builtin_amdgcn_sched_group_barrier(0x008, CB, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, CB * LA, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int a = 0; a < KD / 16; ++a) {
            const f32x4 f = *reinterpret_cast<const f32x4*>(post + 16 * a + 4 * (l >> 4));
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) S.s[a][cb] *= f;
        }
        if constexpr (OUT && GEN && HS) {
            if (c + 1 < c_end) {
                // the lane's offset is formed here, behind an empty asm: hoisted out
                // of the chunk loop, the store's addresses would stay live (and spill)
                int lo = 4 * (l >> 4) * V + col0 + (l & 15);
                int vs = V;
                asm volatile("" : "+v"(lo), "+s"(vs));
                T* dst = hs_out + ((long)bh * N + c + 1) * KD * V + lo;
#pragma unroll
                for (int a = 0; a < KD / 16; ++a)
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            dst[(16 * a + r) * vs + 16 * cb] = Elem<T>::from_f(S.s[a][cb][r]);
            }
        }
        __syncthreads();  // E: buffer bf may be refilled
    }
    if constexpr (OUT) {
        if (s_final && seg == P - 1) S.store(s_final + (long)bh * KD * V, V, col0);
        if (s_final2 && seg == P - 1) S.store(s_final2 + (long)bh * KD * V, V, col0);
    } else {
        S.store(ws_state + ((long)bh * P + seg) * (long)KD * V, V, col0);
    }
}

}  // namespace gla
