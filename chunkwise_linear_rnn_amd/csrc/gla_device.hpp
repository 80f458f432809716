// Device-side building blocks of the gfx950 GLA kernels.
//
// Everything here is written for CDNA4 wave64 and its matrix cores:
//   * one MFMA "k-step" contracts 32 indices: v_mfma_f32_16x16x32_bf16 for
//     bf16 operands, eight v_mfma_f32_16x16x4_f32 for fp32 operands;
//   * every operand fragment is "16 free x 16 contraction" with lane l holding
//     free index (l % 16) and contraction indices 4*(l/16) + e, e = 0..3 --
//     the same placement as the 16x16 accumulator (lane holds rows
//     4*(l/16)+e of column l%16).  A k-step pairs two such fragments.  A and
//     B fragments use the same (lane group, slot) -> contraction-index map, so
//     the product is the intended contraction, and an accumulator tile can be
//     fed straight back as an operand that contracts over its rows.
//   * all LDS tiles are row-major with 16 bytes of padding per row; operands
//     that contract along the row are read with one 8/16-byte load per lane
//     ("rm" fragments), operands that contract down a column with one LDS
//     transpose read for bf16 or four element loads for fp32 ("cm" fragments);
//   * global memory is addressed from a per-chunk uniform base plus 32-bit
//     lane offsets.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

typedef __bf16 bf16;
typedef float __attribute__((ext_vector_type(4))) f32x4;
typedef __bf16 __attribute__((ext_vector_type(4))) bf16x4;
typedef __bf16 __attribute__((ext_vector_type(8))) bf16x8;

constexpr int kChunk = 64;      // chunk length C (Section 4.2)
constexpr int kSub = 16;        // sub-chunk length c (Section 4.3) = MFMA tile edge
constexpr float kLog2e = 1.4426950408889634f;
// Within a chunk the intra-chunk products use one reference row (the chunk's
// last row), so the query side carries factors in [1, 2^R] and the key side
// factors in [2^-R, 1], R = the chunk's gate range in log2 units.  For R up to
// this bound every factor is a normal number in fp32 and bf16 and no product
// can overflow; chunks beyond it take the exact element-wise path (Eq. 4).
constexpr float kRangeLimit = 64.0f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Workgroups are dispatched to the eight XCDs round-robin by block index, and
// each XCD has its own L2.  Kernels whose G sibling workgroups (column or row
// blocks of one head and segment) read the same chunk tiles give the siblings
// block indices eight apart, so they share an L2.  Decodes this workgroup's
// (unit, sibling); the grid is xcd_grid(units, G) and surplus workgroups
// (unit >= units) must exit at once.
constexpr int kXcds = 8;
__host__ __device__ inline long xcd_grid(long units, int G) { return (units + kXcds - 1) / kXcds * kXcds * G; }
__device__ __forceinline__ void xcd_decode(int G, int& unit, int& sib, int bid) {
    const int rest = bid / kXcds;
    sib = rest % G;
    unit = (rest / G) * kXcds + bid % kXcds;
}
__device__ __forceinline__ void xcd_decode(int G, int& unit, int& sib) { xcd_decode(G, unit, sib, blockIdx.x); }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T> struct Elem;
template <> struct Elem<float> {
    using vec4 = f32x4;
    static constexpr int pad = 4;  // 16 bytes of row padding in LDS tiles
    __device__ static __forceinline__ float to_f(float x) { return x; }
    __device__ static __forceinline__ float from_f(float x) { return x; }
};
template <> struct Elem<bf16> {
    using vec4 = bf16x4;
    static constexpr int pad = 8;
    __device__ static __forceinline__ float to_f(bf16 x) { return (float)x; }
    __device__ static __forceinline__ bf16 from_f(float x) { return (bf16)x; }
};

template <typename T> using vec4_t = typename Elem<T>::vec4;

// ---------------------------------------------------------------------------
// MFMA k-step: acc += A(16x32) * B(32x16), operands given as (lo, hi) pairs of
// 16-contraction fragments.
__device__ __forceinline__ f32x4 mma32(f32x4 acc, bf16x4 alo, bf16x4 ahi, bf16x4 blo, bf16x4 bhi) {
    bf16x8 a = __builtin_shufflevector(alo, ahi, 0, 1, 2, 3, 4, 5, 6, 7);
    bf16x8 b = __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(f32x4 acc, f32x4 alo, f32x4 ahi, f32x4 blo, f32x4 bhi) {
    // fp32 operands: step r of a 16-block contracts index 4*(l/16) + r.
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(alo[0], blo[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(alo[1], blo[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(alo[2], blo[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(alo[3], blo[3], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ahi[0], bhi[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ahi[1], bhi[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ahi[2], bhi[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ahi[3], bhi[3], acc, 0, 0, 0);
    return acc;
}

// ---------------------------------------------------------------------------
// Fragment loads from row-major LDS tiles (element (r, c) at base[r*pitch + c]).

// free index = row (r0 + l%16), contraction = columns c0 + 4*(l/16) + e.
template <typename T>
__device__ __forceinline__ vec4_t<T> frag_rm(const T* base, int pitch, int r0, int c0) {
    const int l = lane_id();
    return *reinterpret_cast<const vec4_t<T>*>(base + (r0 + (l & 15)) * pitch + c0 + 4 * (l >> 4));
}

// contraction = rows r0 + 4*(l/16) + e, free index = column c0 + l%16.
// fp32: four element loads.  bf16: one gfx950 LDS transpose read
// (ds_read_b64_tr_b16).  Within each 16-lane group that instruction hands lane
// p element (p % 4) of the 8-byte vectors read by lanes 4e + p/4, e = 0..3; so
// lane s of the group reads row r0 + 4*(l/16) + s/4 at columns c0 + 4*(s%4)..+3
// and every lane ends up holding its column for four consecutive rows.
template <typename T>
__device__ __forceinline__ vec4_t<T> frag_cm(const T* base, int pitch, int r0, int c0) {
    const int l = lane_id();
    const T* p = base + (r0 + 4 * (l >> 4)) * pitch + c0 + (l & 15);
    vec4_t<T> v;
    v[0] = p[0];
    v[1] = p[pitch];
    v[2] = p[2 * pitch];
    v[3] = p[3 * pitch];
    return v;
}
typedef short __attribute__((ext_vector_type(4))) i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
template <>
__device__ __forceinline__ bf16x4 frag_cm<bf16>(const bf16* base, int pitch, int r0, int c0) {
    const int l = lane_id(), s = l & 15;
    const bf16* p = base + (r0 + 4 * (l >> 4) + (s >> 2)) * pitch + c0 + 4 * (s & 3);
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// MFMA k-step with both operands in row-major LDS tiles, contracting columns
// c0 .. c0+31 of rows ra + l%16 (A) and rb + l%16 (B).  The order in which the
// 32 contraction indices meet the hardware's k slots is free as long as both
// operands use the same one: 16-bit tiles hand each lane the 8 consecutive
// columns c0 + 8*(l/16) .. +7 of each operand as one 16-byte LDS read (rows
// must start 16-byte aligned); fp32 tiles take the paired 16-column fragments.
template <typename T>
__device__ __forceinline__ f32x4 mma32_rr(f32x4 acc, const T* a, int pa, int ra, const T* b, int pb, int rb, int c0) {
    if constexpr (sizeof(T) == 2) {
        const int l = lane_id();
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(a + (ra + (l & 15)) * pa + c0 + 8 * (l >> 4));
        const bf16x8 y = *reinterpret_cast<const bf16x8*>(b + (rb + (l & 15)) * pb + c0 + 8 * (l >> 4));
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc, 0, 0, 0);
    } else {
        return mma32(acc, frag_rm<T>(a, pa, ra, c0), frag_rm<T>(a, pa, ra, c0 + 16), frag_rm<T>(b, pb, rb, c0),
                     frag_rm<T>(b, pb, rb, c0 + 16));
    }
}

// 16-bit tiles whose columns are interleaved within each 32-column block
// ("paired" layout): column 32b + c sits at 32b + 8*((c/4)%4) + 4*(c/16) + c%4,
// so the eight columns c0 + 4*(l/16) .. +3 and c0 + 16 + 4*(l/16) .. +3 that an
// MFMA k-step pairs with two stacked accumulator tiles (k slots 0-3 from the
// tile of rows c0..c0+15, 4-7 from the next) are one contiguous 16-byte read.
__host__ __device__ constexpr int paired_col(int c) { return (c & ~31) + 8 * ((c >> 2) & 3) + 4 * ((c >> 4) & 1) + (c & 3); }

// (lo, hi) fragments of rows r0 + l%16 of a paired tile for k-step columns
// c0 .. c0+31 (c0 a multiple of 32), as one 16-byte LDS read.
__device__ __forceinline__ bf16x8 frag_paired(const bf16* base, int pitch, int r0, int c0) {
    const int l = lane_id();
    return *reinterpret_cast<const bf16x8*>(base + (r0 + (l & 15)) * pitch + c0 + 8 * (l >> 4));
}

// k-step of a stacked accumulator tile pair (lo: rows c0..c0+15, hi: the next
// 16) against a paired-layout fragment read with frag_paired.
__device__ __forceinline__ f32x4 mma32_pair(f32x4 acc, bf16x4 lo, bf16x4 hi, bf16x8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), b, acc, 0,
                                                    0, 0);
}

// Store 8 values of logical columns c .. c+7 (c a multiple of 8) of one row of a
// paired tile: two 8-byte halves.
__device__ __forceinline__ void store_paired8(bf16* row, int c, const float* x) {
    bf16x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        a[e] = (bf16)x[e];
        b[e] = (bf16)x[4 + e];
    }
    *reinterpret_cast<bf16x4*>(row + paired_col(c)) = a;
    *reinterpret_cast<bf16x4*>(row + paired_col(c + 4)) = b;
}

template <typename T>
__device__ __forceinline__ vec4_t<T> to_vec4(f32x4 x) {
    vec4_t<T> v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = Elem<T>::from_f(x[e]);
    return v;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// A 64-row x W-column tile held in registers between its global load and its
// use, 16 bytes per vector.  Thread `tid` owns vectors tid, tid+NT, ...; vector
// idx covers row idx / (W/VEC), columns (idx % (W/VEC))*VEC .. +VEC-1.
typedef unsigned int __attribute__((ext_vector_type(4))) u32x4;

template <typename T, int W, int NT>
struct TileRegs {
    static constexpr int VEC = 16 / (int)sizeof(T);
    static constexpr int VPR = W / VEC;           // vectors per row
    static constexpr int NV = kChunk * VPR;       // vectors per tile
    static constexpr int PER = (NV + NT - 1) / NT;
    static_assert(W % VEC == 0, "tile width must be a whole number of 16-byte vectors");
    u32x4 r[PER];

    __device__ __forceinline__ static bool owns(int p, int tid) { return (NV % NT == 0) || (tid + p * NT < NV); }
    __device__ __forceinline__ static int row_of(int p, int tid) { return (tid + p * NT) / VPR; }
    __device__ __forceinline__ static int col_of(int p, int tid) { return ((tid + p * NT) % VPR) * VEC; }

    // `g` (uniform) points at element (row 0, col 0) of the tile; rows are `rs`
    // elements apart.  Offsets stay 32-bit so the loads use a scalar base.
    __device__ __forceinline__ void load(const T* __restrict__ g, int rs, int tid) {
#pragma unroll
        for (int p = 0; p < PER; ++p)
            if (owns(p, tid))
                r[p] = *reinterpret_cast<const u32x4*>(g + (row_of(p, tid) * rs + col_of(p, tid)));
    }
    __device__ __forceinline__ void store_lds(T* s, int pitch, int tid) const {
#pragma unroll
        for (int p = 0; p < PER; ++p)
            if (owns(p, tid))
                *reinterpret_cast<u32x4*>(s + row_of(p, tid) * pitch + col_of(p, tid)) = r[p];
    }
    // 16-bit tiles: store into the paired column layout (two 8-byte halves)
    __device__ __forceinline__ void store_lds_paired(T* s, int pitch, int tid) const {
        static_assert(sizeof(T) == 2, "paired layout is for 16-bit tiles");
#pragma unroll
        for (int p = 0; p < PER; ++p)
            if (owns(p, tid)) {
                T* row = s + row_of(p, tid) * pitch;
                const int c = col_of(p, tid);
                *reinterpret_cast<uint2*>(row + paired_col(c)) = uint2{r[p][0], r[p][1]};
                *reinterpret_cast<uint2*>(row + paired_col(c + 4)) = uint2{r[p][2], r[p][3]};
            }
    }
    // element e (0..VEC-1) of vector p as float
    __device__ __forceinline__ float get(int p, int e) const {
        const T* v = reinterpret_cast<const T*>(&r[p]);
        return Elem<T>::to_f(v[e]);
    }
};

// One wave's slab of a 64-row chunk tile, one token row per lane: lane l holds
// row l, columns c0 .. c0+NC-1 (NC a whole number of 16-byte vectors).
template <typename T, int NC>
struct RowSlab {
    static constexpr bool scalar = false;  // see GateSlab
    static constexpr int VEC = 16 / (int)sizeof(T);
    static constexpr int NV = NC / VEC;
    static_assert(NC % VEC == 0, "slab width must be a whole number of 16-byte vectors");
    u32x4 r[NV];
    // `base` (uniform) points at element (row 0, col 0) of the tile; rows are `rs` apart.
    __device__ __forceinline__ void load(const T* __restrict__ base, int rs, int c0) {
        const T* p = base + (lane_id() * rs + c0);
#pragma unroll
        for (int m = 0; m < NV; ++m) r[m] = *reinterpret_cast<const u32x4*>(p + m * VEC);
    }
    // load, except that the lanes with `skip` set read nothing and hold zeros
    // (a row that lies outside the tensor and stands for a zero row)
    __device__ __forceinline__ void load_unless(const T* __restrict__ base, int rs, int c0, bool skip) {
        if (skip) {
#pragma unroll
            for (int m = 0; m < NV; ++m) r[m] = u32x4{0u, 0u, 0u, 0u};
        } else {
            load(base, rs, c0);
        }
    }
    // only the 16-byte vectors m0 .. m1-1 (columns c0 + m*VEC ..)
    __device__ __forceinline__ void load_part(const T* __restrict__ base, int rs, int c0, int m0, int m1) {
        const T* p = base + (lane_id() * rs + c0);
#pragma unroll
        for (int m = 0; m < NV; ++m)
            if (m >= m0 && m < m1) r[m] = *reinterpret_cast<const u32x4*>(p + m * VEC);
    }
    __device__ __forceinline__ float get(int c) const {
        const T* v = reinterpret_cast<const T*>(&r[c / VEC]);
        return Elem<T>::to_f(v[c % VEC]);
    }
};

// The log gate of one wave's slab.  SG = false: one value per key column,
// the RowSlab of the wave's NC columns.  SG = true (scalar gate per token and
// head, the gates of Mamba-2 / RetNet style layers): lane l holds g of token l,
// shared by every column; `base` then points at the chunk's first token in a
// [B, T, H] tensor and rows are `rs` = H apart.  load_part loads the scalar
// with the last column group, so a slab whose preparation is split over two
// phases keeps one chunk's gate until both parts have used it.
template <typename T, int NC, bool SG>
struct GateSlab : RowSlab<T, NC> {};
template <typename T, int NC>
struct GateSlab<T, NC, true> {
    static constexpr bool scalar = true;
    static constexpr int NV = NC / (16 / (int)sizeof(T));
    T r;
    __device__ __forceinline__ void load(const T* __restrict__ base, int rs, int) { r = base[lane_id() * rs]; }
    __device__ __forceinline__ void load_part(const T* __restrict__ base, int rs, int c0, int, int m1) {
        if (m1 == NV) load(base, rs, c0);
    }
    __device__ __forceinline__ float get(int) const { return Elem<T>::to_f(r); }
};

// Inclusive prefix sum over the 64 lanes of a wave (lane = token): four
// row_shr steps within each 16-lane row, then row_bcast:15 into rows 1 and 3
// and row_bcast:31 into rows 2 and 3 (GFX9 DPP).
__device__ __forceinline__ float wave_incl_scan(float x) {
    x += __builtin_amdgcn_update_dpp(0.0f, x, 0x111, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0.0f, x, 0x112, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0.0f, x, 0x114, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0.0f, x, 0x118, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0.0f, x, 0x142, 0xA, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0.0f, x, 0x143, 0xC, 0xF, false);
    return x;
}

// The same scan over N independent values per lane, step by step across the
// values, so no DPP step waits on the one before it of the same value.
template <int N>
__device__ __forceinline__ void wave_incl_scan_n(float* x) {
#pragma unroll
    for (int e = 0; e < N; ++e) x[e] += __builtin_amdgcn_update_dpp(0.0f, x[e], 0x111, 0xF, 0xF, false);
#pragma unroll
    for (int e = 0; e < N; ++e) x[e] += __builtin_amdgcn_update_dpp(0.0f, x[e], 0x112, 0xF, 0xF, false);
#pragma unroll
    for (int e = 0; e < N; ++e) x[e] += __builtin_amdgcn_update_dpp(0.0f, x[e], 0x114, 0xF, 0xF, false);
#pragma unroll
    for (int e = 0; e < N; ++e) x[e] += __builtin_amdgcn_update_dpp(0.0f, x[e], 0x118, 0xF, 0xF, false);
#pragma unroll
    for (int e = 0; e < N; ++e) x[e] += __builtin_amdgcn_update_dpp(0.0f, x[e], 0x142, 0xA, 0xF, false);
#pragma unroll
    for (int e = 0; e < N; ++e) x[e] += __builtin_amdgcn_update_dpp(0.0f, x[e], 0x143, 0xC, 0xF, false);
}

__device__ __forceinline__ float lane_bcast(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Pack VEC floats into one 16-byte vector of T and store it to LDS.
template <typename T>
__device__ __forceinline__ void store_vec_lds(T* dst, const float* x) {
    constexpr int VEC = 16 / (int)sizeof(T);
    uint4 u;
    T* v = reinterpret_cast<T*>(&u);
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[e] = Elem<T>::from_f(x[e]);
    *reinterpret_cast<uint4*>(dst) = u;
}

// ---------------------------------------------------------------------------
// Intra-chunk inclusive cumulative log gate (Section 4.2: b_{iC+j}/b_{iC} in
// log space; Knowl 3 of the chapter summary: "intra-chunk cumulative log
// gates"), in log2 units:  sB[t][i] = log2(e) * sum_{u<=t} g[u][i].
//
// On entry the raw gate tile is in registers; on exit sB holds the cumsum,
// sLast[i] = sB[63][i], sGam[i] = exp2(sLast[i]) (the chunk decay gamma), and
// *sFlag is set if some column's chunk range sB[0][i] - sB[63][i] exceeds
// kRangeLimit.  NT threads; KD columns.  Three barriers inside.  The caller
// clears *sFlag before the first barrier.
template <typename T, int KD, int NT>
__device__ __forceinline__ void chunk_log_cumsum(const TileRegs<T, KD, NT>& graw, float* sB, int pitchB,
                                                 float* sTot, float* sLast, float* sGam, int* sFlag, int tid) {
    using TR = TileRegs<T, KD, NT>;
#pragma unroll
    for (int p = 0; p < TR::PER; ++p) {
        if (!TR::owns(p, tid)) continue;
        float* dst = sB + TR::row_of(p, tid) * pitchB + TR::col_of(p, tid);
#pragma unroll
        for (int e = 0; e < TR::VEC; ++e) dst[e] = graw.get(p, e) * kLog2e;
    }
    __syncthreads();
    static_assert(NT % KD == 0, "threads must tile the gate columns");
    constexpr int NPART = NT / KD;          // threads per column
    constexpr int R = kChunk / NPART;       // rows per thread
    const int col = tid % KD, part = tid / KD;
    float run = 0.f;
#pragma unroll
    for (int u = 0; u < R; ++u) {
        float* p = sB + (part * R + u) * pitchB + col;
        run += *p;
        *p = run;
    }
    sTot[part * KD + col] = run;
    __syncthreads();
    if (part > 0) {
        float off = 0.f;
        for (int p = 0; p < part; ++p) off += sTot[p * KD + col];
#pragma unroll
        for (int u = 0; u < R; ++u) sB[(part * R + u) * pitchB + col] += off;
        if (part == NPART - 1) {
            const float last = run + off;
            sLast[col] = last;
            sGam[col] = exp2_fast(last);
            if (sB[col] - last > kRangeLimit) *sFlag = 1;
        }
    } else if (NPART == 1) {
        sLast[col] = run;
        sGam[col] = exp2_fast(run);
        if (sB[col] - run > kRangeLimit) *sFlag = 1;
    }
    __syncthreads();
}

}  // namespace gla
