// Host-side launch plan shared by the ABI layer and the kernel launchers.
//
// The plan is a pure function of the problem shape (no device query), so the
// workspace size can be computed without a GPU.  It is sized for MI355X: 256
// compute units, one 512-thread workgroup per CU for the chunk walks.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace gla {

constexpr int kTargetWorkgroups = 256;  // MI355X compute units

struct Shape {
    int64_t B, T, H, K, V;
    bool bf16;
};

struct Plan {
    int64_t BH;      // B*H independent recurrences (Section 4.4)
    int64_t N;       // chunks per sequence, T / 64
    int P;           // sequence segments per recurrence
    int seg_len;     // chunks per segment (the last segment may be shorter)
    int BV;          // state columns held by one workgroup in column-split kernels
    int NW;          // waves per workgroup for column-split kernels
    int BK;          // state rows held by one workgroup in row-split kernels
    int NWK;         // waves per workgroup for row-split kernels
};

// State columns per workgroup: the K x BV fp32 state lives in VGPRs (64 per
// lane at 512 threads) and the chunk tiles in LDS (160 KiB per CU).
inline int plan_bv(const Shape& s) {
    int cap;
    if (s.bf16) cap = (s.K <= 64) ? 256 : (s.K <= 128 ? 256 : 64);
    else cap = 128;
    return (int)(s.V < cap ? s.V : cap);
}

// State rows per workgroup in the backward kernels that contract over V.  The
// workgroup has eight waves; a 64-row block splits V between two waves per
// 16-row key block, which keeps the state slice and the chunk's prefetched
// tiles within 256 registers per lane.  Narrow V takes up to 128 rows whole.
inline int plan_bk(const Shape& s) {
    if (!s.bf16 || s.V >= 128) return 64;
    return (int)(s.K < 128 ? s.K : 128);
}

inline Plan make_plan(const Shape& s, int col_blocks_hint) {
    Plan p;
    p.BH = s.B * s.H;
    p.N = s.T / 64;
    p.BV = plan_bv(s);
    p.NW = p.BV / 16 < 8 ? p.BV / 16 : 8;
    p.BK = plan_bk(s);
    p.NWK = 8;
    int64_t per_seg = p.BH * (int64_t)col_blocks_hint;
    int64_t P = per_seg > 0 ? kTargetWorkgroups / per_seg : 1;
    if (P < 1) P = 1;
    if (P > p.N) P = p.N > 0 ? p.N : 1;
    int64_t len = p.N > 0 ? (p.N + P - 1) / P : 1;
    p.seg_len = (int)len;
    p.P = (int)(p.N > 0 ? (p.N + len - 1) / len : 1);
    return p;
}

// 16-bit heads with 256 key columns: the forward forms each chunk's operands
// once per chunk and head (a record in the workspace), and its state and output
// passes take 128 value columns per four-wave workgroup.
inline bool fwd_wide(const Shape& s) { return s.bf16 && s.K == 256; }
constexpr size_t wide_record_bytes(int64_t K) { return (size_t)(4 * 64 * K + 2 * 64 * 64 + 12 * K + 256); }

inline Plan make_fwd_plan(const Shape& s) {
    if (fwd_wide(s)) {
        const int bv = (int)(s.V < 128 ? s.V : 128);
        Plan p = make_plan(s, (int)(s.V / bv));
        p.BV = bv;
        p.NW = 4;
        return p;
    }
    int bv = plan_bv(s);
    return make_plan(s, (int)(s.V / bv));
}

// The backward's column-split kernels take as many value blocks as the
// row-split kernels take key blocks (never narrower than 64 columns), so both
// kinds launch the same number of workgroups over the same segments.
inline Plan make_bwd_plan(const Shape& s) {
    const int bk = plan_bk(s);
    const int nkb = (int)(s.K / bk);
    int bv = plan_bv(s);
    if (nkb > 1 && s.V / nkb < bv) bv = (int)(s.V / nkb);
    if (bv < 64) bv = s.V < 64 ? (int)s.V : 64;
    const int nvb = (int)(s.V / bv);
    Plan p = make_plan(s, nvb > nkb ? nvb : nkb);
    p.BV = bv;
    p.NW = bv / 16 < 8 ? bv / 16 : 8;
    return p;
}

inline size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// Segment states are kept in the input dtype (2 or 4 bytes per element).
inline size_t state_bytes(const Shape& s, const Plan& p) {
    return round256((size_t)p.BH * p.P * (size_t)s.K * (size_t)s.V * (s.bf16 ? 2 : 4));
}

// 2 when the 16-bit dv walk runs at the forward's (twice wider) value width and
// covers each segment as two halves; 1 otherwise.
inline int dv_split(const Shape& s, const Plan& p) {
    return s.bf16 && p.P > 1 && plan_bv(s) == 2 * p.BV ? 2 : 1;
}

// the backward's chunk-end states for the gate-gradient anchors
inline size_t hs_bytes(const Shape& s, const Plan& p) {
    return (size_t)p.BH * p.N * (size_t)s.K * (size_t)s.V * (s.bf16 ? 2 : 4);
}

// segment states and gate totals (P > 1), then the chunk records (wide heads)
inline size_t fwd_seg_bytes(const Shape& s, const Plan& p) {
    if (p.P <= 1 || p.BH == 0) return 0;
    size_t gt = (size_t)p.BH * p.P * (size_t)s.K * sizeof(float);
    return state_bytes(s, p) + round256(gt);
}

// General gates (16-bit, K in {128, 256}): up to 128 value columns per
// workgroup; records carry the key side and the value side of each chunk.
inline Plan make_fwd_general_plan(const Shape& s) {
    const int bv = (int)(s.V < 128 ? s.V : 128);
    Plan p = make_plan(s, (int)(s.V / bv));
    p.BV = bv;
    p.NW = 4;
    return p;
}
constexpr size_t gen_record_bytes(int64_t K, int64_t V) {
    return wide_record_bytes(K) + (size_t)(6 * 64 * V + 8 * V + 256);
}
// segment states, key-row and value-column gate totals (P > 1), then records
inline size_t fwd_general_seg_bytes(const Shape& s, const Plan& p) {
    if (p.P <= 1 || p.BH == 0) return 0;
    return state_bytes(s, p) + round256((size_t)p.BH * p.P * (size_t)s.K * sizeof(float)) +
           round256((size_t)p.BH * p.P * (size_t)s.V * sizeof(float));
}
inline size_t fwd_general_workspace_bytes(const Shape& s) {
    Plan p = make_fwd_general_plan(s);
    if (p.BH == 0) return 0;
    return fwd_general_seg_bytes(s, p) + (size_t)p.BH * p.N * gen_record_bytes(s.K, s.V);
}

// Backward under general gates: the forward's o and S_T, the chunk-start
// states of the forward and of the time-reversed dS recurrence (the anchors of
// the gate gradients, and the starting states of the transposed passes) with
// the anchors formed from them, and the forward workspace of the largest of the
// four general forwards it runs (shapes K x V and V x K).  The reversed
// recurrences read their inputs in place.
struct BwdGeneralLayout {
    size_t o, st, hsf, hsr, ag, ah, ds0, fws, total;
};
inline BwdGeneralLayout bwd_general_layout(const Shape& s) {
    BwdGeneralLayout w{};
    const size_t BTH = (size_t)(s.B * s.T * s.H), BH = (size_t)(s.B * s.H), KV = (size_t)(s.K * s.V);
    const size_t tv = round256(BTH * s.V * 2), sf = round256(BH * KV * 4);
    Shape st = s;
    st.K = s.V;
    st.V = s.K;
    const size_t f1 = fwd_general_workspace_bytes(s), f2 = fwd_general_workspace_bytes(st);
    size_t at = 0;
    w.o = at; at += tv;
    w.st = at; at += sf;
    const size_t N = (size_t)(s.T / 64);
    w.hsf = at; at += round256(BH * N * KV * 2);
    w.hsr = at; at += round256(BH * N * KV * 2);
    w.ag = at; at += round256(BH * (N + 1) * (size_t)s.K * 4);
    w.ah = at; at += round256(BH * (N + 1) * (size_t)s.V * 4);
    w.ds0 = at; at += sf;  // dS_0 when the caller asks for none (the first chunk's gate anchor needs it)
    w.fws = at; at += round256(f1 > f2 ? f1 : f2);
    w.total = at;
    return w;
}

inline size_t fwd_workspace_bytes(const Shape& s) {
    Plan p = make_fwd_plan(s);
    if (p.BH == 0) return 0;
    size_t n = fwd_seg_bytes(s, p);
    if (fwd_wide(s)) n += (size_t)p.BH * p.N * wide_record_bytes(s.K);
    return n;
}

}  // namespace gla
