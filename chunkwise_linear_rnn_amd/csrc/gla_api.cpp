// C ABI of the gfx950 GLA library: argument validation, launch planning and
// dispatch.  Every check runs on the host before the first HIP call, so an
// invalid call enqueues nothing (see include/gla.h for the contract).
#include "../../include/gla.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "gla_gate.hpp"
#include "gla_launch.hpp"
#include "gla_plan.hpp"

namespace {

// Size limits of the chunked entry points and of decode (see check_shape).
constexpr int64_t kMaxHeads = (int64_t)1 << 20;
constexpr int64_t kMaxTokenHeads = (int64_t)1 << 30;
constexpr int64_t kMaxDecodeGroups = (int64_t)1 << 24;

thread_local std::string g_detail;

gla_status_t fail(gla_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
gla_status_t fail(gla_status_t st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_detail = buf;
    return st;
}

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Head dims of the plain and scalar-gate paths: K and V in {64, 128, 256,
// 512}.  The kernels take K <= 256 (16-bit) or 128 (fp32) and V <= 256 in the
// backward, 128 for fp32 (160 KiB of LDS per CU: fp32 tiles are twice the
// size of bf16 ones, and the backward holds both the value and d_o tiles at
// full V).  Wider heads run as slices: key slices (fwd_any_launch,
// bwd_any_launch), value slices (fwd_split_launch, bwd_split_launch).
bool supported_kv(int64_t K, int64_t V, bool bf16, bool backward) {
    (void)bf16;
    (void)backward;
    const bool k_ok = K == 64 || K == 128 || K == 256 || K == 512;
    const bool v_ok = V == 64 || V == 128 || V == 256 || V == 512;
    return k_ok && v_ok;
}

// Shape checks shared by forward and backward.  On success fills `out`.
gla_status_t check_shape(const gla_shape_t* s, gla::Shape* out, bool backward) {
    if (!s) return fail(GLA_ERR_NULL, "shape is NULL");
    if (s->reserved != 0) return fail(GLA_ERR_UNSUPPORTED, "shape.reserved must be 0 (got %d)", s->reserved);
    if (s->B < 0 || s->T < 0 || s->H < 0)
        return fail(GLA_ERR_SHAPE, "negative size: B=%lld T=%lld H=%lld", (long long)s->B, (long long)s->T,
                    (long long)s->H);
    if (s->K <= 0 || s->V <= 0)
        return fail(GLA_ERR_SHAPE, "head dims must be positive: K=%lld V=%lld", (long long)s->K, (long long)s->V);
    if (s->chunk != 64) return fail(GLA_ERR_UNSUPPORTED, "chunk must be 64 (got %lld)", (long long)s->chunk);
    if (s->dtype != GLA_DTYPE_BF16 && s->dtype != GLA_DTYPE_FP32)
        return fail(GLA_ERR_UNSUPPORTED, "unknown dtype %d", s->dtype);
    const bool bf16 = s->dtype == GLA_DTYPE_BF16;
    if (!supported_kv(s->K, s->V, bf16, backward))
        return fail(GLA_ERR_UNSUPPORTED, "unsupported head dims K=%lld V=%lld for %s %s", (long long)s->K,
                    (long long)s->V, bf16 ? "bf16" : "fp32", backward ? "backward" : "forward");
    if (s->T % 64 != 0) return fail(GLA_ERR_SHAPE, "T=%lld is not a multiple of the chunk 64", (long long)s->T);
    // kernel index arithmetic: sizes and a chunk's 64 rows of row stride H*D in
    // int, grids of at most 2^32 work-items (B*H heads), workgroup indices over
    // chunks and heads (B*H*T token-heads; a shape past that limit would not fit
    // in device memory anyway)
    const int64_t lim = (int64_t)1 << 31;
    if (s->T >= lim || s->H >= lim || s->B >= lim)
        return fail(GLA_ERR_SHAPE, "size too large for this library");
    if (s->B * s->H > kMaxHeads)
        return fail(GLA_ERR_SHAPE, "size too large for this library: B*H=%lld heads (at most %lld)",
                    (long long)(s->B * s->H), (long long)kMaxHeads);
    if (s->B * s->H * s->T >= kMaxTokenHeads)
        return fail(GLA_ERR_SHAPE, "size too large for this library: B*H*T=%lld token-heads (below %lld)",
                    (long long)(s->B * s->H * s->T), (long long)kMaxTokenHeads);
    if (s->H * std::max(s->K, s->V) * 64 >= lim)
        return fail(GLA_ERR_SHAPE, "size too large for this library: H*max(K,V)=%lld (below %lld)",
                    (long long)(s->H * std::max(s->K, s->V)), (long long)(lim / 64));
    out->B = s->B;
    out->T = s->T;
    out->H = s->H;
    out->K = s->K;
    out->V = s->V;
    out->bf16 = bf16;
    return GLA_OK;
}

size_t bwd_workspace_bytes(const gla::Shape& s, bool sg);

// The recurrent decode step: any T >= 0, the chunk field unused.
gla_status_t check_decode_shape(const gla_shape_t* s, gla::Shape* out) {
    if (!s) return fail(GLA_ERR_NULL, "shape is NULL");
    if (s->reserved != 0) return fail(GLA_ERR_UNSUPPORTED, "shape.reserved must be 0 (got %d)", s->reserved);
    if (s->B < 0 || s->T < 0 || s->H < 0)
        return fail(GLA_ERR_SHAPE, "negative size: B=%lld T=%lld H=%lld", (long long)s->B, (long long)s->T,
                    (long long)s->H);
    if (s->dtype != GLA_DTYPE_BF16 && s->dtype != GLA_DTYPE_FP32)
        return fail(GLA_ERR_UNSUPPORTED, "unknown dtype %d", s->dtype);
    const bool k_ok = s->K == 64 || s->K == 128 || s->K == 256 || s->K == 512;
    const bool v_ok = s->V == 64 || s->V == 128 || s->V == 256 || s->V == 512;
    if (!k_ok || !v_ok)
        return fail(GLA_ERR_UNSUPPORTED, "unsupported head dims K=%lld V=%lld for decode", (long long)s->K,
                    (long long)s->V);
    // one 256-thread workgroup per head and 64 value columns: at most 2^32 work-items
    const int64_t lim = (int64_t)1 << 31;
    if (s->T >= lim || s->H >= lim || s->B >= lim || s->B * s->H * (s->V / 64) >= kMaxDecodeGroups)
        return fail(GLA_ERR_SHAPE, "size too large for this library: B*H*V/64=%lld workgroups (below %lld)",
                    (long long)(s->B * s->H * (s->V / 64)), (long long)kMaxDecodeGroups);
    out->B = s->B;
    out->T = s->T;
    out->H = s->H;
    out->K = s->K;
    out->V = s->V;
    out->bf16 = s->dtype == GLA_DTYPE_BF16;
    return GLA_OK;
}

// The output epilogue: rows of V channels, T any length; K and chunk unused.
gla_status_t check_gate_shape(const gla_shape_t* s, gla::Shape* out) {
    if (!s) return fail(GLA_ERR_NULL, "shape is NULL");
    if (s->reserved != 0) return fail(GLA_ERR_UNSUPPORTED, "shape.reserved must be 0 (got %d)", s->reserved);
    if (s->B < 0 || s->T < 0 || s->H < 0)
        return fail(GLA_ERR_SHAPE, "negative size: B=%lld T=%lld H=%lld", (long long)s->B, (long long)s->T,
                    (long long)s->H);
    if (s->dtype != GLA_DTYPE_BF16 && s->dtype != GLA_DTYPE_FP32)
        return fail(GLA_ERR_UNSUPPORTED, "unknown dtype %d", s->dtype);
    if (s->V != 64 && s->V != 128 && s->V != 256 && s->V != 512)
        return fail(GLA_ERR_UNSUPPORTED, "unsupported head dim V=%lld for the output gate", (long long)s->V);
    const int64_t lim = (int64_t)1 << 31;
    if (s->T >= lim || s->H >= lim || s->B >= lim || (s->B * s->H >= lim) || s->B * s->H * s->T >= lim)
        return fail(GLA_ERR_SHAPE, "size too large for this library");
    out->B = s->B;
    out->T = s->T;
    out->H = s->H;
    out->K = s->K;
    out->V = s->V;
    out->bf16 = s->dtype == GLA_DTYPE_BF16;
    return GLA_OK;
}

bool eps_ok(float eps) { return eps >= 0.f && eps <= 3.0e38f; }  // false for NaN and infinities

// Validation of the forward's arguments other than the workspace; fills `s`.
gla_status_t fwd_check(const gla_shape_t* shape, const void* q, const void* k, const void* v, const void* g,
                       const float* s0, void* o, float* s_final, bool sg, gla::Shape* s) {
    gla_status_t st = check_shape(shape, s, false);
    if (st != GLA_OK) return st;
    const bool empty = s->B * s->H == 0 || s->T == 0;
    if (!empty && (!q || !k || !v || !g || !o)) return fail(GLA_ERR_NULL, "q, k, v, g and o are required");
    const void* ptrs[] = {q, k, v, g, s0, o, s_final};
    const char* names[] = {"q", "k", "v", "g", "s0", "o", "s_final"};
    for (int i = 0; i < 7; ++i)
        if (!aligned16(ptrs[i])) return fail(GLA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    return GLA_OK;
}

// Shapes whose backward can start from a checkpointing forward's segment
// states: 16-bit inputs on the pipelined walks (K <= 128) with more than one
// backward segment.  Returns the checkpoint's size in bytes, or 0.
size_t ckpt_bytes(const gla::Shape& s) {
    if (!s.bf16 || s.K > 128 || s.V > 256 || s.B * s.H == 0 || s.T == 0) return 0;
    const gla::Plan pb = gla::make_bwd_plan(s);
    return pb.P > 1 ? gla::state_bytes(s, pb) : 0;
}

// The forward's launches for a validated, non-empty shape on one set of kernels
// (fp32 at V <= 128, 16-bit at any supported V).
hipError_t fwd_launch(const gla::Shape& s, const void* q, const void* k, const void* v, const void* g,
                      const float* s0, void* o, float* s_final, void* workspace, bool sg, void* ckpt,
                      hipStream_t strm) {
    gla::Plan p = gla::make_fwd_plan(s);
    gla::FwdLaunch a{};
    a.bf16 = s.bf16;
    a.sg = sg;
    a.K = (int)s.K;
    a.V = (int)s.V;
    a.BV = p.BV;
    a.T = (int)s.T;
    a.H = (int)s.H;
    a.N = (int)p.N;
    a.P = p.P;
    a.seg_len = p.seg_len;
    a.BH = p.BH;
    a.q = q; a.k = k; a.v = v; a.g = g;
    a.s0 = s0;
    a.o = o;
    a.s_final = s_final;
    if (p.P > 1) {
        a.ws_state = workspace;
        a.ws_gate = reinterpret_cast<float*>(static_cast<char*>(workspace) + gla::state_bytes(s, p));
    }
    if (gla::fwd_wide(s)) a.ws_rec = static_cast<char*>(workspace) + gla::fwd_seg_bytes(s, p);
    if (ckpt && ckpt_bytes(s) > 0) {
        const gla::Plan pb = gla::make_bwd_plan(s);
        a.ckpt = ckpt;
        a.ck_len = pb.seg_len;
        a.ck_P = pb.P;
    }
    a.stream = strm;
    return gla::launch_fwd(a);
}

// fp32 at V = 256 or 512: the recurrence acts on each value column independently
// (Section 4.1, Eq. 3), so the forward is V / 128 forwards over column slices of
// v and S_0 (gathered into the workspace) that share q, k and g; o and S_T are
// the slices side by side.  The same holds for the backward (split_layout).
constexpr long kFp32SliceV = 128;
bool split_fwd(const gla::Shape& s) { return !s.bf16 && s.V > kFp32SliceV; }

struct FwdSplitLayout {
    size_t vh, oh, s0h, sfh, inner, total;
};
FwdSplitLayout fwd_split_layout(const gla::Shape& s) {
    FwdSplitLayout w{};
    gla::Shape h = s;
    h.V = kFp32SliceV;
    const size_t BTH = (size_t)(s.B * s.T * s.H), BH = (size_t)(s.B * s.H);
    size_t at = 0;
    auto take = [&](size_t n) { const size_t o = at; at += gla::round256(n); return o; };
    w.vh = take(BTH * h.V * 4);
    w.oh = take(BTH * h.V * 4);
    w.s0h = take(BH * s.K * h.V * 4);
    w.sfh = take(BH * s.K * h.V * 4);
    w.inner = take(gla::fwd_workspace_bytes(h));
    w.total = at;
    return w;
}

hipError_t fwd_split_launch(const gla::Shape& s, const void* q, const void* k, const void* v, const void* g,
                            const float* s0, void* o, float* s_final, void* workspace, hipStream_t strm) {
    const FwdSplitLayout L = fwd_split_layout(s);
    gla::Shape h = s;
    h.V = kFp32SliceV;
    char* ws = static_cast<char*>(workspace);
    const long W = h.V, VT = s.V;
    const long rows_t = s.B * s.T * s.H, rows_s = s.B * s.H * s.K;
    hipError_t err = hipSuccess;
    for (long off = 0; off < VT && err == hipSuccess; off += W) {
        err = gla::launch_copy_cols(false, v, VT, off, ws + L.vh, W, 0, W, rows_t, strm);
        if (err == hipSuccess && s0) err = gla::launch_copy_cols(false, s0, VT, off, ws + L.s0h, W, 0, W, rows_s, strm);
        if (err != hipSuccess) break;
        err = fwd_launch(h, q, k, ws + L.vh, g, s0 ? (const float*)(ws + L.s0h) : nullptr, ws + L.oh,
                         s_final ? (float*)(ws + L.sfh) : nullptr, ws + L.inner, false, nullptr, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(false, ws + L.oh, W, 0, o, VT, off, W, rows_t, strm);
        if (err == hipSuccess && s_final)
            err = gla::launch_copy_cols(false, ws + L.sfh, W, 0, s_final, VT, off, W, rows_s, strm);
    }
    return err;
}

size_t fwd_total_bytes(const gla::Shape& s) {
    if (s.B * s.H == 0 || s.T == 0) return 0;
    return split_fwd(s) ? fwd_split_layout(s).total : gla::fwd_workspace_bytes(s);
}

hipError_t fwd_v_launch(const gla::Shape& s, const void* q, const void* k, const void* v, const void* g,
                        const float* s0, void* o, float* s_final, void* workspace, bool sg, void* ckpt,
                        hipStream_t strm) {
    return split_fwd(s) ? fwd_split_launch(s, q, k, v, g, s0, o, s_final, workspace, strm)
                        : fwd_launch(s, q, k, v, g, s0, o, s_final, workspace, sg, ckpt, strm);
}

// Key dims past a kernel set's widest (16-bit: 256, fp32: 128) run as slices
// of key columns.  Diag(alpha_t) scales each row of the state on its own and
// k_t^T v_t builds row i from k_t[i] alone (Section 4.1, Eq. 3), so row i of
// S_t depends only on column i of k and g, while o_t = q_t S_t sums over the
// rows: a head with K key columns is K / W heads of width W that share v (and
// a per-token scalar gate, or a value-side gate) and whose outputs add.  Each
// slice's state is a block of W rows of the head's state.
long kslice_width(const gla::Shape& s) { return s.bf16 ? 256 : 128; }
bool split_k(const gla::Shape& s) { return s.K > kslice_width(s); }

// [BH][K][V] rows k0 .. k0 + W - 1  ->  [BH][W][V], and back
hipError_t state_rows_out(const float* src, const gla::Shape& s, long k0, long W, void* dst, hipStream_t strm) {
    return gla::launch_copy_cols(false, src, s.K * s.V, k0 * s.V, dst, W * s.V, 0, W * s.V, s.B * s.H, strm);
}
hipError_t state_rows_in(const void* src, const gla::Shape& s, long k0, long W, float* dst, hipStream_t strm) {
    return gla::launch_copy_cols(false, src, W * s.V, 0, dst, s.K * s.V, k0 * s.V, W * s.V, s.B * s.H, strm);
}

// Workspace of a key-sliced call: per-slice copies of the token tensors with K
// columns (q, k and the gate, unless it is one value per token), the partial
// output, the state row blocks, then the slice's own workspace.
struct KFwdLayout {
    size_t qh, kh, gh, oh, s0h, sfh, inner, total;
};
KFwdLayout kfwd_layout(const gla::Shape& s, bool sg, size_t inner_bytes) {
    KFwdLayout w{};
    const size_t W = (size_t)kslice_width(s);
    const size_t BTH = (size_t)(s.B * s.T * s.H), BH = (size_t)(s.B * s.H), e = s.bf16 ? 2 : 4;
    size_t at = 0;
    auto take = [&](size_t n) { const size_t o = at; at += gla::round256(n); return o; };
    w.qh = take(BTH * W * e);
    w.kh = take(BTH * W * e);
    w.gh = sg ? 0 : take(BTH * W * e);
    w.oh = take(BTH * s.V * e);
    w.s0h = take(BH * W * s.V * 4);
    w.sfh = take(BH * W * s.V * 4);
    w.inner = take(inner_bytes);
    w.total = at;
    return w;
}
gla::Shape kslice_shape(const gla::Shape& s) {
    gla::Shape h = s;
    h.K = kslice_width(s);
    return h;
}

// One forward per key slice: gather its q, k, g columns and S_0 rows, run, add
// its output into o (the first slice writes o) and place its S_T rows.  `run`
// launches the slice's forward on (q, k, g, s0, o, s_final, workspace).
template <class Run>
hipError_t fwd_ksplit(const gla::Shape& s, const void* q, const void* k, const void* g, const float* s0, void* o,
                      float* s_final, void* workspace, bool sg, const KFwdLayout& L, hipStream_t strm, Run run) {
    const long W = kslice_width(s), KT = s.K, rows_t = s.B * s.T * s.H;
    const bool b = s.bf16;
    char* ws = static_cast<char*>(workspace);
    hipError_t err = hipSuccess;
    for (long k0 = 0; k0 < KT && err == hipSuccess; k0 += W) {
        const bool first = k0 == 0;
        err = gla::launch_copy_cols(b, q, KT, k0, ws + L.qh, W, 0, W, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(b, k, KT, k0, ws + L.kh, W, 0, W, rows_t, strm);
        if (err == hipSuccess && !sg) err = gla::launch_copy_cols(b, g, KT, k0, ws + L.gh, W, 0, W, rows_t, strm);
        if (err == hipSuccess && s0) err = state_rows_out(s0, s, k0, W, ws + L.s0h, strm);
        if (err != hipSuccess) break;
        err = run(ws + L.qh, ws + L.kh, sg ? g : ws + L.gh, s0 ? (const float*)(ws + L.s0h) : nullptr,
                  first ? o : ws + L.oh, s_final ? (float*)(ws + L.sfh) : nullptr, ws + L.inner);
        if (err == hipSuccess && !first) err = gla::launch_add_into(b, o, ws + L.oh, rows_t * s.V, strm);
        if (err == hipSuccess && s_final) err = state_rows_in(ws + L.sfh, s, k0, W, s_final, strm);
    }
    return err;
}

// fp32 inputs with one gate per token run the per-column path on the gate
// repeated over the key columns (alpha_t = exp(g_t) times the all-ones row is
// exactly the per-column gate with equal columns); the gate's gradient is then
// the sum over the columns of the per-column one.  The repeated gate (and, in
// the backward, the per-column gradient) sit at the start of the workspace.
bool sg_bcast(const gla::Shape& s, bool sg) { return sg && !s.bf16; }
size_t bcast_gate_bytes(const gla::Shape& s) { return gla::round256((size_t)(s.B * s.T * s.H) * (size_t)s.K * 4); }

size_t fwd_any_bytes(const gla::Shape& s, bool sg) {
    if (s.B * s.H == 0 || s.T == 0) return 0;
    if (sg_bcast(s, sg)) return bcast_gate_bytes(s) + fwd_any_bytes(s, false);
    if (!split_k(s)) return fwd_total_bytes(s);
    return kfwd_layout(s, sg, fwd_total_bytes(kslice_shape(s))).total;
}

// The plain and scalar-gate forward for a validated, non-empty shape.
hipError_t fwd_any_launch(const gla::Shape& s, const void* q, const void* k, const void* v, const void* g,
                          const float* s0, void* o, float* s_final, void* workspace, bool sg, void* ckpt,
                          hipStream_t strm) {
    if (sg_bcast(s, sg)) {
        float* gk = static_cast<float*>(workspace);
        const hipError_t err = gla::launch_bcast_cols(static_cast<const float*>(g), gk, s.K, s.B * s.T * s.H, strm);
        if (err != hipSuccess) return err;
        return fwd_any_launch(s, q, k, v, gk, s0, o, s_final, static_cast<char*>(workspace) + bcast_gate_bytes(s),
                              false, nullptr, strm);
    }
    if (!split_k(s)) return fwd_v_launch(s, q, k, v, g, s0, o, s_final, workspace, sg, ckpt, strm);
    const gla::Shape h = kslice_shape(s);
    const KFwdLayout L = kfwd_layout(s, sg, fwd_total_bytes(h));
    return fwd_ksplit(s, q, k, g, s0, o, s_final, workspace, sg, L, strm,
                      [&](const void* qh, const void* kh, const void* gh, const float* s0h, void* oh, float* sfh,
                          void* inner) { return fwd_v_launch(h, qh, kh, v, gh, s0h, oh, sfh, inner, sg, nullptr, strm); });
}

gla_status_t fwd_impl(const gla_shape_t* shape, const void* q, const void* k, const void* v, const void* g,
                      const float* s0, void* o, float* s_final, void* workspace, size_t workspace_bytes,
                      void* stream, bool sg, void* ckpt = nullptr) {
    g_detail.clear();
    gla::Shape s;
    gla_status_t st = fwd_check(shape, q, k, v, g, s0, o, s_final, sg, &s);
    if (st != GLA_OK) return st;
    if (!aligned16(workspace)) return fail(GLA_ERR_ALIGN, "workspace is not 16-byte aligned");
    const bool empty = s.B * s.H == 0 || s.T == 0;
    const size_t need = fwd_any_bytes(s, sg);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(GLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
    hipError_t err;
    if (empty) {
        // no tokens: the final state is the initial state (Section 2.2)
        err = s_final ? gla::launch_state_copy(s0, s_final, s.B * s.H * s.K * s.V, strm) : hipSuccess;
    } else {
        err = fwd_any_launch(s, q, k, v, g, s0, o, s_final, workspace, sg, ckpt, strm);
    }
    if (err != hipSuccess) return fail(GLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return GLA_OK;
}

// Bytes of the general-gate checkpoint: the state before every chunk [BH][N][K][V]
// bf16, then S_T [BH][K][V] fp32; 0 for shapes the general backward does not take.
size_t general_ckpt_bytes(const gla::Shape& s) {
    if (!s.bf16 || (s.K != 128 && s.K != 256) || (s.V != 128 && s.V != 256)) return 0;
    if (s.B * s.H == 0 || s.T == 0) return 0;
    const size_t BH = (size_t)(s.B * s.H), KV = (size_t)(s.K * s.V);
    return gla::round256(BH * (size_t)(s.T / 64) * KV * 2) + gla::round256(BH * KV * 4);
}
size_t general_ckpt_st_offset(const gla::Shape& s) {
    return gla::round256((size_t)(s.B * s.H) * (size_t)(s.T / 64) * (size_t)(s.K * s.V) * 2);
}

// The general-gate forward for a validated, non-empty shape with K in {128,
// 256}.  ckpt (optional, general_ckpt_bytes(s) bytes): the forward also writes
// the state before every chunk and S_T there, for gla_bwd_general_ckpt.
hipError_t fwd_general_launch(const gla::Shape& s, const void* q, const void* k, const void* v, const void* g,
                              const void* h, const float* s0, void* o, float* s_final, void* workspace, void* ckpt,
                              hipStream_t strm) {
    gla::Plan p = gla::make_fwd_general_plan(s);
    gla::FwdLaunch a{};
    a.bf16 = true;
    a.K = (int)s.K;
    a.V = (int)s.V;
    a.BV = p.BV;
    a.T = (int)s.T;
    a.H = (int)s.H;
    a.N = (int)p.N;
    a.P = p.P;
    a.seg_len = p.seg_len;
    a.BH = p.BH;
    a.q = q; a.k = k; a.v = v; a.g = g; a.h = h;
    a.s0 = s0;
    a.o = o;
    a.s_final = s_final;
    if (ckpt) {
        // S_T goes to the checkpoint, and to s_final too when the caller asks for it
        a.ws_hs = ckpt;
        a.s_final = reinterpret_cast<float*>(static_cast<char*>(ckpt) + general_ckpt_st_offset(s));
        a.s_final2 = s_final;
    }
    char* ws = static_cast<char*>(workspace);
    if (p.P > 1) {
        const size_t sb = gla::state_bytes(s, p);
        a.ws_state = ws;
        a.ws_gate = reinterpret_cast<float*>(ws + sb);
        a.ws_gateb = reinterpret_cast<float*>(ws + sb + gla::round256((size_t)p.BH * p.P * s.K * sizeof(float)));
    }
    a.ws_rec = ws + gla::fwd_general_seg_bytes(s, p);
    a.stream = strm;
    return gla::launch_fwd_general(a);
}

// General gates take K in {128, 256, 512} (512 as two key slices: the gate
// alpha^T beta still scales each state row on its own, so the slices share v
// and the value-side gate h) and V in {64 .. 512} in the forward.
// K = 64 is padded to 128 with zero columns of q, k and g (and zero rows of
// S_0): a zero gate keeps alpha = 1 there, so the padded state rows start and
// stay zero and add nothing to o = q S; the results are exactly the K = 64
// ones.  (The value side pads the same way in the backward: zero columns of
// v, h and d_o.)
bool general_k_ok(int64_t K) { return K == 64 || K == 128 || K == 256 || K == 512; }
constexpr long kGeneralMinDim = 128;
gla::Shape general_kpad_shape(const gla::Shape& s) {
    gla::Shape p = s;
    p.K = kGeneralMinDim;
    return p;
}
struct GKPadFwd {
    size_t qp, kp, gp, s0p, sfp, inner, total;
};
GKPadFwd general_kpad_fwd_layout(const gla::Shape& s) {
    GKPadFwd w{};
    const size_t P = kGeneralMinDim, BTH = (size_t)(s.B * s.T * s.H), BH = (size_t)(s.B * s.H);
    size_t at = 0;
    auto take = [&](size_t n) { const size_t o = at; at += gla::round256(n); return o; };
    w.qp = take(BTH * P * 2);
    w.kp = take(BTH * P * 2);
    w.gp = take(BTH * P * 2);
    w.s0p = take(BH * P * s.V * 4);
    w.sfp = take(BH * P * s.V * 4);
    w.inner = take(gla::fwd_general_workspace_bytes(general_kpad_shape(s)));
    w.total = at;
    return w;
}
size_t fwd_general_any_bytes(const gla::Shape& s) {
    if (s.B * s.H == 0 || s.T == 0) return 0;
    if (s.K < kGeneralMinDim) return general_kpad_fwd_layout(s).total;
    if (!split_k(s)) return gla::fwd_general_workspace_bytes(s);
    return kfwd_layout(s, false, gla::fwd_general_workspace_bytes(kslice_shape(s))).total;
}

hipError_t fwd_general_kpad_launch(const gla::Shape& s, const void* q, const void* k, const void* v, const void* g,
                                   const void* h, const float* s0, void* o, float* s_final, void* workspace,
                                   hipStream_t strm) {
    const GKPadFwd L = general_kpad_fwd_layout(s);
    const gla::Shape p = general_kpad_shape(s);
    char* ws = static_cast<char*>(workspace);
    const long K = s.K, P = p.K, rows_t = s.B * s.T * s.H, BH = s.B * s.H;
    hipError_t err = gla::launch_pad_cols(true, q, K, K, ws + L.qp, P, P, rows_t, strm);
    if (err == hipSuccess) err = gla::launch_pad_cols(true, k, K, K, ws + L.kp, P, P, rows_t, strm);
    if (err == hipSuccess) err = gla::launch_pad_cols(true, g, K, K, ws + L.gp, P, P, rows_t, strm);
    if (err == hipSuccess && s0) err = gla::launch_pad_cols(false, s0, K * s.V, K * s.V, ws + L.s0p, P * s.V, P * s.V, BH, strm);
    if (err != hipSuccess) return err;
    err = fwd_general_launch(p, ws + L.qp, ws + L.kp, v, ws + L.gp, h, s0 ? (const float*)(ws + L.s0p) : nullptr, o,
                             s_final ? (float*)(ws + L.sfp) : nullptr, ws + L.inner, nullptr, strm);
    if (err == hipSuccess && s_final)
        err = gla::launch_copy_cols(false, ws + L.sfp, P * s.V, 0, s_final, K * s.V, 0, K * s.V, BH, strm);
    return err;
}

gla_status_t fwd_general_impl(const gla_shape_t* shape, const void* q, const void* k, const void* v,
                              const void* g, const void* h, const float* s0, void* o, float* s_final,
                              void* workspace, size_t workspace_bytes, void* stream, void* ckpt = nullptr,
                              bool want_ckpt = false) {
    g_detail.clear();
    gla::Shape s;
    gla_status_t st = check_shape(shape, &s, want_ckpt);
    if (st != GLA_OK) return st;
    if (!s.bf16) return fail(GLA_ERR_UNSUPPORTED, "the general-gate path takes bf16 inputs");
    if (!general_k_ok(s.K))
        return fail(GLA_ERR_UNSUPPORTED, "the general-gate path takes K = 64, 128, 256 or 512 (got %lld)", (long long)s.K);
    // shapes without a checkpoint (K or V outside {128, 256}, or empty): the plain forward
    if (want_ckpt && general_ckpt_bytes(s) == 0) {
        want_ckpt = false;
        ckpt = nullptr;
    }
    const bool empty = s.B * s.H == 0 || s.T == 0;
    if (!empty && (!q || !k || !v || !g || !h || !o)) return fail(GLA_ERR_NULL, "q, k, v, g, h and o are required");
    if (want_ckpt && !empty && !ckpt)
        return fail(GLA_ERR_NULL, "ckpt is required (gla_general_ckpt_size = %zu bytes)", general_ckpt_bytes(s));
    const void* ptrs[] = {q, k, v, g, h, s0, o, s_final, workspace, ckpt};
    const char* names[] = {"q", "k", "v", "g", "h", "s0", "o", "s_final", "workspace", "ckpt"};
    for (int i = 0; i < 10; ++i)
        if (!aligned16(ptrs[i])) return fail(GLA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    const size_t need = fwd_general_any_bytes(s);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(GLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
    hipError_t err;
    if (empty) {
        err = s_final ? gla::launch_state_copy(s0, s_final, s.B * s.H * s.K * s.V, strm) : hipSuccess;
    } else if (s.K < kGeneralMinDim) {
        err = fwd_general_kpad_launch(s, q, k, v, g, h, s0, o, s_final, workspace, strm);
    } else if (!split_k(s)) {
        err = fwd_general_launch(s, q, k, v, g, h, s0, o, s_final, workspace, want_ckpt ? ckpt : nullptr, strm);
    } else {
        const gla::Shape hs = kslice_shape(s);
        const KFwdLayout L = kfwd_layout(s, false, gla::fwd_general_workspace_bytes(hs));
        err = fwd_ksplit(s, q, k, g, s0, o, s_final, workspace, false, L, strm,
                         [&](const void* qh, const void* kh, const void* gh, const float* s0h, void* oh, float* sfh,
                             void* inner) {
                             return fwd_general_launch(hs, qh, kh, v, gh, h, s0h, oh, sfh, inner, nullptr, strm);
                         });
    }
    if (err != hipSuccess) return fail(GLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return GLA_OK;
}

// The general-gate backward for a validated, non-empty shape with K and V in
// {128, 256}.  o, ckpt (both or neither): the forward's output and what
// gla_fwd_general_ckpt wrote; the backward then runs no forward of its own.
hipError_t bwd_general_launch(const gla::Shape& s, const void* q, const void* k, const void* v, const void* g,
                              const void* h, const float* s0, const void* d_o, const float* dht, void* dq, void* dk,
                              void* dv, void* dg, void* dh, float* ds0, void* workspace, const void* o,
                              const void* ckpt, hipStream_t strm) {
    gla::BwdGeneralLaunch a{};
    a.B = (int)s.B; a.T = (int)s.T; a.H = (int)s.H; a.K = (int)s.K; a.V = (int)s.V;
    a.q = q; a.k = k; a.v = v; a.g = g; a.h = h; a.d_o = d_o;
    a.s0 = s0; a.dht = dht;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dh = dh; a.ds0 = ds0;
    if (ckpt) {
        a.o_in = o;
        a.hs_in = ckpt;
        a.st_in = reinterpret_cast<const float*>(static_cast<const char*>(ckpt) + general_ckpt_st_offset(s));
    }
    a.workspace = workspace;
    a.stream = strm;
    return gla::launch_bwd_general(a);
}

// V = 512 as two value slices of 256 (each value column of the state, with its
// gate beta_j, evolves on its own): v, h, d_o and the S_0 / dht columns are
// gathered per slice; dv, dh and dS_0 are the slices side by side, dq, dk and
// dg the sums of the slices' values.
constexpr long kGeneralSliceV = 256;
struct GVLayout {
    size_t vh, hh, doh, dq1, dk1, dg1, dvh, dhh, s0h, dhth, ds0h, inner, total;
};
GVLayout general_v_layout(const gla::Shape& s) {
    GVLayout w{};
    gla::Shape sub = s;
    sub.V = kGeneralSliceV;
    const size_t W = kGeneralSliceV, BTH = (size_t)(s.B * s.T * s.H), BH = (size_t)(s.B * s.H);
    size_t at = 0;
    auto take = [&](size_t n) { const size_t o = at; at += gla::round256(n); return o; };
    w.vh = take(BTH * W * 2);
    w.hh = take(BTH * W * 2);
    w.doh = take(BTH * W * 2);
    w.dq1 = take(BTH * s.K * 2);
    w.dk1 = take(BTH * s.K * 2);
    w.dg1 = take(BTH * s.K * 2);
    w.dvh = take(BTH * W * 2);
    w.dhh = take(BTH * W * 2);
    w.s0h = take(BH * s.K * W * 4);
    w.dhth = take(BH * s.K * W * 4);
    w.ds0h = take(BH * s.K * W * 4);
    w.inner = take(gla::bwd_general_layout(sub).total);
    w.total = at;
    return w;
}
// V = 64: v, h and d_o padded with zero columns (S_0, dht with zero columns):
// the padded state columns start and stay zero, so dq, dk and dg are exact and
// dv, dh, dS_0 are the first 64 columns of the padded problem's.
struct GVPad {
    size_t vp, hp, dop, dvp, dhp, s0p, dhtp, ds0p, inner, total;
};
GVPad general_vpad_layout(const gla::Shape& s) {
    GVPad w{};
    gla::Shape p = s;
    p.V = kGeneralMinDim;
    const size_t P = kGeneralMinDim, BTH = (size_t)(s.B * s.T * s.H), BH = (size_t)(s.B * s.H);
    size_t at = 0;
    auto take = [&](size_t n) { const size_t o = at; at += gla::round256(n); return o; };
    w.vp = take(BTH * P * 2);
    w.hp = take(BTH * P * 2);
    w.dop = take(BTH * P * 2);
    w.dvp = take(BTH * P * 2);
    w.dhp = take(BTH * P * 2);
    w.s0p = take(BH * s.K * P * 4);
    w.dhtp = take(BH * s.K * P * 4);
    w.ds0p = take(BH * s.K * P * 4);
    w.inner = take(gla::bwd_general_layout(p).total);
    w.total = at;
    return w;
}
size_t bwd_general_v_bytes(const gla::Shape& s) {
    if (s.V < kGeneralMinDim) return general_vpad_layout(s).total;
    return s.V > kGeneralSliceV ? general_v_layout(s).total : gla::bwd_general_layout(s).total;
}

hipError_t bwd_general_v_launch(const gla::Shape& s, const void* q, const void* k, const void* v, const void* g,
                                const void* h, const float* s0, const void* d_o, const float* dht, void* dq,
                                void* dk, void* dv, void* dg, void* dh, float* ds0, void* workspace,
                                hipStream_t strm) {
    if (s.V < kGeneralMinDim) {
        const GVPad L = general_vpad_layout(s);
        gla::Shape p = s;
        p.V = kGeneralMinDim;
        char* ws = static_cast<char*>(workspace);
        const long V = s.V, P = p.V, rows_t = s.B * s.T * s.H, rows_s = s.B * s.H * s.K;
        hipError_t err = gla::launch_pad_cols(true, v, V, V, ws + L.vp, P, P, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_pad_cols(true, h, V, V, ws + L.hp, P, P, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_pad_cols(true, d_o, V, V, ws + L.dop, P, P, rows_t, strm);
        if (err == hipSuccess && s0) err = gla::launch_pad_cols(false, s0, V, V, ws + L.s0p, P, P, rows_s, strm);
        if (err == hipSuccess && dht) err = gla::launch_pad_cols(false, dht, V, V, ws + L.dhtp, P, P, rows_s, strm);
        if (err != hipSuccess) return err;
        err = bwd_general_launch(p, q, k, ws + L.vp, g, ws + L.hp, s0 ? (const float*)(ws + L.s0p) : nullptr,
                                 ws + L.dop, dht ? (const float*)(ws + L.dhtp) : nullptr, dq, dk, ws + L.dvp, dg,
                                 ws + L.dhp, ds0 ? (float*)(ws + L.ds0p) : nullptr, ws + L.inner, nullptr, nullptr,
                                 strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(true, ws + L.dvp, P, 0, dv, V, 0, V, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(true, ws + L.dhp, P, 0, dh, V, 0, V, rows_t, strm);
        if (err == hipSuccess && ds0)
            err = gla::launch_copy_cols(false, ws + L.ds0p, P, 0, ds0, V, 0, V, rows_s, strm);
        return err;
    }
    if (s.V <= kGeneralSliceV)
        return bwd_general_launch(s, q, k, v, g, h, s0, d_o, dht, dq, dk, dv, dg, dh, ds0, workspace, nullptr,
                                  nullptr, strm);
    const GVLayout L = general_v_layout(s);
    gla::Shape sub = s;
    sub.V = kGeneralSliceV;
    char* ws = static_cast<char*>(workspace);
    const long W = kGeneralSliceV, VT = s.V, rows_t = s.B * s.T * s.H, rows_s = s.B * s.H * s.K;
    const long n_k = rows_t * s.K;
    hipError_t err = hipSuccess;
    for (long off = 0; off < VT && err == hipSuccess; off += W) {
        const bool first = off == 0;
        err = gla::launch_copy_cols(true, v, VT, off, ws + L.vh, W, 0, W, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(true, h, VT, off, ws + L.hh, W, 0, W, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(true, d_o, VT, off, ws + L.doh, W, 0, W, rows_t, strm);
        if (err == hipSuccess && s0) err = gla::launch_copy_cols(false, s0, VT, off, ws + L.s0h, W, 0, W, rows_s, strm);
        if (err == hipSuccess && dht)
            err = gla::launch_copy_cols(false, dht, VT, off, ws + L.dhth, W, 0, W, rows_s, strm);
        if (err != hipSuccess) break;
        err = bwd_general_launch(sub, q, k, ws + L.vh, g, ws + L.hh, s0 ? (const float*)(ws + L.s0h) : nullptr,
                                 ws + L.doh, dht ? (const float*)(ws + L.dhth) : nullptr, first ? dq : ws + L.dq1,
                                 first ? dk : ws + L.dk1, ws + L.dvh, first ? dg : ws + L.dg1, ws + L.dhh,
                                 ds0 ? (float*)(ws + L.ds0h) : nullptr, ws + L.inner, nullptr, nullptr, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(true, ws + L.dvh, W, 0, dv, VT, off, W, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(true, ws + L.dhh, W, 0, dh, VT, off, W, rows_t, strm);
        if (err == hipSuccess && ds0)
            err = gla::launch_copy_cols(false, ws + L.ds0h, W, 0, ds0, VT, off, W, rows_s, strm);
        if (!first) {
            if (err == hipSuccess) err = gla::launch_add_into(true, dq, ws + L.dq1, n_k, strm);
            if (err == hipSuccess) err = gla::launch_add_into(true, dk, ws + L.dk1, n_k, strm);
            if (err == hipSuccess) err = gla::launch_add_into(true, dg, ws + L.dg1, n_k, strm);
        }
    }
    return err;
}

// K = 512 as two key slices of 256 (kbwd_layout's pattern): dq, dk and dg are
// the slices' columns, dv and dh the sums of the slices' values (h is the
// gate of the value columns, which every row shares), dS_0 the row blocks.
struct GKLayout {
    size_t qh, kh, gh, dqh, dkh, dgh, dvh, dhh, s0h, dhth, ds0h, inner, total;
};
GKLayout general_k_layout(const gla::Shape& s) {
    GKLayout w{};
    const size_t W = (size_t)kslice_width(s);
    const size_t BTH = (size_t)(s.B * s.T * s.H), BH = (size_t)(s.B * s.H);
    size_t at = 0;
    auto take = [&](size_t n) { const size_t o = at; at += gla::round256(n); return o; };
    w.qh = take(BTH * W * 2);
    w.kh = take(BTH * W * 2);
    w.gh = take(BTH * W * 2);
    w.dqh = take(BTH * W * 2);
    w.dkh = take(BTH * W * 2);
    w.dgh = take(BTH * W * 2);
    w.dvh = take(BTH * s.V * 2);
    w.dhh = take(BTH * s.V * 2);
    w.s0h = take(BH * W * s.V * 4);
    w.dhth = take(BH * W * s.V * 4);
    w.ds0h = take(BH * W * s.V * 4);
    w.inner = take(bwd_general_v_bytes(kslice_shape(s)));
    w.total = at;
    return w;
}
bool general_bwd_kv_ok(int64_t K, int64_t V) { return general_k_ok(K) && (V == 64 || V == 128 || V == 256 || V == 512); }

// K = 64 (the forward's padding): q, k, g with zero columns, S_0 and dht with
// zero rows; dq, dk, dg and dS_0 are the first 64 columns / rows, dv and dh
// are exact as they are.
struct GKPadBwd {
    size_t qp, kp, gp, dqp, dkp, dgp, s0p, dhtp, ds0p, inner, total;
};
GKPadBwd general_kpad_bwd_layout(const gla::Shape& s) {
    GKPadBwd w{};
    const size_t P = kGeneralMinDim, BTH = (size_t)(s.B * s.T * s.H), BH = (size_t)(s.B * s.H);
    size_t at = 0;
    auto take = [&](size_t n) { const size_t o = at; at += gla::round256(n); return o; };
    w.qp = take(BTH * P * 2);
    w.kp = take(BTH * P * 2);
    w.gp = take(BTH * P * 2);
    w.dqp = take(BTH * P * 2);
    w.dkp = take(BTH * P * 2);
    w.dgp = take(BTH * P * 2);
    w.s0p = take(BH * P * s.V * 4);
    w.dhtp = take(BH * P * s.V * 4);
    w.ds0p = take(BH * P * s.V * 4);
    w.inner = take(bwd_general_v_bytes(general_kpad_shape(s)));
    w.total = at;
    return w;
}

size_t bwd_general_any_bytes(const gla::Shape& s) {
    if (s.B * s.H == 0 || s.T == 0) return 0;
    if (s.K < kGeneralMinDim) return general_kpad_bwd_layout(s).total;
    return split_k(s) ? general_k_layout(s).total : bwd_general_v_bytes(s);
}

hipError_t bwd_general_any_launch(const gla::Shape& s, const void* q, const void* k, const void* v, const void* g,
                                  const void* h, const float* s0, const void* d_o, const float* dht, void* dq,
                                  void* dk, void* dv, void* dg, void* dh, float* ds0, void* workspace,
                                  hipStream_t strm) {
    if (s.K < kGeneralMinDim) {
        const GKPadBwd L = general_kpad_bwd_layout(s);
        const gla::Shape p = general_kpad_shape(s);
        char* ws = static_cast<char*>(workspace);
        const long K = s.K, P = p.K, rows_t = s.B * s.T * s.H, BH = s.B * s.H, KV = s.K * s.V, PV = p.K * s.V;
        hipError_t err = gla::launch_pad_cols(true, q, K, K, ws + L.qp, P, P, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_pad_cols(true, k, K, K, ws + L.kp, P, P, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_pad_cols(true, g, K, K, ws + L.gp, P, P, rows_t, strm);
        if (err == hipSuccess && s0) err = gla::launch_pad_cols(false, s0, KV, KV, ws + L.s0p, PV, PV, BH, strm);
        if (err == hipSuccess && dht) err = gla::launch_pad_cols(false, dht, KV, KV, ws + L.dhtp, PV, PV, BH, strm);
        if (err != hipSuccess) return err;
        err = bwd_general_v_launch(p, ws + L.qp, ws + L.kp, v, ws + L.gp, h, s0 ? (const float*)(ws + L.s0p) : nullptr,
                                   d_o, dht ? (const float*)(ws + L.dhtp) : nullptr, ws + L.dqp, ws + L.dkp, dv,
                                   ws + L.dgp, dh, ds0 ? (float*)(ws + L.ds0p) : nullptr, ws + L.inner, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(true, ws + L.dqp, P, 0, dq, K, 0, K, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(true, ws + L.dkp, P, 0, dk, K, 0, K, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(true, ws + L.dgp, P, 0, dg, K, 0, K, rows_t, strm);
        if (err == hipSuccess && ds0) err = gla::launch_copy_cols(false, ws + L.ds0p, PV, 0, ds0, KV, 0, KV, BH, strm);
        return err;
    }
    if (!split_k(s))
        return bwd_general_v_launch(s, q, k, v, g, h, s0, d_o, dht, dq, dk, dv, dg, dh, ds0, workspace, strm);
    const GKLayout L = general_k_layout(s);
    const gla::Shape sub = kslice_shape(s);
    char* ws = static_cast<char*>(workspace);
    const long W = sub.K, KT = s.K, rows_t = s.B * s.T * s.H;
    hipError_t err = hipSuccess;
    for (long k0 = 0; k0 < KT && err == hipSuccess; k0 += W) {
        const bool first = k0 == 0;
        err = gla::launch_copy_cols(true, q, KT, k0, ws + L.qh, W, 0, W, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(true, k, KT, k0, ws + L.kh, W, 0, W, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(true, g, KT, k0, ws + L.gh, W, 0, W, rows_t, strm);
        if (err == hipSuccess && s0) err = state_rows_out(s0, s, k0, W, ws + L.s0h, strm);
        if (err == hipSuccess && dht) err = state_rows_out(dht, s, k0, W, ws + L.dhth, strm);
        if (err != hipSuccess) break;
        err = bwd_general_v_launch(sub, ws + L.qh, ws + L.kh, v, ws + L.gh, h,
                                   s0 ? (const float*)(ws + L.s0h) : nullptr, d_o,
                                   dht ? (const float*)(ws + L.dhth) : nullptr, ws + L.dqh, ws + L.dkh,
                                   first ? dv : ws + L.dvh, ws + L.dgh, first ? dh : ws + L.dhh,
                                   ds0 ? (float*)(ws + L.ds0h) : nullptr, ws + L.inner, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(true, ws + L.dqh, W, 0, dq, KT, k0, W, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(true, ws + L.dkh, W, 0, dk, KT, k0, W, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(true, ws + L.dgh, W, 0, dg, KT, k0, W, rows_t, strm);
        if (err == hipSuccess && !first) err = gla::launch_add_into(true, dv, ws + L.dvh, rows_t * s.V, strm);
        if (err == hipSuccess && !first) err = gla::launch_add_into(true, dh, ws + L.dhh, rows_t * s.V, strm);
        if (err == hipSuccess && ds0) err = state_rows_in(ws + L.ds0h, s, k0, W, ds0, strm);
    }
    return err;
}

gla_status_t bwd_general_impl(const gla_shape_t* shape, const void* q, const void* k, const void* v,
                              const void* g, const void* h, const float* s0, const void* d_o, const float* dht,
                              void* dq, void* dk, void* dv, void* dg, void* dh, float* ds0, void* workspace,
                              size_t workspace_bytes, void* stream, const void* o = nullptr,
                              const void* ckpt = nullptr, bool want_ckpt = false) {
    g_detail.clear();
    gla::Shape s;
    gla_status_t st = check_shape(shape, &s, true);
    if (st != GLA_OK) return st;
    if (!s.bf16) return fail(GLA_ERR_UNSUPPORTED, "the general-gate path takes bf16 inputs");
    // shapes without a checkpoint (K or V outside {128, 256}, or empty): the plain
    // backward, which recomputes the forward (o and ckpt are not read)
    if (want_ckpt && general_ckpt_bytes(s) == 0) {
        want_ckpt = false;
        o = nullptr;
        ckpt = nullptr;
    }
    if (!general_bwd_kv_ok(s.K, s.V))
        return fail(GLA_ERR_UNSUPPORTED, "the general-gate backward takes K and V in {64, 128, 256, 512} (got K=%lld "
                    "V=%lld)", (long long)s.K, (long long)s.V);
    const bool empty = s.B * s.H == 0 || s.T == 0;
    if (!empty && (!q || !k || !v || !g || !h || !d_o || !dq || !dk || !dv || !dg || !dh))
        return fail(GLA_ERR_NULL, "q, k, v, g, h, d_o, dq, dk, dv, dg and dh are required");
    if (want_ckpt && !empty && (!o || !ckpt))
        return fail(GLA_ERR_NULL, "o and ckpt are required (gla_general_ckpt_size = %zu bytes)", general_ckpt_bytes(s));
    const void* ptrs[] = {q, k, v, g, h, s0, d_o, dht, dq, dk, dv, dg, dh, ds0, workspace, o, ckpt};
    const char* names[] = {"q", "k", "v", "g", "h", "s0", "d_o", "dht", "dq", "dk", "dv", "dg", "dh", "ds0",
                           "workspace", "o", "ckpt"};
    for (int i = 0; i < 17; ++i)
        if (!aligned16(ptrs[i])) return fail(GLA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    const size_t need = empty ? 0 : want_ckpt ? gla::bwd_general_layout(s).total : bwd_general_any_bytes(s);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(GLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
    hipError_t err;
    if (empty) {
        err = ds0 ? gla::launch_state_copy(dht, ds0, s.B * s.H * s.K * s.V, strm) : hipSuccess;
    } else if (want_ckpt) {
        err = bwd_general_launch(s, q, k, v, g, h, s0, d_o, dht, dq, dk, dv, dg, dh, ds0, workspace, o, ckpt, strm);
    } else {
        err = bwd_general_any_launch(s, q, k, v, g, h, s0, d_o, dht, dq, dk, dv, dg, dh, ds0, workspace, strm);
    }
    if (err != hipSuccess) return fail(GLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return GLA_OK;
}

// The backward's launches for a validated, non-empty shape with V <= 256.
hipError_t bwd_launch(const gla::Shape& s, const void* q, const void* k, const void* v, const void* g, const float* s0,
                      const void* d_o, const float* dht, void* dq, void* dk, void* dv, void* dg, float* ds0,
                      void* workspace, bool sg, const void* ckpt, hipStream_t strm) {
    hipError_t err;
    {
        gla::BwdLaunch a{};
        gla::Plan p = gla::make_bwd_plan(s);
        a.bf16 = s.bf16;
        a.sg = sg;
        a.K = (int)s.K;
        a.V = (int)s.V;
        a.BV = p.BV;
        a.BVS = gla::plan_bv(s);
        // 16-bit: the dv walk takes the forward's value width and covers each
        // segment as two halves (same workgroup count, no repeated key-side work)
        a.dv_split = gla::dv_split(s, p);
        a.BVD = a.dv_split == 2 ? a.BVS : a.BV;
        a.BVSEG = a.BVS;
        const bool ck_used = ckpt && ckpt_bytes(s) > 0;
        const int dsub = ck_used && a.dv_split == 2 && p.seg_len % 2 == 0 ? 2 : 1;
        if (ck_used) {
            // only the dS direction runs (over half segments when dsub = 2): half
            // the value width when the full width would leave CUs idle
            const long nsub = dsub == 2 ? (p.N + p.seg_len / 2 - 1) / (p.seg_len / 2) : p.P;
            const long nrev = (nsub - 1 + (a.dv_split == 2 && dsub == 1 ? 1 : 0)) * p.BH * (s.V / a.BVS);
            if (2 * nrev <= gla::kTargetWorkgroups && a.BVS >= 128) a.BVSEG = a.BVS / 2;
        }
        a.BK = p.BK;
        a.T = (int)s.T;
        a.H = (int)s.H;
        a.N = (int)p.N;
        a.P = p.P;
        a.seg_len = p.seg_len;
        a.BH = p.BH;
        a.q = q; a.k = k; a.v = v; a.g = g; a.d_o = d_o;
        a.s0 = s0; a.dht = dht;
        a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.ds0 = ds0;
        const size_t sb = gla::state_bytes(s, p);
        const size_t kk = (size_t)p.BH * p.P * s.K;
        char* ws = static_cast<char*>(workspace);
        // a checkpoint holds S_init(p) in the layout of the workspace's state area
        const bool use_ck = ckpt && ckpt_bytes(s) > 0;
        a.ckpt = use_ck;
        a.ws_state = use_ck ? const_cast<void*>(ckpt) : ws;
        a.ws_dstate = ws + sb;
        // checkpoint with the dv walk in halves: the gradients are combined at
        // every half-segment end, in the workspace's two state areas (the first
        // one is free: the states come from the checkpoint)
        a.dsub = dsub;
        if (a.dsub == 2) a.ws_dstate = ws;
        a.ws_gate = reinterpret_cast<float*>(ws + 2 * sb);
        a.ws_hs = ws + 2 * sb + gla::round256(kk * sizeof(float));
        a.ws_dp = s.bf16 ? static_cast<char*>(a.ws_hs) + gla::round256(gla::hs_bytes(s, p)) : nullptr;
        if (a.dv_split == 2) {
            char* mid = static_cast<char*>(a.ws_dp) + gla::round256((size_t)p.BH * p.N * 64 * 64 * 2);
            a.ws_dmid = mid;
            a.ws_gmid = reinterpret_cast<float*>(mid + sb);
        }
        // scalar gate: each key block's per-token sum of dg, after everything else
        if (sg) a.ws_dgp = reinterpret_cast<float*>(ws + bwd_workspace_bytes(s, false));
        // the half-segment gate totals (dsub = 2) sit in the last area of the
        // per-column layout (the scalar gate's dg partials come after it)
        if (a.dsub == 2) a.ws_gate = reinterpret_cast<float*>(ws + bwd_workspace_bytes(s, false) -
                                                             gla::round256(2 * kk * sizeof(float)));
        // checkpointed, half segments, 16-bit inputs: the dq walk forms the half
        // segments' dS* (no segment pass of its own)
        a.ds_fused = a.dsub == 2 && s.bf16 && p.BK == 64;
        a.stream = strm;
        err = gla::launch_bwd(a);
    }
    return err;
}

// 16-bit V = 512 and fp32 V = 256 or 512: the recurrence acts on each value
// column independently, so the backward is V / W backwards over column slices
// of width W (256 for 16-bit inputs, 128 for fp32) of v, d_o, S_0 and dht
// (gathered into the workspace), sharing q, k and g.  dv and dS_0 are the
// slices side by side; dq, dk and dg are the sums of the slices' values (slice
// 0 writes the caller's buffers, every later slice the workspace, then an add).
bool split_bwd(const gla::Shape& s) { return s.bf16 ? s.V == 512 : s.V > kFp32SliceV; }
long split_width(const gla::Shape& s) { return s.bf16 ? 256 : kFp32SliceV; }

struct SplitLayout {
    size_t vh, doh, dq1, dk1, dg1, dvh, s0h, dhth, ds0h, inner, total;
};
SplitLayout split_layout(const gla::Shape& s, bool sg) {
    SplitLayout w{};
    gla::Shape h = s;
    h.V = split_width(s);
    const size_t BTH = (size_t)(s.B * s.T * s.H), BH = (size_t)(s.B * s.H);
    const size_t e = s.bf16 ? 2 : 4;
    size_t at = 0;
    auto take = [&](size_t n) { const size_t o = at; at += gla::round256(n); return o; };
    w.vh = take(BTH * h.V * e);
    w.doh = take(BTH * h.V * e);
    w.dq1 = take(BTH * s.K * e);
    w.dk1 = take(BTH * s.K * e);
    w.dg1 = take(BTH * (sg ? 1 : s.K) * e);
    w.dvh = take(BTH * h.V * e);
    w.s0h = take(BH * s.K * h.V * 4);
    w.dhth = take(BH * s.K * h.V * 4);
    w.ds0h = take(BH * s.K * h.V * 4);
    w.inner = take(bwd_workspace_bytes(h, sg));
    w.total = at;
    return w;
}

hipError_t bwd_split_launch(const gla::Shape& s, const void* q, const void* k, const void* v, const void* g,
                            const float* s0, const void* d_o, const float* dht, void* dq, void* dk, void* dv, void* dg,
                            float* ds0, void* workspace, bool sg, hipStream_t strm) {
    const SplitLayout L = split_layout(s, sg);
    gla::Shape h = s;
    h.V = split_width(s);
    char* ws = static_cast<char*>(workspace);
    const long W = h.V, VT = s.V;
    const long rows_t = s.B * s.T * s.H, rows_s = s.B * s.H * s.K;
    const long n_k = rows_t * s.K, n_g = rows_t * (sg ? 1 : s.K);
    const bool b = s.bf16;
    hipError_t err = hipSuccess;
    for (long off = 0; off < VT && err == hipSuccess; off += W) {
        const bool first = off == 0;
        err = gla::launch_copy_cols(b, v, VT, off, ws + L.vh, W, 0, W, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(b, d_o, VT, off, ws + L.doh, W, 0, W, rows_t, strm);
        if (err == hipSuccess && s0) err = gla::launch_copy_cols(false, s0, VT, off, ws + L.s0h, W, 0, W, rows_s, strm);
        if (err == hipSuccess && dht)
            err = gla::launch_copy_cols(false, dht, VT, off, ws + L.dhth, W, 0, W, rows_s, strm);
        if (err != hipSuccess) break;
        err = bwd_launch(h, q, k, ws + L.vh, g, s0 ? (const float*)(ws + L.s0h) : nullptr, ws + L.doh,
                         dht ? (const float*)(ws + L.dhth) : nullptr, first ? dq : ws + L.dq1,
                         first ? dk : ws + L.dk1, ws + L.dvh, first ? dg : ws + L.dg1,
                         ds0 ? (float*)(ws + L.ds0h) : nullptr, ws + L.inner, sg, nullptr, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(b, ws + L.dvh, W, 0, dv, VT, off, W, rows_t, strm);
        if (err == hipSuccess && ds0)
            err = gla::launch_copy_cols(false, ws + L.ds0h, W, 0, ds0, VT, off, W, rows_s, strm);
        if (!first) {
            if (err == hipSuccess) err = gla::launch_add_into(b, dq, ws + L.dq1, n_k, strm);
            if (err == hipSuccess) err = gla::launch_add_into(b, dk, ws + L.dk1, n_k, strm);
            if (err == hipSuccess) err = gla::launch_add_into(b, dg, ws + L.dg1, n_g, strm);
        }
    }
    return err;
}

size_t bwd_total_bytes(const gla::Shape& s, bool sg) {
    if (s.B * s.H == 0 || s.T == 0) return 0;
    return split_bwd(s) ? split_layout(s, sg).total : bwd_workspace_bytes(s, sg);
}

hipError_t bwd_v_launch(const gla::Shape& s, const void* q, const void* k, const void* v, const void* g,
                        const float* s0, const void* d_o, const float* dht, void* dq, void* dk, void* dv, void* dg,
                        float* ds0, void* workspace, bool sg, const void* ckpt, hipStream_t strm) {
    return split_bwd(s) ? bwd_split_launch(s, q, k, v, g, s0, d_o, dht, dq, dk, dv, dg, ds0, workspace, sg, strm)
                        : bwd_launch(s, q, k, v, g, s0, d_o, dht, dq, dk, dv, dg, ds0, workspace, sg, ckpt, strm);
}

// Backward over key slices (the forward's kfwd_layout): a slice's dq, dk and
// dg are its columns of the head's; dv is the sum of the slices' (and so is
// dg for a scalar gate, which every row shares); dS_0 is the slices' row
// blocks.
struct KBwdLayout {
    size_t qh, kh, gh, dqh, dkh, dgh, dvh, s0h, dhth, ds0h, inner, total;
};
KBwdLayout kbwd_layout(const gla::Shape& s, bool sg, size_t inner_bytes) {
    KBwdLayout w{};
    const size_t W = (size_t)kslice_width(s);
    const size_t BTH = (size_t)(s.B * s.T * s.H), BH = (size_t)(s.B * s.H), e = s.bf16 ? 2 : 4;
    size_t at = 0;
    auto take = [&](size_t n) { const size_t o = at; at += gla::round256(n); return o; };
    w.qh = take(BTH * W * e);
    w.kh = take(BTH * W * e);
    w.gh = sg ? 0 : take(BTH * W * e);
    w.dqh = take(BTH * W * e);
    w.dkh = take(BTH * W * e);
    w.dgh = take(BTH * (sg ? 1 : W) * e);
    w.dvh = take(BTH * s.V * e);
    w.s0h = take(BH * W * s.V * 4);
    w.dhth = take(BH * W * s.V * 4);
    w.ds0h = take(BH * W * s.V * 4);
    w.inner = take(inner_bytes);
    w.total = at;
    return w;
}

size_t bwd_any_bytes(const gla::Shape& s, bool sg) {
    if (s.B * s.H == 0 || s.T == 0) return 0;
    if (sg_bcast(s, sg)) return 2 * bcast_gate_bytes(s) + bwd_any_bytes(s, false);
    if (!split_k(s)) return bwd_total_bytes(s, sg);
    return kbwd_layout(s, sg, bwd_total_bytes(kslice_shape(s), sg)).total;
}

// The plain and scalar-gate backward for a validated, non-empty shape.
hipError_t bwd_any_launch(const gla::Shape& s, const void* q, const void* k, const void* v, const void* g,
                          const float* s0, const void* d_o, const float* dht, void* dq, void* dk, void* dv, void* dg,
                          float* ds0, void* workspace, bool sg, const void* ckpt, hipStream_t strm) {
    if (sg_bcast(s, sg)) {
        const size_t gb = bcast_gate_bytes(s);
        const long rows_t = s.B * s.T * s.H;
        char* ws = static_cast<char*>(workspace);
        float* gk = reinterpret_cast<float*>(ws);
        float* dgk = reinterpret_cast<float*>(ws + gb);
        hipError_t err = gla::launch_bcast_cols(static_cast<const float*>(g), gk, s.K, rows_t, strm);
        if (err == hipSuccess)
            err = bwd_any_launch(s, q, k, v, gk, s0, d_o, dht, dq, dk, dv, dgk, ds0, ws + 2 * gb, false, nullptr, strm);
        if (err == hipSuccess) err = gla::launch_row_sums(dgk, s.K, static_cast<float*>(dg), rows_t, strm);
        return err;
    }
    if (!split_k(s)) return bwd_v_launch(s, q, k, v, g, s0, d_o, dht, dq, dk, dv, dg, ds0, workspace, sg, ckpt, strm);
    const gla::Shape h = kslice_shape(s);
    const KBwdLayout L = kbwd_layout(s, sg, bwd_total_bytes(h, sg));
    const long W = h.K, KT = s.K, rows_t = s.B * s.T * s.H;
    const bool b = s.bf16;
    char* ws = static_cast<char*>(workspace);
    hipError_t err = hipSuccess;
    for (long k0 = 0; k0 < KT && err == hipSuccess; k0 += W) {
        const bool first = k0 == 0;
        err = gla::launch_copy_cols(b, q, KT, k0, ws + L.qh, W, 0, W, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(b, k, KT, k0, ws + L.kh, W, 0, W, rows_t, strm);
        if (err == hipSuccess && !sg) err = gla::launch_copy_cols(b, g, KT, k0, ws + L.gh, W, 0, W, rows_t, strm);
        if (err == hipSuccess && s0) err = state_rows_out(s0, s, k0, W, ws + L.s0h, strm);
        if (err == hipSuccess && dht) err = state_rows_out(dht, s, k0, W, ws + L.dhth, strm);
        if (err != hipSuccess) break;
        err = bwd_v_launch(h, ws + L.qh, ws + L.kh, v, sg ? g : ws + L.gh, s0 ? (const float*)(ws + L.s0h) : nullptr,
                           d_o, dht ? (const float*)(ws + L.dhth) : nullptr, ws + L.dqh, ws + L.dkh,
                           first ? dv : ws + L.dvh, sg && first ? dg : ws + L.dgh,
                           ds0 ? (float*)(ws + L.ds0h) : nullptr, ws + L.inner, sg, nullptr, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(b, ws + L.dqh, W, 0, dq, KT, k0, W, rows_t, strm);
        if (err == hipSuccess) err = gla::launch_copy_cols(b, ws + L.dkh, W, 0, dk, KT, k0, W, rows_t, strm);
        if (err == hipSuccess && !sg) err = gla::launch_copy_cols(b, ws + L.dgh, W, 0, dg, KT, k0, W, rows_t, strm);
        if (err == hipSuccess && !first) err = gla::launch_add_into(b, dv, ws + L.dvh, rows_t * s.V, strm);
        if (err == hipSuccess && !first && sg) err = gla::launch_add_into(b, dg, ws + L.dgh, rows_t, strm);
        if (err == hipSuccess && ds0) err = state_rows_in(ws + L.ds0h, s, k0, W, ds0, strm);
    }
    return err;
}

gla_status_t bwd_impl(const gla_shape_t* shape, const void* q, const void* k, const void* v, const void* g,
                      const float* s0, const void* d_o, const float* dht, void* dq, void* dk, void* dv, void* dg,
                      float* ds0, void* workspace, size_t workspace_bytes, void* stream, bool sg,
                      const void* ckpt = nullptr) {
    g_detail.clear();
    gla::Shape s;
    gla_status_t st = check_shape(shape, &s, true);
    if (st != GLA_OK) return st;
    const bool empty = s.B * s.H == 0 || s.T == 0;
    if (!empty && (!q || !k || !v || !g || !d_o || !dq || !dk || !dv || !dg))
        return fail(GLA_ERR_NULL, "q, k, v, g, d_o, dq, dk, dv and dg are required");
    const void* ptrs[] = {q, k, v, g, s0, d_o, dht, dq, dk, dv, dg, ds0, workspace};
    const char* names[] = {"q", "k", "v", "g", "s0", "d_o", "dht", "dq", "dk", "dv", "dg", "ds0", "workspace"};
    for (int i = 0; i < 13; ++i)
        if (!aligned16(ptrs[i])) return fail(GLA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    const size_t need = bwd_any_bytes(s, sg);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(GLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
    hipError_t err;
    if (empty) {
        // no tokens: dS_0 = dht (the state passes through unchanged)
        err = ds0 ? gla::launch_state_copy(dht, ds0, s.B * s.H * s.K * s.V, strm) : hipSuccess;
    } else {
        err = bwd_any_launch(s, q, k, v, g, s0, d_o, dht, dq, dk, dv, dg, ds0, workspace, sg, ckpt, strm);
    }
    if (err != hipSuccess) return fail(GLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return GLA_OK;
}

// The training pair for per-column (sg = false) or per-token (sg = true) gates.
gla_status_t fwd_ckpt_impl(const gla_shape_t* shape, const void* q, const void* k, const void* v, const void* g,
                           const float* s0, void* o, float* s_final, void* ckpt, void* workspace,
                           size_t workspace_bytes, void* stream, bool sg) {
    g_detail.clear();
    gla::Shape s;
    gla_status_t st = check_shape(shape, &s, true);
    if (st != GLA_OK) return st;
    const size_t need = ckpt_bytes(s);
    if (need > 0 && !ckpt) return fail(GLA_ERR_NULL, "ckpt is required (gla_ckpt_size = %zu bytes)", need);
    if (!aligned16(ckpt)) return fail(GLA_ERR_ALIGN, "ckpt is not 16-byte aligned");
    return fwd_impl(shape, q, k, v, g, s0, o, s_final, workspace, workspace_bytes, stream, sg,
                    need > 0 ? ckpt : nullptr);
}

gla_status_t bwd_ckpt_impl(const gla_shape_t* shape, const void* q, const void* k, const void* v, const void* g,
                           const float* s0, const void* ckpt, const void* d_o, const float* dht, void* dq, void* dk,
                           void* dv, void* dg, float* ds0, void* workspace, size_t workspace_bytes, void* stream,
                           bool sg) {
    g_detail.clear();
    gla::Shape s;
    gla_status_t st = check_shape(shape, &s, true);
    if (st != GLA_OK) return st;
    const size_t need = ckpt_bytes(s);
    if (need > 0 && !ckpt) return fail(GLA_ERR_NULL, "ckpt is required (gla_ckpt_size = %zu bytes)", need);
    if (!aligned16(ckpt)) return fail(GLA_ERR_ALIGN, "ckpt is not 16-byte aligned");
    return bwd_impl(shape, q, k, v, g, s0, d_o, dht, dq, dk, dv, dg, ds0, workspace, workspace_bytes, stream, sg,
                    need > 0 ? ckpt : nullptr);
}

}  // namespace

extern "C" {

int gla_abi_version(void) { return GLA_ABI_VERSION; }

const char* gla_status_string(gla_status_t st) {
    switch (st) {
        case GLA_OK: return "GLA_OK: success";
        case GLA_ERR_NULL: return "GLA_ERR_NULL: a required pointer is NULL";
        case GLA_ERR_SHAPE: return "GLA_ERR_SHAPE: invalid problem size";
        case GLA_ERR_UNSUPPORTED: return "GLA_ERR_UNSUPPORTED: head dims, chunk or dtype not supported";
        case GLA_ERR_ALIGN: return "GLA_ERR_ALIGN: pointer not 16-byte aligned";
        case GLA_ERR_WORKSPACE: return "GLA_ERR_WORKSPACE: workspace missing or too small";
        case GLA_ERR_HIP: return "GLA_ERR_HIP: HIP runtime error";
    }
    return "unknown gla_status_t";
}

const char* gla_last_error_detail(void) { return g_detail.c_str(); }

size_t gla_fwd_workspace_size(const gla_shape_t* shape) {
    gla::Shape s;
    if (check_shape(shape, &s, false) != GLA_OK) return 0;
    return fwd_any_bytes(s, false);
}

size_t gla_bwd_workspace_size(const gla_shape_t* shape) {
    gla::Shape s;
    if (check_shape(shape, &s, true) != GLA_OK) return 0;
    return bwd_any_bytes(s, false);
}

size_t gla_fwd_scalar_workspace_size(const gla_shape_t* shape) {
    gla::Shape s;
    if (check_shape(shape, &s, false) != GLA_OK) return 0;
    return fwd_any_bytes(s, true);
}

size_t gla_bwd_scalar_workspace_size(const gla_shape_t* shape) {
    gla::Shape s;
    if (check_shape(shape, &s, true) != GLA_OK) return 0;
    return bwd_any_bytes(s, true);
}

gla_status_t gla_fwd(const gla_shape_t* shape, const void* q, const void* k, const void* v, const void* g,
                     const float* s0, void* o, float* s_final, void* workspace, size_t workspace_bytes,
                     void* stream) {
    return fwd_impl(shape, q, k, v, g, s0, o, s_final, workspace, workspace_bytes, stream, false);
}

gla_status_t gla_fwd_noalloc(const gla_shape_t* shape, const void* q, const void* k, const void* v,
                             const void* g, const float* s0, void* o, float* s_final, void* stream) {
    static_assert(GLA_NOALLOC_SCRATCH_BYTES == gla::kNoAllocScratchBytes, "one scratch size");
    g_detail.clear();
    gla::Shape s;
    // every argument is checked before the first HIP call (the scratch lookup)
    gla_status_t st = fwd_check(shape, q, k, v, g, s0, o, s_final, false, &s);
    if (st != GLA_OK) return st;
    const size_t need = fwd_any_bytes(s, false);
    if (need > gla::kNoAllocScratchBytes)
        return fail(GLA_ERR_WORKSPACE, "this shape needs %zu bytes of scratch; the fixed scratch of gla_fwd_noalloc "
                    "holds %zu (call gla_fwd with a workspace)", need, gla::kNoAllocScratchBytes);
    void* ws = nullptr;
    if (need > 0) {
        const hipError_t err = gla::noalloc_scratch(&ws);
        if (err != hipSuccess)
            return fail(GLA_ERR_HIP, "scratch address lookup failed: %s", hipGetErrorString(err));
    }
    return fwd_impl(shape, q, k, v, g, s0, o, s_final, ws, need > 0 ? gla::kNoAllocScratchBytes : 0, stream, false);
}

size_t gla_ckpt_size(const gla_shape_t* shape) {
    gla::Shape s;
    if (check_shape(shape, &s, true) != GLA_OK) return 0;
    return ckpt_bytes(s);
}

gla_status_t gla_fwd_ckpt(const gla_shape_t* shape, const void* q, const void* k, const void* v, const void* g,
                          const float* s0, void* o, float* s_final, void* ckpt, void* workspace,
                          size_t workspace_bytes, void* stream) {
    return fwd_ckpt_impl(shape, q, k, v, g, s0, o, s_final, ckpt, workspace, workspace_bytes, stream, false);
}

gla_status_t gla_bwd_ckpt(const gla_shape_t* shape, const void* q, const void* k, const void* v, const void* g,
                          const float* s0, const void* ckpt, const void* d_o, const float* dht, void* dq, void* dk,
                          void* dv, void* dg, float* ds0, void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_ckpt_impl(shape, q, k, v, g, s0, ckpt, d_o, dht, dq, dk, dv, dg, ds0, workspace, workspace_bytes,
                         stream, false);
}

gla_status_t gla_fwd_scalar_ckpt(const gla_shape_t* shape, const void* q, const void* k, const void* v,
                                 const void* g, const float* s0, void* o, float* s_final, void* ckpt,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    return fwd_ckpt_impl(shape, q, k, v, g, s0, o, s_final, ckpt, workspace, workspace_bytes, stream, true);
}

gla_status_t gla_bwd_scalar_ckpt(const gla_shape_t* shape, const void* q, const void* k, const void* v,
                                 const void* g, const float* s0, const void* ckpt, const void* d_o, const float* dht,
                                 void* dq, void* dk, void* dv, void* dg, float* ds0, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    return bwd_ckpt_impl(shape, q, k, v, g, s0, ckpt, d_o, dht, dq, dk, dv, dg, ds0, workspace, workspace_bytes,
                         stream, true);
}

gla_status_t gla_fwd_scalar(const gla_shape_t* shape, const void* q, const void* k, const void* v, const void* g,
                            const float* s0, void* o, float* s_final, void* workspace, size_t workspace_bytes,
                            void* stream) {
    return fwd_impl(shape, q, k, v, g, s0, o, s_final, workspace, workspace_bytes, stream, true);
}

size_t gla_fwd_general_workspace_size(const gla_shape_t* shape) {
    gla::Shape s;
    if (check_shape(shape, &s, false) != GLA_OK || !s.bf16 || !general_k_ok(s.K)) return 0;
    return fwd_general_any_bytes(s);
}

gla_status_t gla_fwd_general(const gla_shape_t* shape, const void* q, const void* k, const void* v, const void* g,
                             const void* h, const float* s0, void* o, float* s_final, void* workspace,
                             size_t workspace_bytes, void* stream) {
    return fwd_general_impl(shape, q, k, v, g, h, s0, o, s_final, workspace, workspace_bytes, stream);
}

size_t gla_bwd_general_workspace_size(const gla_shape_t* shape) {
    gla::Shape s;
    if (check_shape(shape, &s, true) != GLA_OK || !s.bf16 || !general_bwd_kv_ok(s.K, s.V)) return 0;
    return bwd_general_any_bytes(s);
}

gla_status_t gla_bwd_general(const gla_shape_t* shape, const void* q, const void* k, const void* v, const void* g,
                             const void* h, const float* s0, const void* d_o, const float* dht, void* dq, void* dk,
                             void* dv, void* dg, void* dh, float* ds0, void* workspace, size_t workspace_bytes,
                             void* stream) {
    return bwd_general_impl(shape, q, k, v, g, h, s0, d_o, dht, dq, dk, dv, dg, dh, ds0, workspace, workspace_bytes,
                            stream);
}

size_t gla_general_ckpt_size(const gla_shape_t* shape) {
    gla::Shape s;
    if (check_shape(shape, &s, true) != GLA_OK) return 0;
    return general_ckpt_bytes(s);
}

gla_status_t gla_fwd_general_ckpt(const gla_shape_t* shape, const void* q, const void* k, const void* v,
                                  const void* g, const void* h, const float* s0, void* o, float* s_final, void* ckpt,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    return fwd_general_impl(shape, q, k, v, g, h, s0, o, s_final, workspace, workspace_bytes, stream, ckpt, true);
}

gla_status_t gla_bwd_general_ckpt(const gla_shape_t* shape, const void* q, const void* k, const void* v,
                                  const void* g, const void* h, const float* s0, const void* o, const void* ckpt,
                                  const void* d_o, const float* dht, void* dq, void* dk, void* dv, void* dg, void* dh,
                                  float* ds0, void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_general_impl(shape, q, k, v, g, h, s0, d_o, dht, dq, dk, dv, dg, dh, ds0, workspace, workspace_bytes,
                            stream, o, ckpt, true);
}

gla_status_t gla_bwd(const gla_shape_t* shape, const void* q, const void* k, const void* v, const void* g,
                     const float* s0, const void* d_o, const float* dht, void* dq, void* dk, void* dv, void* dg,
                     float* ds0, void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_impl(shape, q, k, v, g, s0, d_o, dht, dq, dk, dv, dg, ds0, workspace, workspace_bytes, stream, false);
}

gla_status_t gla_bwd_scalar(const gla_shape_t* shape, const void* q, const void* k, const void* v, const void* g,
                            const float* s0, const void* d_o, const float* dht, void* dq, void* dk, void* dv,
                            void* dg, float* ds0, void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_impl(shape, q, k, v, g, s0, d_o, dht, dq, dk, dv, dg, ds0, workspace, workspace_bytes, stream, true);
}

}  // extern "C"

namespace {

// gate: 0 per key column, 1 one per token, 2 per key column and per value column (h)
gla_status_t decode_impl(const gla_shape_t* shape, const void* q, const void* k, const void* v, const void* g,
                         const void* h, float* state, void* o, void* stream, int gate) {
    g_detail.clear();
    gla::Shape s;
    gla_status_t st = check_decode_shape(shape, &s);
    if (st != GLA_OK) return st;
    if (s.B * s.H == 0 || s.T == 0) return GLA_OK;
    if (!q || !k || !v || !g || !state || !o) return fail(GLA_ERR_NULL, "q, k, v, g, state and o are required");
    if (gate == 2 && !h) return fail(GLA_ERR_NULL, "h is required");
    const void* ptrs[] = {q, k, v, g, state, o, h};
    const char* names[] = {"q", "k", "v", "g", "state", "o", "h"};
    for (int i = 0; i < 7; ++i)
        if (!aligned16(ptrs[i])) return fail(GLA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    gla::DecodeLaunch a{};
    a.bf16 = s.bf16;
    a.K = (int)s.K;
    a.V = (int)s.V;
    a.T = (int)s.T;
    a.H = (int)s.H;
    a.BH = s.B * s.H;
    a.gate = gate;
    a.q = q; a.k = k; a.v = v; a.g = g; a.h = h;
    a.state = state;
    a.o = o;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    const hipError_t err = gla::launch_decode(a);
    if (err != hipSuccess) return fail(GLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return GLA_OK;
}

}  // namespace

extern "C" {

gla_status_t gla_decode(const gla_shape_t* shape, const void* q, const void* k, const void* v, const void* g,
                        float* state, void* o, void* stream) {
    return decode_impl(shape, q, k, v, g, nullptr, state, o, stream, 0);
}

gla_status_t gla_decode_scalar(const gla_shape_t* shape, const void* q, const void* k, const void* v, const void* g,
                               float* state, void* o, void* stream) {
    return decode_impl(shape, q, k, v, g, nullptr, state, o, stream, 1);
}

gla_status_t gla_decode_general(const gla_shape_t* shape, const void* q, const void* k, const void* v,
                                const void* g, const void* h, float* state, void* o, void* stream) {
    return decode_impl(shape, q, k, v, g, h, state, o, stream, 2);
}

gla_status_t gla_out_gate(const gla_shape_t* shape, const void* o, const void* z, const float* ln_w,
                          const float* ln_b, float eps, void* y, void* stream) {
    g_detail.clear();
    gla::Shape s;
    gla_status_t st = check_gate_shape(shape, &s);
    if (st != GLA_OK) return st;
    if (!eps_ok(eps)) return fail(GLA_ERR_UNSUPPORTED, "eps must be finite and >= 0 (got %g)", (double)eps);
    const long R = (long)(s.B * s.T * s.H);
    if (R == 0) return GLA_OK;
    if (!o || !z || !ln_w || !y) return fail(GLA_ERR_NULL, "o, z, ln_w and y are required");
    const void* ptrs[] = {o, z, ln_w, ln_b, y};
    const char* names[] = {"o", "z", "ln_w", "ln_b", "y"};
    for (int i = 0; i < 5; ++i)
        if (!aligned16(ptrs[i])) return fail(GLA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    gla::GateLaunch a{};
    a.bf16 = s.bf16;
    a.backward = false;
    a.V = (int)s.V;
    a.R = R;
    a.o = o; a.z = z; a.w = ln_w; a.b = ln_b; a.eps = eps;
    a.y = y;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    const hipError_t err = gla::launch_out_gate(a);
    if (err != hipSuccess) return fail(GLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return GLA_OK;
}

size_t gla_out_gate_bwd_workspace_size(const gla_shape_t* shape) {
    gla::Shape s;
    if (check_gate_shape(shape, &s) != GLA_OK) return 0;
    return gla::round256((size_t)2 * gla::kGateMaxBlocks * (size_t)s.V * sizeof(float));
}

gla_status_t gla_out_gate_bwd(const gla_shape_t* shape, const void* o, const void* z, const float* ln_w,
                              const float* ln_b, float eps, const void* dy, void* d_o, void* dz, float* dln_w,
                              float* dln_b, void* workspace, size_t workspace_bytes, void* stream) {
    g_detail.clear();
    gla::Shape s;
    gla_status_t st = check_gate_shape(shape, &s);
    if (st != GLA_OK) return st;
    if (!eps_ok(eps)) return fail(GLA_ERR_UNSUPPORTED, "eps must be finite and >= 0 (got %g)", (double)eps);
    const long R = (long)(s.B * s.T * s.H);
    const size_t need = gla::round256((size_t)2 * gla::kGateMaxBlocks * (size_t)s.V * sizeof(float));
    hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
    if (R == 0) {
        // no rows: the column sums are zero (written by a kernel, not a memset,
        // so that the call can be captured in a graph)
        if (!aligned16(dln_w) || !aligned16(dln_b)) return fail(GLA_ERR_ALIGN, "dln_w or dln_b is not 16-byte aligned");
        gla::GateLaunch a{};
        a.backward = true;
        a.V = (int)s.V;
        a.R = 0;
        a.dw = dln_w; a.db = dln_b;
        a.stream = strm;
        const hipError_t err = gla::launch_out_gate(a);
        if (err != hipSuccess) return fail(GLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
        return GLA_OK;
    }
    if (!o || !z || !ln_w || !dy || !d_o || !dz)
        return fail(GLA_ERR_NULL, "o, z, ln_w, dy, d_o and dz are required");
    const void* ptrs[] = {o, z, ln_w, ln_b, dy, d_o, dz, dln_w, dln_b, workspace};
    const char* names[] = {"o", "z", "ln_w", "ln_b", "dy", "d_o", "dz", "dln_w", "dln_b", "workspace"};
    for (int i = 0; i < 10; ++i)
        if (!aligned16(ptrs[i])) return fail(GLA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    if (!workspace || workspace_bytes < need)
        return fail(GLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    gla::GateLaunch a{};
    a.bf16 = s.bf16;
    a.backward = true;
    a.V = (int)s.V;
    a.R = R;
    a.o = o; a.z = z; a.w = ln_w; a.b = ln_b; a.eps = eps;
    a.dy = dy; a.dx = d_o; a.dz = dz; a.dw = dln_w; a.db = dln_b;
    a.ws = static_cast<float*>(workspace);
    a.stream = strm;
    const hipError_t err = gla::launch_out_gate(a);
    if (err != hipSuccess) return fail(GLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return GLA_OK;
}

}  // extern "C"

namespace {
size_t bwd_workspace_bytes(const gla::Shape& s, bool sg) {
    gla::Plan p = gla::make_bwd_plan(s);
    if (p.BH == 0) return 0;
    // scalar gate: each key block's fp32 per-token sum of dg, after the rest
    const size_t dgp = sg ? gla::round256((size_t)(s.K / p.BK) * p.BH * p.N * 64 * sizeof(float)) : 0;
    const size_t kk = (size_t)p.BH * p.P * s.K;
    // 16-bit inputs: the dq walk's dP tiles for the dk walk, and (split dv
    // walk) the segments' midpoint states and half gate totals
    const size_t dp = s.bf16 ? gla::round256((size_t)p.BH * p.N * 64 * 64 * 2) : 0;
    const size_t mid = gla::dv_split(s, p) == 2 ? gla::state_bytes(s, p) + gla::round256(kk * sizeof(float)) : 0;
    // last: [BH][2P][K] fp32 half-segment gate totals of the checkpointed backward
    const size_t gsub = gla::round256(2 * kk * sizeof(float));
    return 2 * gla::state_bytes(s, p) + gla::round256(kk * sizeof(float)) + gla::round256(gla::hs_bytes(s, p)) + dp +
           mid + dgp + gsub;
}
}  // namespace
