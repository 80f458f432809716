// Backward of general gated linear attention (forget gate exp(g_t)^T exp(h_t);
// "Gated Linear Attention Transformers with Hardware-Efficient Training", the
// chapter summary's Knowl 12 and Appendix C), built from the general forward's
// kernels on three related recurrences:
//   dq_t = do_t S_t^T: the forward of the transposed state S^T, whose recurrence
//        is the general one with (do, v, k) as (q, k, v) and the gates swapped;
//   dS, the gradient with respect to S_t, runs backwards in time:
//        dS_t = q_t^T do_t + (alpha_{t+1}^T beta_{t+1}) * dS_{t+1},  dS_{T-1} also + dht,
//        a general recurrence over the reversed sequence with keys q, values do
//        and the gates shifted by one token (run in place: the general
//        forward's kernels read token T-1-t and write row T-1-t); dv_t = k_t dS_t
//        is its output for queries k, and its final state gives
//        dS_0 = (alpha_0^T beta_0) * dS_0';
//   dk_t = v_t dS_t^T: the same reversed recurrence for dS^T, queries v.
// The gate gradients take the closed forms (GLA paper Section 4.3 and the
// appendix general form), reverse cumulative sums of q*dq - k*dk and
// o*do - v*dv, within each chunk only: every chunk starts from an exact anchor
// at its end boundary (below), so rounding does not build up over the sequence.
// Everything runs in the kernels below and those of gla_fwd_wide.hip, on the
// caller's stream, with every intermediate in the caller's workspace.
#include "gla_device.hpp"
#include "gla_launch.hpp"
#include "gla_plan.hpp"
#include "gla_timing.hpp"

namespace gla {

// ds0[bh][i][j] *= exp(g[b,0,h,i] + h[b,0,h,j]): the gradient one gate further back
__global__ void __launch_bounds__(256)
gla_scale_ds0(float* __restrict__ ds0, const bf16* __restrict__ g, const bf16* __restrict__ hg, int T, int H, int K,
              int V, long n) {
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    const long KV = (long)K * V;
    const long bh = e / KV, r = e % KV;
    const int i = (int)(r / V), j = (int)(r % V);
    const long b = bh / H, h = bh % H;
    const float gi = Elem<bf16>::to_f(g[(b * T * H + h) * K + i]);
    const float hj = Elem<bf16>::to_f(hg[(b * T * H + h) * V + j]);
    ds0[e] *= __expf(gi + hj);
}

// Gate-gradient anchors at the chunk boundaries.  With dg_t the key-side gate
// gradient, dg_t = q_t*dq_t - k_t*dk_t + dg_{t+1} and, at a boundary 64m,
//   dg_{64m}[i] = sum_j (G_{64m} .* dS_{64m})[i,j] S_{64m-1}[i,j] ,
// (dh the same summed over i), with G_{64m} = alpha^T beta of token 64m; at
// m = N the term is sum_j dht S_T (no gate), and at m = 0 it is sum_j dS_0'
// S_0 with dS_0' = G_0 .* dS_0 the gradient of the initial state (blocks for
// m = 0 run only when there is an S_0: without one, dg_0 = 0).  S_{64m-1} is
// the forward walk's state before chunk m (hsf), dS_{64m} the reversed walk's
// state before its chunk N - m (hsr).
// One workgroup per (head, boundary m = 1..N): W[i][j] = alpha_i beta_j
// dS[i][j] S[i][j] over the K x V tile read as 16-byte vectors; thread
// (row group rg, column vector cv) takes rows rg, rg + RG, ... of columns
// 8cv .. 8cv+7.  Row sums reduce across the V/8 lanes of a row by shuffles,
// column sums across the row groups through LDS.
template <int V>
__global__ void __launch_bounds__(256)
gla_gate_anchor(const bf16* __restrict__ hsf, const bf16* __restrict__ hsr, const float* __restrict__ st,
                const float* __restrict__ dht, const bf16* __restrict__ g, const bf16* __restrict__ hg,
                float* __restrict__ ag, float* __restrict__ ah, int T, int H, int K,
                const float* __restrict__ s0 = nullptr, const float* __restrict__ ds0 = nullptr) {
    constexpr int CVN = V / 8, RG = 256 / CVN;
    static_assert(CVN <= 64 && (CVN & (CVN - 1)) == 0, "a row's lanes sit in one wave");
    __shared__ float alpha[256];
    __shared__ float beta[V];
    __shared__ float colp[RG][V];
    const int N = T / 64;
    const int m = blockIdx.x + (s0 ? 0 : 1);
    const long bh = blockIdx.y, b = bh / H, h = bh % H, KV = (long)K * V;
    const int tid = threadIdx.x, cv = tid % CVN, rg = tid / CVN;
    const bool last = m == N;   // S_T and dht, no gate
    const bool first = m == 0;  // S_0 and dS_0', the gate already applied
    const bool edge = last || first;
    const long tok = edge ? 0 : (b * T + 64L * m) * H + h;
    for (int i = tid; i < K; i += 256) alpha[i] = edge ? 1.f : __expf(Elem<bf16>::to_f(g[tok * K + i]));
    for (int j = tid; j < V; j += 256) beta[j] = edge ? 1.f : __expf(Elem<bf16>::to_f(hg[tok * V + j]));
    __syncthreads();
    float cs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) cs[e] = 0.f;
    const bf16* S16 = hsf + (bh * N + (edge ? 0 : m)) * KV;
    const bf16* D16 = hsr + (bh * N + (edge ? 0 : N - m)) * KV;
    const float* S32 = first ? s0 + bh * KV : st + bh * KV;
    const float* D32 = first ? ds0 + bh * KV : (dht ? dht + bh * KV : nullptr);
    // rows in groups of four: the group's loads are independent, then its four
    // row reductions (also independent) follow
    constexpr int GR = 4;
#pragma unroll 1
    for (int i0 = rg; i0 < K; i0 += GR * RG) {
        float rsum[GR];
#pragma unroll
        for (int r = 0; r < GR; ++r) {
            const int i = i0 + r * RG;
            rsum[r] = 0.f;
            if (i >= K) continue;
            float p[8];
            const long off = (long)i * V + 8 * cv;
            if (!edge) {
                const u32x4 sv = *reinterpret_cast<const u32x4*>(S16 + off);
                const u32x4 dv = *reinterpret_cast<const u32x4*>(D16 + off);
                const bf16* sx = reinterpret_cast<const bf16*>(&sv);
                const bf16* dx = reinterpret_cast<const bf16*>(&dv);
#pragma unroll
                for (int e = 0; e < 8; ++e) p[e] = Elem<bf16>::to_f(sx[e]) * Elem<bf16>::to_f(dx[e]);
            } else if (D32) {
#pragma unroll
                for (int e = 0; e < 8; ++e) p[e] = S32[off + e] * D32[off + e];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) p[e] = 0.f;
            }
            const float a = alpha[i];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float wv = a * beta[8 * cv + e] * p[e];
                rsum[r] += wv;
                cs[e] += wv;
            }
        }
#pragma unroll
        for (int r = 0; r < GR; ++r) {
            const int i = i0 + r * RG;
            float rs = rsum[r];
#pragma unroll
            for (int o = CVN / 2; o >= 1; o >>= 1) rs += __shfl_xor(rs, o, CVN);
            if (cv == 0 && i < K) ag[(bh * (N + 1) + m) * K + i] = rs;
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) colp[rg][8 * cv + e] = cs[e];
    __syncthreads();
    for (int j = tid; j < V; j += 256) {
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) acc += colp[r][j];
        ah[(bh * (N + 1) + m) * V + j] = acc;
    }
}

// out_t = the anchor of the chunk's end boundary + the chunk's own reverse
// cumulative sum of a*da - c*dc (tensors [B,T,H,D]), pinned to the anchor of
// the chunk's start boundary as well: that anchor is the exact value at the
// chunk's first token, and its mismatch delta with (end anchor + the chunk's
// whole sum) is the sum's accumulated rounding, which is spread linearly over
// the chunk (token p of 64 gets delta * (64 - p) / 64), so both ends are exact
// and the error in between is that of a path pinned at both ends rather than
// one free at the start.  The first chunk's start anchor is zero when the
// initial state is (zero_start), else the anchor of boundary 0.  One
// workgroup per chunk and head: thread (part, cv) takes
// columns 8cv .. 8cv+7 over the tokens part*TPP .. +TPP-1 with 16-byte loads,
// sums them in reverse, and adds the totals of the later parts (through LDS)
// and the anchors.
template <int D>
__device__ __forceinline__ void gate_grad_chunk(const bf16* __restrict__ a, const bf16* __restrict__ da,
                                                const bf16* __restrict__ c, const bf16* __restrict__ dc,
                                                const float* __restrict__ anchor, bf16* __restrict__ out, int T,
                                                int H, bool zero_start) {
    constexpr int CV = D / 8, NPART = 256 / CV, TPP = kChunk / NPART;
    static_assert(NPART * CV == 256 && NPART * TPP == kChunk, "gate-gradient tiling");
    __shared__ float tot[NPART][D];
    const int n = blockIdx.x, N = T / kChunk;
    const long bh = blockIdx.y, b = bh / H, h = bh % H;
    const int tid = threadIdx.x, cv = tid % CV, part = tid / CV, jv = 8 * cv;
    const long rs = (long)H * D;
    const long base = ((b * T + (long)n * kChunk + part * TPP) * H + h) * D + jv;
    float x[TPP][8];
#pragma unroll
    for (int i = 0; i < TPP; ++i) {
        const long o = base + i * rs;
        const u32x4 ra = *reinterpret_cast<const u32x4*>(a + o), rda = *reinterpret_cast<const u32x4*>(da + o);
        const u32x4 rc = *reinterpret_cast<const u32x4*>(c + o), rdc = *reinterpret_cast<const u32x4*>(dc + o);
        const bf16 *pa = reinterpret_cast<const bf16*>(&ra), *pda = reinterpret_cast<const bf16*>(&rda);
        const bf16 *pc = reinterpret_cast<const bf16*>(&rc), *pdc = reinterpret_cast<const bf16*>(&rdc);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            x[i][e] = Elem<bf16>::to_f(pa[e]) * Elem<bf16>::to_f(pda[e]) -
                      Elem<bf16>::to_f(pc[e]) * Elem<bf16>::to_f(pdc[e]);
    }
#pragma unroll
    for (int i = TPP - 2; i >= 0; --i)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[i][e] += x[i + 1][e];
#pragma unroll
    for (int e = 0; e < 8; ++e) tot[part][jv + e] = x[0][e];
    __syncthreads();
    float off[8], all[8], del[8];
    const float* an = anchor + (bh * (N + 1) + n + 1) * D + jv;
    const float* an0 = anchor + (bh * (N + 1) + n) * D + jv;  // n = 0: written only when there is an S_0
#pragma unroll
    for (int e = 0; e < 8; ++e) off[e] = all[e] = an[e];
    for (int p = 0; p < NPART; ++p)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float t = tot[p][jv + e];
            all[e] += t;
            off[e] += p > part ? t : 0.f;
        }
#pragma unroll
    for (int e = 0; e < 8; ++e) del[e] = (n > 0 || !zero_start ? an0[e] : 0.f) - all[e];
#pragma unroll
    for (int i = 0; i < TPP; ++i) {
        const float wt = (float)(kChunk - (part * TPP + i)) * (1.f / kChunk);
        alignas(16) bf16 y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = Elem<bf16>::from_f(x[i][e] + off[e] + del[e] * wt);
        *reinterpret_cast<u32x4*>(out + base + i * rs) = *reinterpret_cast<const u32x4*>(y);
    }
}

// Both gate gradients in one launch: blockIdx.z = 0 the key side (dg from q,
// dq, k, dk), 1 the value side (dh from o, d_o, v, dv).
template <int DK, int DV>
__global__ void __launch_bounds__(256)
gla_gate_grad_out(const bf16* __restrict__ q, const bf16* __restrict__ dq, const bf16* __restrict__ k,
                  const bf16* __restrict__ dk, const float* __restrict__ ag, bf16* __restrict__ dg,
                  const bf16* __restrict__ o, const bf16* __restrict__ d_o, const bf16* __restrict__ v,
                  const bf16* __restrict__ dv, const float* __restrict__ ah, bf16* __restrict__ dh, int T, int H,
                  int zero_start) {
    if (blockIdx.z == 0)
        gate_grad_chunk<DK>(q, dq, k, dk, ag, dg, T, H, zero_start != 0);
    else
        gate_grad_chunk<DV>(o, d_o, v, dv, ah, dh, T, H, zero_start != 0);
}

static FwdLaunch general_fwd_args(int B, int T, int H, int K, int V, const void* q, const void* k, const void* v,
                                  const void* g, const void* h, const float* s0, void* o, float* s_final, char* ws,
                                  void* hs, int rev, hipStream_t stream, const void* init_t = nullptr) {
    Shape s{B, T, H, K, V, true};
    Plan p = make_fwd_general_plan(s);
    FwdLaunch a{};
    a.bf16 = true;
    a.K = K; a.V = V; a.BV = p.BV;
    a.T = T; a.H = H; a.N = (int)p.N; a.P = p.P; a.seg_len = p.seg_len; a.BH = p.BH;
    a.q = q; a.k = k; a.v = v; a.g = g; a.h = h; a.s0 = s0; a.o = o; a.s_final = s_final;
    if (p.P > 1) {
        const size_t sb = state_bytes(s, p);
        a.ws_state = ws;
        a.ws_gate = reinterpret_cast<float*>(ws + sb);
        a.ws_gateb = reinterpret_cast<float*>(ws + sb + round256((size_t)p.BH * p.P * K * sizeof(float)));
    }
    a.ws_rec = ws + fwd_general_seg_bytes(s, p);
    a.ws_hs = hs;
    a.rev = rev;
    a.init_t = init_t;
    a.stream = stream;
    return a;
}

hipError_t launch_bwd_general(const BwdGeneralLaunch& L) {
    const int B = L.B, T = L.T, H = L.H, K = L.K, V = L.V;
    const long BH = (long)B * H, KV = (long)K * V;
    const BwdGeneralLayout w = bwd_general_layout(Shape{B, T, H, K, V, true});
    char* ws = static_cast<char*>(L.workspace);
    const bool ck = L.hs_in != nullptr;  // the forward's results come in
    const bf16* o = ck ? static_cast<const bf16*>(L.o_in) : reinterpret_cast<bf16*>(ws + w.o);
    const float* st = ck ? L.st_in : reinterpret_cast<float*>(ws + w.st);
    const bf16* hsf = ck ? static_cast<const bf16*>(L.hs_in) : reinterpret_cast<bf16*>(ws + w.hsf);
    bf16* hsr = reinterpret_cast<bf16*>(ws + w.hsr);
    float* ag = reinterpret_cast<float*>(ws + w.ag);
    float* ah = reinterpret_cast<float*>(ws + w.ah);
    char* fws = ws + w.fws;
    hipStream_t sm = L.stream;
    hipError_t err;
    // forward (o, S_T and the state before every chunk), unless given
    if (!ck) {
        err = launch_fwd_general(general_fwd_args(B, T, H, K, V, L.q, L.k, L.v, L.g, L.h, L.s0, ws + w.o,
                                                  reinterpret_cast<float*>(ws + w.st), fws, ws + w.hsf, 0, sm));
        if (err != hipSuccess) return err;
    }
    // dq: the transposed state's forward; its states at every chunk boundary are
    // the transposes of the forward's, so each segment starts from one of those
    // (segment 0 from S_0^T) and no state pass runs
    err = launch_fwd_general(general_fwd_args(B, T, H, V, K, L.d_o, L.v, L.k, L.h, L.g, L.s0, L.dq, nullptr, fws,
                                              nullptr, 0, sm, hsf));
    if (err != hipSuccess) return err;
    // dv and dS_0' from the time-reversed recurrence of dS (its gates one token
    // later), read and written in place in the input's token order
    // (dS_0' goes to the workspace when the caller asks for none but there is an
    // S_0: the first chunk's gate anchor is sum dS_0' S_0)
    float* ds0 = L.ds0 ? L.ds0 : (L.s0 ? reinterpret_cast<float*>(ws + w.ds0) : nullptr);
    err = launch_fwd_general(general_fwd_args(B, T, H, K, V, L.k, L.q, L.d_o, L.g, L.h, L.dht, L.dv, ds0, fws, hsr, 1, sm));
    if (err != hipSuccess) return err;
    if (ds0) {
        const long nst = BH * KV;
        GLA_LAUNCH("bwdg_scale_ds0", gla_scale_ds0, dim3((unsigned)((nst + 255) / 256)), dim3(256), sm, ds0,
                   (const bf16*)L.g, (const bf16*)L.h, T, H, K, V, nst);
    }
    // dk from the time-reversed recurrence of dS^T, whose segments start from
    // the transposes of the dv pass's states (segment 0 from dht^T)
    err = launch_fwd_general(general_fwd_args(B, T, H, V, K, L.v, L.d_o, L.q, L.h, L.g, L.dht, L.dk, nullptr, fws,
                                              nullptr, 1, sm, hsr));
    if (err != hipSuccess) return err;
    // gate gradients: anchors at the chunk boundaries, then each chunk's reverse sums
    const unsigned N = (unsigned)(T / 64);
    {
        // boundaries 1 .. N, and 0 when there is an S_0
        const dim3 ga(N + (L.s0 ? 1 : 0), (unsigned)BH);
        if (V == 128)
            GLA_LAUNCH("bwdg_gate_anchor", gla_gate_anchor<128>, ga, dim3(256), sm, (const bf16*)hsf,
                       (const bf16*)hsr, (const float*)st, L.dht, (const bf16*)L.g, (const bf16*)L.h, ag, ah, T, H, K,
                       L.s0, ds0);
        else
            GLA_LAUNCH("bwdg_gate_anchor", gla_gate_anchor<256>, ga, dim3(256), sm, (const bf16*)hsf,
                       (const bf16*)hsr, (const float*)st, L.dht, (const bf16*)L.g, (const bf16*)L.h, ag, ah, T, H, K,
                       L.s0, ds0);
    }
    const dim3 gg(N, (unsigned)BH, 2);
#define GLA_GATE_OUT(DK_, DV_)                                                                                  \
    GLA_LAUNCH("bwdg_gate_out", (gla_gate_grad_out<DK_, DV_>), gg, dim3(256), sm, (const bf16*)L.q,           \
               (const bf16*)L.dq, (const bf16*)L.k, (const bf16*)L.dk, (const float*)ag, static_cast<bf16*>(L.dg), \
               o, (const bf16*)L.d_o, (const bf16*)L.v, (const bf16*)L.dv, (const float*)ah,                      \
               static_cast<bf16*>(L.dh), T, H, L.s0 == nullptr ? 1 : 0)
    if (K == 128 && V == 128) GLA_GATE_OUT(128, 128);
    else if (K == 128) GLA_GATE_OUT(128, 256);
    else if (V == 128) GLA_GATE_OUT(256, 128);
    else GLA_GATE_OUT(256, 256);
#undef GLA_GATE_OUT
    return hipGetLastError();
}

}  // namespace gla
