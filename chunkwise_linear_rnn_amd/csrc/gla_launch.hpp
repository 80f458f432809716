// Internal interface between the ABI layer (gla_api.cpp) and the kernel
// launchers (gla_fwd.hip, gla_bwd.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

// Size of the fixed device scratch behind gla_fwd_noalloc (gla_noalloc.hip).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(void** ptr);

struct FwdLaunch {
    bool bf16;
    bool sg;  // g is one value per token and head, [B,T,H] (16-bit inputs only)
    int K, V, BV;
    int T, H, N, P, seg_len;
    long BH;
    const void *q, *k, *v, *g;
    const float* s0;
    void* o;
    float* s_final;
    void* ws_state;   // [BH][P][K][V] in the input dtype
    float* ws_gate;   // [BH][P][K]    fp32 (log2 of the segment decay)
    void* ws_rec;     // [BH][N] chunk records of the wide-head forward
    const void* h;    // general gates: log beta, [B,T,H,V] (null otherwise)
    float* ws_gateb;  // general gates: [BH][P][V] fp32 (log2 of the segment's column decay)
    void* ws_hs;      // general gates, optional: the state before every chunk, [BH][N][K][V] bf16
    int rev;          // general gates: run the time-reversed sequence in place (token t = input token T-1-t,
                      // its gate the input's gate of token T-t, none at t = 0; o written at row T-1-t)
    float* s_final2;     // general gates, optional: S_T also here (the forward's checkpoint)
    const void* init_t;  // general gates, optional: the state before every chunk of the transposed recurrence,
                         // [BH][N][V][K] bf16; segments start from its transposes (s0 then also given as
                         // [V][K]) and no state pass or combine runs
    void* ckpt;       // optional: the state before every ck_len-th chunk, [BH][ck_P][K][V] input dtype
    int ck_len, ck_P;
    hipStream_t stream;
};

struct BwdLaunch {
    bool bf16;
    bool sg;  // g and dg are one value per token and head, [B,T,H] (16-bit inputs only)
    int K, V, BV, BK;
    int BVS;  // value columns per workgroup of the forward's segment-state pass
    int BVSEG;  // value columns per workgroup of the backward's segment-state pass
    int BVD;  // value columns per workgroup of the dv walk
    int dv_split;  // 2: the dv walk takes each segment in two halves (from the midpoint states)
    bool ds_fused;  // the dq walk forms the half segments' dS* (checkpointed, dsub = 2, 16-bit, per-column gates)
    int T, H, N, P, seg_len;
    long BH;
    const void *q, *k, *v, *g, *d_o;
    const float *s0, *dht;
    void *dq, *dk, *dv, *dg;
    float* ds0;
    void* ws_state;    // [BH][P][K][V] input dtype: S*_p, then S_init(p)
    void* ws_dstate;   // [BH][P][K][V] input dtype: dS*_p, then dS_end(p)
    float* ws_gate;    // [BH][P][K]
    void* ws_hs;       // [BH][N][K*V] dtype: state after every chunk, in the walks' tile order
    void* ws_dp;       // [BH][N][64][64] dtype (16-bit inputs): each chunk's dP = dO V^T, [t][s]
    void* ws_dmid;     // [BH][P][K][V] dtype (dv_split == 2): local dS* of each segment's second half
    float* ws_gmid;    // [BH][P][K] fp32: that half's gate total (log2)
    float* ws_dgp;     // scalar gate: [K/BK][BH*T] fp32, each key block's sum of dg over its columns
    bool ckpt;         // ws_state already holds S_init(p) (a checkpointing forward's): only dS is combined
    int dsub;          // 2 (checkpoint, dv walk in halves, even seg_len): ws_dstate holds [BH][2P][K][V],
                       // the combined gradient at every half-segment end, and ws_gate [BH][2P][K]
    hipStream_t stream;
};

struct DecodeLaunch {
    bool bf16;
    int K, V, T, H;
    long BH;
    int gate;  // 0: g per key column [B,T,H,K]; 1: one g per token [B,T,H]; 2: g per key column and h per value column
    const void *q, *k, *v, *g, *h;
    float* state;  // [BH][K][V] fp32, read and written in place
    void* o;
    hipStream_t stream;
};

hipError_t launch_fwd(const FwdLaunch& a);
hipError_t launch_fwd_wide(const FwdLaunch& a);
hipError_t launch_fwd_general(const FwdLaunch& a);

// general-gate backward (bf16): inputs, outputs and the caller's workspace
struct BwdGeneralLaunch {
    int B, T, H, K, V;
    const void *q, *k, *v, *g, *h, *d_o;
    const float *s0, *dht;
    void *dq, *dk, *dv, *dg, *dh;
    float* ds0;
    // optional, all three or none: the forward's output o, its state before every
    // chunk [BH][N][K][V] bf16 and S_T [BH][K][V]; the backward then runs no forward
    const void* o_in;
    const void* hs_in;
    const float* st_in;
    void* workspace;
    hipStream_t stream;
};
hipError_t launch_bwd_general(const BwdGeneralLaunch& a);  // 16-bit, K = 256
hipError_t launch_decode(const DecodeLaunch& a);
hipError_t launch_bwd(const BwdLaunch& a);
hipError_t launch_state_copy(const float* src, float* dst, long n, hipStream_t stream);
// dst[r][off_d + c] = src[r][off_s + c], c < W, r < rows (bf16 or fp32; 16-byte multiples)
hipError_t launch_copy_cols(bool bf16, const void* src, long ld_s, long off_s, void* dst, long ld_d, long off_d, long W,
                            long rows, hipStream_t stream);
hipError_t launch_add_into(bool bf16, void* a, const void* b, long n, hipStream_t stream);  // a += b (bf16 or fp32)
// dst[r][c] = c < W_src ? src[r][c] : 0, c < W_dst (bf16 or fp32; 16-byte multiples)
hipError_t launch_pad_cols(bool bf16, const void* src, long ld_s, long W_src, void* dst, long ld_d, long W_dst,
                           long rows, hipStream_t stream);
hipError_t launch_bcast_cols(const float* src, float* dst, long W, long rows, hipStream_t stream);  // dst[r][:] = src[r]
hipError_t launch_row_sums(const float* src, long W, float* dst, long rows, hipStream_t stream);    // dst[r] = sum src[r][:]

}  // namespace gla
