/*
 * gla.h -- C ABI of the MI355X (gfx950) chunkwise gated linear attention library.
 *
 * The operator is the gated linear attention recurrence of "Gated Linear
 * Attention Transformers with Hardware-Efficient Training" (Yang, Wang, Shen,
 * Panda, Kim), Section 4.1, Eq. 3, per head:
 *
 *     S_t = Diag(alpha_t) S_{t-1} + k_t^T v_t ,     o_t = q_t S_t ,
 *
 * with the forget gate passed in log space, g_t = log(alpha_t) <= 0, and the
 * initial state S_0 either zero or a caller-supplied state carried over from an
 * earlier segment of the sequence (Section 2.2).  The library computes it in
 * the chunkwise form of Section 4.2 (chunk C = 64) with the secondary
 * sub-chunking of Section 4.3 (sub-chunk c = 16), on hand-written HIP kernels.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layout (row-major, fully contiguous, no padding):
 *      q, k, g, dq, dk, dg        [B, T, H, K]
 *      v, o, d_o, dv              [B, T, H, V]
 *      s0, s_final, dht, ds0      [B, H, K, V]   (always float32)
 *  dtype: GLA_DTYPE_BF16 or GLA_DTYPE_FP32 applies to q, k, v, g, o, d_o and
 *      to the gradients dq, dk, dv, dg.  Accumulation is always float32.
 *  Pointers are DEVICE pointers (hipMalloc'd or equivalent), 16-byte aligned.
 *  Ownership: the caller allocates every buffer including the workspace; the
 *      library allocates nothing, frees nothing and keeps no pointer after
 *      the call returns.
 *  Execution: stream-ordered and asynchronous.  A call validates its
 *      arguments on the host, then only enqueues kernels on `stream` (a
 *      hipStream_t; NULL = the default stream) and returns.  Inputs must stay
 *      alive and unmodified until the stream has passed the call.  Results are
 *      deterministic: no atomics take part in any sum.
 *  Errors: every argument is validated before anything is enqueued, so on
 *      any error other than GLA_ERR_HIP nothing has been launched.  Detail
 *      text for the last error of the calling thread is available from
 *      gla_last_error_detail().  No C++ exception crosses this interface.
 *  Preconditions not checked (checking would cost a pass over the data):
 *      all inputs finite and g <= 0 (alpha in (0, 1], as the gate's
 *      definition in Section 4.1 requires; g = 0 is ungated linear attention,
 *      Eq. 1).  Violations give unspecified values, never an out-of-bounds
 *      access.
 *  Supported sizes: chunk == 64; T a multiple of 64; K and V in {64, 128,
 *      256, 512}, bf16 or fp32.  Heads wider than the kernels run as slices
 *      whose staging copies sit in the workspace: value slices (the
 *      recurrence never mixes value columns: the 16-bit backward at V = 512
 *      in two slices of 256, fp32 at V = 256 and 512 in slices of 128) and key
 *      slices (Diag(alpha_t) never mixes state rows and o_t sums over them:
 *      16-bit K = 512 in two slices of 256, fp32 K = 256 and 512 in slices of
 *      128; the slices' outputs and dv add).  B, H >= 0 and T >= 0; B*H == 0 or T == 0
 *      is a valid no-op (s_final is then s0, or zero; ds0 is dht, or zero).
 *  Size limits (GLA_ERR_SHAPE beyond them; the kernels index in 32 bits):
 *      B*H <= 2^20 heads, B*H*T < 2^30 token-heads (larger inputs would not
 *      fit in one GPU's memory), H*max(K, V) < 2^25 (a chunk's 64 rows of
 *      row stride); decode: B*H*V/64 < 2^24; the output gate: B*H*T < 2^31
 *      rows.
 */
#ifndef GLA_H_
#define GLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GLA_ABI_VERSION 1

typedef enum {
    GLA_OK = 0,
    GLA_ERR_NULL = 1,        /* a required pointer is NULL                          */
    GLA_ERR_SHAPE = 2,       /* negative size, T not a multiple of the chunk, or a
                                size past the limits above                          */
    GLA_ERR_UNSUPPORTED = 3, /* K, V, chunk or dtype outside the supported set      */
    GLA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                    */
    GLA_ERR_WORKSPACE = 5,   /* workspace smaller than the *_workspace_size() value */
    GLA_ERR_HIP = 6          /* the HIP runtime rejected a launch (see detail text) */
} gla_status_t;

typedef enum { GLA_DTYPE_FP32 = 0, GLA_DTYPE_BF16 = 1 } gla_dtype_t;

/* Problem description.  chunk must be 64 (the chunk size C of Section 4.2). */
typedef struct {
    int64_t B, T, H, K, V;
    int64_t chunk;
    int32_t dtype; /* gla_dtype_t */
    int32_t reserved; /* must be 0 */
} gla_shape_t;

/*
 * gla_fwd -- forward pass (Section 4.2 chunkwise form of Eq. 3).
 *   q, k, g : [B,T,H,K] dtype        (g = log forget gate, <= 0)
 *   v       : [B,T,H,V] dtype
 *   s0      : [B,H,K,V] float32 initial state, or NULL for a zero state
 *   o       : [B,T,H,V] dtype output, o_t = q_t S_t (S_t after token t)
 *   s_final : [B,H,K,V] float32 final state S_T, or NULL to skip
 *   workspace / workspace_bytes : device scratch of at least
 *             gla_fwd_workspace_size(shape) bytes (may be NULL when that is 0)
 *   stream  : hipStream_t to enqueue on (NULL = default stream)
 * Returns GLA_OK or an error code (see above).
 */
gla_status_t gla_fwd(const gla_shape_t* shape,
                     const void* q, const void* k, const void* v, const void* g,
                     const float* s0, void* o, float* s_final,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace gla_fwd needs for `shape` (0 for an invalid shape).
 * A pure function of the shape: it makes no HIP call.  It holds the sequence
 * segments' states and log-decays (B*H*P*K*V elements in the input dtype plus
 * B*H*P*K floats, P <= T/64), and for 16-bit inputs with K = 256 also one
 * 77056-byte record of prepared chunk operands per chunk and head
 * (B*H*T/64 records: about 1.2 KB per token and head).  Heads run as slices
 * (16-bit K = 512; fp32 K or V above 128) add the staging copies of one slice
 * (its q, k, g columns or v columns, its partial output and state rows) in
 * front of the slice's own workspace. */
size_t gla_fwd_workspace_size(const gla_shape_t* shape);

/*
 * gla_fwd_noalloc -- gla_fwd for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The arguments, results, validation and errors are gla_fwd's,
 * without the workspace: the forward's scratch (segment states and segment
 * gate totals) lives in a fixed device array inside the library,
 * GLA_NOALLOC_SCRATCH_BYTES per GPU, which that GPU holds until the process
 * ends.  The call allocates nothing (no hipMalloc, no library allocation).
 *  - Shapes whose gla_fwd_workspace_size() exceeds GLA_NOALLOC_SCRATCH_BYTES
 *    return GLA_ERR_WORKSPACE before anything is enqueued (16-bit heads with
 *    K = 256, whose forward keeps per-chunk records, always need gla_fwd).
 *  - Every call on one GPU uses that GPU's single array, and its contents
 *    are whatever the last call left (nothing in it needs to start at zero).
 *    Calls that overlap on one GPU -- on different streams, or from several
 *    threads without ordering them on one stream -- race on the array and
 *    give wrong results; order them.
 *  - The first call on each device looks up the array's address on that
 *    device (hipGetSymbolAddress, the device current at the call); a failure
 *    there is GLA_ERR_HIP.
 */
#define GLA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
gla_status_t gla_fwd_noalloc(const gla_shape_t* shape,
                             const void* q, const void* k, const void* v, const void* g,
                             const float* s0, void* o, float* s_final, void* stream);

/*
 * gla_bwd -- gradients of the loss L = <o, d_o> + <S_T, dht> with respect to
 * q, k, v, g and S_0, for the same forward as gla_fwd.  States are recomputed
 * (Section 3.3: hidden states are discarded after the forward pass and
 * recomputed in the backward pass).  The gate gradient uses the closed form of
 * Section 4.3, dlog b_t = q_t*dq_t - k_t*dk_t, dg_t = sum_{i>=t} dlog b_i, plus
 * the final-state term sum_j S_T[i,j] dht[i,j] added to every dg_t.
 *   q, k, g, v, s0 : as for gla_fwd (s0 may be NULL)
 *   d_o     : [B,T,H,V] dtype upstream gradient of o
 *   dht     : [B,H,K,V] float32 gradient of S_T, or NULL for zero
 *             (truncated BPTT passes no gradient across segments, Section 5.2)
 *   dq, dk, dg : [B,T,H,K] dtype outputs;  dv : [B,T,H,V] dtype output
 *   ds0     : [B,H,K,V] float32 gradient of S_0, or NULL to skip
 *   workspace : at least gla_bwd_workspace_size(shape) bytes
 * Returns GLA_OK or an error code.
 */
gla_status_t gla_bwd(const gla_shape_t* shape,
                     const void* q, const void* k, const void* v, const void* g,
                     const float* s0, const void* d_o, const float* dht,
                     void* dq, void* dk, void* dv, void* dg, float* ds0,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace gla_bwd needs for `shape` (0 for an invalid shape; no
 * HIP call).  It holds the segment states and gradients, the backward's chunk
 * anchors and the dP tiles handed from the dq walk to the dk walk; heads run as
 * slices (16-bit V = 512 or K = 512, fp32 K or V above 128) add one slice's staging
 * copies and partial gradients in front of the slice's own workspace. */
size_t gla_bwd_workspace_size(const gla_shape_t* shape);

/*
 * Checkpointed training pair: gla_fwd_ckpt + gla_bwd_ckpt.
 * Section 3.3 weighs materialising the hidden states in the forward pass
 * against recomputing them in the backward pass.  This pair keeps a small
 * part: the state at the start of each sequence segment the backward splits a
 * head into (one K x V state per segment), written by the forward's segment
 * combine (or, when such a start is not one of the forward's own segment
 * starts, by the forward walk as it passes that chunk boundary).  The backward
 * then recomputes every chunk state
 * inside its segments from those starting states (instead of first running
 * its own pass over k, v and g to find them); everything else is gla_bwd.
 *   gla_ckpt_size(shape) : bytes of the checkpoint, [B,H,P,K,V] in the
 *     token dtype (P = the backward's segment count; entry 0 of each head is
 *     not written: segment 0 starts from s0).  0 when the shape has no
 *     checkpoint: fp32 inputs, K above 128, V = 512, a single segment, or an
 *     invalid or empty shape; both calls then behave exactly like gla_fwd /
 *     gla_bwd and ckpt may be NULL.  The shape must be a valid backward shape.
 *   gla_fwd_ckpt : gla_fwd (same arguments, results and workspace), plus
 *     writes ckpt (device, caller-owned, 16-byte aligned).
 *   gla_bwd_ckpt : gla_bwd (same arguments, results and workspace), plus
 *     reads ckpt, which must hold what gla_fwd_ckpt wrote for the same shape,
 *     q, k, v, g and s0, unmodified since.  A checkpoint from other inputs
 *     gives wrong gradients (it is not checked).
 * Errors: as gla_fwd / gla_bwd; GLA_ERR_NULL for a NULL ckpt when
 * gla_ckpt_size(shape) > 0, GLA_ERR_ALIGN for a misaligned one.
 */
size_t gla_ckpt_size(const gla_shape_t* shape);
gla_status_t gla_fwd_ckpt(const gla_shape_t* shape,
                          const void* q, const void* k, const void* v, const void* g,
                          const float* s0, void* o, float* s_final, void* ckpt,
                          void* workspace, size_t workspace_bytes, void* stream);
gla_status_t gla_bwd_ckpt(const gla_shape_t* shape,
                          const void* q, const void* k, const void* v, const void* g,
                          const float* s0, const void* ckpt, const void* d_o, const float* dht,
                          void* dq, void* dk, void* dv, void* dg, float* ds0,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * gla_fwd_scalar / gla_bwd_scalar -- the same operator with a scalar forget
 * gate per token and head, alpha_t = exp(g_t) * 1 (every key column decays
 * alike: the data-dependent decay of Mamba-2 and the gated retention form,
 * the scalar-decay special case of Eq. 3 discussed with Eq. 1 and Section 4.1).
 * Intra-chunk attention is then a masked product with a rank-one decay mask,
 * and each chunk needs one cumulative gate per token instead of one per key
 * column, which the kernels exploit (one scan and two exponentials per token).
 *   g  : [B,T,H] dtype (instead of [B,T,H,K]), g <= 0
 *   dg : [B,T,H] dtype output of gla_bwd_scalar, the gradient with respect to
 *        the scalar log gate (the sum over key columns of the per-column one)
 * Every other argument, layout and convention is that of gla_fwd / gla_bwd.
 * bf16 or fp32.  fp32 runs the per-column path on the gate repeated over the
 * key columns (exactly the same gate) and sums its per-column dg, so its
 * workspace also holds the repeated gate and that dg ([B,T,H,K] fp32 each).
 * gla_fwd_scalar takes gla_fwd_scalar_workspace_size(shape) bytes of workspace
 * (equal to gla_fwd_workspace_size for bf16); gla_bwd_scalar takes
 * gla_bwd_scalar_workspace_size(shape).  Both sizes are 0 for an invalid or
 * empty shape.
 */
gla_status_t gla_fwd_scalar(const gla_shape_t* shape,
                            const void* q, const void* k, const void* v, const void* g,
                            const float* s0, void* o, float* s_final,
                            void* workspace, size_t workspace_bytes, void* stream);
gla_status_t gla_bwd_scalar(const gla_shape_t* shape,
                            const void* q, const void* k, const void* v, const void* g,
                            const float* s0, const void* d_o, const float* dht,
                            void* dq, void* dk, void* dv, void* dg, float* ds0,
                            void* workspace, size_t workspace_bytes, void* stream);
size_t gla_fwd_scalar_workspace_size(const gla_shape_t* shape);
size_t gla_bwd_scalar_workspace_size(const gla_shape_t* shape);

/*
 * The training pair of the scalar gate: gla_fwd_ckpt / gla_bwd_ckpt (above) with
 * g and dg [B,T,H] as for gla_fwd_scalar / gla_bwd_scalar.  The checkpoint has the
 * layout and size of gla_ckpt_size(shape) and the same contract (written by
 * gla_fwd_scalar_ckpt, read unmodified by gla_bwd_scalar_ckpt for the same inputs);
 * shapes without one (gla_ckpt_size == 0: fp32, K > 128, V > 256, a single
 * backward segment) run the plain pair.  Workspaces: gla_fwd_scalar_workspace_size
 * and gla_bwd_scalar_workspace_size.  Errors: as gla_fwd_scalar / gla_bwd_scalar,
 * plus GLA_ERR_NULL for a NULL ckpt the shape needs and GLA_ERR_ALIGN for a
 * misaligned one.
 */
gla_status_t gla_fwd_scalar_ckpt(const gla_shape_t* shape,
                                 const void* q, const void* k, const void* v, const void* g,
                                 const float* s0, void* o, float* s_final, void* ckpt,
                                 void* workspace, size_t workspace_bytes, void* stream);
gla_status_t gla_bwd_scalar_ckpt(const gla_shape_t* shape,
                                 const void* q, const void* k, const void* v, const void* g,
                                 const float* s0, const void* ckpt, const void* d_o, const float* dht,
                                 void* dq, void* dk, void* dv, void* dg, float* ds0,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * gla_fwd_general -- forward pass of general gated linear attention, whose
 * forget gate is an outer product G_t = alpha_t^T beta_t of a key-side gate
 * alpha_t = exp(g_t) and a value-side gate beta_t = exp(h_t) ("Gated Linear
 * Attention Transformers with Hardware-Efficient Training", the chapter
 * summary's Knowl 12 and Appendix C):
 *     S_t = (alpha_t^T beta_t) .* S_{t-1} + k_t^T v_t ,   o_t = q_t S_t .
 * h = 0 gives gla_fwd.  Chunkwise: per chunk, with B_t / C_t the cumulative
 * log2 gates of the key / value columns, the output is
 * (q_t exp2(B_t)) S exp2(C_t) plus the intra-chunk term, and the state's rows
 * and columns decay by exp2(B_63) and exp2(C_63).
 *   q, k, g : [B,T,H,K] bf16   (g <= 0)
 *   v, h    : [B,T,H,V] bf16   (h = log beta <= 0)
 *   s0, o, s_final, stream : as for gla_fwd
 *   workspace : at least gla_fwd_general_workspace_size(shape) bytes
 * bf16 with K in {128, 256, 512} (512 as two key slices of 256 that share v
 * and h, their outputs added) and V in {64, 128, 256, 512}; other shapes and
 * fp32 return GLA_ERR_UNSUPPORTED.  Results are deterministic.  The backward is
 * gla_bwd_general.
 */
gla_status_t gla_fwd_general(const gla_shape_t* shape,
                             const void* q, const void* k, const void* v, const void* g,
                             const void* h, const float* s0, void* o, float* s_final,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace gla_fwd_general needs (0 for fp32, K = 64 or an invalid
 * shape; no HIP call).  At K = 512 the key slice's q, k, g, partial output and
 * state rows, then the K = 256 workspace.  Segment states and the segments' key-row and
 * value-column log-decays, and one record per chunk and head of
 * 268 K + 392 V + 8704 bytes (prepared key-side operands and A, v * exp2(C_63 - C_t),
 * exp2(C_t), the intra-chunk output (kept only where the walk cannot form it) and the
 * column decays). */
size_t gla_fwd_general_workspace_size(const gla_shape_t* shape);

/*
 * gla_bwd_general -- gradients of L = <o, d_o> + <S_T, dht> for gla_fwd_general
 * with respect to q, k, v, both log gates g and h, and S_0.  States are
 * recomputed.  dq is the output of the transposed state's recurrence
 * (S_t^T = (beta_t^T alpha_t) .* S_{t-1}^T + v_t^T k_t, queried by do); dv and dk
 * are the outputs of the gradient dS_t and of dS_t^T, which follow the general
 * recurrence backwards in time with the gates one token later; the gate
 * gradients take the closed forms of Section 4.3 and the appendix general form,
 * dg_t = sum_{s>=t} (q_s*dq_s - k_s*dk_s) + sum_j S_T[i,j] dht[i,j] and
 * dh_t = sum_{s>=t} (o_s*do_s - v_s*dv_s) + sum_i S_T[i,j] dht[i,j].
 *   q, k, g, v, h, s0 : as for gla_fwd_general;  d_o, dht : as for gla_bwd
 *   dq, dk, dg : [B,T,H,K] bf16;  dv, dh : [B,T,H,V] bf16;  ds0 : [B,H,K,V] fp32 or NULL
 *   workspace : at least gla_bwd_general_workspace_size(shape) bytes
 * bf16 with K and V in {128, 256, 512}; 512 runs as two slices of 256: key
 * slices share v and h (dq, dk, dg side by side, dv and dh added), value
 * slices share q, k and g (dv, dh side by side, dq, dk, dg added).  Other
 * shapes and fp32 return GLA_ERR_UNSUPPORTED.  Results are deterministic.
 */
gla_status_t gla_bwd_general(const gla_shape_t* shape,
                             const void* q, const void* k, const void* v, const void* g,
                             const void* h, const float* s0, const void* d_o, const float* dht,
                             void* dq, void* dk, void* dv, void* dg, void* dh, float* ds0,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace gla_bwd_general needs (0 for an unsupported or
 * invalid shape; no HIP call): the forward's o and S_T, the states before every
 * chunk of the forward and of the time-reversed dS recurrence, the gate-gradient
 * anchors and the general forward's workspace.  The time-reversed recurrences
 * read q, k, v, d_o and the gates in place.  At K or V = 512, the slices'
 * gathered inputs and partial gradients come first. */
size_t gla_bwd_general_workspace_size(const gla_shape_t* shape);

/*
 * General-gate training pair: gla_fwd_general_ckpt + gla_bwd_general_ckpt.
 * gla_bwd_general recomputes the forward for the output o (in the closed form
 * of dh) and for the state before every chunk (the gate-gradient anchors at the
 * chunk boundaries).  This pair keeps them instead (Section 3.3's
 * materialisation side): the forward also writes its state before every chunk
 * and S_T into a caller-owned checkpoint, and the backward takes that and the
 * forward's o and runs no forward.
 *   gla_general_ckpt_size(shape) : bytes of the checkpoint, the states
 *     [B,H,T/64,K,V] bf16 (entry 0 of each head is not used), then S_T
 *     [B,H,K,V] fp32 at a 256-byte aligned offset; 0 for an empty or invalid
 *     shape and for one without a checkpoint (K or V outside {128, 256}): both
 *     calls then behave exactly like gla_fwd_general / gla_bwd_general, and
 *     ckpt (and the backward's o) may be NULL.
 *   gla_fwd_general_ckpt : gla_fwd_general (same arguments, results and
 *     workspace), plus, for bf16 with K and V in {128, 256}, writes ckpt (device,
 *     16-byte aligned, required unless the shape is empty).
 *   gla_bwd_general_ckpt : gla_bwd_general (same arguments, results and
 *     workspace), plus reads o and ckpt, which must hold what
 *     gla_fwd_general_ckpt returned for the same shape, q, k, v, g, h and s0,
 *     unmodified since (not checked: other contents give wrong gradients).
 * Errors: as gla_fwd_general / gla_bwd_general; GLA_ERR_NULL for a NULL o or
 * ckpt on a shape with a checkpoint, GLA_ERR_ALIGN for a misaligned one.
 */
size_t gla_general_ckpt_size(const gla_shape_t* shape);
gla_status_t gla_fwd_general_ckpt(const gla_shape_t* shape,
                                  const void* q, const void* k, const void* v, const void* g,
                                  const void* h, const float* s0, void* o, float* s_final, void* ckpt,
                                  void* workspace, size_t workspace_bytes, void* stream);
gla_status_t gla_bwd_general_ckpt(const gla_shape_t* shape,
                                  const void* q, const void* k, const void* v, const void* g,
                                  const void* h, const float* s0, const void* o, const void* ckpt,
                                  const void* d_o, const float* dht,
                                  void* dq, void* dk, void* dv, void* dg, void* dh, float* ds0,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * gla_decode -- the recurrent form of Eq. 3 (Section 3.1), for token-by-token
 * inference with the state carried between calls: for t = 1..T,
 *     S <- Diag(exp g_t) S + k_t^T v_t ,   o_t = q_t S ,
 * starting from and ending in `state`.  O(K V) work per token and head, no
 * chunking, so T need not be a multiple of 64 (shape.chunk is not used; it is
 * meant for a few tokens per call, the state staying on chip between them).
 *   q, k, g : [B,T,H,K] dtype;  v : [B,T,H,V] dtype
 *   state   : [B,H,K,V] float32, read and overwritten in place (required)
 *   o       : [B,T,H,V] dtype output
 *   stream  : as for gla_fwd.  No workspace.
 * Supported: K and V in {64, 128, 256, 512}, bf16 or fp32.
 * T == 0 or B*H == 0 is a no-op.  Returns GLA_OK or an error code.
 */
gla_status_t gla_decode(const gla_shape_t* shape,
                        const void* q, const void* k, const void* v, const void* g,
                        float* state, void* o, void* stream);

/*
 * gla_decode_scalar / gla_decode_general -- gla_decode for the other two gate
 * forms of the chunked paths (same arguments, sizes, state contract and errors):
 *   gla_decode_scalar  : g is [B,T,H] dtype, one log gate per token and head
 *                        (alpha_t = exp(g_t) times the all-ones row, as for
 *                        gla_fwd_scalar);
 *   gla_decode_general : g is [B,T,H,K] and h is [B,T,H,V] dtype (required,
 *                        16-byte aligned), S <- (exp(g_t)^T exp(h_t)) .* S +
 *                        k_t^T v_t, as for gla_fwd_general.
 */
gla_status_t gla_decode_scalar(const gla_shape_t* shape,
                               const void* q, const void* k, const void* v, const void* g,
                               float* state, void* o, void* stream);
gla_status_t gla_decode_general(const gla_shape_t* shape,
                                const void* q, const void* k, const void* v, const void* g, const void* h,
                                float* state, void* o, void* stream);

/*
 * gla_out_gate -- the output epilogue of the multi-head GLA layer (Section 4.4,
 * "GLA Transformer"): every head's output row is normalised by LayerNorm on its
 * own, then multiplied elementwise by the Swish output gate r = Swish(z),
 *     y[b,t,h,:] = Swish(z[b,t,h,:]) * (LN(o[b,t,h,:]) * ln_w + ln_b),
 *     LN(x) = (x - mean(x)) / sqrt(var(x) + eps)   (mean and biased variance
 *             over the row's V channels),   Swish(z) = z / (1 + exp(-z)).
 * z is the gate's pre-activation x W_r + b_r; that projection is a plain GEMM
 * and not part of this call.  Only B, T, H, V and dtype of `shape` are used
 * (K and chunk are ignored; T need not be a multiple of 64).
 *   o, z    : [B,T,H,V] dtype inputs;  y : [B,T,H,V] dtype output
 *   ln_w    : [V] float32 scale shared by the heads (required)
 *   ln_b    : [V] float32 shift, or NULL for zero
 *   eps     : finite, >= 0 (a row with zero variance and eps == 0 gives
 *             non-finite values)
 *   stream  : as for gla_fwd.  No workspace.
 * Supported: V in {64, 128, 256, 512}, bf16 or fp32.  B*T*H == 0 is a no-op.
 * Returns GLA_OK or an error code.
 */
gla_status_t gla_out_gate(const gla_shape_t* shape, const void* o, const void* z,
                          const float* ln_w, const float* ln_b, float eps, void* y, void* stream);

/*
 * gla_out_gate_bwd -- gradients of <y, dy> for gla_out_gate with respect to o,
 * z, ln_w and ln_b.  The ln_w and ln_b gradients are sums over all B*T*H rows,
 * formed per workgroup and then added in a fixed order (deterministic).
 *   o, z, ln_w, ln_b, eps : as for gla_out_gate
 *   dy      : [B,T,H,V] dtype upstream gradient of y
 *   d_o, dz : [B,T,H,V] dtype outputs (required)
 *   dln_w, dln_b : [V] float32 outputs, either may be NULL to skip
 *   workspace : at least gla_out_gate_bwd_workspace_size(shape) bytes
 * B*T*H == 0 writes zero column sums.  Returns GLA_OK or an error code.
 */
gla_status_t gla_out_gate_bwd(const gla_shape_t* shape, const void* o, const void* z,
                              const float* ln_w, const float* ln_b, float eps, const void* dy,
                              void* d_o, void* dz, float* dln_w, float* dln_b,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace gla_out_gate_bwd needs (depends on V only; 0 for an
 * invalid shape).  A pure function of the shape: it makes no HIP call. */
size_t gla_out_gate_bwd_workspace_size(const gla_shape_t* shape);

/* Static description of a status code (never NULL). */
const char* gla_status_string(gla_status_t status);

/* Detail text of the last error reported on the calling thread ("" if none).
 * The pointer stays valid until the next gla_* call on that thread. */
const char* gla_last_error_detail(void);

/* GLA_ABI_VERSION of the loaded library. */
int gla_abi_version(void);

/*
 * Per-kernel timing, for benchmarks and profiling (off by default).
 * gla_set_launch_recorder(rec): until it is called again with NULL, every
 *   library call made by the CALLING THREAD brackets each kernel it enqueues
 *   with two of the caller's HIP events, recorded on that call's stream (so
 *   the interval between them is that kernel on that stream).  For the i-th
 *   launch seen (i = rec->count before the launch; count is then incremented)
 *   the library records start[i] and stop[i] and sets name[i] to a static,
 *   NUL-terminated kernel name, as long as i < capacity; later launches only
 *   increment count, so count > capacity tells the caller that entries were
 *   dropped.  A failed hipEventRecord sets failed = 1.
 * Ownership: the record, its arrays and the events (created by the caller
 *   with timing enabled) stay the caller's and must outlive their use; the
 *   library creates, destroys and synchronises no event and keeps only the
 *   pointer, per thread.  Reading the times (hipEventElapsedTime) is the
 *   caller's job once the stream has passed the stop events.
 */
typedef struct {
    int32_t capacity;     /* entries in start, stop and name                 */
    int32_t count;        /* launches seen while set; the library increments */
    int32_t failed;       /* set to 1 by the library if an event record fails */
    int32_t reserved;
    void* const* start;   /* hipEvent_t[capacity]                            */
    void* const* stop;    /* hipEvent_t[capacity]                            */
    const char** name;    /* written by the library                          */
} gla_launch_recorder_t;

void gla_set_launch_recorder(gla_launch_recorder_t* recorder);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H_ */
