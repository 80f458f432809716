/*
 * Reference oracle for gated linear attention (GLA) -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the slow, obviously-correct CPU definition that the GPU path is
 * checked against.  Only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it; the product library never links it, and it
 * shares no code, header or table with the HIP kernels.
 *
 * Arithmetic is IEEE fp64 throughout, token by token, exactly as the
 * recurrence is written -- no chunking, no blocking, no reordering:
 *
 *   "Gated Linear Attention Transformers with Hardware-Efficient Training"
 *   (Yang, Wang, Shen, Panda, Kim), Section 4.1, Eq. (3):
 *       S_t = Diag(alpha_t) S_{t-1} + k_t^T v_t ,   o_t = q_t S_t
 *   with alpha_t = exp(g_t) given as the log forget gate g_t (Section 4.3 and
 *   the chapter summary's Knowl 3 take the gate in log space).  S_0 is zero or
 *   the state an earlier segment of the sequence ended with (Section 2.2); the
 *   final state S_T is returned so that segments can be chained (truncated
 *   BPTT, Section 5.2).
 *
 * The backward pass is reverse-mode differentiation of that same loop (the
 * hand-computed gradient of the recurrence).  It does NOT use the paper's
 * closed-form gate gradient (Section 4.3, "Memory-efficient dalpha_t
 * computation"); the gate gradient here comes from dS_t and S_{t-1} directly,
 * which is the quantity the paper says earlier work had to materialise.  The
 * agreement of the two routes is itself one of the tests.
 *
 * Layouts (row-major, contiguous):
 *   q, k, g, dq, dk, dg : [B, T, H, K]
 *   v, o, do, dv        : [B, T, H, V]
 *   s0, s_final, dht, ds0 : [B, H, K, V]
 * Heads are independent (Section 4.4, multi-head GLA), so (b, h) pairs are
 * processed in parallel with OpenMP when it is available.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX_TOK(b, t, h, d, T, H, D) ((((size_t)(b) * (T) + (t)) * (H) + (h)) * (D) + (d))
#define IDX_ST(b, h, i, j, H, K, V) ((((size_t)(b) * (H) + (h)) * (K) + (i)) * (V) + (j))

/* Length of the recompute segments used by the backward pass.  States are
 * checkpointed at every multiple of this many tokens and recomputed forward
 * inside a segment; they are never obtained by dividing by the gate. */
#define ORACLE_CKPT 64

int oracle_version(void) { return 1; }

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One recurrence step on a single head: S <- Diag(exp(g_t)) S + k_t^T v_t. */
static void step_state(double *S, const double *k_t, const double *g_t, const double *v_t,
                       long K, long V) {
    for (long i = 0; i < K; ++i) {
        const double a = exp(g_t[i]);
        const double ki = k_t[i];
        double *row = S + i * V;
        for (long j = 0; j < V; ++j) row[j] = a * row[j] + ki * v_t[j];
    }
}

/* Forward: o_t = q_t S_t with S_t the state AFTER token t's update (the causal
 * mask of Section 2.1 has M_tt = 1, so token t attends to itself). */
int oracle_gla_fwd(long B, long T, long H, long K, long V,
                   const double *q, const double *k, const double *v, const double *g,
                   const double *s0, double *o, double *s_final) {
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0) return 1;
    long nbh = B * H;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        long b = bh / H, h = bh % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)K * (size_t)V);
        double *qt = (double *)malloc(sizeof(double) * (size_t)K);
        double *kt = (double *)malloc(sizeof(double) * (size_t)K);
        double *gt = (double *)malloc(sizeof(double) * (size_t)K);
        double *vt = (double *)malloc(sizeof(double) * (size_t)V);
        if (!S || !qt || !kt || !gt || !vt) {
#pragma omp atomic write
            err = 2;
            free(S); free(qt); free(kt); free(gt); free(vt);
            continue;
        }
        for (long i = 0; i < K; ++i)
            for (long j = 0; j < V; ++j)
                S[i * V + j] = s0 ? s0[IDX_ST(b, h, i, j, H, K, V)] : 0.0;
        for (long t = 0; t < T; ++t) {
            for (long i = 0; i < K; ++i) {
                qt[i] = q[IDX_TOK(b, t, h, i, T, H, K)];
                kt[i] = k[IDX_TOK(b, t, h, i, T, H, K)];
                gt[i] = g[IDX_TOK(b, t, h, i, T, H, K)];
            }
            for (long j = 0; j < V; ++j) vt[j] = v[IDX_TOK(b, t, h, j, T, H, V)];
            step_state(S, kt, gt, vt, K, V);
            for (long j = 0; j < V; ++j) {
                double acc = 0.0;
                for (long i = 0; i < K; ++i) acc += qt[i] * S[i * V + j];
                o[IDX_TOK(b, t, h, j, T, H, V)] = acc;
            }
        }
        if (s_final)
            for (long i = 0; i < K; ++i)
                for (long j = 0; j < V; ++j) s_final[IDX_ST(b, h, i, j, H, K, V)] = S[i * V + j];
        free(S); free(qt); free(kt); free(gt); free(vt);
    }
    return err;
}

/* General gated linear attention ("Gated Linear Attention Transformers with
 * Hardware-Efficient Training", the chapter summary's Knowl 12 and Appendix C):
 * the forget gate is the outer product of a key-side gate alpha_t = exp(g_t)
 * (1 x K) and a value-side gate beta_t = exp(h_t) (1 x V),
 *   S_t = (alpha_t^T beta_t) .* S_{t-1} + k_t^T v_t ,   o_t = q_t S_t ,
 * token by token, with S_0 = s0 or zero.  h is laid out like v: [B, T, H, V]. */
int oracle_gla_fwd_general(long B, long T, long H, long K, long V,
                           const double *q, const double *k, const double *v, const double *g,
                           const double *h, const double *s0, double *o, double *s_final) {
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0) return 1;
    long nbh = B * H;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        long b = bh / H, hh = bh % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)K * (size_t)V);
        double *av = (double *)malloc(sizeof(double) * (size_t)K);
        double *bv = (double *)malloc(sizeof(double) * (size_t)V);
        if (!S || !av || !bv) {
#pragma omp atomic write
            err = 2;
            free(S); free(av); free(bv);
            continue;
        }
        for (long i = 0; i < K; ++i)
            for (long j = 0; j < V; ++j)
                S[i * V + j] = s0 ? s0[IDX_ST(b, hh, i, j, H, K, V)] : 0.0;
        for (long t = 0; t < T; ++t) {
            for (long i = 0; i < K; ++i) av[i] = exp(g[IDX_TOK(b, t, hh, i, T, H, K)]);
            for (long j = 0; j < V; ++j) bv[j] = exp(h[IDX_TOK(b, t, hh, j, T, H, V)]);
            for (long i = 0; i < K; ++i) {
                const double ki = k[IDX_TOK(b, t, hh, i, T, H, K)];
                double *row = S + i * V;
                for (long j = 0; j < V; ++j)
                    row[j] = (av[i] * bv[j]) * row[j] + ki * v[IDX_TOK(b, t, hh, j, T, H, V)];
            }
            for (long j = 0; j < V; ++j) {
                double acc = 0.0;
                for (long i = 0; i < K; ++i) acc += q[IDX_TOK(b, t, hh, i, T, H, K)] * S[i * V + j];
                o[IDX_TOK(b, t, hh, j, T, H, V)] = acc;
            }
        }
        if (s_final)
            for (long i = 0; i < K; ++i)
                for (long j = 0; j < V; ++j) s_final[IDX_ST(b, hh, i, j, H, K, V)] = S[i * V + j];
        free(S); free(av); free(bv);
    }
    return err;
}

/* One token of the general recurrence in place: S <- (alpha^T beta) .* S + k^T v,
 * with alpha = exp(g_t), beta = exp(h_t) already exponentiated in av, bv. */
static void step_general(double *S, const double *kt, const double *av, const double *vt, const double *bv,
                         long K, long V) {
    for (long i = 0; i < K; ++i) {
        double *row = S + i * V;
        for (long j = 0; j < V; ++j) row[j] = (av[i] * bv[j]) * row[j] + kt[i] * vt[j];
    }
}

/* Reverse-mode gradient of oracle_gla_fwd_general for the loss
 * L = <o, d_o> + <S_T, dht> (same pages and notation).  With dS the running
 * gradient with respect to the post-update state S_t and G_t = alpha_t^T beta_t,
 * for t = T-1 .. 0:
 *   dS += q_t^T do_t ;  dq_t = do_t S_t^T ;  dk_t = v_t dS^T ;  dv_t = k_t dS ;
 *   dg_t[i] = sum_j dS[i,j] G_t[i,j] S_{t-1}[i,j] ,  dh_t[j] = sum_i (the same) ;
 *   dS <- G_t .* dS            (now the gradient with respect to S_{t-1}),
 * and ds0 is the last dS.  g and h are log gates, so d/dg of alpha = alpha.
 * States come from checkpoints every ORACLE_CKPT tokens and a forward replay. */
int oracle_gla_bwd_general(long B, long T, long H, long K, long V,
                           const double *q, const double *k, const double *v, const double *g,
                           const double *h, const double *s0, const double *d_o, const double *dht,
                           double *dq, double *dk, double *dv, double *dg, double *dh, double *ds0) {
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0) return 1;
    const long KV = K * V;
    const long nseg = (T + ORACLE_CKPT - 1) / ORACLE_CKPT;
    long nbh = B * H;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        long b = bh / H, hh = bh % H;
        double *ckpt = (double *)malloc(sizeof(double) * (size_t)KV * (size_t)(nseg > 0 ? nseg : 1));
        double *seg = (double *)malloc(sizeof(double) * (size_t)KV * (ORACLE_CKPT + 1));
        double *dS = (double *)malloc(sizeof(double) * (size_t)KV);
        double *kt = (double *)malloc(sizeof(double) * (size_t)K);
        double *av = (double *)malloc(sizeof(double) * (size_t)K);
        double *vt = (double *)malloc(sizeof(double) * (size_t)V);
        double *bv = (double *)malloc(sizeof(double) * (size_t)V);
        double *dhacc = (double *)malloc(sizeof(double) * (size_t)V);
        if (!ckpt || !seg || !dS || !kt || !av || !vt || !bv || !dhacc) {
#pragma omp atomic write
            err = 2;
            free(ckpt); free(seg); free(dS); free(kt); free(av); free(vt); free(bv); free(dhacc);
            continue;
        }
#define LOAD_TOKEN(t)                                                        \
        do {                                                                 \
            for (long i = 0; i < K; ++i) {                                   \
                kt[i] = k[IDX_TOK(b, (t), hh, i, T, H, K)];                  \
                av[i] = exp(g[IDX_TOK(b, (t), hh, i, T, H, K)]);             \
            }                                                                \
            for (long j = 0; j < V; ++j) {                                   \
                vt[j] = v[IDX_TOK(b, (t), hh, j, T, H, V)];                  \
                bv[j] = exp(h[IDX_TOK(b, (t), hh, j, T, H, V)]);             \
            }                                                                \
        } while (0)
        double *S = seg;
        for (long i = 0; i < K; ++i)
            for (long j = 0; j < V; ++j) S[i * V + j] = s0 ? s0[IDX_ST(b, hh, i, j, H, K, V)] : 0.0;
        for (long t = 0; t < T; ++t) {
            if (t % ORACLE_CKPT == 0) memcpy(ckpt + (t / ORACLE_CKPT) * KV, S, sizeof(double) * KV);
            LOAD_TOKEN(t);
            step_general(S, kt, av, vt, bv, K, V);
        }
        for (long i = 0; i < K; ++i)
            for (long j = 0; j < V; ++j) dS[i * V + j] = dht ? dht[IDX_ST(b, hh, i, j, H, K, V)] : 0.0;
        for (long m = nseg - 1; m >= 0; --m) {
            long t0 = m * ORACLE_CKPT;
            long t1 = t0 + ORACLE_CKPT < T ? t0 + ORACLE_CKPT : T;
            memcpy(seg, ckpt + m * KV, sizeof(double) * KV);
            for (long t = t0; t < t1; ++t) {
                double *dst = seg + (t - t0 + 1) * KV;
                memcpy(dst, seg + (t - t0) * KV, sizeof(double) * KV);
                LOAD_TOKEN(t);
                step_general(dst, kt, av, vt, bv, K, V);
            }
            for (long t = t1 - 1; t >= t0; --t) {
                const double *St = seg + (t - t0 + 1) * KV;
                const double *Sp = seg + (t - t0) * KV;
                LOAD_TOKEN(t);
                for (long i = 0; i < K; ++i) {
                    const double qi = q[IDX_TOK(b, t, hh, i, T, H, K)];
                    for (long j = 0; j < V; ++j) dS[i * V + j] += qi * d_o[IDX_TOK(b, t, hh, j, T, H, V)];
                }
                for (long j = 0; j < V; ++j) dhacc[j] = 0.0;
                for (long i = 0; i < K; ++i) {
                    double aq = 0.0, ak = 0.0, ag = 0.0;
                    for (long j = 0; j < V; ++j) {
                        const double decayed = (av[i] * bv[j]) * Sp[i * V + j];  /* G_t .* S_{t-1} */
                        aq += d_o[IDX_TOK(b, t, hh, j, T, H, V)] * St[i * V + j];
                        ak += dS[i * V + j] * vt[j];
                        ag += dS[i * V + j] * decayed;
                        dhacc[j] += dS[i * V + j] * decayed;
                    }
                    dq[IDX_TOK(b, t, hh, i, T, H, K)] = aq;
                    dk[IDX_TOK(b, t, hh, i, T, H, K)] = ak;
                    dg[IDX_TOK(b, t, hh, i, T, H, K)] = ag;
                }
                for (long j = 0; j < V; ++j) {
                    double acc = 0.0;
                    for (long i = 0; i < K; ++i) acc += kt[i] * dS[i * V + j];
                    dv[IDX_TOK(b, t, hh, j, T, H, V)] = acc;
                    dh[IDX_TOK(b, t, hh, j, T, H, V)] = dhacc[j];
                }
                for (long i = 0; i < K; ++i)
                    for (long j = 0; j < V; ++j) dS[i * V + j] *= av[i] * bv[j];
            }
        }
#undef LOAD_TOKEN
        if (ds0)
            for (long i = 0; i < K; ++i)
                for (long j = 0; j < V; ++j) ds0[IDX_ST(b, hh, i, j, H, K, V)] = dS[i * V + j];
        free(ckpt); free(seg); free(dS); free(kt); free(av); free(vt); free(bv); free(dhacc);
    }
    return err;
}

/* Backward of the same loop.  With S_t the post-update state and dS the
 * running gradient with respect to it, for t = T..1:
 *   dS      += q_t^T do_t                       (o_t = q_t S_t)
 *   dq_t[i]  = sum_j do_t[j] S_t[i,j]
 *   dk_t[i]  = sum_j dS[i,j] v_t[j]             (S_t contains k_t^T v_t)
 *   dv_t[j]  = sum_i k_t[i] dS[i,j]
 *   dg_t[i]  = exp(g_t[i]) sum_j dS[i,j] S_{t-1}[i,j]   (d/dg of exp(g) S_{t-1})
 *   dS      <- Diag(exp(g_t)) dS                (gradient flowing into S_{t-1})
 * The loss is <o, do> + <S_T, dht>, so dS starts at dht (zero when absent),
 * and after t = 1 it is the gradient with respect to S_0. */
int oracle_gla_bwd(long B, long T, long H, long K, long V,
                   const double *q, const double *k, const double *v, const double *g,
                   const double *s0, const double *d_o, const double *dht,
                   double *dq, double *dk, double *dv, double *dg, double *ds0) {
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0) return 1;
    const long KV = K * V;
    const long nseg = (T + ORACLE_CKPT - 1) / ORACLE_CKPT;
    long nbh = B * H;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        long b = bh / H, h = bh % H;
        /* ckpt[m] = state before token m*ORACLE_CKPT (i.e. S_{m*CKPT}). */
        double *ckpt = (double *)malloc(sizeof(double) * (size_t)KV * (size_t)(nseg > 0 ? nseg : 1));
        /* seg[u] = state after token (segment start + u), u = 0..CKPT-1,
         * plus seg_prev = state before the segment. */
        double *seg = (double *)malloc(sizeof(double) * (size_t)KV * (ORACLE_CKPT + 1));
        double *dS = (double *)malloc(sizeof(double) * (size_t)KV);
        double *kt = (double *)malloc(sizeof(double) * (size_t)K);
        double *gt = (double *)malloc(sizeof(double) * (size_t)K);
        double *vt = (double *)malloc(sizeof(double) * (size_t)V);
        if (!ckpt || !seg || !dS || !kt || !gt || !vt) {
#pragma omp atomic write
            err = 2;
            free(ckpt); free(seg); free(dS); free(kt); free(gt); free(vt);
            continue;
        }
        /* Forward sweep storing checkpoints. */
        double *S = seg; /* scratch for the sweep */
        for (long i = 0; i < K; ++i)
            for (long j = 0; j < V; ++j)
                S[i * V + j] = s0 ? s0[IDX_ST(b, h, i, j, H, K, V)] : 0.0;
        for (long t = 0; t < T; ++t) {
            if (t % ORACLE_CKPT == 0) memcpy(ckpt + (t / ORACLE_CKPT) * KV, S, sizeof(double) * KV);
            for (long i = 0; i < K; ++i) {
                kt[i] = k[IDX_TOK(b, t, h, i, T, H, K)];
                gt[i] = g[IDX_TOK(b, t, h, i, T, H, K)];
            }
            for (long j = 0; j < V; ++j) vt[j] = v[IDX_TOK(b, t, h, j, T, H, V)];
            step_state(S, kt, gt, vt, K, V);
        }
        for (long i = 0; i < K; ++i)
            for (long j = 0; j < V; ++j)
                dS[i * V + j] = dht ? dht[IDX_ST(b, h, i, j, H, K, V)] : 0.0;
        /* Reverse sweep, one checkpoint segment at a time. */
        for (long m = nseg - 1; m >= 0; --m) {
            long t0 = m * ORACLE_CKPT;
            long t1 = t0 + ORACLE_CKPT < T ? t0 + ORACLE_CKPT : T;
            /* seg[0] = S before token t0; seg[u+1] = S after token t0+u. */
            memcpy(seg, ckpt + m * KV, sizeof(double) * KV);
            for (long t = t0; t < t1; ++t) {
                double *dst = seg + (t - t0 + 1) * KV;
                memcpy(dst, seg + (t - t0) * KV, sizeof(double) * KV);
                for (long i = 0; i < K; ++i) {
                    kt[i] = k[IDX_TOK(b, t, h, i, T, H, K)];
                    gt[i] = g[IDX_TOK(b, t, h, i, T, H, K)];
                }
                for (long j = 0; j < V; ++j) vt[j] = v[IDX_TOK(b, t, h, j, T, H, V)];
                step_state(dst, kt, gt, vt, K, V);
            }
            for (long t = t1 - 1; t >= t0; --t) {
                const double *St = seg + (t - t0 + 1) * KV;
                const double *Sp = seg + (t - t0) * KV;
                /* dS += q_t^T do_t */
                for (long i = 0; i < K; ++i) {
                    const double qi = q[IDX_TOK(b, t, h, i, T, H, K)];
                    for (long j = 0; j < V; ++j) dS[i * V + j] += qi * d_o[IDX_TOK(b, t, h, j, T, H, V)];
                }
                for (long i = 0; i < K; ++i) {
                    double aq = 0.0, ak = 0.0, ag = 0.0;
                    for (long j = 0; j < V; ++j) {
                        aq += d_o[IDX_TOK(b, t, h, j, T, H, V)] * St[i * V + j];
                        ak += dS[i * V + j] * v[IDX_TOK(b, t, h, j, T, H, V)];
                        ag += dS[i * V + j] * Sp[i * V + j];
                    }
                    const double a = exp(g[IDX_TOK(b, t, h, i, T, H, K)]);
                    dq[IDX_TOK(b, t, h, i, T, H, K)] = aq;
                    dk[IDX_TOK(b, t, h, i, T, H, K)] = ak;
                    dg[IDX_TOK(b, t, h, i, T, H, K)] = a * ag;
                }
                for (long j = 0; j < V; ++j) {
                    double av = 0.0;
                    for (long i = 0; i < K; ++i) av += k[IDX_TOK(b, t, h, i, T, H, K)] * dS[i * V + j];
                    dv[IDX_TOK(b, t, h, j, T, H, V)] = av;
                }
                for (long i = 0; i < K; ++i) {
                    const double a = exp(g[IDX_TOK(b, t, h, i, T, H, K)]);
                    for (long j = 0; j < V; ++j) dS[i * V + j] *= a;
                }
            }
        }
        if (ds0)
            for (long i = 0; i < K; ++i)
                for (long j = 0; j < V; ++j) ds0[IDX_ST(b, h, i, j, H, K, V)] = dS[i * V + j];
        free(ckpt); free(seg); free(dS); free(kt); free(gt); free(vt);
    }
    return err;
}

/* ------------------------------------------------------------------------
 * Output epilogue of the multi-head GLA layer (Section 4.4, "GLA
 * Transformer"): each head's output row o (V channels) goes through
 * LayerNorm on its own, and the result is multiplied elementwise by the
 * output gate r = Swish(z), z being the gate's pre-activation x W_r + b_r:
 *     mu = mean_j o_j,  var = mean_j (o_j - mu)^2,  n_j = (o_j - mu) / sqrt(var + eps),
 *     a_j = n_j w_j + b_j,  y_j = a_j * z_j * sigmoid(z_j).
 * w and b (length V) are shared by every row; b may be NULL (zero).
 * Rows are R = B*T*H contiguous runs of V values.
 */
static double sigmoid_d(double z) { return 1.0 / (1.0 + exp(-z)); }

int oracle_out_gate_fwd(long R, long V, const double *o, const double *z, const double *w, const double *b,
                        double eps, double *y) {
    if (R < 0 || V <= 0 || !o || !z || !w || !y) return 1;
    for (long r = 0; r < R; ++r) {
        const double *x = o + r * V;
        double mu = 0.0, var = 0.0;
        for (long j = 0; j < V; ++j) mu += x[j];
        mu /= (double)V;
        for (long j = 0; j < V; ++j) var += (x[j] - mu) * (x[j] - mu);
        var /= (double)V;
        const double inv = 1.0 / sqrt(var + eps);
        for (long j = 0; j < V; ++j) {
            const double a = (x[j] - mu) * inv * w[j] + (b ? b[j] : 0.0);
            const double zj = z[r * V + j];
            y[r * V + j] = a * zj * sigmoid_d(zj);
        }
    }
    return 0;
}

/* Reverse-mode gradient of the loss sum_{r,j} dy_{r,j} y_{r,j} for the function
 * above, by the chain rule through each step as written:
 *   y = a * s with s = z sigmoid(z):   da = dy s,   dz = dy a s'(z),
 *       s'(z) = sigmoid(z) + z sigmoid(z) (1 - sigmoid(z));
 *   a = n w + b:                        dw += da n,  db += da,  dn = da w;
 *   n = (x - mu) inv, inv = (var + eps)^(-1/2):
 *       dinv = sum_j dn_j (x_j - mu),   dvar = -dinv inv^3 / 2,
 *       dx_j = dn_j inv + dvar 2 (x_j - mu) / V + dmu / V,
 *       dmu = -inv sum_j dn_j - dvar 2 sum_j (x_j - mu) / V  (the last sum is 0).
 * dw and db are summed over all rows (either may be NULL). */
int oracle_out_gate_bwd(long R, long V, const double *o, const double *z, const double *w, const double *b,
                        double eps, const double *dy, double *dx, double *dz, double *dw, double *db) {
    if (R < 0 || V <= 0 || !o || !z || !w || !dy || !dx || !dz) return 1;
    if (dw) for (long j = 0; j < V; ++j) dw[j] = 0.0;
    if (db) for (long j = 0; j < V; ++j) db[j] = 0.0;
    double *dn = (double *)malloc(sizeof(double) * (size_t)V);
    if (!dn) return 2;
    for (long r = 0; r < R; ++r) {
        const double *x = o + r * V;
        double mu = 0.0, var = 0.0;
        for (long j = 0; j < V; ++j) mu += x[j];
        mu /= (double)V;
        for (long j = 0; j < V; ++j) var += (x[j] - mu) * (x[j] - mu);
        var /= (double)V;
        const double inv = 1.0 / sqrt(var + eps);
        double dinv = 0.0, sdn = 0.0;
        for (long j = 0; j < V; ++j) {
            const double n = (x[j] - mu) * inv;
            const double a = n * w[j] + (b ? b[j] : 0.0);
            const double zj = z[r * V + j], sg = sigmoid_d(zj);
            const double s = zj * sg;
            const double g = dy[r * V + j];
            const double da = g * s;
            dz[r * V + j] = g * a * (sg + zj * sg * (1.0 - sg));
            if (dw) dw[j] += da * n;
            if (db) db[j] += da;
            dn[j] = da * w[j];
            dinv += dn[j] * (x[j] - mu);
            sdn += dn[j];
        }
        const double dvar = -0.5 * dinv * inv * inv * inv;
        const double dmu = -inv * sdn;
        for (long j = 0; j < V; ++j)
            dx[r * V + j] = dn[j] * inv + dvar * 2.0 * (x[j] - mu) / (double)V + dmu / (double)V;
    }
    free(dn);
    return 0;
}
