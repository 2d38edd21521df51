/*
 * kda_oracle.c -- fp64 CPU oracle for Kimi Delta Attention (KDA): the forward
 * pass and its gradients.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
 * definition that the GPU library is checked against.  Only tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or helper with the HIP library, and the library never calls it.
 *
 * Pages cited (by title):
 *   [K3-explainer]  lshu.cn news 263999, the Kimi K3 explainer (KDA, AttnRes,
 *                   MoE, agent harness) -- the only page with KDA's equations.
 *   [K3-memory]     "Kimi K3 Changed the Memory Math for Agentic AI Forever"
 *                   (hubwiz.com translation, "Kimi K3 混合线性注意力").
 *   [Kimi-Linear]   "Kimi Linear 最多砍掉 75% KV Cache：全注意力真要退场了吗？"
 *                   (ai.concitech.org).
 *
 * What is computed.  Per sequence and per head, one state matrix
 * S in R^{d_k x d_v} that maps keys to values ([K3-explainer] §二.1, the
 * linear-memory definition).  For every token t, in order:
 *
 *   S'    = Diag(alpha_t) S_{t-1}            per-channel decay over the d_k rows,
 *                                            alpha_t in [0,1]^{d_k}  ([K3-explainer] §四)
 *   vhat  = S'^T k_t                         the memory's prediction for k_t
 *   e_t   = v_t - vhat                       prediction error         ([K3-explainer] §三)
 *   S_t   = S' + beta_t k_t e_t^T            write only the error     ([K3-explainer] §三)
 *   o_t   = S_t^T q_t                        read with the query      ([K3-explainer] §二.1)
 *
 * Expanding S_t gives (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 * the KDA update printed in [K3-explainer] §四 (the decay is applied first,
 * then the erase along k_t, as printed).  The page's formulas lost their '+'
 * and '=' signs in extraction; the reading above is the only one consistent
 * with the page's own expansion of the delta rule in §三.
 *
 * Interface conventions (not fixed by the pages; chosen to match the library):
 *   - Gates arrive as natural-log decays: alpha_t[c] = exp(log_alpha[t,h,c]).
 *   - No 1/sqrt(d_k) query scale and no normalisation: o_t = S_t^T q_t as printed.
 *   - States are stored transposed, M = S^T with shape [d_v][d_k] (row = value
 *     index, contiguous along the key index), the [batch, heads, value_dim,
 *     key_dim] layout that [K3-memory] §3 reports for Moonshot's kernel.
 *   - Sequences are packed along the token axis; sequence n covers tokens
 *     [seq_start[n], seq_start[n+1]).  A dense [B, T] batch is B sequences of
 *     length T.  Each sequence starts from its own initial state (zeros if NULL).
 *
 * Every input is double precision; the caller upcasts bf16/fp32 data exactly.
 * Build:  gcc -O2 -fopenmp -shared -fPIC -o libkda_oracle.so kda_oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Returns 0 on success, -1 on bad arguments, -2 if memory runs out. */
int kda_oracle_forward(int64_t n_seqs, const int64_t *seq_start, int64_t n_heads,
                       int64_t d_k, int64_t d_v, const double *q, const double *k,
                       const double *v, const double *log_alpha, const double *beta,
                       const double *state_in, double *out, double *state_out,
                       int n_threads)
{
    if (n_seqs < 0 || n_heads <= 0 || d_k <= 0 || d_v <= 0 || !seq_start)
        return -1;
    for (int64_t n = 0; n < n_seqs; ++n)
        if (seq_start[n + 1] < seq_start[n] || seq_start[n] < 0)
            return -1;

    int failed = 0;
    const int64_t units = n_seqs * n_heads;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (int64_t u = 0; u < units; ++u) {
        const int64_t n = u / n_heads, h = u % n_heads;
        /* S[i*d_v + j] = S[i][j]: i runs over key channels, j over value channels. */
        double *S = (double *)malloc(sizeof(double) * (size_t)(d_k * d_v));
        double *vhat = (double *)malloc(sizeof(double) * (size_t)d_v);
        if (!S || !vhat) {
            free(S);
            free(vhat);
            failed |= 1;
            continue;
        }
        const double *M0 = state_in ? state_in + u * d_v * d_k : NULL;
        for (int64_t i = 0; i < d_k; ++i)
            for (int64_t j = 0; j < d_v; ++j)
                S[i * d_v + j] = M0 ? M0[j * d_k + i] : 0.0;

        for (int64_t t = seq_start[n]; t < seq_start[n + 1]; ++t) {
            const double *qt = q + (t * n_heads + h) * d_k;
            const double *kt = k + (t * n_heads + h) * d_k;
            const double *vt = v + (t * n_heads + h) * d_v;
            const double *gt = log_alpha + (t * n_heads + h) * d_k;
            const double bt = beta[t * n_heads + h];

            /* S' = Diag(alpha_t) S_{t-1}: row i of S is key channel i. */
            for (int64_t i = 0; i < d_k; ++i) {
                const double alpha_i = exp(gt[i]);
                for (int64_t j = 0; j < d_v; ++j)
                    S[i * d_v + j] *= alpha_i;
            }
            /* vhat = S'^T k_t */
            for (int64_t j = 0; j < d_v; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < d_k; ++i)
                    acc += S[i * d_v + j] * kt[i];
                vhat[j] = acc;
            }
            /* S_t = S' + beta_t k_t e_t^T with e_t = v_t - vhat */
            for (int64_t i = 0; i < d_k; ++i)
                for (int64_t j = 0; j < d_v; ++j)
                    S[i * d_v + j] += bt * kt[i] * (vt[j] - vhat[j]);
            /* o_t = S_t^T q_t */
            double *ot = out + (t * n_heads + h) * d_v;
            for (int64_t j = 0; j < d_v; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < d_k; ++i)
                    acc += S[i * d_v + j] * qt[i];
                ot[j] = acc;
            }
        }

        if (state_out) {
            double *M1 = state_out + u * d_v * d_k;
            for (int64_t i = 0; i < d_k; ++i)
                for (int64_t j = 0; j < d_v; ++j)
                    M1[j * d_k + i] = S[i * d_v + j];
        }
        free(S);
        free(vhat);
    }
    return failed ? -2 : 0;
}

/*
 * Backward pass (gradients of the forward above).
 *
 * The pages state the forward recurrence only.  They give training as the
 * reason for the chunkwise kernel (so that training runs as matrix products
 * rather than a token-serial RNN: [Kimi-Linear], the section on KDA's
 * per-channel forgetting) but no gradient.  What follows is the reverse-mode derivative of each step of the
 * recurrence, written token by token in reverse order.  With G = dL/dS_t (the
 * loss gradient with respect to the state after token t) and the forward
 * quantities S_prev = S_{t-1}, S' = Diag(alpha_t) S_prev, e_t = v_t - S'^T k_t:
 *
 *   o_t = S_t^T q_t:         G += q_t do_t^T,  dq_t = S_t do_t
 *   S_t = S' + beta k e^T:   with r = G^T k_t (a d_v vector),
 *                            dv_t    = beta_t r
 *                            dbeta_t = r . e_t
 *                            dk_t    = beta_t (G e_t - S' r)
 *                            dL/dS'  = G - beta_t k_t r^T
 *   S' = Diag(alpha) S_prev: dalpha_t[i] = sum_j (dL/dS')[i][j] S_prev[i][j],
 *                            dlog_alpha_t[i] = alpha_t[i] dalpha_t[i],
 *                            dL/dS_prev = Diag(alpha_t) dL/dS'
 *
 * and G for the state before the first token is the initial state's gradient.
 * The loss enters through d_out (dL/do_t) and d_state_out (dL/dS_final, may be
 * NULL for zero); both and all gradients use the forward's layouts.  States
 * before each token are recomputed from checkpoints kept every CK tokens.
 * Returns 0 on success, -1 on bad arguments, -2 if memory runs out.
 */
#define CK 64

/* One forward step: S <- S' + beta k e^T with S' = Diag(alpha) S (S is d_k x d_v). */
static void fwd_step(double *S, int64_t d_k, int64_t d_v, const double *kt, const double *vt,
                     const double *gt, double bt, double *tmp)
{
    for (int64_t i = 0; i < d_k; ++i) {
        const double a = exp(gt[i]);
        for (int64_t j = 0; j < d_v; ++j)
            S[i * d_v + j] *= a;
    }
    for (int64_t j = 0; j < d_v; ++j) {
        double p = 0.0;
        for (int64_t i = 0; i < d_k; ++i)
            p += S[i * d_v + j] * kt[i];
        tmp[j] = vt[j] - p;
    }
    for (int64_t i = 0; i < d_k; ++i)
        for (int64_t j = 0; j < d_v; ++j)
            S[i * d_v + j] += bt * kt[i] * tmp[j];
}

int kda_oracle_backward(int64_t n_seqs, const int64_t *seq_start, int64_t n_heads,
                        int64_t d_k, int64_t d_v, const double *q, const double *k,
                        const double *v, const double *log_alpha, const double *beta,
                        const double *state_in, const double *d_out,
                        const double *d_state_out, double *dq, double *dk, double *dv,
                        double *dlog_alpha, double *dbeta, double *d_state_in, int n_threads)
{
    if (n_seqs < 0 || n_heads <= 0 || d_k <= 0 || d_v <= 0 || !seq_start)
        return -1;
    for (int64_t n = 0; n < n_seqs; ++n)
        if (seq_start[n + 1] < seq_start[n] || seq_start[n] < 0)
            return -1;

    int failed = 0;
    const int64_t units = n_seqs * n_heads;
    const int64_t sz = d_k * d_v;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (int64_t u = 0; u < units; ++u) {
        const int64_t n = u / n_heads, h = u % n_heads;
        const int64_t t_beg = seq_start[n], t_end = seq_start[n + 1];
        const int64_t nblk = (t_end - t_beg + CK - 1) / CK;
        double *ckpt = (double *)malloc(sizeof(double) * (size_t)((nblk + 1) * sz));
        double *blk = (double *)malloc(sizeof(double) * (size_t)((CK + 1) * sz));
        double *G = (double *)malloc(sizeof(double) * (size_t)sz);
        double *tmp = (double *)malloc(sizeof(double) * (size_t)(d_v > d_k ? d_v : d_k));
        double *e = (double *)malloc(sizeof(double) * (size_t)d_v);
        double *r = (double *)malloc(sizeof(double) * (size_t)d_v);
        if (!ckpt || !blk || !G || !tmp || !e || !r) {
            free(ckpt); free(blk); free(G); free(tmp); free(e); free(r);
            failed |= 1;
            continue;
        }
        /* forward, keeping the state before every CK-th token (math layout S[i][j]) */
        double *S = ckpt;
        const double *M0 = state_in ? state_in + u * d_v * d_k : NULL;
        for (int64_t i = 0; i < d_k; ++i)
            for (int64_t j = 0; j < d_v; ++j)
                S[i * d_v + j] = M0 ? M0[j * d_k + i] : 0.0;
        for (int64_t b = 0; b + 1 < nblk; ++b) {
            memcpy(ckpt + (b + 1) * sz, ckpt + b * sz, sizeof(double) * (size_t)sz);
            for (int64_t t = t_beg + b * CK; t < t_beg + (b + 1) * CK; ++t)
                fwd_step(ckpt + (b + 1) * sz, d_k, d_v, k + (t * n_heads + h) * d_k,
                         v + (t * n_heads + h) * d_v, log_alpha + (t * n_heads + h) * d_k,
                         beta[t * n_heads + h], tmp);
        }
        /* G = dL/dS_final */
        const double *dM1 = d_state_out ? d_state_out + u * d_v * d_k : NULL;
        for (int64_t i = 0; i < d_k; ++i)
            for (int64_t j = 0; j < d_v; ++j)
                G[i * d_v + j] = dM1 ? dM1[j * d_k + i] : 0.0;

        for (int64_t b = nblk - 1; b >= 0; --b) {
            const int64_t t0 = t_beg + b * CK;
            const int64_t t1 = t0 + CK < t_end ? t0 + CK : t_end;
            /* blk[j] = state before token t0 + j, blk[t1 - t0] = state after the block */
            memcpy(blk, ckpt + b * sz, sizeof(double) * (size_t)sz);
            for (int64_t t = t0; t < t1; ++t) {
                double *nxt = blk + (t - t0 + 1) * sz;
                memcpy(nxt, blk + (t - t0) * sz, sizeof(double) * (size_t)sz);
                fwd_step(nxt, d_k, d_v, k + (t * n_heads + h) * d_k,
                         v + (t * n_heads + h) * d_v, log_alpha + (t * n_heads + h) * d_k,
                         beta[t * n_heads + h], tmp);
            }
            for (int64_t t = t1 - 1; t >= t0; --t) {
                const double *Sprev = blk + (t - t0) * sz, *Snow = blk + (t - t0 + 1) * sz;
                const double *qt = q + (t * n_heads + h) * d_k;
                const double *kt = k + (t * n_heads + h) * d_k;
                const double *vt = v + (t * n_heads + h) * d_v;
                const double *gt = log_alpha + (t * n_heads + h) * d_k;
                const double *dot = d_out + (t * n_heads + h) * d_v;
                const double bt = beta[t * n_heads + h];
                /* the read o_t = S_t^T q_t */
                for (int64_t i = 0; i < d_k; ++i)
                    for (int64_t j = 0; j < d_v; ++j)
                        G[i * d_v + j] += qt[i] * dot[j];
                double *dqt = dq + (t * n_heads + h) * d_k;
                for (int64_t i = 0; i < d_k; ++i) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < d_v; ++j)
                        acc += Snow[i * d_v + j] * dot[j];
                    dqt[i] = acc;
                }
                /* forward quantities of the step: e_t from S' = Diag(alpha) S_prev */
                for (int64_t j = 0; j < d_v; ++j) {
                    double p = 0.0;
                    for (int64_t i = 0; i < d_k; ++i)
                        p += exp(gt[i]) * Sprev[i * d_v + j] * kt[i];
                    e[j] = vt[j] - p;
                }
                /* r = G^T k_t */
                for (int64_t j = 0; j < d_v; ++j) {
                    double acc = 0.0;
                    for (int64_t i = 0; i < d_k; ++i)
                        acc += G[i * d_v + j] * kt[i];
                    r[j] = acc;
                }
                double *dvt = dv + (t * n_heads + h) * d_v;
                double db = 0.0;
                for (int64_t j = 0; j < d_v; ++j) {
                    dvt[j] = bt * r[j];
                    db += r[j] * e[j];
                }
                dbeta[t * n_heads + h] = db;
                double *dkt = dk + (t * n_heads + h) * d_k;
                for (int64_t i = 0; i < d_k; ++i) {
                    const double a = exp(gt[i]);
                    double ge = 0.0, sr = 0.0;
                    for (int64_t j = 0; j < d_v; ++j) {
                        ge += G[i * d_v + j] * e[j];
                        sr += a * Sprev[i * d_v + j] * r[j];
                    }
                    dkt[i] = bt * (ge - sr);
                }
                /* dL/dS' = G - beta k r^T, then through the decay */
                double *dgt = dlog_alpha + (t * n_heads + h) * d_k;
                for (int64_t i = 0; i < d_k; ++i) {
                    const double a = exp(gt[i]);
                    double da = 0.0;
                    for (int64_t j = 0; j < d_v; ++j) {
                        const double dsp = G[i * d_v + j] - bt * kt[i] * r[j];
                        da += dsp * Sprev[i * d_v + j];
                        G[i * d_v + j] = a * dsp;
                    }
                    dgt[i] = a * da;
                }
            }
        }
        if (d_state_in) {
            double *dM0 = d_state_in + u * d_v * d_k;
            for (int64_t i = 0; i < d_k; ++i)
                for (int64_t j = 0; j < d_v; ++j)
                    dM0[j * d_k + i] = G[i * d_v + j];
        }
        free(ckpt); free(blk); free(G); free(tmp); free(e); free(r);
    }
    return failed ? -2 : 0;
}

/* Number of threads an OpenMP parallel region would use (1 without OpenMP). */
int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
