/*
 * kda_oracle.c -- fp64 CPU oracle for Kimi Delta Attention (KDA), forward pass.
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

/* Number of threads an OpenMP parallel region would use (1 without OpenMP). */
int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
