/*
 * gdn_oracle.c -- fp64 CPU oracle for the gated delta-rule token mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (the Gated DeltaNet layer of InfiniteVL; explainer page
 * "InfiniteVL: Synergizing Linear and Sparse Attention for Highly-Efficient,
 * Unlimited-Input Vision-Language Models", section "The Concept: Gated
 * DeltaNet", its five steps; the project README "hustvl/InfiniteVL", section
 * "Accelerated Streaming Inference", for the state carried across calls).
 * The pages name the mixer but print no formula; the recurrence used is the
 * published gated delta rule (Yang, Kautz, Hatamizadeh, "Gated Delta Networks",
 * ICLR 2025), which maps onto those five steps one to one:
 *
 *   step 1  a fixed-size memory      S (d_v x d_k per head)
 *   step 2  gate keeps old memory    a_t = exp(g_t)
 *   step 3  "rotation-like" step     S (I - b_t k_t k_t^T)   (generalised Householder)
 *   step 4  write new info           + b_t v_t k_t^T
 *   step 5  read with the query      o_t = S_t q_t
 *
 *   S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T ,   o_t = S_t q_t .
 *
 * The product S_{t-1}(I - b k k^T) is evaluated as S_{t-1} - b (S_{t-1} k) k^T:
 * the same matrix, by associativity of the matrix product, without forming the
 * d_k x d_k factor.  Everything is IEEE double; no fast-math.
 *
 * Layout (row-major, contiguous):
 *   q, k      [B][T][H][d_k]      v, o   [B][T][H][d_v]
 *   g, beta   [B][T][H]           (g = log a, the per-token log-decay)
 *   state     [B][H][d_k][d_v]    stored element [i][j] is S[j][i]
 *                                 (i runs over keys, j over values)
 * state_in may be NULL (zero initial state).  state_out receives S_T in the
 * same stored layout.  o may be NULL (state only).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int gdn_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Returns 0 on success, -1 on bad sizes, -2 on allocation failure. */
int gdn_oracle_recurrence(const double *q, const double *k, const double *v,
                          const double *g, const double *beta,
                          const double *state_in, double *state_out, double *o,
                          long B, long T, long H, long dk, long dv, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (nthreads <= 0) nthreads = 1;
    int failed = 0;

#ifdef _OPENMP
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
#endif
    for (long bh = 0; bh < B * H; ++bh) {
        const long b = bh / H, h = bh % H;
        /* St holds S transposed, St[i*dv + j] = S[j][i] (the stored layout), so
         * that every loop below runs over the value index j innermost; each
         * sum over the key index i is still accumulated in increasing i. */
        double *St = (double *)malloc(sizeof(double) * (size_t)(dk * dv));
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!St || !u) {
            free(St); free(u);
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
            continue;
        }
        for (long e = 0; e < dk * dv; ++e)
            St[e] = state_in ? state_in[bh * dk * dv + e] : 0.0;

        for (long t = 0; t < T; ++t) {
            const long tok = (b * T + t) * H + h;
            const double *kt = k + tok * dk;
            const double *qt = q + tok * dk;
            const double *vt = v + tok * dv;
            const double a = exp(g[tok]);   /* step 2: decay gate */
            const double bt = beta[tok];

            /* step 3: S (I - b k k^T) = S - b (S k) k^T ; u = S k */
            for (long j = 0; j < dv; ++j) u[j] = 0.0;
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j) u[j] += St[i * dv + j] * kt[i];
            /* steps 2-4: S <- a (S - b u k^T) + b v k^T */
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j)
                    St[i * dv + j] = a * (St[i * dv + j] - bt * u[j] * kt[i]) + bt * vt[j] * kt[i];

            /* step 5: o_t = S_t q_t (readout after the update) */
            if (o) {
                double *ot = o + tok * dv;
                for (long j = 0; j < dv; ++j) ot[j] = 0.0;
                for (long i = 0; i < dk; ++i)
                    for (long j = 0; j < dv; ++j) ot[j] += St[i * dv + j] * qt[i];
            }
        }
        for (long e = 0; e < dk * dv; ++e) state_out[bh * dk * dv + e] = St[e];
        free(St);
        free(u);
    }
    return failed ? -2 : 0;
}
