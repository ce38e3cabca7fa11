/*
 * Host sanitizer driver for the fp64 oracle (test infrastructure).  Built with
 * gcc -fsanitize=address,undefined together with oracle/gdn_oracle.c by
 * tests/test_host_sanitizers.py: every shape below runs under the address and
 * undefined-behaviour checkers, and the one-token case is checked against its
 * closed form S_1 = a S_0 (I - b k k^T) + b v k^T, o_1 = S_1 q (the gated
 * delta rule of the explainer "InfiniteVL: Synergizing Linear and Sparse
 * Attention ...", "The Concept: Gated DeltaNet").
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int gdn_oracle_recurrence(const double *q, const double *k, const double *v,
                          const double *g, const double *beta,
                          const double *state_in, double *state_out, double *o,
                          long B, long T, long H, long dk, long dv, int nthreads);

static unsigned long long rng = 0x9e3779b97f4a7c15ull;
static double urand(void) {  /* xorshift64*, uniform in (-1, 1) */
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return (double)((rng * 2685821657736338717ull) >> 11) / 4503599627370496.0 - 1.0;
}

static double *fill(long n, double lo, double hi) {
    double *x = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (long i = 0; i < n; ++i) x[i] = lo + (hi - lo) * 0.5 * (urand() + 1.0);
    return x;
}

static int run(long B, long T, long H, long d, int with_state, int with_o) {
    const long tok = B * T * H;
    double *q = fill(tok * d, -1, 1), *k = fill(tok * d, -1, 1), *v = fill(tok * d, -1, 1);
    double *g = fill(tok, -2, 0), *beta = fill(tok, 0, 1);
    double *s0 = with_state ? fill(B * H * d * d, -0.1, 0.1) : NULL;
    double *s1 = fill(B * H * d * d, 0, 0);
    double *o = with_o ? fill(tok * d, 0, 0) : NULL;
    int bad = gdn_oracle_recurrence(q, k, v, g, beta, s0, s1, o, B, T, H, d, d, 1) != 0;
    if (!bad && T == 1 && with_o) {
        /* closed form, stored layout st[i][j] = S[j][i] */
        for (long bh = 0; bh < B * H && !bad; ++bh) {
            const long b = bh / H, h = bh % H, t = (b * T) * H + h;
            const double a = exp(g[t]), bt = beta[t];
            for (long j = 0; j < d && !bad; ++j) {
                double oj = 0.0;
                for (long i = 0; i < d; ++i) {
                    double sk = 0.0;  /* (S_0 k)_j */
                    for (long l = 0; l < d; ++l) sk += (s0 ? s0[bh * d * d + l * d + j] : 0.0) * k[t * d + l];
                    const double s = a * ((s0 ? s0[bh * d * d + i * d + j] : 0.0) - bt * sk * k[t * d + i]) +
                                     bt * v[t * d + j] * k[t * d + i];
                    if (fabs(s - s1[bh * d * d + i * d + j]) > 1e-12) bad = 1;
                    oj += s * q[t * d + i];
                }
                if (fabs(oj - o[t * d + j]) > 1e-12) bad = 1;
            }
        }
    }
    free(q); free(k); free(v); free(g); free(beta); free(s0); free(s1); free(o);
    if (bad) printf("FAIL B=%ld T=%ld H=%ld d=%ld state=%d o=%d\n", B, T, H, d, with_state, with_o);
    return bad;
}

int main(void) {
    int fails = 0;
    const long shapes[][4] = {{1, 1, 1, 2}, {2, 1, 3, 4}, {1, 3, 2, 64}, {2, 65, 2, 8}, {1, 7, 1, 128}};
    for (unsigned s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (int st = 0; st < 2; ++st)
            for (int wo = 0; wo < 2; ++wo)
                fails += run(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], st, wo);
    /* T = 0 (no tokens) and bad sizes */
    fails += run(1, 0, 2, 4, 1, 1);
    double x = 0.0;
    if (gdn_oracle_recurrence(&x, &x, &x, &x, &x, NULL, &x, NULL, 1, 1, 1, 0, 1, 1) != -1) ++fails;
    printf(fails ? "oracle sanitizer run: %d failures\n" : "oracle sanitizer run: ok\n", fails);
    return fails != 0;
}
