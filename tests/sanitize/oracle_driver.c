/*
 * oracle_driver.c -- runs the fp64 oracle (oracle/kda_oracle.c, compiled into
 * this program) on small packed cases under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Inputs come from a fixed linear congruential
 * generator; every input and output array is written to the file named by
 * argv[1] so that the test can rerun the same inputs through the normal
 * build of the oracle and compare.  Test infrastructure only.
 *
 * Layout of the file, all little-endian: int64 n_cases, then per case
 *   int64 N, H, dk, dv, T, has_state, has_dstate; int64 seq_start[N + 1];
 *   double q[T H dk], k[T H dk], v[T H dv], g[T H dk], b[T H], d_out[T H dv],
 *   [state0[N H dv dk]], [d_state[N H dv dk]];
 *   double out[T H dv], state[N H dv dk];
 *   double dq[T H dk], dk[T H dk], dv[T H dv], dg[T H dk], db[T H], ds0[N H dv dk].
 */
#include "../../oracle/kda_oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* in [-1, 1) */
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng_state >> 11) / (double)(1ull << 52) - 1.0;
}

static double *fill(int64_t n, double lo, double hi) {
    double *p = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5 * (uniform() + 1.0);
    return p;
}

static void put(FILE *f, const void *p, size_t bytes) {
    if (bytes && fwrite(p, 1, bytes, f) != bytes) exit(3);
}

int main(int argc, char **argv) {
    if (argc != 2) return 2;
    FILE *f = fopen(argv[1], "wb");
    if (!f) return 2;
    /* sequence lengths per case (an empty one, one token, ragged, a checkpoint boundary) */
    static const int64_t lens[3][5] = {{0, 1, 17, 64, 3}, {70, 0, 0, 0, 0}, {2, 65, 0, 129, 1}};
    static const int64_t nseq[3] = {5, 1, 5};
    static const int64_t dims[3][2] = {{8, 8}, {16, 4}, {4, 12}};
    const int64_t n_cases = 3;
    put(f, &n_cases, 8);
    for (int c = 0; c < n_cases; ++c) {
        const int64_t N = nseq[c], H = 2, dk = dims[c][0], dv = dims[c][1];
        int64_t *st = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N + 1));
        st[0] = 0;
        for (int64_t n = 0; n < N; ++n) st[n + 1] = st[n] + lens[c][n];
        const int64_t T = st[N];
        const int64_t has_state = c != 1, has_dstate = c != 2;
        double *q = fill(T * H * dk, -1, 1), *k = fill(T * H * dk, -0.5, 0.5),
               *v = fill(T * H * dv, -1, 1), *g = fill(T * H * dk, -0.3, 0),
               *b = fill(T * H, 0, 1), *dout = fill(T * H * dv, -1, 1);
        double *s0 = has_state ? fill(N * H * dv * dk, -0.1, 0.1) : NULL;
        double *ds = has_dstate ? fill(N * H * dv * dk, -0.1, 0.1) : NULL;
        double *out = fill(T * H * dv, 0, 0), *sT = fill(N * H * dv * dk, 0, 0);
        double *gq = fill(T * H * dk, 0, 0), *gk = fill(T * H * dk, 0, 0),
               *gv = fill(T * H * dv, 0, 0), *gg = fill(T * H * dk, 0, 0),
               *gb = fill(T * H, 0, 0), *gs = fill(N * H * dv * dk, 0, 0);
        if (kda_oracle_forward(N, st, H, dk, dv, q, k, v, g, b, s0, out, sT, 1) != 0) return 4;
        if (kda_oracle_backward(N, st, H, dk, dv, q, k, v, g, b, s0, dout, ds, gq, gk, gv, gg,
                                gb, gs, 1) != 0)
            return 5;
        const int64_t hdr[7] = {N, H, dk, dv, T, has_state, has_dstate};
        put(f, hdr, sizeof hdr);
        put(f, st, sizeof(int64_t) * (size_t)(N + 1));
        const size_t tk = sizeof(double) * (size_t)(T * H * dk), tv = sizeof(double) * (size_t)(T * H * dv),
                     th = sizeof(double) * (size_t)(T * H), ss = sizeof(double) * (size_t)(N * H * dv * dk);
        put(f, q, tk); put(f, k, tk); put(f, v, tv); put(f, g, tk); put(f, b, th); put(f, dout, tv);
        if (s0) put(f, s0, ss);
        if (ds) put(f, ds, ss);
        put(f, out, tv); put(f, sT, ss);
        put(f, gq, tk); put(f, gk, tk); put(f, gv, tv); put(f, gg, tk); put(f, gb, th); put(f, gs, ss);
        free(st); free(q); free(k); free(v); free(g); free(b); free(dout); free(s0); free(ds);
        free(out); free(sT); free(gq); free(gk); free(gv); free(gg); free(gb); free(gs);
    }
    /* bad arguments are rejected, not dereferenced */
    const int64_t bad[3] = {0, 5, 2};
    if (kda_oracle_forward(2, bad, 1, 4, 4, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1) != -1)
        return 6;
    fclose(f);
    return 0;
}
