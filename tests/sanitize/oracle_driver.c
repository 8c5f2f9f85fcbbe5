/*
 * Runs every entry point of the CPU oracle (oracle/kda_oracle.c) on small
 * seeded inputs, edge sizes included, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer: any out-of-bounds access, use after free, leak
 * or undefined operation aborts the run.  A few identities are checked on the
 * way (they are pinned properly in tests/test_oracle_pins.py); exit code 0
 * means everything ran clean.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda_oracle.h"

static unsigned long long rng_state = 0x9e3779b97f4a7c15ull;
static double urand(void) /* uniform in [0, 1), xorshift64* */
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 2685821657736338717ull) >> 11) / 9007199254740992.0;
}
static double *arr(long n, double lo, double hi)
{
    double *a = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    long i;
    for (i = 0; i < n; ++i) a[i] = lo + (hi - lo) * urand();
    return a;
}
static int fails = 0;
static void check(int cond, const char *what)
{
    if (!cond) {
        fprintf(stderr, "FAILED: %s\n", what);
        ++fails;
    }
}

static void run_fwd_bwd(long B, long T, long H, long HV, long K, long V)
{
    const long nq = B * T * H * K, nv = B * T * HV * V, ng = B * T * HV * K, nb = B * T * HV;
    const long ns = B * HV * K * V, every = 2, NS = T / every;
    double *q = arr(nq, -1, 1), *k = arr(nq, -1, 1), *v = arr(nv, -1, 1);
    double *g = arr(ng, -5, 0), *beta = arr(nb, 0, 1), *S0 = arr(ns, -0.5, 0.5);
    double *o = arr(nv, 0, 0), *S = arr(ns, 0, 0), *snaps = arr(B * NS * HV * K * V, 0, 0);
    double *dout = arr(nv, -1, 1), *dST = arr(ns, -1, 1);
    double *dq = arr(nq, 0, 0), *dk = arr(nq, 0, 0), *dv = arr(nv, 0, 0), *dg = arr(ng, 0, 0);
    double *db = arr(nb, 0, 0), *dS0 = arr(ns, 0, 0);
    check(kda_oracle_fwd(q, k, v, g, beta, S0, o, S, B, T, H, HV, K, V, 0.0) == 0, "fwd");
    check(kda_oracle_fwd_snapshots(q, k, v, g, beta, NULL, o, S, snaps, every, B, T, H, HV, K, V, 0.3) == 0,
          "fwd snapshots");
    if (T > 0 && T % every == 0 && B > 0)
        check(memcmp(snaps + ((B - 1) * NS + NS - 1) * HV * K * V, S + (B - 1) * HV * K * V,
                     (size_t)(HV * K * V) * sizeof(double)) == 0, "last snapshot equals the final state");
    check(kda_oracle_bwd(q, k, v, g, beta, S0, dout, dST, dq, dk, dv, dg, db, dS0, B, T, H, HV, K, V, 0.0) == 0,
          "bwd");
    check(kda_oracle_bwd(q, k, v, g, beta, NULL, dout, NULL, dq, dk, dv, dg, db, NULL, B, T, H, HV, K, V, 0.0) == 0,
          "bwd without states");
    free(q); free(k); free(v); free(g); free(beta); free(S0); free(o); free(S); free(snaps);
    free(dout); free(dST); free(dq); free(dk); free(dv); free(dg); free(db); free(dS0);
}

static void run_layer(long B, long T, long H, long HV, long K, long V, long KW)
{
    const long C = 2 * H * K + HV * V;
    double *x = arr(B * T * C, -2, 2), *w = arr(C * KW, -1, 1), *cs = arr(B * C * KW, -1, 1);
    double *z = arr(B * T * HV * K, -3, 3), *al = arr(HV, -1, 1), *dt = arr(HV * K, -1, 1);
    double *bl = arr(B * T * HV, -2, 2);
    double *q = arr(B * T * H * K, 0, 0), *k = arr(B * T * H * K, 0, 0), *v = arr(B * T * HV * V, 0, 0);
    double *g = arr(B * T * HV * K, 0, 0), *bo = arr(B * T * HV, 0, 0);
    double *st = arr(B * HV * K * V, 0, 0), *out = arr(B * HV * V, 0, 0), *y = arr(B * T * HV * V, 0, 0);
    double *yc = arr(B * C, 0, 0);
    long i;
    int bounded;
    for (bounded = 0; bounded < 2; ++bounded) {
        check(kda_oracle_prefill_prologue(x, w, cs, KW, 1, 1e-6, z, al, dt, bounded, -5.0, bl, 1, q, k, v, g, bo,
                                          B, T, H, HV, K, V) == 0, "prologue");
        for (i = 0; i < B * T * HV * K; ++i) check(g[i] <= 0.0, "gate is a decay");
        check(kda_oracle_prefill_prologue(x, NULL, NULL, 0, 0, 0.0, z, NULL, NULL, bounded, -5.0, bl, 0, q, k, v,
                                          g, bo, B, T, H, HV, K, V) == 0, "prologue, no stages");
        if (T > 0)
            check(kda_oracle_decode_step(x, w, cs, KW, 1, 1e-6, z, al, dt, bounded, -5.0, bl, 1, st, out,
                                         B, H, HV, K, V, 0.0) == 0, "decode step");
        check(kda_oracle_gate(z, al, dt, bounded, -5.0, g, B * T, HV, K) == 0, "gate");
    }
    if (T > 0) check(kda_oracle_conv_update(cs, x, w, yc, B, C, KW) == 0, "conv update"); /* x holds B rows */
    check(kda_oracle_l2norm_rows(x, B * T * C / K, K, 1e-6) == 0, "l2norm rows");
    check(kda_oracle_output_gate(v, v, y, B * T * HV, V, 1e-6) == 0, "output gate");
    free(x); free(w); free(cs); free(z); free(al); free(dt); free(bl); free(q); free(k); free(v);
    free(g); free(bo); free(st); free(out); free(y); free(yc);
}

int main(void)
{
    long shapes[][6] = {{1, 5, 1, 1, 3, 2}, {2, 4, 1, 2, 4, 3}, {1, 1, 2, 4, 2, 2}, {1, 0, 1, 1, 2, 2},
                        {0, 3, 1, 1, 2, 2}, {2, 7, 2, 2, 8, 5}};
    size_t i;
    for (i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i) {
        long *s = shapes[i];
        run_fwd_bwd(s[0], s[1], s[2], s[3], s[4], s[5]);
        if (s[4] >= 2) run_layer(s[0], s[1], s[2], s[3], s[4], s[5], 4);
        run_layer(s[0], s[1], s[2], s[3], s[4] + 1, s[5], 1);
    }
    check(kda_oracle_fwd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 2, 3, 1, 1, 0.0) == 1,
          "rejects HV % H != 0");
    printf("oracle driver: %d failure(s)\n", fails);
    return fails ? 1 : 0;
}
