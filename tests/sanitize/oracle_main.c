/*
 * Sanitizer driver for oracle/kda_oracle.c (built by tests/test_sanitizers.py
 * with -fsanitize=address,undefined; CPU only).  It runs every entry point of
 * the oracle on small packed batches that include an empty sequence, a
 * one-token sequence and sequences longer than the backward's checkpoint
 * interval, with and without initial states, value-column subsets and unit
 * subsets, so that every loop bound and every optional-pointer branch is
 * exercised under the sanitizers.  Besides "no sanitizer report", it checks
 * facts that need no formula: a column subset reproduces those columns of the
 * full run, a unit subset those units, one decode step equals a one-token
 * sequence, and invalid arguments are refused.  Exit status 0 = all good.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_forward(const double*, const double*, const double*, const double*,
                       const double*, const double*, const int64_t*, int64_t, int64_t,
                       int64_t, int64_t, int64_t, int64_t, const int64_t*, int64_t,
                       double*, double*, int);
int kda_oracle_decode_step(const double*, const double*, const double*, const double*,
                           const double*, double*, int64_t, int64_t, int64_t, int64_t,
                           double*, int);
int kda_oracle_backward(const double*, const double*, const double*, const double*,
                        const double*, const double*, const int64_t*, int64_t, int64_t,
                        int64_t, int64_t, const double*, const double*, const int64_t*,
                        int64_t, double*, double*, double*, double*, double*, double*, int);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
/* uniform in [-1, 1) from a 64-bit linear congruential generator */
static double urand(void) {
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng_state >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}
static double* fill(size_t n, double lo, double hi) {
    double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5 * (urand() + 1.0);
    return p;
}
static double* zeros(size_t n) { return (double*)calloc(n ? n : 1, sizeof(double)); }

static int fails = 0;
#define CHECK(c)                                                    \
    do {                                                            \
        if (!(c)) {                                                 \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++fails;                                                \
        }                                                           \
    } while (0)

int main(void) {
    enum { N = 4, H = 2, DK = 8, DV = 6 };
    const int64_t cu[N + 1] = {0, 0, 1, 71, 140};   /* lengths 0, 1, 70, 69 */
    const int64_t T = cu[N];
    double* q = fill((size_t)T * H * DK, -1, 1);
    double* k = fill((size_t)T * H * DK, -0.4, 0.4);
    double* v = fill((size_t)T * H * DV, -1, 1);
    double* la = fill((size_t)T * H * DK, -5, 0);
    double* be = fill((size_t)T * H, 0, 1);
    double* s0 = fill((size_t)N * H * DK * DV, -0.1, 0.1);
    const size_t no = (size_t)T * H * DV, ns = (size_t)N * H * DK * DV;

    for (int with_s0 = 0; with_s0 < 2; ++with_s0) {
        const double* S0 = with_s0 ? s0 : NULL;
        double* o = zeros(no);
        double* st = zeros(ns);
        CHECK(kda_oracle_forward(q, k, v, la, be, S0, cu, N, H, DK, DV, 0, DV, NULL, 0, o, st, 2) == 0);
        for (size_t i = 0; i < no; ++i) CHECK(isfinite(o[i]));
        /* columns [2, 5) alone */
        double* oc = zeros(no);
        double* sc = zeros(ns);
        CHECK(kda_oracle_forward(q, k, v, la, be, S0, cu, N, H, DK, DV, 2, 5, NULL, 0, oc, sc, 1) == 0);
        for (int64_t t = 0; t < T * H; ++t)
            for (int j = 0; j < DV; ++j)
                CHECK(oc[t * DV + j] == ((j >= 2 && j < 5) ? o[t * DV + j] : 0.0));
        /* units (3, 1) and (1, 0) alone, without the state output */
        const int64_t units[4] = {3, 1, 1, 0};
        double* ou = zeros(no);
        CHECK(kda_oracle_forward(q, k, v, la, be, S0, cu, N, H, DK, DV, 0, DV, units, 2, ou, NULL, 1) == 0);
        for (int64_t t = 0; t < T; ++t)
            for (int h = 0; h < H; ++h) {
                const int in_unit = (t >= cu[3] && h == 1) || (t >= cu[1] && t < cu[2] && h == 0);
                for (int j = 0; j < DV; ++j) {
                    const size_t e = ((size_t)t * H + h) * DV + j;
                    CHECK(ou[e] == (in_unit ? o[e] : 0.0));
                }
            }
        /* backward, with and without dL/dS_T and dS0 */
        double* dO = fill(no, -1, 1);
        double* dST = fill(ns, -1, 1);
        for (int variant = 0; variant < 2; ++variant) {
            double* dq = zeros((size_t)T * H * DK);
            double* dk = zeros((size_t)T * H * DK);
            double* dv = zeros(no);
            double* dla = zeros((size_t)T * H * DK);
            double* db = zeros((size_t)T * H);
            double* ds0 = variant ? NULL : zeros(ns);
            CHECK(kda_oracle_backward(q, k, v, la, be, S0, cu, N, H, DK, DV, dO,
                                      variant ? NULL : dST, NULL, 0, dq, dk, dv, dla, db, ds0,
                                      2) == 0);
            for (size_t i = 0; i < (size_t)T * H * DK; ++i) CHECK(isfinite(dq[i]) && isfinite(dla[i]));
            free(dq); free(dk); free(dv); free(dla); free(db); free(ds0);
        }
        free(dO); free(dST); free(o); free(st); free(oc); free(sc); free(ou);
    }

    /* decode step on 3 requests == a one-token sequence each */
    {
        enum { B = 3 };
        double* S = fill((size_t)B * H * DK * DV, -0.1, 0.1);
        double* S1 = (double*)malloc(sizeof(double) * B * H * DK * DV);
        memcpy(S1, S, sizeof(double) * B * H * DK * DV);
        double* od = zeros((size_t)B * H * DV);
        double* of = zeros((size_t)B * H * DV);
        double* sf = zeros((size_t)B * H * DK * DV);
        const int64_t cud[B + 1] = {0, 1, 2, 3};
        CHECK(kda_oracle_decode_step(q, k, v, la, be, S1, B, H, DK, DV, od, 1) == 0);
        CHECK(kda_oracle_forward(q, k, v, la, be, S, cud, B, H, DK, DV, 0, DV, NULL, 0, of, sf, 1) == 0);
        CHECK(memcmp(od, of, sizeof(double) * B * H * DV) == 0);
        CHECK(memcmp(S1, sf, sizeof(double) * B * H * DK * DV) == 0);
        free(S); free(S1); free(od); free(of); free(sf);
    }

    /* invalid arguments are refused */
    {
        double* o = zeros(no);
        const int64_t bad[3] = {0, 5, 2};
        CHECK(kda_oracle_forward(q, k, v, la, be, NULL, bad, 2, H, DK, DV, 0, DV, NULL, 0, o, NULL, 1) != 0);
        CHECK(kda_oracle_forward(q, k, v, la, be, NULL, cu, N, H, DK, DV, 3, 3, NULL, 0, o, NULL, 1) != 0);
        CHECK(kda_oracle_forward(q, k, v, la, be, NULL, cu, N, 0, DK, DV, 0, DV, NULL, 0, o, NULL, 1) != 0);
        CHECK(kda_oracle_forward(NULL, k, v, la, be, NULL, cu, N, H, DK, DV, 0, DV, NULL, 0, o, NULL, 1) != 0);
        free(o);
    }
    free(q); free(k); free(v); free(la); free(be); free(s0);
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("oracle sanitizer driver: all checks passed\n");
    return 0;
}
