/*
 * The fp64 oracle (oracle/gdn_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer, on small inputs: argument errors, a closed form
 * (beta = 0: nothing is written, the state only decays, o_t = (prod alpha)
 * S_0 q^_t), split invariance (two calls with the state carried give the
 * same bits as one), and thread-count invariance (the column split does not
 * change any arithmetic).  Built and run by tests/test_sanitize.py; prints one
 * line per failed expectation and exits non-zero if any failed.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gdn_oracle_scan(const double* q, const double* k, const double* v, const double* alpha,
                    const double* beta, const double* state_in, double* out, double* state_out,
                    long B, long H, long T, long dk, long dv, int qk_l2norm, double scale, double eps,
                    int reverse, int nthreads);

static int g_fail = 0;
#define EXPECT(cond, msg)                                       \
    do {                                                        \
        if (!(cond)) { ++g_fail; printf("FAIL line %d: %s\n", __LINE__, msg); } \
    } while (0)

static unsigned long long g_rng = 88172645463325252ULL;
static double urand(void) {               /* xorshift64, uniform in [-1, 1) */
    g_rng ^= g_rng << 13; g_rng ^= g_rng >> 7; g_rng ^= g_rng << 17;
    return (double)(g_rng >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}
static double* arr(long n, double lo, double hi) {
    double* a = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (long i = 0; i < n; ++i) a[i] = lo + (hi - lo) * 0.5 * (urand() + 1.0);
    return a;
}

int main(void) {
    const long B = 2, H = 3, T = 37, dk = 8, dv = 20, Ts = 15;
    const double eps = 1e-6;
    double *q = arr(B * H * T * dk, -1, 1), *k = arr(B * H * T * dk, -1, 1), *v = arr(B * H * T * dv, -1, 1);
    double *al = arr(B * H * T, 0.8, 1.0), *be = arr(B * H * T, 0.0, 1.0), *s0 = arr(B * H * dk * dv, -0.3, 0.3);
    double *o1 = arr(B * H * T * dv, 0, 0), *o2 = arr(B * H * T * dv, 0, 0), *s1 = arr(B * H * dk * dv, 0, 0);
    double *s2 = arr(B * H * dk * dv, 0, 0);

    /* argument errors */
    EXPECT(gdn_oracle_scan(q, k, v, al, be, s0, o1, s1, -1, H, T, dk, dv, 1, 1.0, eps, 0, 1) == -1, "B < 0");
    EXPECT(gdn_oracle_scan(q, k, v, al, be, s0, o1, s1, B, H, T, 0, dv, 1, 1.0, eps, 0, 1) == -1, "dk = 0");
    EXPECT(gdn_oracle_scan(NULL, k, v, al, be, s0, o1, s1, B, H, T, dk, dv, 1, 1.0, eps, 0, 1) == -1, "q NULL");
    EXPECT(gdn_oracle_scan(q, k, v, al, be, s0, o1, s0, B, H, T, dk, dv, 1, 1.0, eps, 0, 1) == -1, "aliased state");
    EXPECT(gdn_oracle_scan(q, k, v, al, be, s0, o1, s1, B, H, 0, dk, dv, 1, 1.0, eps, 0, 1) == 0, "T = 0");
    EXPECT(memcmp(s0, s1, sizeof(double) * B * H * dk * dv) == 0, "T = 0 copies the state");

    /* split invariance: [0, Ts) then [Ts, T) with the state carried, against one call */
    EXPECT(gdn_oracle_scan(q, k, v, al, be, s0, o1, s1, B, H, T, dk, dv, 1, 1.0, eps, 0, 1) == 0, "one call");
    {
        const long T2 = T - Ts;
        double *qa = arr(B * H * Ts * dk, 0, 0), *ka = arr(B * H * Ts * dk, 0, 0), *va = arr(B * H * Ts * dv, 0, 0);
        double *aa = arr(B * H * Ts, 0, 0), *ba = arr(B * H * Ts, 0, 0), *oa = arr(B * H * Ts * dv, 0, 0);
        double *qb = arr(B * H * T2 * dk, 0, 0), *kb = arr(B * H * T2 * dk, 0, 0), *vb = arr(B * H * T2 * dv, 0, 0);
        double *ab = arr(B * H * T2, 0, 0), *bb = arr(B * H * T2, 0, 0), *ob = arr(B * H * T2 * dv, 0, 0);
        double* mid = arr(B * H * dk * dv, 0, 0);
        for (long bh = 0; bh < B * H; ++bh) {
            memcpy(qa + bh * Ts * dk, q + bh * T * dk, sizeof(double) * Ts * dk);
            memcpy(ka + bh * Ts * dk, k + bh * T * dk, sizeof(double) * Ts * dk);
            memcpy(va + bh * Ts * dv, v + bh * T * dv, sizeof(double) * Ts * dv);
            memcpy(aa + bh * Ts, al + bh * T, sizeof(double) * Ts);
            memcpy(ba + bh * Ts, be + bh * T, sizeof(double) * Ts);
            memcpy(qb + bh * T2 * dk, q + bh * T * dk + Ts * dk, sizeof(double) * T2 * dk);
            memcpy(kb + bh * T2 * dk, k + bh * T * dk + Ts * dk, sizeof(double) * T2 * dk);
            memcpy(vb + bh * T2 * dv, v + bh * T * dv + Ts * dv, sizeof(double) * T2 * dv);
            memcpy(ab + bh * T2, al + bh * T + Ts, sizeof(double) * T2);
            memcpy(bb + bh * T2, be + bh * T + Ts, sizeof(double) * T2);
        }
        EXPECT(gdn_oracle_scan(qa, ka, va, aa, ba, s0, oa, mid, B, H, Ts, dk, dv, 1, 1.0, eps, 0, 2) == 0, "part 1");
        EXPECT(gdn_oracle_scan(qb, kb, vb, ab, bb, mid, ob, s2, B, H, T2, dk, dv, 1, 1.0, eps, 0, 3) == 0, "part 2");
        int same = memcmp(s1, s2, sizeof(double) * B * H * dk * dv) == 0;
        for (long bh = 0; bh < B * H; ++bh) {
            same &= memcmp(o1 + bh * T * dv, oa + bh * Ts * dv, sizeof(double) * Ts * dv) == 0;
            same &= memcmp(o1 + bh * T * dv + Ts * dv, ob + bh * T2 * dv, sizeof(double) * T2 * dv) == 0;
        }
        EXPECT(same, "split invariance (bitwise)");
        free(qa); free(ka); free(va); free(aa); free(ba); free(oa);
        free(qb); free(kb); free(vb); free(ab); free(bb); free(ob); free(mid);
    }

    /* thread-count invariance, forward and reverse */
    for (int rev = 0; rev < 2; ++rev) {
        EXPECT(gdn_oracle_scan(q, k, v, al, be, s0, o1, s1, B, H, T, dk, dv, 1, 0.5, eps, rev, 1) == 0, "1 thread");
        EXPECT(gdn_oracle_scan(q, k, v, al, be, s0, o2, s2, B, H, T, dk, dv, 1, 0.5, eps, rev, 4) == 0, "4 threads");
        EXPECT(memcmp(o1, o2, sizeof(double) * B * H * T * dv) == 0, "outputs independent of threads");
        EXPECT(memcmp(s1, s2, sizeof(double) * B * H * dk * dv) == 0, "state independent of threads");
    }

    /* beta = 0: o_t = (alpha_0 ... alpha_t) S_0 q^_t, with M = S^T stored [dk][dv] */
    {
        double* zb = arr(B * H * T, 0, 0);
        EXPECT(gdn_oracle_scan(q, k, v, al, zb, s0, o1, s1, B, H, T, dk, dv, 1, 1.0, eps, 0, 2) == 0, "beta = 0");
        double worst = 0.0;
        for (long bh = 0; bh < B * H; ++bh) {
            double decay = 1.0;
            for (long t = 0; t < T; ++t) {
                decay *= al[bh * T + t];
                const double* qt = q + (bh * T + t) * dk;
                double n2 = 0.0;
                for (long i = 0; i < dk; ++i) n2 += qt[i] * qt[i];
                const double r = 1.0 / sqrt(n2 + eps);
                for (long j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (long i = 0; i < dk; ++i) acc += s0[(bh * dk + i) * dv + j] * qt[i] * r;
                    const double d = fabs(o1[(bh * T + t) * dv + j] - decay * acc);
                    if (d > worst) worst = d;
                }
            }
        }
        EXPECT(worst < 1e-12, "beta = 0 closed form");
        free(zb);
    }
    printf("oracle sanitize: %d failures\n", g_fail);
    free(q); free(k); free(v); free(al); free(be); free(s0); free(o1); free(o2); free(s1); free(s2);
    return g_fail ? 1 : 0;
}
