/*
 * gdn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, token-by-token fp64 CPU evaluation of the gated delta rule
 * (Gated DeltaNet forward), used as the parity oracle for the GPU library.
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this code.  It shares no source, header or helper with
 * the GPU library.
 *
 * What it computes (SANA-Streaming, paperpeel page, section 2.1 "Frame-wise
 * Gated DeltaNet for Global Accumulated Memory": each GDN head keeps a
 * fixed-size recurrent state corrected by the delta rule of Gated DeltaNet
 * [35] and carried across streaming chunks; appendix G.3 gives the roles of
 * the decay gate alpha and the write gate beta.  The update equation itself
 * did not survive on the page, so the token-wise reading is used):
 *
 *   per (b, h), with state S (d_v x d_k) and unit-normalised q_t, k_t:
 *       S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *       o_t = S_t q_t
 *
 * The state is stored transposed, M = S^T with shape [d_k][d_v], so that
 * element (i, j) is the weight from key dimension i to value dimension j.
 * Expanding the product gives the equivalent per-token steps used below:
 *       y   = M^T k_t                       (= S_{t-1} k_t)
 *       u   = beta_t (v_t - alpha_t y)
 *       M  <- alpha_t M + k_t u^T
 *       o_t = M^T q_t
 * Columns j of M never mix, so work is split over (b, h, column block)
 * without changing any arithmetic.
 *
 * Backward scan (bidirectional GDN: SANA-Streaming section 4.1 runs a forward
 * scan from the previous cache and a backward scan within the chunk; section
 * 2.3 "Efficient GDN Kernel" combines the forward and reverse histories for
 * the output): the same recurrence over the tokens in reverse order, from a
 * zero state, each token with its own alpha_t, beta_t:
 *       S^b_t = alpha_t S^b_{t+1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *       o^b_t = S^b_t q_t,   S^b_T = 0.
 * gdn_oracle_scan with reverse = 1 is that loop (t = T-1 down to 0); the
 * bidirectional output o^f_t + o^b_t is formed by the Python wrapper.
 *
 * L2 normalisation (when qk_l2norm != 0): x_hat = x / sqrt(sum x^2 + eps),
 * then q is multiplied by `scale`.
 *
 * Parity pins for every function here live in tests/test_oracle_pins.py:
 * closed forms (beta = 0, orthonormal keys, identical keys, d_k = 1), an
 * explicitly unrolled product of d_k x d_k matrices, split invariance,
 * per-step identities, and a hand-derived worked example in tests/golden/.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_COLBLOCK 16

/* Normalise one vector of length n into dst (fp64). */
static void l2_unit(const double* src, double* dst, long n, double eps, double mult) {
    double ss = 0.0;
    for (long i = 0; i < n; ++i) ss += src[i] * src[i];
    double r = mult / sqrt(ss + eps);
    for (long i = 0; i < n; ++i) dst[i] = src[i] * r;
}

/*
 * One (b, h, column block) work item: runs the token recurrence over all T
 * tokens for value columns [j0, j1).
 */
static void run_item(const double* q, const double* k, const double* v,
                     const double* alpha, const double* beta,
                     const double* m_in, double* out, double* m_out,
                     long T, long dk, long dv, long j0, long j1,
                     int qk_l2norm, double scale, double eps, int reverse,
                     double* M, double* kh, double* qh) {
    long w = j1 - j0;
    for (long i = 0; i < dk; ++i)
        for (long j = 0; j < w; ++j)
            M[i * w + j] = m_in ? m_in[i * dv + j0 + j] : 0.0;

    for (long n = 0; n < T; ++n) {
        const long t = reverse ? T - 1 - n : n;  /* token visited n-th */
        const double* qt = q + t * dk;
        const double* kt = k + t * dk;
        const double* vt = v + t * dv;
        if (qk_l2norm) {
            l2_unit(kt, kh, dk, eps, 1.0);
            l2_unit(qt, qh, dk, eps, scale);
        } else {
            for (long i = 0; i < dk; ++i) { kh[i] = kt[i]; qh[i] = qt[i] * scale; }
        }
        double a = alpha[t], b = beta[t];
        for (long j = 0; j < w; ++j) {
            double y = 0.0;                      /* y_j = sum_i M[i][j] k_i */
            for (long i = 0; i < dk; ++i) y += M[i * w + j] * kh[i];
            double u = b * (vt[j0 + j] - a * y); /* delta-rule write value */
            double o = 0.0;
            for (long i = 0; i < dk; ++i) {
                double mij = a * M[i * w + j] + kh[i] * u;
                M[i * w + j] = mij;
                o += mij * qh[i];                /* readout with the new state */
            }
            out[t * dv + j0 + j] = o;
        }
    }
    if (m_out)
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < w; ++j)
                m_out[i * dv + j0 + j] = M[i * w + j];
}

/*
 * gdn_oracle_scan: full scan over B*H independent heads, tokens in order
 * (reverse = 0, the forward recurrence) or in reverse (reverse = 1, the
 * backward scan above).
 *   q, k     [B][H][T][dk]   fp64
 *   v        [B][H][T][dv]   fp64
 *   alpha    [B][H][T]       decay in (0, 1]
 *   beta     [B][H][T]       write strength
 *   state_in [B][H][dk][dv]  or NULL for a zero state
 *   out      [B][H][T][dv]
 *   state_out[B][H][dk][dv]  or NULL; must not alias state_in
 *   nthreads <= 0 uses the OpenMP default.
 * Returns 0, or -1 on a bad argument.
 */
int gdn_oracle_scan(const double* q, const double* k, const double* v,
                    const double* alpha, const double* beta,
                    const double* state_in, double* out, double* state_out,
                    long B, long H, long T, long dk, long dv,
                    int qk_l2norm, double scale, double eps, int reverse, int nthreads) {
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
    if (T > 0 && (!q || !k || !v || !alpha || !beta || !out)) return -1;
    if (state_out && state_in && state_out == state_in) return -1;
    long nblk = (dv + ORACLE_COLBLOCK - 1) / ORACLE_COLBLOCK;
    long items = B * H * nblk;
    int err = 0;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
    {
        double* M = (double*)malloc(sizeof(double) * (size_t)dk * ORACLE_COLBLOCK);
        double* kh = (double*)malloc(sizeof(double) * (size_t)dk);
        double* qh = (double*)malloc(sizeof(double) * (size_t)dk);
        if (!M || !kh || !qh) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            err = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (long it = 0; it < items; ++it) {
                long bh = it / nblk, blk = it % nblk;
                long j0 = blk * ORACLE_COLBLOCK;
                long j1 = j0 + ORACLE_COLBLOCK < dv ? j0 + ORACLE_COLBLOCK : dv;
                size_t tk = (size_t)bh * T * dk, tv = (size_t)bh * T * dv;
                size_t ts = (size_t)bh * T, ss = (size_t)bh * dk * dv;
                run_item(q + tk, k + tk, v + tv, alpha + ts, beta + ts,
                         state_in ? state_in + ss : NULL, out + tv,
                         state_out ? state_out + ss : NULL,
                         T, dk, dv, j0, j1, qk_l2norm, scale, eps, reverse, M, kh, qh);
            }
        }
        free(M); free(kh); free(qh);
    }
    return err ? -2 : 0;
}

/* gdn_oracle_fwd: the forward scan (gdn_oracle_scan with reverse = 0). */
int gdn_oracle_fwd(const double* q, const double* k, const double* v,
                   const double* alpha, const double* beta,
                   const double* state_in, double* out, double* state_out,
                   long B, long H, long T, long dk, long dv,
                   int qk_l2norm, double scale, double eps, int nthreads) {
    return gdn_oracle_scan(q, k, v, alpha, beta, state_in, out, state_out, B, H, T, dk, dv,
                           qk_l2norm, scale, eps, 0, nthreads);
}

/*
 * gdn_oracle_gates: the decay and write gates from their logits, n values.
 * SANA-Streaming (paperpeel page, appendix G.3 "Gate parameterization") names
 * a frame-wise decay gate, a token-wise write gate and an output gate but the
 * formulas did not survive on the page; the maps used are those the benchmark
 * inputs are drawn with:
 *     alpha = exp(-softplus(a)),  softplus(a) = log(1 + exp(a))
 *     beta  = 1 / (1 + exp(-b))
 * softplus is evaluated as max(a, 0) + log1p(exp(-|a|)), the same number
 * without overflow of exp for large a.
 */
void gdn_oracle_gates(const double* a, const double* b, double* alpha, double* beta, long n) {
    for (long i = 0; i < n; ++i) {
        double sp = (a[i] > 0.0 ? a[i] : 0.0) + log1p(exp(-fabs(a[i])));
        alpha[i] = exp(-sp);
        beta[i] = 1.0 / (1.0 + exp(-b[i]));
    }
}

int gdn_oracle_abi_version(void) { return 3; }
