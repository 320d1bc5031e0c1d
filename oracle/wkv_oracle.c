/*
 * wkv_oracle.c -- plain fp64 CPU reference for the RWKV WKV recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file or the library built from it; only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark do.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * Every loop below is the serial recurrence written out one token at a time,
 * in double precision, with no chunking, no log-domain rescaling and no
 * reordering beyond what the definitions state.  Independent units
 * (batch x channel, or batch x head) are spread over OpenMP threads; the work
 * inside a unit is strictly serial, so results do not depend on the thread
 * count.
 *
 * Sources (the pages print prose only; their equation slots are empty, so
 * the exact formulas are the plainest reading of that prose):
 *
 *  RWKV-4  -- RWKV paper summary (cafeforensic.com, zhuanlan/310315):
 *    section "Temporal structure for sequential data processing": the time
 *    decay e^{-w} and the current-token bonus e^{u} of the WKV (eq. 14);
 *    section "Transformer-like parallelization": wkv_t is a serial scan,
 *    O(BTd).  The WKV output is the decayed weighted average
 *        y_t = (sum_{i<t} e^{-(t-1-i)w + k_i} v_i + e^{u+k_t} v_t)
 *            / (sum_{i<t} e^{-(t-1-i)w + k_i}     + e^{u+k_t}),
 *    evaluated here through the numerator / denominator recurrences
 *        Num_t = e^{-w} Num_{t-1} + e^{k_t} v_t,
 *        Den_t = e^{-w} Den_{t-1} + e^{k_t}.
 *    The values are unscaled: valid while every exponent fits a double
 *    (|k| + |u| well below 700).
 *
 *  Eagle / Finch -- RWKV-5/6 (Eagle and Finch) summary (blob.wenxiaobai.com):
 *    section 4 (notation: per-head row vectors of size D/h, matrices act on
 *    the right); 4.1.2 "Eagle time mixing": w = exp(-exp(omega)) in (0,1);
 *    the state is a sum of k^T v, each key channel decayed by its w every
 *    step; the learned bonus u scales the current token's k^T v, which is
 *    added to the state before the receptance r multiplies it like a query;
 *    4.2.2 "Finch time mixing": w_t varies per token and channel.  Per head:
 *        o_t      = r_t (S_{t-1} + diag(u) k_t^T v_t)
 *        S_t      = diag(w_t) S_{t-1} + k_t^T v_t,   w_t = exp(-exp(x_t)),
 *    with S[i][j]: i = key channel, j = value channel.  Eagle is the case
 *    where x_t = omega for every t.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG (-1)

/*
 * RWKV-4 forward over B sequences of T tokens and C channels.
 *   k, v      [B][T][C] (float values, promoted to double)
 *   w         [C] decay rate (the per-step factor is e^{-w})
 *   u         [C] bonus
 *   num_in, den_in  [B][C] history numerator / denominator, or NULL for an
 *             empty history (both zero)
 *   y         [B][T][C] output
 *   scale     [B][T][C] or NULL: the same weighted average taken over |v|,
 *             the natural size of y for relative error checks; a non-empty
 *             history contributes |num_in| to it
 *   num_out, den_out [B][C] or NULL: the state after the last token
 */
int oracle_rwkv4_fwd(long B, long T, long C,
                     const float *k, const float *v,
                     const float *w, const float *u,
                     const double *num_in, const double *den_in,
                     double *y, double *scale,
                     double *num_out, double *den_out, int nthreads)
{
    if (B < 0 || T < 0 || C < 0 || nthreads < 1) return ORACLE_BAD_ARG;
    long units = B * C;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (long unit = 0; unit < units; ++unit) {
        long b = unit / C, c = unit % C;
        double num = num_in ? num_in[b * C + c] : 0.0;
        double den = den_in ? den_in[b * C + c] : 0.0;
        double absnum = fabs(num);
        double decay = exp(-(double)w[c]);
        double bonus = (double)u[c];
        for (long t = 0; t < T; ++t) {
            long idx = (b * T + t) * C + c;
            double kt = (double)k[idx], vt = (double)v[idx];
            double cur = exp(bonus + kt);
            y[idx] = (num + cur * vt) / (den + cur);
            if (scale) scale[idx] = (absnum + cur * fabs(vt)) / (den + cur);
            double ek = exp(kt);
            num = decay * num + ek * vt;
            den = decay * den + ek;
            absnum = decay * absnum + ek * fabs(vt);
        }
        if (num_out) num_out[b * C + c] = num;
        if (den_out) den_out[b * C + c] = den;
    }
    return ORACLE_OK;
}

/*
 * Eagle / Finch forward, one head at a time, one token at a time.
 *   r, k, v   [B][T][H][N]
 *   x         decay logit: [B][T][H][N] when x_per_token != 0 (Finch),
 *             [H][N] otherwise (Eagle: x = omega for every token)
 *   u         [H][N] bonus
 *   s_in      [B][H][N][N] initial state, or NULL for zeros
 *   o         [B][T][H][N] output
 *   s_out     [B][H][N][N] final state (may be NULL)
 */
int oracle_wkv_matrix(long B, long T, long H, long N,
                      const float *r, const float *k, const float *v,
                      const float *x, int x_per_token, const float *u,
                      const double *s_in, double *o, double *s_out,
                      int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || N < 1 || nthreads < 1) return ORACLE_BAD_ARG;
    long units = B * H;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (long unit = 0; unit < units; ++unit) {
        long b = unit / H, h = unit % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)(N * N));
        double *wt = (double *)malloc(sizeof(double) * (size_t)N);
        if (!S || !wt) {
            free(S); free(wt);
#pragma omp atomic write
            bad = 1;
            continue;
        }
        for (long i = 0; i < N * N; ++i)
            S[i] = s_in ? s_in[(b * H + h) * N * N + i] : 0.0;
        for (long t = 0; t < T; ++t) {
            long base = ((b * T + t) * H + h) * N;
            const float *rt = r + base, *kt = k + base, *vt = v + base;
            const float *xt = x_per_token ? x + base : x + h * N;
            const float *uh = u + h * N;
            /* per-channel decay of this token: w = exp(-exp(x)) */
            for (long i = 0; i < N; ++i) wt[i] = exp(-exp((double)xt[i]));
            /* bonus term: r_t diag(u) k_t^T = sum_i r_i u_i k_i */
            double ruk = 0.0;
            for (long i = 0; i < N; ++i)
                ruk += (double)rt[i] * (double)uh[i] * (double)kt[i];
            /* output from the previous state plus the current token's bonus */
            for (long j = 0; j < N; ++j) {
                double acc = 0.0;
                for (long i = 0; i < N; ++i) acc += (double)rt[i] * S[i * N + j];
                o[base + j] = acc + ruk * (double)vt[j];
            }
            /* state update: decay each key row, add k^T v */
            for (long i = 0; i < N; ++i)
                for (long j = 0; j < N; ++j)
                    S[i * N + j] = wt[i] * S[i * N + j] + (double)kt[i] * (double)vt[j];
        }
        if (s_out)
            for (long i = 0; i < N * N; ++i) s_out[(b * H + h) * N * N + i] = S[i];
        free(S);
        free(wt);
    }
    return bad ? ORACLE_BAD_ARG : ORACLE_OK;
}
