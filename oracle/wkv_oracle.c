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

/*
 * Eagle / Finch backward: the gradients of a loss L through the forward
 * above, given dL/do and dL/dS_T.  This is reverse-mode differentiation of
 * the serial recurrence, one token at a time from the last to the first
 * (no chunking, no closed forms).  With S the state before token t (the one
 * o_t reads), beta = sum_i r_i u_i k_i and dbeta = sum_j do_j v_j:
 *     dr_i = sum_j do_j S_ij + u_i k_i dbeta
 *     dk_i = sum_j dS'_ij v_j + u_i r_i dbeta      (dS' = dL/dS after token t)
 *     dv_j = sum_i dS'_ij k_i + beta do_j
 *     dw_i = sum_j dS'_ij S_ij,   dx_i = dw_i w_i (-exp(x_i))
 *     du_i += r_i k_i dbeta
 *     dS_ij = w_i dS'_ij + r_i do_j                 (dL/dS before token t)
 * The forward states are needed in reverse order: every CK-th state is kept
 * and the states of one segment are recomputed from it.
 *   r, k, v, x, x_per_token, u, s_in   as in oracle_wkv_matrix
 *   d_o       [B][T][H][N]
 *   d_sT      [B][H][N][N], or NULL for zero
 *   d_r, d_k, d_v   [B][T][H][N]
 *   d_x       [B][T][H][N] (Finch), or [H][N] summed over b and t (Eagle)
 *   d_u       [H][N], summed over b and t
 *   d_s0      [B][H][N][N], or NULL
 * Sums over sequences are taken in sequence order after the parallel loop,
 * so results do not depend on the thread count.
 */
#define CK 64
int oracle_wkv_matrix_bwd(long B, long T, long H, long N,
                          const float *r, const float *k, const float *v,
                          const float *x, int x_per_token, const float *u,
                          const double *s_in, const double *d_o, const double *d_sT,
                          double *d_r, double *d_k, double *d_v, double *d_x,
                          double *d_u, double *d_s0, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || N < 1 || nthreads < 1) return ORACLE_BAD_ARG;
    long units = B * H, NN = N * N, nseg = (T + CK - 1) / CK;
    /* per-unit partial sums of d_u (and of Eagle's d_x) */
    double *pu = (double *)calloc((size_t)(units * N), sizeof(double));
    double *px = x_per_token ? NULL : (double *)calloc((size_t)(units * N), sizeof(double));
    if (!pu || (!x_per_token && !px)) {
        free(pu); free(px);
        return ORACLE_BAD_ARG;
    }
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (long unit = 0; unit < units; ++unit) {
        long b = unit / H, h = unit % H;
        double *ck = (double *)malloc(sizeof(double) * (size_t)((nseg + 1) * NN));
        double *seg = (double *)malloc(sizeof(double) * (size_t)(CK * NN));
        double *dS = (double *)malloc(sizeof(double) * (size_t)NN);
        double *wt = (double *)malloc(sizeof(double) * (size_t)N);
        if (!ck || !seg || !dS || !wt) {
            free(ck); free(seg); free(dS); free(wt);
#pragma omp atomic write
            bad = 1;
            continue;
        }
        const float *uh = u + h * N;
        /* forward, in dS as the running state: keep the state before tokens
           0, CK, 2 CK, ... */
        double *S = dS;
        for (long i = 0; i < NN; ++i) S[i] = s_in ? s_in[(b * H + h) * NN + i] : 0.0;
        for (long t = 0; t < T; ++t) {
            long base = ((b * T + t) * H + h) * N;
            const float *xt = x_per_token ? x + base : x + h * N;
            if (t % CK == 0)
                for (long i = 0; i < NN; ++i) ck[(t / CK) * NN + i] = S[i];
            for (long i = 0; i < N; ++i) wt[i] = exp(-exp((double)xt[i]));
            for (long i = 0; i < N; ++i)
                for (long j = 0; j < N; ++j)
                    S[i * N + j] = wt[i] * S[i * N + j] + (double)k[base + i] * (double)v[base + j];
        }
        /* reverse */
        for (long i = 0; i < NN; ++i) dS[i] = d_sT ? d_sT[(b * H + h) * NN + i] : 0.0;
        for (long sg = nseg - 1; sg >= 0; --sg) {
            long t0 = sg * CK, t1 = t0 + CK < T ? t0 + CK : T;
            /* states before tokens t0 .. t1-1 */
            for (long i = 0; i < NN; ++i) seg[i] = ck[sg * NN + i];
            for (long t = t0; t + 1 < t1; ++t) {
                long base = ((b * T + t) * H + h) * N;
                const float *xt = x_per_token ? x + base : x + h * N;
                const double *Sp = seg + (t - t0) * NN;
                double *Sn = seg + (t - t0 + 1) * NN;
                for (long i = 0; i < N; ++i) wt[i] = exp(-exp((double)xt[i]));
                for (long i = 0; i < N; ++i)
                    for (long j = 0; j < N; ++j)
                        Sn[i * N + j] = wt[i] * Sp[i * N + j] +
                                        (double)k[base + i] * (double)v[base + j];
            }
            for (long t = t1 - 1; t >= t0; --t) {
                long base = ((b * T + t) * H + h) * N;
                const float *rt = r + base, *kt = k + base, *vt = v + base;
                const float *xt = x_per_token ? x + base : x + h * N;
                const double *dot = d_o + base;
                const double *Sp = seg + (t - t0) * NN;
                for (long i = 0; i < N; ++i) wt[i] = exp(-exp((double)xt[i]));
                double beta = 0.0, dbeta = 0.0;
                for (long i = 0; i < N; ++i) beta += (double)rt[i] * (double)uh[i] * (double)kt[i];
                for (long j = 0; j < N; ++j) dbeta += dot[j] * (double)vt[j];
                for (long i = 0; i < N; ++i) {
                    double ar = 0.0, ak = 0.0, aw = 0.0;
                    for (long j = 0; j < N; ++j) {
                        ar += dot[j] * Sp[i * N + j];
                        ak += dS[i * N + j] * (double)vt[j];
                        aw += dS[i * N + j] * Sp[i * N + j];
                    }
                    d_r[base + i] = ar + (double)uh[i] * (double)kt[i] * dbeta;
                    d_k[base + i] = ak + (double)uh[i] * (double)rt[i] * dbeta;
                    double dx = aw * wt[i] * (-exp((double)xt[i]));
                    if (x_per_token) d_x[base + i] = dx;
                    else px[unit * N + i] += dx;
                    pu[unit * N + i] += (double)rt[i] * (double)kt[i] * dbeta;
                }
                for (long j = 0; j < N; ++j) {
                    double av = 0.0;
                    for (long i = 0; i < N; ++i) av += dS[i * N + j] * (double)kt[i];
                    d_v[base + j] = av + beta * dot[j];
                }
                for (long i = 0; i < N; ++i)
                    for (long j = 0; j < N; ++j)
                        dS[i * N + j] = wt[i] * dS[i * N + j] + (double)rt[i] * dot[j];
            }
        }
        if (d_s0)
            for (long i = 0; i < NN; ++i) d_s0[(b * H + h) * NN + i] = dS[i];
        free(ck); free(seg); free(dS); free(wt);
    }
    if (!bad) {
        for (long h = 0; h < H; ++h)
            for (long i = 0; i < N; ++i) {
                double su = 0.0, sx = 0.0;
                for (long b = 0; b < B; ++b) {
                    su += pu[(b * H + h) * N + i];
                    if (!x_per_token) sx += px[(b * H + h) * N + i];
                }
                d_u[h * N + i] = su;
                if (!x_per_token) d_x[h * N + i] = sx;
            }
    }
    free(pu); free(px);
    return bad ? ORACLE_BAD_ARG : ORACLE_OK;
}

/*
 * Output epilogue of Eagle / Finch time mixing (RWKV-5/6 summary, 4.1.2
 * "Eagle time mixing": a LayerNorm on each of the h heads separately, i.e. a
 * GroupNorm over h groups, and a SiLU gate on the attention output, before
 * the output weights):
 *     y = (LayerNorm_head(o) * ln_w + ln_b) * silu(g),   silu(g) = g / (1 + e^-g),
 * with the mean and the (biased) variance over the N channels of one head
 * of one token, and eps added to the variance.
 *   o, g      [rows][H][N]   (rows = B * T)
 *   ln_w, ln_b  [H][N]
 *   y         [rows][H][N]
 */
int oracle_norm_gate(long rows, long H, long N, const double *o, const float *g,
                     const float *ln_w, const float *ln_b, double eps, double *y,
                     int nthreads)
{
    if (rows < 0 || H < 1 || N < 1 || nthreads < 1) return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (long unit = 0; unit < rows * H; ++unit) {
        long h = unit % H;
        const double *ou = o + unit * N;
        double mean = 0.0, var = 0.0;
        for (long i = 0; i < N; ++i) mean += ou[i];
        mean /= (double)N;
        for (long i = 0; i < N; ++i) var += (ou[i] - mean) * (ou[i] - mean);
        var /= (double)N;
        double rstd = 1.0 / sqrt(var + eps);
        for (long i = 0; i < N; ++i) {
            double gi = (double)g[unit * N + i];
            double silu = gi / (1.0 + exp(-gi));
            double n = (ou[i] - mean) * rstd * (double)ln_w[h * N + i] + (double)ln_b[h * N + i];
            y[unit * N + i] = n * silu;
        }
    }
    return ORACLE_OK;
}

/*
 * Finch decay producer (RWKV-5/6 summary: 4.1.1 "Eagle token shift", the
 * linear interpolation between x_t and x_{t-1} with a learned mix per
 * channel; 4.2.1 "Finch token shift", the data-dependent interpolation
 * (ddlerp) whose mix is a learned vector lam plus a low-rank (LoRA) term
 * with A in R^{D x R1}, B in R^{R1 x D}, the LoRA taking the Eagle-style
 * shifted value, made with mu_x, as its input; LoRA_omega with
 * A in R^{D x 64}, B in R^{64 x D}; 4.2.2 "Finch time mixing": the decay
 * varies per token and channel, LoRA applied again after the interpolation).
 * No formula is printed; the reading taken, per sequence and token t, with
 * x_{-1} = shift (zeros when NULL):
 *     dx  = x_{t-1} - x_t
 *     y   = x_t + dx * mu_x                    (Eagle-style lerp)
 *     m   = lam + act(y A1) B1                 (LoRA of the mix)
 *     z   = x_t + dx * m                       (ddlerp)
 *     d_t = omega + act(z A2) B2               (LoRA_omega: the decay logit)
 * act is the identity (act = 0) or tanh (act = 1); w_t = exp(-exp(d_t)) is
 * then the Finch decay of the WKV above.  Products are plain sums in order.
 *   x       [B][T][D]      shift [B][D] or NULL
 *   mu_x, lam, omega [D]
 *   A1 [D][R1]  B1 [R1][D]  A2 [D][R2]  B2 [R2][D]
 *   d       [B][T][D] output
 */
int oracle_decay_lora(long B, long T, long D, long R1, long R2, const float *x,
                      const float *shift, const float *mu_x, const float *lam,
                      const float *A1, const float *B1, const float *omega,
                      const float *A2, const float *B2, int act, double *d, int nthreads)
{
    if (B < 0 || T < 0 || D < 1 || R1 < 1 || R2 < 1 || (act != 0 && act != 1) || nthreads < 1)
        return ORACLE_BAD_ARG;
    int bad = 0;
#pragma omp parallel num_threads(nthreads) reduction(|| : bad)
    {
        double *dx = malloc(sizeof(double) * D), *y = malloc(sizeof(double) * D);
        double *z = malloc(sizeof(double) * D);
        double *h1 = malloc(sizeof(double) * R1), *h2 = malloc(sizeof(double) * R2);
        if (!dx || !y || !z || !h1 || !h2) {
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (long bt = 0; bt < B * T; ++bt) {
                long b = bt / T, t = bt % T;
                const float *xt = x + bt * D;
                for (long i = 0; i < D; ++i) {
                    double prev = t > 0 ? (double)xt[i - D] : (shift ? (double)shift[b * D + i] : 0.0);
                    dx[i] = prev - (double)xt[i];
                    y[i] = (double)xt[i] + dx[i] * (double)mu_x[i];
                }
                for (long j = 0; j < R1; ++j) {
                    double s = 0.0;
                    for (long i = 0; i < D; ++i) s += y[i] * (double)A1[i * R1 + j];
                    h1[j] = act ? tanh(s) : s;
                }
                for (long i = 0; i < D; ++i) {
                    double m = (double)lam[i];
                    for (long j = 0; j < R1; ++j) m += h1[j] * (double)B1[j * D + i];
                    z[i] = (double)xt[i] + dx[i] * m;
                }
                for (long j = 0; j < R2; ++j) {
                    double s = 0.0;
                    for (long i = 0; i < D; ++i) s += z[i] * (double)A2[i * R2 + j];
                    h2[j] = act ? tanh(s) : s;
                }
                for (long i = 0; i < D; ++i) {
                    double s = (double)omega[i];
                    for (long j = 0; j < R2; ++j) s += h2[j] * (double)B2[j * D + i];
                    d[bt * D + i] = s;
                }
            }
        }
        free(dx); free(y); free(z); free(h1); free(h2);
    }
    return bad ? ORACLE_BAD_ARG : ORACLE_OK;
}
