/*
 * gdn_oracle.c -- fp64 CPU oracle of the Gated DeltaNet (GDN) token mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or constant with the HIP path.
 *
 * What it computes, step by step, in the order of the definition:
 *
 *  1. Short causal depthwise convolution of width 4 over the raw q, k and v
 *     channels (hybrid-attention explainer, jianying88.com, section 3: the GDN
 *     layers add a short convolution of kernel width 4),
 *     followed by SiLU.  Tap 3 multiplies the current token; the three older
 *     rows come from a carried conv state or are zero.
 *  2. L2 normalisation of q and k per (token, QK head), eps = 1e-6 inside the
 *     square root.  v is not normalised.
 *  3. Gates per (token, V head): beta = sigmoid(b) is the write strength,
 *     alpha = exp(-c * softplus(a)) is the data-dependent forget gate
 *     (local-inference walkthrough, bjdmk.com.cn, section 2.1: alpha_t
 *     forgets, beta_t sets the write strength).
 *  4. The state update of section 2.1 of the same walkthrough,
 *        S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *     evaluated token by token in the equivalent "delta" form the walkthrough
 *     describes in words (the new value is corrected by what the memory
 *     already predicts):
 *        S <- alpha S;  p = S^T k;  S <- S + beta k (v - p)^T.
 *     S has d_k rows and d_v columns (the outer product k v^T fixes this).
 *  5. Readout o_t = q_scale * S_t^T q_t with the post-update state.
 *
 * Head sharing: V head h reads QK head h / (Hv / Hqk) (contiguous groups; the
 * explainer gives 16 QK heads shared by 48 V heads).
 *
 * All arithmetic is IEEE double; bf16 and fp32 inputs convert to double
 * exactly.  No blocking, chunking or reordering beyond the definition: the
 * only parallelism is over independent (sequence, V head) pairs.
 *
 * Every entry point also takes its inputs in double ("_f64" variants, or the
 * f64 flag), so that derivatives can be checked by finite differences.
 *
 * Backward (gdn_ref_prefill_backward): the gradient of
 *     L = sum_t <dO_t, o_t> + <dS_T, S_T>
 * with respect to every input (q, k, v, a, b, the conv weights and carried
 * conv rows, the initial state), by reverse-mode differentiation of the same
 * token-by-token definition, written out by hand: the state update is undone
 * step by step from the last token, and each step's local derivatives are the
 * chain rule applied to the five operations above.  Section 9 of the
 * architecture deep dive (alwayszhang.cn) names forward and backward kernels
 * of the chunked form (FlashQLA) as what training needs; no chunking is used
 * here.  All forward states of a (sequence, V head) are kept, so the
 * backward is meant for test sizes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* One input element as double: bf16 (f64 == 0) or double (f64 != 0). */
static double in_x(const void *p, int f64, long i)
{
    return f64 ? ((const double *)p)[i] : bf16_to_double(((const uint16_t *)p)[i]);
}
/* One gate pre-activation as double: fp32 (f64 == 0) or double. */
static double in_g(const void *p, int f64, long i)
{
    return f64 ? ((const double *)p)[i] : (double)((const float *)p)[i];
}

double gdn_ref_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* softplus(x) = log(1 + e^x), written so that it neither overflows nor
 * loses the small tail: max(x, 0) + log1p(e^{-|x|}). */
double gdn_ref_softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

double gdn_ref_silu(double x) { return x * gdn_ref_sigmoid(x); }

int gdn_ref_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Step 1: y[t][c] = sum_{j=0..3} w[c][j] * x[t-3+j][c], then SiLU.
 *   x     : bf16 rows, x[t*ldx + c] for t in [0, T), c in [0, nc)
 *   w     : bf16 [nc][4] (tap 3 = current token)
 *   hist  : bf16 rows hist[r*ldh + c], r = 0..2 oldest first (x[-3..-1]);
 *           NULL means zeros
 *   out   : double [T][nc]
 */
/* The conv alone (pre-activation y), inputs of either kind. */
static void conv_any(const void *x, long ldx, int T, int nc, const void *w,
                     const void *hist, long ldh, int f64, double *y_out)
{
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < nc; ++c) {
            double y = 0.0;
            for (int j = 0; j < 4; ++j) {
                int tau = t - 3 + j;
                double xv;
                if (tau >= 0)
                    xv = in_x(x, f64, (long)tau * ldx + c);
                else if (hist)
                    xv = in_x(hist, f64, (long)(3 + tau) * ldh + c);
                else
                    xv = 0.0;
                y += in_x(w, f64, (long)c * 4 + j) * xv;
            }
            y_out[(long)t * nc + c] = y;
        }
    }
}

static void conv_silu_any(const void *x, long ldx, int T, int nc, const void *w,
                          const void *hist, long ldh, int f64, double *out)
{
    conv_any(x, ldx, T, nc, w, hist, ldh, f64, out);
    for (long e = 0; e < (long)T * nc; ++e)
        out[e] = gdn_ref_silu(out[e]);
}

void gdn_ref_conv_silu(const uint16_t *x, long ldx, int T, int nc,
                       const uint16_t *w, const uint16_t *hist, long ldh,
                       double *out)
{
    conv_silu_any(x, ldx, T, nc, w, hist, ldh, 0, out);
}

/* Step 2: each row of x[T][n] divided by sqrt(sum of squares + eps). */
void gdn_ref_l2norm(double *x, int T, int n, double eps)
{
    for (int t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int i = 0; i < n; ++i)
            ss += x[(long)t * n + i] * x[(long)t * n + i];
        double r = 1.0 / sqrt(ss + eps);
        for (int i = 0; i < n; ++i)
            x[(long)t * n + i] *= r;
    }
}

/* Step 3: alpha_t = exp(-c softplus(a_t)), beta_t = sigmoid(b_t). */
static void gates_any(const void *a, const void *b, long ld, int T, double c,
                      int f64, double *alpha, double *beta)
{
    for (int t = 0; t < T; ++t) {
        alpha[t] = exp(-c * gdn_ref_softplus(in_g(a, f64, (long)t * ld)));
        beta[t] = gdn_ref_sigmoid(in_g(b, f64, (long)t * ld));
    }
}

void gdn_ref_gates(const float *a, const float *b, long ld, int T, double c,
                   double *alpha, double *beta)
{
    gates_any(a, b, ld, T, c, 0, alpha, beta);
}

/*
 * Steps 4-5 for one (sequence, V head), on already-prepared q^, k^, v^.
 *   qh, kh : double [T][dk];  vh : double [T][dv]
 *   alpha, beta : double [T]
 *   S      : double [dk][dv]; in = initial state, out = final state
 *   o      : double [T][dv]
 */
void gdn_ref_recurrence(const double *qh, const double *kh, const double *vh,
                        const double *alpha, const double *beta, int T, int dk,
                        int dv, double q_scale, double *S, double *o)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)dv);
    for (int t = 0; t < T; ++t) {
        const double *k = kh + (long)t * dk;
        const double *q = qh + (long)t * dk;
        const double *v = vh + (long)t * dv;
        /* forget: S <- alpha S */
        for (long e = 0; e < (long)dk * dv; ++e)
            S[e] *= alpha[t];
        /* what the (decayed) memory predicts for key k: p = S^T k */
        for (int j = 0; j < dv; ++j)
            p[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                p[j] += S[(long)i * dv + j] * k[i];
        /* write the corrected value: S <- S + beta k (v - p)^T */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[(long)i * dv + j] += beta[t] * k[i] * (v[j] - p[j]);
        /* read out with the updated state: o = q_scale S^T q */
        for (int j = 0; j < dv; ++j)
            o[(long)t * dv + j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                o[(long)t * dv + j] += S[(long)i * dv + j] * q[i];
        for (int j = 0; j < dv; ++j)
            o[(long)t * dv + j] *= q_scale;
    }
    free(p);
}

/*
 * Whole mixer over packed sequences.
 *   q, k          : bf16 [T_tot][Hqk][dk];  v : bf16 [T_tot][Hv][dv]
 *   a, b          : fp32 [T_tot][Hv]
 *   conv_w        : bf16 [C_tot][4], channels q | k | v
 *   conv_state_in : bf16 [N][3][C_tot] or NULL (zero history)
 *   state_in      : double [N][Hv][dk][dv] or NULL (zero state)
 *   cu_seqlens    : int32 [N+1]
 *   heads, n_heads: V heads to evaluate (NULL: all)
 *   o             : double [T_tot][Hv][dv] (only selected heads written)
 *   state_out     : double [N][Hv][dk][dv] or NULL (only selected heads)
 *   conv_state_out: bf16 [N][3][C_tot] or NULL: the last three raw input
 *                   rows of every channel, oldest first
 * Returns 0, or -1 on bad arguments.
 */
static int prefill_any(const void *q, const void *k, const void *v,
                       const void *a, const void *b, const void *conv_w,
                       const void *conv_state_in, const double *state_in,
                       const int32_t *cu_seqlens, int N, int Hqk, int Hv, int dk,
                       int dv, double gate_scale, double q_scale,
                       const int32_t *heads, int n_heads, int f64, double *o,
                       double *state_out)
{
    if (N < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hqk != 0)
        return -1;
    const int G = Hv / Hqk;
    const long C_tot = 2L * Hqk * dk + (long)Hv * dv;
    if (!heads)
        n_heads = Hv;
    long n_tasks = (long)N * n_heads;

#pragma omp parallel for schedule(dynamic, 1)
    for (long task = 0; task < n_tasks; ++task) {
        int s = (int)(task / n_heads);
        int h = heads ? heads[task % n_heads] : (int)(task % n_heads);
        int g = h / G;
        long t0 = cu_seqlens[s];
        int L = cu_seqlens[s + 1] - cu_seqlens[s];
        const long hist0 = (long)s * 3 * C_tot;  /* this sequence's carried rows */
        long cq = (long)g * dk, ck = (long)Hqk * dk + (long)g * dk,
             cv = 2L * Hqk * dk + (long)h * dv;
#define HIST_AT(ch) (conv_state_in ? (f64 ? (const void *)((const double *)conv_state_in + hist0 + (ch)) \
                                          : (const void *)((const uint16_t *)conv_state_in + hist0 + (ch))) : NULL)
#define X_AT(p, off) (f64 ? (const void *)((const double *)(p) + (off)) : (const void *)((const uint16_t *)(p) + (off)))
#define G_AT(p, off) (f64 ? (const void *)((const double *)(p) + (off)) : (const void *)((const float *)(p) + (off)))

        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        if (state_in)
            memcpy(S, state_in + ((long)s * Hv + h) * dk * dv, sizeof(double) * (size_t)dk * dv);
        else
            memset(S, 0, sizeof(double) * (size_t)dk * dv);

        if (L > 0) {
            double *qh = (double *)malloc(sizeof(double) * (size_t)L * dk);
            double *kh = (double *)malloc(sizeof(double) * (size_t)L * dk);
            double *vh = (double *)malloc(sizeof(double) * (size_t)L * dv);
            double *al = (double *)malloc(sizeof(double) * (size_t)L);
            double *be = (double *)malloc(sizeof(double) * (size_t)L);
            double *oh = (double *)malloc(sizeof(double) * (size_t)L * dv);
            conv_silu_any(X_AT(q, t0 * Hqk * dk + (long)g * dk), (long)Hqk * dk, L, dk,
                          X_AT(conv_w, cq * 4), HIST_AT(cq), C_tot, f64, qh);
            conv_silu_any(X_AT(k, t0 * Hqk * dk + (long)g * dk), (long)Hqk * dk, L, dk,
                          X_AT(conv_w, ck * 4), HIST_AT(ck), C_tot, f64, kh);
            conv_silu_any(X_AT(v, t0 * Hv * dv + (long)h * dv), (long)Hv * dv, L, dv,
                          X_AT(conv_w, cv * 4), HIST_AT(cv), C_tot, f64, vh);
            gdn_ref_l2norm(qh, L, dk, 1e-6);
            gdn_ref_l2norm(kh, L, dk, 1e-6);
            gates_any(G_AT(a, t0 * Hv + h), G_AT(b, t0 * Hv + h), Hv, L, gate_scale, f64, al, be);
            gdn_ref_recurrence(qh, kh, vh, al, be, L, dk, dv, q_scale, S, oh);
            for (int t = 0; t < L; ++t)
                memcpy(o + ((t0 + t) * Hv + h) * dv, oh + (long)t * dv, sizeof(double) * (size_t)dv);
            free(qh); free(kh); free(vh); free(al); free(be); free(oh);
        }
        if (state_out)
            memcpy(state_out + ((long)s * Hv + h) * dk * dv, S, sizeof(double) * (size_t)dk * dv);
        free(S);
    }
    return 0;
}

int gdn_ref_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const float *a, const float *b, const uint16_t *conv_w,
                    const uint16_t *conv_state_in, const double *state_in,
                    const int32_t *cu_seqlens, int N, int Hqk, int Hv, int dk,
                    int dv, double gate_scale, double q_scale,
                    const int32_t *heads, int n_heads, double *o,
                    double *state_out, uint16_t *conv_state_out)
{
    int rc = prefill_any(q, k, v, a, b, conv_w, conv_state_in, state_in, cu_seqlens, N, Hqk,
                         Hv, dk, dv, gate_scale, q_scale, heads, n_heads, 0, o, state_out);
    if (rc != 0)
        return rc;
    const long C_tot = 2L * Hqk * dk + (long)Hv * dv;

    /* carried conv state: raw rows x[L-3], x[L-2], x[L-1] of each sequence,
     * reaching back into the incoming history when L < 3 */
    if (conv_state_out) {
        for (int s = 0; s < N; ++s) {
            long t0 = cu_seqlens[s];
            int L = cu_seqlens[s + 1] - cu_seqlens[s];
            for (int r = 0; r < 3; ++r) {
                int tau = L - 3 + r;
                uint16_t *dst = conv_state_out + ((long)s * 3 + r) * C_tot;
                for (long c = 0; c < C_tot; ++c) {
                    uint16_t val;
                    if (tau >= 0) {
                        long t = t0 + tau;
                        if (c < (long)Hqk * dk)
                            val = q[t * Hqk * dk + c];
                        else if (c < 2L * Hqk * dk)
                            val = k[t * Hqk * dk + (c - (long)Hqk * dk)];
                        else
                            val = v[t * Hv * dv + (c - 2L * Hqk * dk)];
                    } else {
                        val = conv_state_in ? conv_state_in[((long)s * 3 + (3 + tau)) * C_tot + c] : 0;
                    }
                    dst[c] = val;
                }
            }
        }
    }
    return 0;
}

/* The same mixer with every input in double (q, k, v, conv_w, conv rows,
 * a, b): the forward that the finite-difference checks of the backward
 * perturb.  No conv state is emitted. */
int gdn_ref_prefill_f64(const double *q, const double *k, const double *v,
                        const double *a, const double *b, const double *conv_w,
                        const double *conv_state_in, const double *state_in,
                        const int32_t *cu_seqlens, int N, int Hqk, int Hv, int dk,
                        int dv, double gate_scale, double q_scale, double *o,
                        double *state_out)
{
    return prefill_any(q, k, v, a, b, conv_w, conv_state_in, state_in, cu_seqlens, N, Hqk,
                       Hv, dk, dv, gate_scale, q_scale, NULL, 0, 1, o, state_out);
}

/* d/dy of silu(y) = y sigma(y): sigma(y) (1 + y (1 - sigma(y))). */
static double silu_grad(double y)
{
    double sg = gdn_ref_sigmoid(y);
    return sg * (1.0 + y * (1.0 - sg));
}

/*
 * Reverse of the conv for one plane of nc channels of one sequence:
 * y[t][c] = sum_j w[c][j] x[t-3+j][c].  Given dy, adds
 *   gx[tau][c]   += w[c][j] dy[t][c]  for tau = t-3+j >= 0,
 *   ghist[r][c]  += w[c][j] dy[t][c]  for tau = r-3 < 0 (if ghist),
 *   gw[c][j]     += dy[t][c] x[t-3+j][c]  (x from the carried rows, or 0).
 */
static void conv_backward(const double *dy, const void *x, long ldx, int T, int nc,
                          const void *w, const void *hist, long ldh, int f64,
                          double *gx, long ldgx, double *ghist, long ldgh, double *gw)
{
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < nc; ++c) {
            const double d = dy[(long)t * nc + c];
            for (int j = 0; j < 4; ++j) {
                int tau = t - 3 + j;
                double xv;
                if (tau >= 0)
                    xv = in_x(x, f64, (long)tau * ldx + c);
                else if (hist)
                    xv = in_x(hist, f64, (long)(3 + tau) * ldh + c);
                else
                    xv = 0.0;
                gw[(long)c * 4 + j] += d * xv;
                const double wd = in_x(w, f64, (long)c * 4 + j) * d;
                if (tau >= 0)
                    gx[(long)tau * ldgx + c] += wd;
                else if (ghist)
                    ghist[(long)(3 + tau) * ldgh + c] += wd;
            }
        }
    }
}

/*
 * Reverse of the L2 normalisation xh = z / r, r = sqrt(|z|^2 + eps), row by
 * row: dz = dxh / r - z (z . dxh) / r^3.  z, dxh: [T][n]; dz written.
 */
static void l2norm_backward(const double *z, const double *dxh, int T, int n, double eps,
                            double *dz)
{
    for (int t = 0; t < T; ++t) {
        double ss = 0.0, zd = 0.0;
        for (int i = 0; i < n; ++i) {
            ss += z[(long)t * n + i] * z[(long)t * n + i];
            zd += z[(long)t * n + i] * dxh[(long)t * n + i];
        }
        const double r = sqrt(ss + eps);
        for (int i = 0; i < n; ++i)
            dz[(long)t * n + i] = dxh[(long)t * n + i] / r - z[(long)t * n + i] * zd / (r * r * r);
    }
}

/*
 * Reverse of the token recurrence for one (sequence, V head).  Forward, per
 * token: Sd = alpha S_{t-1};  p = Sd^T k;  u = v - p;  S_t = Sd + beta k u^T;
 * o_t = q_scale S_t^T q.  With G = dL/dS_t (starting from dS_T), going back:
 *   G   += q_scale q dO^T;          dq  += q_scale S_t dO
 *   du   = beta G^T k;              dbeta = k^T G u;   dv = du
 *   dk  += beta G u - Sd du         (the write, then the prediction p)
 *   dSd  = G - k du^T;              dalpha = <dSd, S_{t-1}>
 *   G    = alpha dSd                (dL/dS_{t-1})
 * and G after the first token is dL/dS_0.
 *   S_all : [T+1][dk][dv] forward states (S_all[0] = S_0); u_all: [T][dv]
 *   dqh, dkh accumulate ([T][dk]); dvh, dal, dbe are written ([T][dv], [T])
 *   G : in = dS_T (dk x dv), out = dS_0
 */
static void recurrence_backward(const double *qh, const double *kh, const double *alpha,
                                const double *beta, const double *S_all, const double *u_all,
                                const double *dO, int T, int dk, int dv, double q_scale,
                                double *G, double *dqh, double *dkh, double *dvh,
                                double *dal, double *dbe)
{
    const long DD = (long)dk * dv;
    double *du = (double *)malloc(sizeof(double) * (size_t)dv);
    for (int t = T - 1; t >= 0; --t) {
        const double *q = qh + (long)t * dk, *k = kh + (long)t * dk;
        const double *St = S_all + (long)(t + 1) * DD, *Sp = S_all + (long)t * DD;
        const double *u = u_all + (long)t * dv, *g = dO + (long)t * dv;
        /* readout o_t = q_scale S_t^T q */
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) {
                G[(long)i * dv + j] += q_scale * q[i] * g[j];
                acc += St[(long)i * dv + j] * g[j];
            }
            dqh[(long)t * dk + i] += q_scale * acc;
        }
        /* write S_t = Sd + beta k u^T */
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += G[(long)i * dv + j] * k[i];
            du[j] = beta[t] * acc;
            dvh[(long)t * dv + j] = du[j];
        }
        double db = 0.0;
        for (int i = 0; i < dk; ++i) {
            double gu = 0.0, sdu = 0.0;
            for (int j = 0; j < dv; ++j) {
                gu += G[(long)i * dv + j] * u[j];
                sdu += alpha[t] * Sp[(long)i * dv + j] * du[j];  /* Sd du */
            }
            db += k[i] * gu;
            dkh[(long)t * dk + i] += beta[t] * gu - sdu;
        }
        dbe[t] = db;
        /* prediction p = Sd^T k, u = v - p: dSd = G - k du^T; decay Sd = alpha S_{t-1} */
        double da = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) {
                const double dsd = G[(long)i * dv + j] - k[i] * du[j];
                da += dsd * Sp[(long)i * dv + j];
                G[(long)i * dv + j] = alpha[t] * dsd;
            }
        dal[t] = da;
    }
    free(du);
}

/*
 * Gradient of L = sum <dO, o> + <dS_T, S_T> of the whole mixer over packed
 * sequences, with respect to all of its inputs.
 *   inputs as gdn_ref_prefill (f64 = 0: bf16 / fp32) or all double (f64 = 1)
 *   d_o           : double [T_tot][Hv][dv]
 *   d_state_out   : double [N][Hv][dk][dv] or NULL (zero)
 *   gq, gk        : double [T_tot][Hqk][dk];  gv : double [T_tot][Hv][dv]
 *   ga, gb        : double [T_tot][Hv]
 *   gw            : double [C_tot][4] (summed over sequences)
 *   g_conv_state  : double [N][3][C_tot] or NULL: gradient of the carried
 *                   conv rows (the rows themselves, or zeros, are the history)
 *   g_state_in    : double [N][Hv][dk][dv] or NULL
 * All outputs are overwritten.  Returns 0, or -1 on bad arguments.
 */
int gdn_ref_prefill_backward(const void *q, const void *k, const void *v, const void *a,
                             const void *b, const void *conv_w, const void *conv_state_in,
                             const double *state_in, const int32_t *cu_seqlens, int N,
                             int Hqk, int Hv, int dk, int dv, double gate_scale,
                             double q_scale, int f64, const double *d_o,
                             const double *d_state_out, double *gq, double *gk, double *gv,
                             double *ga, double *gb, double *gw, double *g_conv_state,
                             double *g_state_in)
{
    if (N < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hqk != 0)
        return -1;
    const int G = Hv / Hqk;
    const long C_tot = 2L * Hqk * dk + (long)Hv * dv;
    const long T_tot = N > 0 ? cu_seqlens[N] : 0;
    memset(gq, 0, sizeof(double) * (size_t)(T_tot * Hqk * dk));
    memset(gk, 0, sizeof(double) * (size_t)(T_tot * Hqk * dk));
    memset(gv, 0, sizeof(double) * (size_t)(T_tot * Hv * dv));
    memset(ga, 0, sizeof(double) * (size_t)(T_tot * Hv));
    memset(gb, 0, sizeof(double) * (size_t)(T_tot * Hv));
    memset(gw, 0, sizeof(double) * (size_t)(C_tot * 4));
    if (g_conv_state)
        memset(g_conv_state, 0, sizeof(double) * (size_t)((long)N * 3 * C_tot));
    /* per-sequence conv weight gradients, summed in a fixed order at the end */
    double *gw_seq = (double *)calloc((size_t)(N > 0 ? N : 1) * C_tot * 4, sizeof(double));
    const long DD = (long)dk * dv;
    long n_tasks = (long)N * Hqk;

#pragma omp parallel for schedule(dynamic, 1)
    for (long task = 0; task < n_tasks; ++task) {
        const int s = (int)(task / Hqk), g = (int)(task % Hqk);
        const long t0 = cu_seqlens[s];
        const int L = cu_seqlens[s + 1] - cu_seqlens[s];
        const long hist0 = (long)s * 3 * C_tot;
        double *gws = gw_seq + (long)s * C_tot * 4;
        double *ghs = g_conv_state ? g_conv_state + hist0 : NULL;
        const long cq = (long)g * dk, ck = (long)Hqk * dk + (long)g * dk;
        const int Lm = L > 0 ? L : 1;
        double *yq = (double *)malloc(sizeof(double) * (size_t)Lm * dk);
        double *yk = (double *)malloc(sizeof(double) * (size_t)Lm * dk);
        double *zq = (double *)malloc(sizeof(double) * (size_t)Lm * dk);
        double *zk = (double *)malloc(sizeof(double) * (size_t)Lm * dk);
        double *qh = (double *)malloc(sizeof(double) * (size_t)Lm * dk);
        double *kh = (double *)malloc(sizeof(double) * (size_t)Lm * dk);
        double *dqh = (double *)calloc((size_t)Lm * dk, sizeof(double));
        double *dkh = (double *)calloc((size_t)Lm * dk, sizeof(double));
        double *dz = (double *)malloc(sizeof(double) * (size_t)Lm * (dk > dv ? dk : dv));
        /* q^, k^ of the group: conv, SiLU, L2 norm (pre-activations kept) */
        conv_any(X_AT(q, t0 * Hqk * dk + cq), (long)Hqk * dk, L, dk, X_AT(conv_w, cq * 4),
                 HIST_AT(cq), C_tot, f64, yq);
        conv_any(X_AT(k, t0 * Hqk * dk + (long)g * dk), (long)Hqk * dk, L, dk, X_AT(conv_w, ck * 4),
                 HIST_AT(ck), C_tot, f64, yk);
        for (long e = 0; e < (long)L * dk; ++e) {
            zq[e] = gdn_ref_silu(yq[e]);
            zk[e] = gdn_ref_silu(yk[e]);
        }
        memcpy(qh, zq, sizeof(double) * (size_t)L * dk);
        memcpy(kh, zk, sizeof(double) * (size_t)L * dk);
        gdn_ref_l2norm(qh, L, dk, 1e-6);
        gdn_ref_l2norm(kh, L, dk, 1e-6);

        for (int jh = 0; jh < G; ++jh) {
            const int h = g * G + jh;
            const long cv = 2L * Hqk * dk + (long)h * dv;
            double *yv = (double *)malloc(sizeof(double) * (size_t)Lm * dv);
            double *vh = (double *)malloc(sizeof(double) * (size_t)Lm * dv);
            double *al = (double *)malloc(sizeof(double) * (size_t)Lm);
            double *be = (double *)malloc(sizeof(double) * (size_t)Lm);
            double *S_all = (double *)malloc(sizeof(double) * (size_t)(L + 1) * DD);
            double *u_all = (double *)malloc(sizeof(double) * (size_t)Lm * dv);
            double *dO = (double *)malloc(sizeof(double) * (size_t)Lm * dv);
            double *dvh = (double *)malloc(sizeof(double) * (size_t)Lm * dv);
            double *dal = (double *)malloc(sizeof(double) * (size_t)Lm);
            double *dbe = (double *)malloc(sizeof(double) * (size_t)Lm);
            double *Gm = (double *)malloc(sizeof(double) * (size_t)DD);
            conv_any(X_AT(v, t0 * Hv * dv + (long)h * dv), (long)Hv * dv, L, dv, X_AT(conv_w, cv * 4),
                     HIST_AT(cv), C_tot, f64, yv);
            for (long e = 0; e < (long)L * dv; ++e)
                vh[e] = gdn_ref_silu(yv[e]);
            gates_any(G_AT(a, t0 * Hv + h), G_AT(b, t0 * Hv + h), Hv, L, gate_scale, f64, al, be);
            /* forward, keeping every state and every correction u_t */
            if (state_in)
                memcpy(S_all, state_in + ((long)s * Hv + h) * DD, sizeof(double) * (size_t)DD);
            else
                memset(S_all, 0, sizeof(double) * (size_t)DD);
            for (int t = 0; t < L; ++t) {
                const double *Sp = S_all + (long)t * DD;
                double *St = S_all + (long)(t + 1) * DD;
                const double *kt = kh + (long)t * dk, *vt = vh + (long)t * dv;
                double *u = u_all + (long)t * dv;
                for (int j = 0; j < dv; ++j) {
                    double p = 0.0;
                    for (int i = 0; i < dk; ++i)
                        p += al[t] * Sp[(long)i * dv + j] * kt[i];
                    u[j] = vt[j] - p;
                }
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j)
                        St[(long)i * dv + j] = al[t] * Sp[(long)i * dv + j] + be[t] * kt[i] * u[j];
            }
            for (int t = 0; t < L; ++t)
                for (int j = 0; j < dv; ++j)
                    dO[(long)t * dv + j] = d_o[((t0 + t) * Hv + h) * dv + j];
            if (d_state_out)
                memcpy(Gm, d_state_out + ((long)s * Hv + h) * DD, sizeof(double) * (size_t)DD);
            else
                memset(Gm, 0, sizeof(double) * (size_t)DD);
            recurrence_backward(qh, kh, al, be, S_all, u_all, dO, L, dk, dv, q_scale, Gm, dqh, dkh,
                                dvh, dal, dbe);
            if (g_state_in)
                memcpy(g_state_in + ((long)s * Hv + h) * DD, Gm, sizeof(double) * (size_t)DD);
            /* gates: alpha = exp(-c softplus(a)), d alpha / da = -c sigma(a) alpha;
             * beta = sigma(b), d beta / db = beta (1 - beta) */
            for (int t = 0; t < L; ++t) {
                const double av = in_g(a, f64, (t0 + t) * Hv + h);
                ga[(t0 + t) * Hv + h] = dal[t] * al[t] * (-gate_scale * gdn_ref_sigmoid(av));
                gb[(t0 + t) * Hv + h] = dbe[t] * be[t] * (1.0 - be[t]);
            }
            /* v: SiLU, then the conv */
            for (long e = 0; e < (long)L * dv; ++e)
                dz[e] = dvh[e] * silu_grad(yv[e]);
            conv_backward(dz, X_AT(v, t0 * Hv * dv + (long)h * dv), (long)Hv * dv, L, dv,
                          X_AT(conv_w, cv * 4), HIST_AT(cv), C_tot, f64,
                          gv + t0 * Hv * dv + (long)h * dv, (long)Hv * dv,
                          ghs ? ghs + cv : NULL, C_tot, gws + cv * 4);
            free(yv); free(vh); free(al); free(be); free(S_all); free(u_all);
            free(dO); free(dvh); free(dal); free(dbe); free(Gm);
        }
        /* q, k: L2 norm, SiLU, conv */
        double *dzn = (double *)malloc(sizeof(double) * (size_t)Lm * dk);
        l2norm_backward(zq, dqh, L, dk, 1e-6, dzn);
        for (long e = 0; e < (long)L * dk; ++e)
            dz[e] = dzn[e] * silu_grad(yq[e]);
        conv_backward(dz, X_AT(q, t0 * Hqk * dk + cq), (long)Hqk * dk, L, dk, X_AT(conv_w, cq * 4),
                      HIST_AT(cq), C_tot, f64, gq + t0 * Hqk * dk + cq, (long)Hqk * dk,
                      ghs ? ghs + cq : NULL, C_tot, gws + cq * 4);
        l2norm_backward(zk, dkh, L, dk, 1e-6, dzn);
        for (long e = 0; e < (long)L * dk; ++e)
            dz[e] = dzn[e] * silu_grad(yk[e]);
        conv_backward(dz, X_AT(k, t0 * Hqk * dk + (long)g * dk), (long)Hqk * dk, L, dk,
                      X_AT(conv_w, ck * 4), HIST_AT(ck), C_tot, f64,
                      gk + t0 * Hqk * dk + (long)g * dk, (long)Hqk * dk,
                      ghs ? ghs + ck : NULL, C_tot, gws + ck * 4);
        free(dzn);
        free(yq); free(yk); free(zq); free(zk); free(qh); free(kh); free(dqh); free(dkh); free(dz);
    }
    for (int s = 0; s < N; ++s)
        for (long e = 0; e < C_tot * 4; ++e)
            gw[e] += gw_seq[(long)s * C_tot * 4 + e];
    free(gw_seq);
    return 0;
}

/*
 * One decode step for B sequences: the mixer on a single new token per
 * sequence, with the carried conv rows as history and the carried state.
 *   q, k       : bf16 [B][Hqk][dk];  v : bf16 [B][Hv][dv]
 *   a, b       : fp32 [B][Hv]
 *   conv_state : bf16 [B][3][C_tot], updated in place (shift, append token)
 *   state      : double [B][Hv][dk][dv], updated in place
 *   o          : double [B][Hv][dv]
 */
int gdn_ref_decode_step(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        const float *a, const float *b, const uint16_t *conv_w,
                        uint16_t *conv_state, double *state, int B, int Hqk,
                        int Hv, int dk, int dv, double gate_scale,
                        double q_scale, double *o)
{
    if (B < 0)
        return -1;
    int32_t *cu = (int32_t *)malloc(sizeof(int32_t) * (size_t)(B + 1));
    for (int i = 0; i <= B; ++i)
        cu[i] = i;
    const long C_tot = 2L * Hqk * dk + (long)Hv * dv;
    uint16_t *cs_new = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(B > 0 ? B : 1) * 3 * C_tot);
    int rc = gdn_ref_prefill(q, k, v, a, b, conv_w, conv_state, state, cu, B, Hqk, Hv,
                             dk, dv, gate_scale, q_scale, NULL, 0, o, state, cs_new);
    if (rc == 0)
        memcpy(conv_state, cs_new, sizeof(uint16_t) * (size_t)B * 3 * C_tot);
    free(cs_new);
    free(cu);
    return rc;
}
