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
void gdn_ref_conv_silu(const uint16_t *x, long ldx, int T, int nc,
                       const uint16_t *w, const uint16_t *hist, long ldh,
                       double *out)
{
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < nc; ++c) {
            double y = 0.0;
            for (int j = 0; j < 4; ++j) {
                int tau = t - 3 + j;
                double xv;
                if (tau >= 0)
                    xv = bf16_to_double(x[(long)tau * ldx + c]);
                else if (hist)
                    xv = bf16_to_double(hist[(long)(3 + tau) * ldh + c]);
                else
                    xv = 0.0;
                y += bf16_to_double(w[c * 4 + j]) * xv;
            }
            out[(long)t * nc + c] = gdn_ref_silu(y);
        }
    }
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
void gdn_ref_gates(const float *a, const float *b, long ld, int T, double c,
                   double *alpha, double *beta)
{
    for (int t = 0; t < T; ++t) {
        alpha[t] = exp(-c * gdn_ref_softplus((double)a[(long)t * ld]));
        beta[t] = gdn_ref_sigmoid((double)b[(long)t * ld]);
    }
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
int gdn_ref_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const float *a, const float *b, const uint16_t *conv_w,
                    const uint16_t *conv_state_in, const double *state_in,
                    const int32_t *cu_seqlens, int N, int Hqk, int Hv, int dk,
                    int dv, double gate_scale, double q_scale,
                    const int32_t *heads, int n_heads, double *o,
                    double *state_out, uint16_t *conv_state_out)
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
        const uint16_t *hist = conv_state_in ? conv_state_in + (long)s * 3 * C_tot : NULL;
        long cq = (long)g * dk, ck = (long)Hqk * dk + (long)g * dk,
             cv = 2L * Hqk * dk + (long)h * dv;

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
            gdn_ref_conv_silu(q + t0 * Hqk * dk + (long)g * dk, (long)Hqk * dk, L, dk,
                              conv_w + cq * 4, hist ? hist + cq : NULL, C_tot, qh);
            gdn_ref_conv_silu(k + t0 * Hqk * dk + (long)g * dk, (long)Hqk * dk, L, dk,
                              conv_w + ck * 4, hist ? hist + ck : NULL, C_tot, kh);
            gdn_ref_conv_silu(v + t0 * Hv * dv + (long)h * dv, (long)Hv * dv, L, dv,
                              conv_w + cv * 4, hist ? hist + cv : NULL, C_tot, vh);
            gdn_ref_l2norm(qh, L, dk, 1e-6);
            gdn_ref_l2norm(kh, L, dk, 1e-6);
            gdn_ref_gates(a + t0 * Hv + h, b + t0 * Hv + h, Hv, L, gate_scale, al, be);
            gdn_ref_recurrence(qh, kh, vh, al, be, L, dk, dv, q_scale, S, oh);
            for (int t = 0; t < L; ++t)
                memcpy(o + ((t0 + t) * Hv + h) * dv, oh + (long)t * dv, sizeof(double) * (size_t)dv);
            free(qh); free(kh); free(vh); free(al); free(be); free(oh);
        }
        if (state_out)
            memcpy(state_out + ((long)s * Hv + h) * dk * dv, S, sizeof(double) * (size_t)dk * dv);
        free(S);
    }

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
