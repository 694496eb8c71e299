/* Sanitizer driver for the fp64 oracle: every entry point on small inputs
 * (empty, one-token and multi-chunk sequences, carries on and off, a head
 * subset, both input kinds of the backward), built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_sanitizers.py.  Any out-of-bounds
 * access, leak or undefined operation aborts the run; the driver itself only
 * checks the return codes and that the outputs are finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double gdn_ref_sigmoid(double x);
double gdn_ref_softplus(double x);
double gdn_ref_silu(double x);
int gdn_ref_num_threads(void);
void gdn_ref_conv_silu(const uint16_t *x, long ldx, int T, int nc, const uint16_t *w, const uint16_t *hist,
                       long ldh, double *out);
void gdn_ref_l2norm(double *x, int T, int n, double eps);
void gdn_ref_gates(const float *a, const float *b, long ld, int T, double c, double *alpha, double *beta);
void gdn_ref_recurrence(const double *qh, const double *kh, const double *vh, const double *alpha,
                        const double *beta, int T, int dk, int dv, double q_scale, double *S, double *o);
int gdn_ref_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a, const float *b,
                    const uint16_t *conv_w, const uint16_t *conv_state_in, const double *state_in,
                    const int32_t *cu_seqlens, int N, int Hqk, int Hv, int dk, int dv, double gate_scale,
                    double q_scale, const int32_t *heads, int n_heads, double *o, double *state_out,
                    uint16_t *conv_state_out);
int gdn_ref_prefill_f64(const double *q, const double *k, const double *v, const double *a, const double *b,
                        const double *conv_w, const double *conv_state_in, const double *state_in,
                        const int32_t *cu_seqlens, int N, int Hqk, int Hv, int dk, int dv, double gate_scale,
                        double q_scale, double *o, double *state_out);
int gdn_ref_prefill_backward(const void *q, const void *k, const void *v, const void *a, const void *b,
                             const void *conv_w, const void *conv_state_in, const double *state_in,
                             const int32_t *cu_seqlens, int N, int Hqk, int Hv, int dk, int dv,
                             double gate_scale, double q_scale, int f64, const double *d_o,
                             const double *d_state_out, double *gq, double *gk, double *gv, double *ga,
                             double *gb, double *gw, double *g_conv_state, double *g_state_in);
int gdn_ref_decode_step(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a, const float *b,
                        const uint16_t *conv_w, uint16_t *conv_state, double *state, int B, int Hqk, int Hv,
                        int dk, int dv, double gate_scale, double q_scale, double *o);

static uint64_t rng = 88172645463325252ull;
static double unif(void) /* xorshift64, in (-1, 1) */
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
static uint16_t bf16(double x) /* truncating conversion is enough for inputs */
{
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}
static void *xmalloc(size_t n) { void *p = malloc(n ? n : 1); if (!p) abort(); return p; }
static uint16_t *rand_bf16(size_t n, double s) { uint16_t *p = xmalloc(n * 2); for (size_t i = 0; i < n; ++i) p[i] = bf16(s * unif()); return p; }
static float *rand_f32(size_t n, double s) { float *p = xmalloc(n * 4); for (size_t i = 0; i < n; ++i) p[i] = (float)(s * unif()); return p; }
static double *rand_f64(size_t n, double s) { double *p = xmalloc(n * 8); for (size_t i = 0; i < n; ++i) p[i] = s * unif(); return p; }
static void finite(const double *x, size_t n, const char *what)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) { fprintf(stderr, "%s: non-finite at %zu\n", what, i); exit(2); }
}
#define CHECK(e) do { if ((e) != 0) { fprintf(stderr, "failed: %s\n", #e); exit(3); } } while (0)

int main(void)
{
    const int Hqk = 1, Hv = 2, d = 128, N = 4;
    const int32_t cu[5] = {0, 0, 1, 71, 75}; /* empty, one token, two chunks, ragged */
    const int T = cu[N];
    const long C = 2L * Hqk * d + (long)Hv * d;
    uint16_t *q = rand_bf16((size_t)T * Hqk * d, 2), *k = rand_bf16((size_t)T * Hqk * d, 2);
    uint16_t *v = rand_bf16((size_t)T * Hv * d, 2), *w = rand_bf16((size_t)C * 4, 0.5);
    uint16_t *cs = rand_bf16((size_t)N * 3 * C, 1);
    float *a = rand_f32((size_t)T * Hv, 2), *b = rand_f32((size_t)T * Hv, 2);
    double *st = rand_f64((size_t)N * Hv * d * d, 0.05);
    double *o = xmalloc(sizeof(double) * T * Hv * d), *so = xmalloc(sizeof(double) * N * Hv * d * d);
    uint16_t *cso = xmalloc(2 * (size_t)N * 3 * C);
    (void)gdn_ref_sigmoid(0.3); (void)gdn_ref_softplus(-40.0); (void)gdn_ref_silu(3.0);
    (void)gdn_ref_num_threads();
    /* carries on, then off, then a head subset */
    CHECK(gdn_ref_prefill(q, k, v, a, b, w, cs, st, cu, N, Hqk, Hv, d, d, 0.1, 0.9, NULL, 0, o, so, cso));
    finite(o, (size_t)T * Hv * d, "prefill o");
    CHECK(gdn_ref_prefill(q, k, v, a, b, w, NULL, NULL, cu, N, Hqk, Hv, d, d, 0.1, 1.0, NULL, 0, o, so, cso));
    const int32_t heads[1] = {1};
    CHECK(gdn_ref_prefill(q, k, v, a, b, w, cs, st, cu, N, Hqk, Hv, d, d, 0.1, 1.0, heads, 1, o, so, NULL));
    /* every input in double */
    double *qd = rand_f64((size_t)T * Hqk * d, 2), *kd = rand_f64((size_t)T * Hqk * d, 2);
    double *vd = rand_f64((size_t)T * Hv * d, 2), *wd = rand_f64((size_t)C * 4, 0.5);
    double *csd = rand_f64((size_t)N * 3 * C, 1), *ad = rand_f64((size_t)T * Hv, 2), *bd = rand_f64((size_t)T * Hv, 2);
    CHECK(gdn_ref_prefill_f64(qd, kd, vd, ad, bd, wd, csd, st, cu, N, Hqk, Hv, d, d, 0.1, 1.0, o, so));
    finite(so, (size_t)N * Hv * d * d, "prefill_f64 state");
    /* backward, bf16 and double inputs, carries on and off */
    double *dO = rand_f64((size_t)T * Hv * d, 1), *dS = rand_f64((size_t)N * Hv * d * d, 1);
    double *gq = xmalloc(8 * (size_t)T * Hqk * d), *gk = xmalloc(8 * (size_t)T * Hqk * d);
    double *gv = xmalloc(8 * (size_t)T * Hv * d), *ga = xmalloc(8 * (size_t)T * Hv), *gb = xmalloc(8 * (size_t)T * Hv);
    double *gw = xmalloc(8 * (size_t)C * 4), *gcs = xmalloc(8 * (size_t)N * 3 * C);
    double *gs = xmalloc(8 * (size_t)N * Hv * d * d);
    CHECK(gdn_ref_prefill_backward(q, k, v, a, b, w, cs, st, cu, N, Hqk, Hv, d, d, 0.1, 0.8, 0, dO, dS, gq, gk, gv,
                                   ga, gb, gw, gcs, gs));
    finite(gw, (size_t)C * 4, "backward conv_w");
    CHECK(gdn_ref_prefill_backward(qd, kd, vd, ad, bd, wd, NULL, NULL, cu, N, Hqk, Hv, d, d, 0.1, 1.0, 1, dO, NULL,
                                   gq, gk, gv, ga, gb, gw, NULL, NULL));
    finite(gq, (size_t)T * Hqk * d, "backward q");
    /* decode steps, in place */
    const int B = 3;
    uint16_t *dcs = rand_bf16((size_t)B * 3 * C, 1);
    double *dst = rand_f64((size_t)B * Hv * d * d, 0.05), *dout = xmalloc(8 * (size_t)B * Hv * d);
    for (int step = 0; step < 4; ++step)
        CHECK(gdn_ref_decode_step(q, k, v, a, b, w, dcs, dst, B, Hqk, Hv, d, d, 0.1, 1.0, dout));
    finite(dst, (size_t)B * Hv * d * d, "decode state");
    /* bad arguments are rejected */
    if (gdn_ref_decode_step(q, k, v, a, b, w, dcs, dst, -1, Hqk, Hv, d, d, 0.1, 1.0, dout) == 0) return 4;
    void *all[] = {q, k, v, w, cs, a, b, st, o, so, cso, qd, kd, vd, wd, csd, ad, bd, dO, dS,
                   gq, gk, gv, ga, gb, gw, gcs, gs, dcs, dst, dout};
    for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) free(all[i]);
    puts("oracle sanitizer run ok");
    return 0;
}
