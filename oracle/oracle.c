/*
 * oracle.c -- plain, slow CPU forward pass of a llama-family decoder.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  It shares no code
 * with the GPU path and is written from the pages' definitions:
 *
 *   - RMSNorm: mean of squares, plus epsilon, inverse square root, then two
 *     multiplications (by that scale and by the learned weight)
 *     ["Building a GPU compiler from scratch ... (Emmy)", Tensor IR section].
 *   - Decoder block: RMSNorm blocks, rotary attention with GQA, optional
 *     per-head qk RMSNorm, SwiGLU MLP, plain unscaled rope, LM head and
 *     greedy argmax, each operation rounded to bf16 where an eager bf16
 *     reference run rounds it ["model-as-a-kernel", API and Method sections].
 *   - Masked positions contribute nothing to the softmax (the causal-mask
 *     argument of "GPT-2 on the GPU", section "The Whole Model as One
 *     Kernel").
 *
 * Rounding schedule (our reading of the card's eager-bf16 claim; the pages
 * do not list the rounding points):
 *   r32(v) = round-to-nearest-even to fp32, rbf(v) = bf16(RNE) of r32(v).
 *   A dot product of bf16 vectors is the fp64 sum of the (exact) products in
 *   ascending index order.  Transcendentals are evaluated in fp64 on the
 *   fp32 operand, then rounded as stated at each call site.
 *
 * Every function takes `rnd`: 1 applies the schedule, 0 is the fp64 mode in
 * which every r32/rbf is the identity (used for closed-form checks).
 *
 * Activations are double arrays (bf16-valued when rnd=1); weights are bf16
 * bit patterns (uint16) in [out, in] row-major layout.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* number formats                                                      */
/* ------------------------------------------------------------------ */

static float f32_of_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN. */
static uint16_t bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static double r32(double v, int rnd) { return rnd ? (double)(float)v : v; }

static double rbf(double v, int rnd)
{
    return rnd ? (double)f32_of_bf16(bf16_rne((float)v)) : v;
}

static double wval(const uint16_t *w, int64_t i) { return (double)f32_of_bf16(w[i]); }

void orc_bf16_from_f32(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = bf16_rne(in[i]);
}

void orc_round_bf(const double *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = rbf(in[i], 1);
}

/* ------------------------------------------------------------------ */
/* contractions                                                        */
/* ------------------------------------------------------------------ */

/* sum_k w[k] * x[k] in fp64, k ascending. */
double orc_dot(const uint16_t *w, const double *x, int64_t K)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; k++)
        acc += wval(w, k) * x[k];
    return acc;
}

/* Output rounding of a linear layer: 0 = none (fp64), 1 = fp32, 2 = bf16. */
static double round_out(double v, int out_mode, int rnd)
{
    if (out_mode == 2) return rbf(v, rnd);
    if (out_mode == 1) return r32(v, rnd);
    return v;
}

/*
 * Y[t][i] = round(dot(W[i], X[t])) for T rows of input X [T][K] and the
 * weight W [N][K].  Rows i are independent; the threads split i.
 */
void orc_linear(const uint16_t *W, int64_t N, int64_t K, const double *X, int64_t T,
                double *Y, int out_mode, int rnd)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < N; i++)
        for (int64_t t = 0; t < T; t++)
            Y[t * N + i] = round_out(orc_dot(W + i * K, X + t * K, K), out_mode, rnd);
}

/* ------------------------------------------------------------------ */
/* RMSNorm                                                             */
/* ------------------------------------------------------------------ */

/*
 * out = rbf(w * rbf(x * r)), r = r32(1 / sqrt(r32(r32(sum x^2 / n) + eps))).
 * With rnd=1 eps is first rounded to fp32 (the variance is an fp32 tensor).
 */
void orc_rmsnorm(const double *x, int64_t n, const uint16_t *w, double eps,
                 double *out, int rnd)
{
    double ss = 0.0;
    for (int64_t k = 0; k < n; k++)
        ss += x[k] * x[k];
    double ms = r32(ss / (double)n, rnd);
    double v = r32(ms + r32(eps, rnd), rnd);
    double r = r32(1.0 / sqrt(v), rnd);
    for (int64_t k = 0; k < n; k++) {
        double xh = rbf(r32(x[k] * r, rnd), rnd);
        out[k] = rbf(wval(w, k) * xh, rnd);
    }
}

/* ------------------------------------------------------------------ */
/* rotary embedding                                                    */
/* ------------------------------------------------------------------ */

/*
 * cos/sin of one position: inv_i = r32(theta^(-2i/d)), a = r32(r32(pos) * inv_i),
 * c_i = rbf(cos a), s_i = rbf(sin a), i < d/2.
 */
void orc_rope_table(int64_t pos, int64_t d, double theta, double *c, double *s, int rnd)
{
    for (int64_t i = 0; i < d / 2; i++) {
        double inv = r32(pow(theta, -2.0 * (double)i / (double)d), rnd);
        double a = r32(r32((double)pos, rnd) * inv, rnd);
        c[i] = rbf(cos(a), rnd);
        s[i] = rbf(sin(a), rnd);
    }
}

/*
 * Rotate one head vector u[d] in place, pairing element i with i + d/2:
 *   u'_i       = rbf(rbf(u_i c_i)       - rbf(u_{i+d/2} s_i))
 *   u'_{i+d/2} = rbf(rbf(u_{i+d/2} c_i) + rbf(u_i s_i))
 */
void orc_rope(double *u, int64_t d, int64_t pos, double theta, int rnd)
{
    double c[512], s[512];
    int64_t h = d / 2;
    orc_rope_table(pos, d, theta, c, s, rnd);
    for (int64_t i = 0; i < h; i++) {
        double a = u[i], b = u[i + h];
        u[i] = rbf(rbf(a * c[i], rnd) - rbf(b * s[i], rnd), rnd);
        u[i + h] = rbf(rbf(b * c[i], rnd) + rbf(a * s[i], rnd), rnd);
    }
}

/* ------------------------------------------------------------------ */
/* attention of one query head over n cached positions                 */
/* ------------------------------------------------------------------ */

/*
 * q[d]; K, V: n rows of d values, row j at K + j * ld.  scores[n] is
 * caller-provided workspace.
 *   sigma_j = rbf(rbf(q . K_j) * r32(scale))
 *   e_j = r32(exp(sigma_j - max sigma)),  Z = r32(sum_j e_j)   (j ascending)
 *   P_j = rbf(r32(e_j / Z)),  o_i = rbf(sum_j P_j V_j[i])      (j ascending)
 */
void orc_attend(const double *q, const double *K, const double *V, int64_t n, int64_t d,
                int64_t ld, double scale, double *o, double *scores, int rnd)
{
    double sc = r32(scale, rnd);
    double m = -INFINITY;
    for (int64_t j = 0; j < n; j++) {
        double acc = 0.0;
        for (int64_t i = 0; i < d; i++)
            acc += q[i] * K[j * ld + i];
        scores[j] = rbf(rbf(acc, rnd) * sc, rnd);
        if (scores[j] > m) m = scores[j];
    }
    double z = 0.0;
    for (int64_t j = 0; j < n; j++) {
        scores[j] = r32(exp(scores[j] - m), rnd);
        z += scores[j];
    }
    z = r32(z, rnd);
    for (int64_t j = 0; j < n; j++)
        scores[j] = rbf(r32(scores[j] / z, rnd), rnd);
    for (int64_t i = 0; i < d; i++) {
        double acc = 0.0;
        for (int64_t j = 0; j < n; j++)
            acc += scores[j] * V[j * ld + i];
        o[i] = rbf(acc, rnd);
    }
}

/* ------------------------------------------------------------------ */
/* MLP and residual                                                    */
/* ------------------------------------------------------------------ */

/* m_i = rbf(rbf(g_i / (1 + exp(-g_i))) * u_i)   (SwiGLU with SiLU = x * sigmoid(x)) */
void orc_swiglu(const double *g, const double *u, int64_t n, double *m, int rnd)
{
    for (int64_t i = 0; i < n; i++) {
        double z = rbf(g[i] / (1.0 + exp(-g[i])), rnd);
        m[i] = rbf(z * u[i], rnd);
    }
}

/* x_i = rbf(x_i + y_i) */
void orc_residual(double *x, const double *y, int64_t n, int rnd)
{
    for (int64_t i = 0; i < n; i++)
        x[i] = rbf(x[i] + y[i], rnd);
}

/* ------------------------------------------------------------------ */
/* greedy choice                                                       */
/* ------------------------------------------------------------------ */

/* Smallest index attaining the maximum. */
int64_t orc_argmax(const double *v, int64_t n)
{
    int64_t best = 0;
    for (int64_t i = 1; i < n; i++)
        if (v[i] > v[best]) best = i;
    return best;
}
