/*
 * CPU oracle, fp32 router part. TEST INFRASTRUCTURE ONLY: nothing on the
 * product path may link or call this file; only the tests, the smoke check
 * and the benchmark's CPU-baseline leg do.
 *
 * The router runs in fp32 ("Scalable Training of Mixture-of-Experts Models
 * with Megatron Core", section 5.1: the router is kept in FP32; the handbook
 * page "Mixture-of-Experts from Architecture to Large-Scale Training",
 * section 2.5, runs it with --moe-router-dtype fp32). Its logits decide the
 * top-k selection, an integer result, so the order of the fp32 summation is
 * fixed here (no page states one):
 *
 *   gate order G: 64 partial sums part[r], r = i mod 64; for i = 0..h-1
 *   ascending, part[r] = fma(x[i], w[i], part[r]); then for s = 32,16,8,4,2,1
 *   and j < s, part[j] = part[j] + part[j+s]; the logit is part[0], plus the
 *   gate bias (one fp32 add) when the gate has one.
 *
 * The DeepSeek-V3 style sigmoid score enters the selection key as
 * sigma(l) + bias (section 2.2 of the Megatron Core page), so sigma is fixed
 * too. sigma_c(l): clamp l to [-80, 80]; in fp64, d = 1 + exp_c(-l) and
 * s = 1 / d (correctly rounded divide); round s to fp32. exp_c(y) is Cody and
 * Waite's range reduction, n = rint(y log2 e), r = y - n ln2 with ln2 split
 * into a high part with 32 trailing zero bits and a low part (two fmas),
 * followed by the Taylor polynomial of e^r to degree 13 in Horner form (fma)
 * with coefficients 1/m! rounded to nearest, and a scaling by 2^n. Every step
 * is an IEEE-exact or correctly rounded operation, so any implementation of
 * these steps gives the same bits.
 *
 * Compiled with -ffp-contract=off: every product and sum below rounds as
 * written.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ gate */

static float gate_dot(const float *x, const float *w, long h)
{
    float part[64];
    for (int r = 0; r < 64; r++)
        part[r] = 0.0f;
    /* i = 64 c + r: within each residue r, i ascends with c. */
    long full = h / 64;
    for (long c = 0; c < full; c++)
        for (int r = 0; r < 64; r++)
            part[r] = fmaf(x[64 * c + r], w[64 * c + r], part[r]);
    for (long i = 64 * full; i < h; i++)
        part[i % 64] = fmaf(x[i], w[i], part[i % 64]);
    for (int s = 32; s >= 1; s >>= 1)
        for (int j = 0; j < s; j++)
            part[j] = part[j] + part[j + s];
    return part[0];
}

/* logits[t*E + e] = gate order G of x[t,:] . w[e,:] (+ bias[e]).
 * x: [T,h] fp32, w: [E,h] fp32 (bf16 inputs are widened exactly by the
 * caller), bias: [E] or NULL. */
void oracle_gate_logits(const float *x, const float *w, const float *bias,
                        long T, long h, long E, float *logits)
{
#pragma omp parallel for schedule(static)
    for (long t = 0; t < T; t++) {
        for (long e = 0; e < E; e++) {
            float l = gate_dot(x + t * h, w + e * h, h);
            if (bias)
                l = l + bias[e];
            logits[t * E + e] = l;
        }
    }
}

/* --------------------------------------------------------- exp_c, sigma_c */

/* sigma_c is evaluated in fp64 and rounded once to fp32, which keeps it
 * within a hair of the correctly rounded sigmoid and monotone over fp32
 * inputs. The argument is clamped to [-80, 80] first: sigma(80) rounds to
 * 1.0f and sigma(-80) is still a normal fp32 number. */
#define SIGC_CLAMP 80.0f
#define EXPD_LOG2E 1.4426950408889634        /* log2 e */
#define EXPD_LN2_HI 6.93147180369123816490e-01 /* 0x3FE62E42FEE00000 */
#define EXPD_LN2_LO 1.90821492927058770002e-10 /* ln 2 - LN2_HI */

double oracle_exp_c(double y)
{
    double n = rint(y * EXPD_LOG2E);
    double r = fma(-n, EXPD_LN2_HI, y);
    r = fma(-n, EXPD_LN2_LO, r);
    /* Taylor polynomial of e^r to degree 13, coefficients 1/m! rounded to
     * fp64, Horner form from the top. */
    double c[14];
    double fact = 1.0; /* m! is exact in fp64 for m <= 13 */
    for (int m = 0; m < 14; m++) {
        if (m > 0)
            fact = fact * (double)m;
        c[m] = 1.0 / fact;
    }
    double p = c[13];
    for (int m = 12; m >= 0; m--)
        p = fma(p, r, c[m]);
    return ldexp(p, (int)n);
}

float oracle_sigmoid_c(float l)
{
    if (l != l)
        return l;
    if (l > SIGC_CLAMP)
        l = SIGC_CLAMP;
    if (l < -SIGC_CLAMP)
        l = -SIGC_CLAMP;
    double d = 1.0 + oracle_exp_c(-(double)l);
    return (float)(1.0 / d);
}

void oracle_sigmoid_c_array(const float *l, long n, float *out)
{
#pragma omp parallel for schedule(static)
    for (long i = 0; i < n; i++)
        out[i] = oracle_sigmoid_c(l[i]);
}

/* Self-check sweep of sigma_c over every fp32 value in [lo, hi] (lo < hi,
 * both finite). Reports the largest distance in ulps of sigma_c from the
 * fp64 sigmoid rounded to fp32, and the number of adjacent pairs where
 * sigma_c decreases. The distance is measured in units of the fp32 spacing
 * at the fp64 value. */
static uint32_t f2ord(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

static float ord2f(uint32_t o)
{
    uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

void oracle_sigmoid_c_sweep(float lo, float hi, double *max_ulp, long *n_decreasing,
                            long *n_checked)
{
    uint32_t a = f2ord(lo), b = f2ord(hi);
    double worst = 0.0;
    long dec = 0, cnt = 0;
#pragma omp parallel for schedule(static, 1 << 16) reduction(max : worst) reduction(+ : dec, cnt)
    for (int64_t o = (int64_t)a; o <= (int64_t)b; o++) {
        float l = ord2f((uint32_t)o);
        float s = oracle_sigmoid_c(l);
        double ref = 1.0 / (1.0 + exp(-(double)l));
        float rf = (float)ref;
        double ulp = (double)nextafterf(rf, INFINITY) - (double)rf;
        if (ulp <= 0.0)
            ulp = (double)rf - (double)nextafterf(rf, -INFINITY);
        double d = fabs((double)s - ref) / ulp;
        if (d > worst)
            worst = d;
        if (o > (int64_t)a) {
            float sp = oracle_sigmoid_c(ord2f((uint32_t)(o - 1)));
            if (s < sp)
                dec++;
        }
        cnt++;
    }
    *max_ulp = worst;
    *n_decreasing = dec;
    *n_checked = cnt;
}
