/*
 * hc_oracle.c -- plain CPU oracle for the hyper-connection read.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library path may include, link,
 * load or call this file: only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP implementation.
 *
 * What it computes, per token t (the definition, written out directly; every
 * loop runs in ascending index order, no blocking, no fusion):
 *
 *   R'[t,s,c]  = fl32(R[t,s,c] + P[t,s,c])           pending write applied first
 *                (P = 0 when no pending write is given)
 *        -- "#315 hc: the multi-token hyper-connection read split finer",
 *           section Exactness (reads with and without the pending write);
 *           "#2488 sycl/A770 ...", Summary item 4 (the norm sees the
 *           pending-updated residual).
 *   rs[t,s]    = 1 / sqrt( (1/C) * sum_c R'[t,s,c]^2 + eps )
 *        -- #315, section "What changes", Norm bullet: one sum of squares per
 *           token and stream gives rs; eps is added to the mean of squares.
 *   xn[t,k]    = R'[t,s,c] * w_norm[s,c] * rs[t,s],   k = s*C + c
 *        -- #315, Norm bullet (R' times w_norm, scaled by rs).
 *   lo[t,j]    = sum_k W_down[j,k] * xn[t,k]          (down projection)
 *        -- #315, "Down projection" bullet; #2226 Summary (column-sliced down
 *           projection reduced into lo); #2488 items 1 and 3.
 *   up[t,k]    = sum_j W_up[k,j] * lo[t,j]            (up projection)
 *        -- "#1370 prefill: ... gr_mix_r as its epilogue", "What it does"
 *           (K = r = 320); #2070 item 1.
 *   gated      = up                                   (the up epilogue; the
 *           pages name it but never give its function -- read as identity)
 *        -- #2226 Summary ("the same epilogue as gr_up_kernel"); #1370 "Why"
 *           (the up GEMM writes gated directly).
 *   mixed[t,c] = sum_{s=0..n-1} gated[t, s*C+c] * R'[t,s,c]
 *        -- #1370 "Why" (gr_mix_r reads gated back with R) and "What it does"
 *           (a lane holds a (token, column) pair for all 4 streams and mixes
 *           them in registers).
 *   images     = round-to-nearest-even of fl32(mixed) to bf16 and to fp16
 *        -- #1370 "What it does" (mixed with its BF16 / FP16 images).
 *
 * Weights are bf16 bit patterns, widened exactly from the format's fields.
 * Three modes:
 *   fp64 (mode 0) is the parity reference: every quantity after R' is a
 *        double.
 *   fp32 (mode 1) is a diagnostic: the same loops with float accumulators,
 *        each sum taken in ascending index order one rounded addition at a
 *        time, rs = 1 / sqrtf(fl(ss / C) + eps), and the two roundings of xn
 *        (R' * w_norm stored, then scaled by rs), as the Norm bullet of #315
 *        describes.
 *   bf16-lo (mode 2) is the fp64 read with lo rounded to bf16 (nearest, ties
 *        to even) before the up projection: the operand the fused up + mix
 *        of #1370 "What it does" feeds its BF16 mma (FP32 accumulation).  It
 *        is the reference of the library's bf16-lo mode; lo itself (lo_out)
 *        is reported before the rounding.
 * Build with -O2 -ffp-contract=off and without fast-math so the arithmetic is
 * exactly what is written.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>

#define HC_ORACLE_OK 0
#define HC_ORACLE_EARG 1
#define HC_ORACLE_ENOMEM 2

/* ------------------------------------------------------------------------ */
/* Number formats, from their definitions.                                   */
/* ------------------------------------------------------------------------ */

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double hc_oracle_bf16_to_double(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 7) & 0xFF;
    int frac = bits & 0x7F;
    double mag;
    if (expo == 0xFF) {
        mag = frac ? NAN : INFINITY;
    } else if (expo == 0) {
        mag = ldexp((double)frac, -126 - 7); /* subnormal: 0.frac * 2^-126 */
    } else {
        mag = ldexp(128.0 + (double)frac, expo - 127 - 7); /* 1.frac * 2^(e-127) */
    }
    return sign ? -mag : mag;
}

/*
 * Nearest value of a binary floating-point format with `sig` significand bits
 * (implicit bit included), minimum normal exponent `emin` and maximum finite
 * exponent `emax`, ties to even; returns the rounded value as a double (which
 * holds it exactly) or +-inf on overflow.  x must be finite.
 */
static double round_to_format(double x, int sig, int emin, int emax)
{
    if (x == 0.0)
        return x;
    int e2;
    (void)frexp(fabs(x), &e2); /* |x| = m * 2^e2, m in [0.5, 1) */
    int e = e2 - 1;            /* |x| in [2^e, 2^(e+1)) */
    if (e < emin)
        e = emin;              /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, e - (sig - 1));
    double n = x / quantum;    /* exact: a power-of-two scaling */
    double r = nearbyint(n);   /* default rounding mode: nearest, ties even */
    double v = r * quantum;
    if (fabs(v) >= ldexp(1.0, emax + 1))
        return x < 0 ? -INFINITY : INFINITY;
    return v;
}

/* Encode a double that is exactly representable in the format (or +-inf). */
static uint16_t encode_format(double v, int sig, int ebits, int is_neg)
{
    int bias = (1 << (ebits - 1)) - 1;
    int fbits = sig - 1;
    uint16_t s = (uint16_t)(is_neg ? (1u << (ebits + fbits)) : 0u);
    double a = fabs(v);
    if (isinf(a))
        return (uint16_t)(s | (((1u << ebits) - 1u) << fbits));
    if (a == 0.0)
        return s;
    int e2;
    (void)frexp(a, &e2);
    int e = e2 - 1;
    int emin = 1 - bias;
    if (e < emin) { /* subnormal */
        double f = ldexp(a, -(emin - fbits));
        return (uint16_t)(s | (uint16_t)f);
    }
    double f = ldexp(a, -(e - fbits)) - ldexp(1.0, fbits);
    return (uint16_t)(s | ((uint16_t)(e + bias) << fbits) | (uint16_t)f);
}

/* float -> bfloat16 bits, round to nearest even. */
uint16_t hc_oracle_f32_to_bf16(float x)
{
    if (isnan(x))
        return (uint16_t)(signbit(x) ? 0xFFC0u : 0x7FC0u);
    if (isinf(x))
        return (uint16_t)(signbit(x) ? 0xFF80u : 0x7F80u);
    double v = round_to_format((double)x, 8, -126, 127);
    return encode_format(v, 8, 8, signbit(x) != 0);
}

/* float -> IEEE binary16 bits, round to nearest even, subnormals kept. */
uint16_t hc_oracle_f32_to_f16(float x)
{
    if (isnan(x))
        return (uint16_t)(signbit(x) ? 0xFE00u : 0x7E00u);
    if (isinf(x))
        return (uint16_t)(signbit(x) ? 0xFC00u : 0x7C00u);
    double v = round_to_format((double)x, 11, -14, 15);
    return encode_format(v, 11, 5, signbit(x) != 0);
}

/* The images of a double-valued output: RNE of fl32(m) to bf16 and fp16. */
void hc_oracle_images(const double* mixed, int64_t count,
                      uint16_t* out_bf16, uint16_t* out_f16)
{
    for (int64_t i = 0; i < count; ++i) {
        float f = (float)mixed[i]; /* fl32: the fp32 output the images round */
        if (out_bf16)
            out_bf16[i] = hc_oracle_f32_to_bf16(f);
        if (out_f16)
            out_f16[i] = hc_oracle_f32_to_f16(f);
    }
}

/* ------------------------------------------------------------------------ */
/* The read.                                                                 */
/* ------------------------------------------------------------------------ */

typedef struct {
    int n, C, r;
    double eps;
    const float* R;
    const float* P;
    const float* w_norm;
    const uint16_t* W_down;
    const uint16_t* W_up;
    double* mixed;
    double* rs_out;
    double* lo_out;
    const double* wd; /* widened weights (shared, read only) */
    const double* wu;
    int mode; /* 0 = fp64, 1 = fp32, 2 = fp64 with lo rounded to bf16 */
    int64_t t_begin, t_end;
    int status;
} oracle_job;

/* fp64 mode: one token. */
static void read_token_f64(const oracle_job* jb, int64_t t, double* rp,
                           double* xn, double* lo, double* up)
{
    const int n = jb->n, C = jb->C, r = jb->r;
    const int64_t D = (int64_t)n * C;
    const float* Rt = jb->R + t * D;
    const float* Pt = jb->P ? jb->P + t * D : NULL;

    /* R' = fl32(R + P) */
    for (int64_t k = 0; k < D; ++k) {
        float v = Rt[k];
        if (Pt) {
            float sum = Rt[k] + Pt[k];
            v = sum;
        }
        rp[k] = (double)v;
    }
    /* per-stream RMS norm */
    for (int s = 0; s < n; ++s) {
        double ss = 0.0;
        for (int c = 0; c < C; ++c)
            ss += rp[(int64_t)s * C + c] * rp[(int64_t)s * C + c];
        double rs = 1.0 / sqrt(ss / (double)C + jb->eps);
        if (jb->rs_out)
            jb->rs_out[t * n + s] = rs;
        for (int c = 0; c < C; ++c) {
            int64_t k = (int64_t)s * C + c;
            xn[k] = rp[k] * (double)jb->w_norm[k] * rs;
        }
    }
    /* down projection */
    for (int j = 0; j < r; ++j) {
        const double* wrow = jb->wd + (int64_t)j * D;
        double acc = 0.0;
        for (int64_t k = 0; k < D; ++k)
            acc += wrow[k] * xn[k];
        lo[j] = acc;
    }
    if (jb->lo_out)
        memcpy(jb->lo_out + t * r, lo, sizeof(double) * (size_t)r);
    /* bf16-lo mode: the up projection's operand is lo rounded to bf16 */
    if (jb->mode == 2)
        for (int j = 0; j < r; ++j)
            lo[j] = isfinite(lo[j]) ? round_to_format(lo[j], 8, -126, 127) : lo[j];
    /* up projection; epilogue = identity */
    for (int64_t k = 0; k < D; ++k) {
        const double* wrow = jb->wu + k * r;
        double acc = 0.0;
        for (int j = 0; j < r; ++j)
            acc += wrow[j] * lo[j];
        up[k] = acc;
    }
    /* gr_mix_r: sum over streams, stream 0 first */
    for (int c = 0; c < C; ++c) {
        double m = 0.0;
        for (int s = 0; s < n; ++s)
            m += up[(int64_t)s * C + c] * rp[(int64_t)s * C + c];
        jb->mixed[t * C + c] = m;
    }
}

/* fp32 mode: the same loops in float (diagnostic, not the parity gate). */
static void read_token_f32(const oracle_job* jb, int64_t t, float* rp,
                           float* xn, float* lo, float* up)
{
    const int n = jb->n, C = jb->C, r = jb->r;
    const int64_t D = (int64_t)n * C;
    const float* Rt = jb->R + t * D;
    const float* Pt = jb->P ? jb->P + t * D : NULL;
    const float eps = (float)jb->eps;

    for (int64_t k = 0; k < D; ++k)
        rp[k] = Pt ? Rt[k] + Pt[k] : Rt[k];
    for (int s = 0; s < n; ++s) {
        float ss = 0.0f;
        for (int c = 0; c < C; ++c) {
            float v = rp[(int64_t)s * C + c];
            float sq = v * v;
            ss = ss + sq;
        }
        float mean = ss / (float)C;
        float rs = 1.0f / sqrtf(mean + eps);
        if (jb->rs_out)
            jb->rs_out[t * n + s] = (double)rs;
        for (int c = 0; c < C; ++c) {
            int64_t k = (int64_t)s * C + c;
            float prod = rp[k] * jb->w_norm[k]; /* first rounding (store) */
            xn[k] = prod * rs;                  /* second rounding (scale) */
        }
    }
    for (int j = 0; j < r; ++j) {
        const double* wrow = jb->wd + (int64_t)j * D;
        float acc = 0.0f;
        for (int64_t k = 0; k < D; ++k) {
            float p = (float)wrow[k] * xn[k];
            acc = acc + p;
        }
        lo[j] = acc;
    }
    if (jb->lo_out)
        for (int j = 0; j < r; ++j)
            jb->lo_out[t * r + j] = (double)lo[j];
    for (int64_t k = 0; k < D; ++k) {
        const double* wrow = jb->wu + k * r;
        float acc = 0.0f;
        for (int j = 0; j < r; ++j) {
            float p = (float)wrow[j] * lo[j];
            acc = acc + p;
        }
        up[k] = acc;
    }
    for (int c = 0; c < C; ++c) {
        float m = 0.0f;
        for (int s = 0; s < n; ++s) {
            float p = up[(int64_t)s * C + c] * rp[(int64_t)s * C + c];
            m = m + p;
        }
        jb->mixed[t * C + c] = (double)m;
    }
}

static void* run_job(void* arg)
{
    oracle_job* jb = (oracle_job*)arg;
    const int64_t D = (int64_t)jb->n * jb->C;
    size_t elt = jb->mode == 1 ? sizeof(float) : sizeof(double);
    void* rp = malloc(elt * (size_t)D);
    void* xn = malloc(elt * (size_t)D);
    void* lo = malloc(elt * (size_t)jb->r);
    void* up = malloc(elt * (size_t)D);
    if (!rp || !xn || !lo || !up) {
        jb->status = HC_ORACLE_ENOMEM;
    } else {
        for (int64_t t = jb->t_begin; t < jb->t_end; ++t) {
            if (jb->mode == 1)
                read_token_f32(jb, t, rp, xn, lo, up);
            else
                read_token_f64(jb, t, rp, xn, lo, up);
        }
        jb->status = HC_ORACLE_OK;
    }
    free(rp);
    free(xn);
    free(lo);
    free(up);
    return NULL;
}

/*
 * The read for T tokens.
 *   R, P       fp32 [T][n][C]; P may be NULL (no pending write)
 *   w_norm     fp32 [n][C]
 *   W_down     bf16 bits [r][n*C];  W_up bf16 bits [n*C][r]
 *   mode       0 = fp64 (parity reference), 1 = fp32 (diagnostic),
 *              2 = fp64 with lo rounded to bf16 before the up projection
 *   threads    >= 1; tokens are split into contiguous ranges, one per thread
 *              (every token is computed by the same code, so the result does
 *              not depend on the thread count)
 *   mixed      out, double [T][C]; rs_out [T][n] and lo_out [T][r] optional
 * Returns 0 on success, 1 on a bad argument, 2 when memory runs out.
 */
int hc_oracle_read(int64_t T, int n, int C, int r, double eps,
                   const float* R, const float* P, const float* w_norm,
                   const uint16_t* W_down, const uint16_t* W_up,
                   int mode, int threads,
                   double* mixed, double* rs_out, double* lo_out)
{
    if (T < 0 || n < 1 || C < 1 || r < 1 || !(eps >= 0.0) || !R || !w_norm ||
        !W_down || !W_up || !mixed || mode < 0 || mode > 2 || threads < 1)
        return HC_ORACLE_EARG;
    if (T == 0)
        return HC_ORACLE_OK;
    const int64_t D = (int64_t)n * C;
    double* wd = malloc(sizeof(double) * (size_t)(D * r));
    double* wu = malloc(sizeof(double) * (size_t)(D * r));
    if (!wd || !wu) {
        free(wd);
        free(wu);
        return HC_ORACLE_ENOMEM;
    }
    for (int64_t i = 0; i < D * r; ++i) {
        wd[i] = hc_oracle_bf16_to_double(W_down[i]);
        wu[i] = hc_oracle_bf16_to_double(W_up[i]);
    }
    if (threads > T)
        threads = (int)T;
    oracle_job* jobs = calloc((size_t)threads, sizeof(oracle_job));
    pthread_t* tids = calloc((size_t)threads, sizeof(pthread_t));
    int status = HC_ORACLE_OK;
    if (!jobs || !tids) {
        status = HC_ORACLE_ENOMEM;
    } else {
        for (int i = 0; i < threads; ++i) {
            oracle_job* jb = &jobs[i];
            jb->n = n;
            jb->C = C;
            jb->r = r;
            jb->eps = eps;
            jb->R = R;
            jb->P = P;
            jb->w_norm = w_norm;
            jb->W_down = W_down;
            jb->W_up = W_up;
            jb->mixed = mixed;
            jb->rs_out = rs_out;
            jb->lo_out = lo_out;
            jb->wd = wd;
            jb->wu = wu;
            jb->mode = mode;
            jb->t_begin = T * i / threads;
            jb->t_end = T * (i + 1) / threads;
        }
        if (threads == 1) {
            run_job(&jobs[0]);
        } else {
            char* started = calloc((size_t)threads, 1);
            for (int i = 0; i < threads; ++i) {
                if (started && pthread_create(&tids[i], NULL, run_job, &jobs[i]) == 0)
                    started[i] = 1;
                else
                    run_job(&jobs[i]); /* no thread: run it here instead */
            }
            for (int i = 0; i < threads; ++i)
                if (started && started[i])
                    pthread_join(tids[i], NULL);
            free(started);
        }
        for (int i = 0; i < threads; ++i)
            if (jobs[i].status != HC_ORACLE_OK)
                status = jobs[i].status;
    }
    free(jobs);
    free(tids);
    free(wd);
    free(wu);
    return status;
}

/*
 * The pending write committed: R'[i] = fl32(R[i] + P[i]) for `count`
 * elements, the same R' the read above starts from ("#2488 sycl/A770: faster
 * hyper-connection read", Summary item 4: the pending-updated residual; "#315
 * hc: the multi-token hyper-connection read split finer", Exactness: reads
 * with and without the pending write).  Writing it back into R is an
 * extension of the library, not a step of the pages; this is its reference.
 * P == NULL copies R (nothing to commit).  out may be R itself.
 * Returns 0, or 1 on a bad argument.
 */
int hc_oracle_commit(int64_t count, const float* R, const float* P, float* out)
{
    if (count < 0 || !R || !out)
        return HC_ORACLE_EARG;
    for (int64_t i = 0; i < count; ++i) {
        float v = R[i];
        if (P) {
            float sum = R[i] + P[i];
            v = sum;
        }
        out[i] = v;
    }
    return HC_ORACLE_OK;
}
