/*
 * kvq_oracle.c -- CPU oracle for the paged, quantized KV-cache decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or constant table with
 * the HIP library.
 *
 * It is deliberately plain and slow: every quantity is computed the way its
 * definition reads, floating point in fp64 unless the method fixes fp32
 * (the INT8 scale and the division x/scale are fp32 by definition, so that
 * the integer codes are decided in the same precision as the GPU kernel).
 *
 * Sources (web pages; section names as printed on them):
 *  [P3] "KV Cache优化实战：大模型推理显存占用与加速方案详解" (0539edu.com)
 *       s1.1  decode appends the new token's K/V and attends with the current
 *             query over all cached K/V; same result as recomputation.
 *       s1.2  KV byte formula 2*batch*seq_len*layers*kv_heads*head_dim*bytes.
 *       s2.1  GQA: query heads are split into groups, each group shares one
 *             KV head.
 *       s2.3  INT8 absmax symmetric quantization with a stored scale,
 *             dequantized at run time; per-group variant (e.g. 128 elements
 *             per group, each with its own scale); FP8 option.
 *       s3.3  per_group granularity with group size 128 or 64.
 *  [P1] xpshop.cn article 402, s3 / [P2] xpshop.cn article 312, s2-s3: INT8 /
 *       FP8 KV cache in paged 16/32-token blocks.
 *
 * Readings where the pages are silent:
 *  - INT8 scale s = fl32(absmax / 127), code = clamp(rne(fl32(x / s)), -127,
 *    127); an all-zero group stores s = 0 and codes 0.
 *  - FP8 is OCP E4M3FN (bias 7, max 448, no infinities); encode rounds to
 *    nearest, ties to even, and saturates to +-448; a negative value that
 *    rounds to zero keeps its sign (code 0x80).  The scale is a static fp32
 *    per KV head, applied as fl32(x / S); a zero scale (a head whose
 *    calibration data are all zero) gives code 0.
 *  - FP8 E5M2 (the kv_cache_dtype "fp8_e5m2" of xpshop.cn article 312 s3) is
 *    the OCP E5M2 format (bias 15, 2 mantissa bits, infinities and NaNs);
 *    encode rounds to nearest, ties to even, and saturates to +-57344.
 *  - FP8 with dynamic scales (either format): per (token, head, group of G
 *    consecutive elements), s = fl32(absmax / FP8_MAX), code =
 *    fp8(fl32(x / s)); an all-zero group stores s = 0 and codes 0.  G =
 *    head_dim is the per-token case.
 *  - INT8 per-channel ("per_channel" granularity, [P3] s2.3, s3.3, s4.2):
 *    one static fp32 scale per (KV head, channel), given as an input like the
 *    FP8 static scale; code = clamp(rne(fl32(x / s_c)), -127, 127); a zero
 *    scale gives code 0.
 *  - softmax scale defaults to 1/sqrt(head_dim); query head g reads KV head
 *    g / (Hq / Hkv) (contiguous grouping).
 *
 * Parity pins: every exported function is pinned by a CPU test against
 * something other than itself (a library routine, brute force, a closed form
 * or an invariant); see the test files tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------ */
/* IEEE-754 binary16 -> double, read off the bit layout                */
/* (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits).       */
/* ------------------------------------------------------------------ */
ORC_API double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

ORC_API void orc_f16_to_f64_array(const uint16_t *x, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f16_to_f64(x[i]);
}

/* ------------------------------------------------------------------ */
/* INT8 per-group absmax symmetric codec  ([P3] s2.3, s3.3)             */
/* ------------------------------------------------------------------ */

/* Quantize one group of G fp16 values.  Returns 0, or -1 on a non-finite
 * input (the method is defined for finite K/V only). */
ORC_API int orc_int8_quantize_group(const uint16_t *x, int G, int8_t *codes,
                                    float *scale)
{
    float absmax = 0.0f;
    for (int i = 0; i < G; ++i) {
        double xd = orc_f16_to_f64(x[i]);
        if (!isfinite(xd))
            return -1;
        float ax = fabsf((float)xd);               /* exact: fp16 fits fp32 */
        if (ax > absmax)
            absmax = ax;
    }
    float s = absmax / 127.0f;                     /* IEEE fp32 division     */
    *scale = s;
    for (int i = 0; i < G; ++i) {
        if (s == 0.0f) {
            codes[i] = 0;
            continue;
        }
        float xf = (float)orc_f16_to_f64(x[i]);
        float y = xf / s;                          /* fp32, correctly rounded */
        float r = rintf(y);                        /* nearest, ties to even   */
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        codes[i] = (int8_t)r;
    }
    return 0;
}

/* Rows of d elements, groups of G consecutive elements along the row.
 * x: [rows][d] fp16 bits; codes: [rows][d]; scales: [rows][d/G]. */
ORC_API int orc_int8_quantize_rows(const uint16_t *x, int64_t rows, int d,
                                   int G, int8_t *codes, float *scales)
{
    if (G <= 0 || d % G != 0)
        return -2;
    int ng = d / G;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r)
        for (int j = 0; j < ng; ++j)
            bad |= orc_int8_quantize_group(x + r * d + j * G, G,
                                           codes + r * d + j * G,
                                           scales + r * ng + j) != 0;
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* INT4 per-group absmax symmetric codec ([P3] s2.3 lists int4 among the */
/* cache quantization methods; s3.3 and xpshop.cn article 402 s3 report  */
/* its quality loss): the INT8 rule with 7 in place of 127.              */
/* x: [rows][d] fp16 bits; codes: [rows][d] in [-7, 7]; scales [rows][d/G]*/
/* ------------------------------------------------------------------ */
ORC_API int orc_int4_quantize_rows(const uint16_t *x, int64_t rows, int d,
                                   int G, int8_t *codes, float *scales)
{
    if (G <= 0 || d % G != 0)
        return -2;
    int ng = d / G;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r)
        for (int j = 0; j < ng; ++j) {
            const uint16_t *xg = x + r * d + j * G;
            float absmax = 0.0f;
            for (int i = 0; i < G; ++i) {
                double xd = orc_f16_to_f64(xg[i]);
                if (!isfinite(xd))
                    bad = 1;
                else if (fabsf((float)xd) > absmax)
                    absmax = fabsf((float)xd);
            }
            float s = absmax / 7.0f;                  /* IEEE fp32 division */
            scales[r * ng + j] = s;
            for (int i = 0; i < G; ++i) {
                int8_t c = 0;
                if (s != 0.0f) {
                    float y = (float)orc_f16_to_f64(xg[i]) / s;
                    float q = rintf(y);
                    if (q > 7.0f) q = 7.0f;
                    if (q < -7.0f) q = -7.0f;
                    c = (int8_t)q;
                }
                codes[r * d + j * G + i] = c;
            }
        }
    return bad ? -1 : 0;
}

/* x_hat = code * scale, exact in fp64 (INT8 and INT4 alike). */
ORC_API void orc_int8_dequantize_rows(const int8_t *codes, const float *scales,
                                      int64_t rows, int d, int G, double *out)
{
    int ng = d / G;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int i = 0; i < d; ++i)
            out[r * d + i] = (double)codes[r * d + i] * (double)scales[r * ng + i / G];
}

/* ------------------------------------------------------------------ */
/* FP8 E4M3 (OCP "FN" variant)                                          */
/* value(code) for exponent field e and mantissa m:                      */
/*   e == 0 : m/8 * 2^-6   (subnormal)                                   */
/*   e >= 1 : (1 + m/8) * 2^(e-7); e == 15 and m == 7 is NaN             */
/* ------------------------------------------------------------------ */
ORC_API double orc_e4m3_decode(uint8_t c)
{
    int sign = c >> 7;
    int e = (c >> 3) & 0xf;
    int m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return sign ? -v : v;
}

/* Round a finite fp32 value to E4M3: nearest representable, ties to the
 * even mantissa, magnitudes beyond the largest finite value saturate. */
ORC_API uint8_t orc_e4m3_encode(float yf)
{
    double y = (double)yf;
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs(y);
    if (!(a < 448.0))                   /* 448 = 1.75 * 2^8, largest finite */
        return (uint8_t)(sign | 0x7e);
    if (a == 0.0)
        return sign;
    int ex;
    frexp(a, &ex);                      /* a = f * 2^ex, f in [0.5, 1) */
    int E = ex - 1;                     /* a in [2^E, 2^(E+1))          */
    if (E < -6)
        E = -6;                         /* below 2^-6: subnormal spacing */
    double quantum = ldexp(1.0, E - 3); /* 3 fraction bits               */
    double n = nearbyint(a / quantum);  /* exact quotient, then RNE      */
    double v = n * quantum;             /* representable (or 2^(E+1))    */
    if (v == 0.0)
        return sign;                    /* negative underflow keeps -0   */
    int e2;
    frexp(v, &e2);
    int E2 = e2 - 1;
    int efield, mfield;
    if (E2 < -6) {                      /* subnormal: v = m * 2^-9       */
        efield = 0;
        mfield = (int)(v / ldexp(1.0, -9));
    } else {
        efield = E2 + 7;
        mfield = (int)(v / ldexp(1.0, E2 - 3)) - 8;
    }
    return (uint8_t)(sign | (efield << 3) | mfield);
}

/* ------------------------------------------------------------------ */
/* FP8 E5M2 (OCP)                                                       */
/* value(code) for exponent field e and mantissa m:                      */
/*   e == 0  : m/4 * 2^-14  (subnormal)                                  */
/*   e == 31 : infinity (m == 0) or NaN                                  */
/*   else    : (1 + m/4) * 2^(e-15)                                      */
/* ------------------------------------------------------------------ */
ORC_API double orc_e5m2_decode(uint8_t c)
{
    int sign = c >> 7;
    int e = (c >> 2) & 0x1f;
    int m = c & 3;
    double v;
    if (e == 31) {
        if (m)
            return NAN;
        v = INFINITY;
    } else if (e == 0) {
        v = ldexp((double)m, -16);
    } else {
        v = ldexp((double)(4 + m), e - 17);
    }
    return sign ? -v : v;
}

/* Round a finite fp32 value to E5M2: nearest representable, ties to the
 * even mantissa, magnitudes beyond the largest finite value (57344)
 * saturate. */
ORC_API uint8_t orc_e5m2_encode(float yf)
{
    double y = (double)yf;
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs(y);
    if (!(a < 57344.0))                 /* 1.75 * 2^15, largest finite */
        return (uint8_t)(sign | 0x7b);
    if (a == 0.0)
        return sign;
    int ex;
    frexp(a, &ex);
    int E = ex - 1;                     /* a in [2^E, 2^(E+1))          */
    if (E < -14)
        E = -14;                        /* below 2^-14: subnormal spacing */
    double quantum = ldexp(1.0, E - 2); /* 2 fraction bits               */
    double n = nearbyint(a / quantum);
    double v = n * quantum;
    if (v == 0.0)
        return sign;
    int e2;
    frexp(v, &e2);
    int E2 = e2 - 1;
    int efield, mfield;
    if (E2 < -14) {                     /* subnormal: v = m * 2^-16      */
        efield = 0;
        mfield = (int)(v / ldexp(1.0, -16));
    } else {
        efield = E2 + 15;
        mfield = (int)(v / ldexp(1.0, E2 - 2)) - 4;
    }
    return (uint8_t)(sign | (efield << 2) | mfield);
}

/* fmt: 0 = E4M3, 1 = E5M2 */
static double fp8_decode(uint8_t c, int fmt)
{
    return fmt ? orc_e5m2_decode(c) : orc_e4m3_decode(c);
}

static uint8_t fp8_encode(float y, int fmt)
{
    return fmt ? orc_e5m2_encode(y) : orc_e4m3_encode(y);
}

static float fp8_max(int fmt)
{
    return fmt ? 57344.0f : 448.0f;
}

/* Static per-head scale.  x: [rows][Hkv][d] fp16 bits; S: [Hkv]; codes same
 * shape as x.  code = fp8(fl32(x / S[h])). */
ORC_API int orc_fp8_quantize_rows_fmt(const uint16_t *x, int64_t rows, int Hkv,
                                      int d, const float *S, int fmt,
                                      uint8_t *codes)
{
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r)
        for (int h = 0; h < Hkv; ++h)
            for (int i = 0; i < d; ++i) {
                int64_t k = (r * Hkv + h) * d + i;
                double xd = orc_f16_to_f64(x[k]);
                if (!isfinite(xd)) {
                    bad = 1;
                    continue;
                }
                if (S[h] == 0.0f) {           /* no scale: code 0 */
                    codes[k] = 0;
                    continue;
                }
                float y = (float)xd / S[h];
                codes[k] = fp8_encode(y, fmt);
            }
    return bad ? -1 : 0;
}

ORC_API int orc_fp8_quantize_rows(const uint16_t *x, int64_t rows, int Hkv,
                                  int d, const float *S, uint8_t *codes)
{
    return orc_fp8_quantize_rows_fmt(x, rows, Hkv, d, S, 0, codes);
}

ORC_API void orc_fp8_dequantize_rows_fmt(const uint8_t *codes, int64_t rows,
                                         int Hkv, int d, const float *S,
                                         int fmt, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int h = 0; h < Hkv; ++h)
            for (int i = 0; i < d; ++i) {
                int64_t k = (r * Hkv + h) * d + i;
                out[k] = fp8_decode(codes[k], fmt) * (double)S[h];
            }
}

ORC_API void orc_fp8_dequantize_rows(const uint8_t *codes, int64_t rows,
                                     int Hkv, int d, const float *S,
                                     double *out)
{
    orc_fp8_dequantize_rows_fmt(codes, rows, Hkv, d, S, 0, out);
}

/* Dynamic per-group scale: rows of d elements, groups of G consecutive
 * elements; s = fl32(absmax / FP8_MAX), code = fp8(fl32(x / s)); an
 * all-zero group stores s = 0 and codes 0.  codes: [rows][d]; scales:
 * [rows][d/G]. */
ORC_API int orc_fp8_quantize_groups(const uint16_t *x, int64_t rows, int d,
                                    int G, int fmt, uint8_t *codes,
                                    float *scales)
{
    if (G <= 0 || d % G != 0)
        return -2;
    int ng = d / G;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r)
        for (int j = 0; j < ng; ++j) {
            const uint16_t *xg = x + r * d + j * G;
            float absmax = 0.0f;
            for (int i = 0; i < G; ++i) {
                double xd = orc_f16_to_f64(xg[i]);
                if (!isfinite(xd))
                    bad = 1;
                else if (fabsf((float)xd) > absmax)
                    absmax = fabsf((float)xd);
            }
            float s = absmax / fp8_max(fmt);          /* IEEE fp32 division */
            scales[r * ng + j] = s;
            for (int i = 0; i < G; ++i) {
                if (s == 0.0f) {
                    codes[r * d + j * G + i] = 0;
                    continue;
                }
                float y = (float)orc_f16_to_f64(xg[i]) / s;
                codes[r * d + j * G + i] = fp8_encode(y, fmt);
            }
        }
    return bad ? -1 : 0;
}

ORC_API void orc_fp8_dequantize_groups(const uint8_t *codes,
                                       const float *scales, int64_t rows,
                                       int d, int G, int fmt, double *out)
{
    int ng = d / G;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int i = 0; i < d; ++i)
            out[r * d + i] = fp8_decode(codes[r * d + i], fmt) *
                             (double)scales[r * ng + i / G];
}

/* ------------------------------------------------------------------ */
/* INT8 per-channel, static scales ([P3] s2.3 per_channel)              */
/* x: [rows][Hkv][d] fp16 bits; S: [Hkv][d]; codes same shape as x.      */
/* ------------------------------------------------------------------ */
ORC_API int orc_int8_quantize_channels(const uint16_t *x, int64_t rows,
                                       int Hkv, int d, const float *S,
                                       int8_t *codes)
{
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r)
        for (int h = 0; h < Hkv; ++h)
            for (int i = 0; i < d; ++i) {
                int64_t k = (r * Hkv + h) * d + i;
                double xd = orc_f16_to_f64(x[k]);
                float s = S[h * d + i];
                if (!isfinite(xd)) {
                    bad = 1;
                    continue;
                }
                if (s == 0.0f) {
                    codes[k] = 0;
                    continue;
                }
                float y = (float)xd / s;              /* fp32, correctly rounded */
                float q = rintf(y);                   /* nearest, ties to even   */
                if (q > 127.0f) q = 127.0f;
                if (q < -127.0f) q = -127.0f;
                codes[k] = (int8_t)q;
            }
    return bad ? -1 : 0;
}

ORC_API void orc_int8_dequantize_channels(const int8_t *codes, int64_t rows,
                                          int Hkv, int d, const float *S,
                                          double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int h = 0; h < Hkv; ++h)
            for (int i = 0; i < d; ++i) {
                int64_t k = (r * Hkv + h) * d + i;
                out[k] = (double)codes[k] * (double)S[h * d + i];
            }
}

/* ------------------------------------------------------------------ */
/* Decode attention on contiguous (un-paged) dequantized K/V            */
/* ([P3] s1.1 and s2.1).                                                 */
/*                                                                      */
/* q     : [B][Hq][d] fp16 bits                                         */
/* K, V  : all sequences concatenated, [sum ctx][Hkv][d] fp64            */
/* cu    : [B+1] token offsets of each sequence inside K / V            */
/* out   : [B][Hq][d] fp64                                              */
/* For query head g, KV head h = g / (Hq / Hkv):                        */
/*   z_t = sm * sum_i q[g][i] * K[t][h][i],  t < ctx                    */
/*   p   = softmax(z) (max-subtracted, fp64),                            */
/*   o   = sum_t p_t * V[t][h][:].                                       */
/* ------------------------------------------------------------------ */
ORC_API int orc_decode_attention(const uint16_t *q, const double *K,
                                 const double *V, const int64_t *cu, int B,
                                 int Hq, int Hkv, int d, double sm, double *out)
{
    if (Hkv <= 0 || Hq % Hkv != 0)
        return -2;
    for (int b = 0; b < B; ++b)
        if (cu[b + 1] - cu[b] < 1)
            return -2;                  /* a decode step needs ctx >= 1 */
    int r = Hq / Hkv;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) collapse(2) reduction(| : err)
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < Hq; ++g) {
            int h = g / r;
            int64_t t0 = cu[b], ctx = cu[b + 1] - cu[b];
            double *z = (double *)malloc(sizeof(double) * (size_t)ctx);
            double *qd = (double *)malloc(sizeof(double) * (size_t)d);
            if (!z || !qd) {
                free(z);
                free(qd);
                err = 1;
                continue;
            }
            for (int i = 0; i < d; ++i)
                qd[i] = orc_f16_to_f64(q[((int64_t)b * Hq + g) * d + i]);
            double zmax = -INFINITY;
            for (int64_t t = 0; t < ctx; ++t) {
                const double *kr = K + ((t0 + t) * Hkv + h) * d;
                double acc = 0.0;
                for (int i = 0; i < d; ++i)
                    acc += qd[i] * kr[i];
                z[t] = acc * sm;
                if (z[t] > zmax)
                    zmax = z[t];
            }
            double L = 0.0;
            for (int64_t t = 0; t < ctx; ++t) {
                z[t] = exp(z[t] - zmax);
                L += z[t];
            }
            double *o = out + ((int64_t)b * Hq + g) * d;
            for (int i = 0; i < d; ++i)
                o[i] = 0.0;
            for (int64_t t = 0; t < ctx; ++t) {
                const double *vr = V + ((t0 + t) * Hkv + h) * d;
                double w = z[t] / L;
                for (int i = 0; i < d; ++i)
                    o[i] += w * vr[i];
            }
            free(z);
            free(qd);
        }
    return err ? -3 : 0;
}

/* ------------------------------------------------------------------ */
/* Prefill (chunked) attention over contiguous dequantized K/V          */
/* ([P3] s1.1: prefill computes the K/V of every prompt token and each   */
/* token attends to the tokens before it; xpshop.cn article 312 s6:      */
/* long prompts are processed in chunks).                                */
/*                                                                      */
/* Sequence b holds ctx_b tokens (its cached ones and then the n_b of    */
/* this chunk, whose K/V are already in the cache); chunk token i is at  */
/* position ctx_b - n_b + i and attends to tokens t <= that position.    */
/* q     : [sum n][Hq][d] fp16 bits, chunks concatenated in batch order  */
/* K, V  : [sum ctx][Hkv][d] fp64, sequences concatenated                */
/* cu_q  : [B+1] chunk offsets in q;  cu_k : [B+1] offsets in K / V      */
/* out   : [sum n][Hq][d] fp64                                          */
/* ------------------------------------------------------------------ */
ORC_API int orc_prefill_attention(const uint16_t *q, const double *K,
                                  const double *V, const int64_t *cu_q,
                                  const int64_t *cu_k, int B, int Hq, int Hkv,
                                  int d, double sm, double *out)
{
    if (Hkv <= 0 || Hq % Hkv != 0)
        return -2;
    for (int b = 0; b < B; ++b) {
        int64_t n = cu_q[b + 1] - cu_q[b], ctx = cu_k[b + 1] - cu_k[b];
        if (n < 0 || n > ctx)
            return -2;                  /* the chunk is part of the context */
    }
    int r = Hq / Hkv;
    int64_t total = cu_q[B];
    int err = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : err)
    for (int64_t row = 0; row < total; ++row) {
        int b = 0;
        while (cu_q[b + 1] <= row)
            ++b;
        int64_t n = cu_q[b + 1] - cu_q[b], ctx = cu_k[b + 1] - cu_k[b];
        int64_t pos = ctx - n + (row - cu_q[b]);
        int64_t len = pos + 1;          /* causal: tokens 0 .. pos */
        double *z = (double *)malloc(sizeof(double) * (size_t)len);
        double *qd = (double *)malloc(sizeof(double) * (size_t)d);
        if (!z || !qd) {
            free(z);
            free(qd);
            err = 1;
            continue;
        }
        for (int g = 0; g < Hq; ++g) {
            int h = g / r;
            for (int i = 0; i < d; ++i)
                qd[i] = orc_f16_to_f64(q[(row * Hq + g) * d + i]);
            double zmax = -INFINITY;
            for (int64_t t = 0; t < len; ++t) {
                const double *kr = K + ((cu_k[b] + t) * Hkv + h) * d;
                double acc = 0.0;
                for (int i = 0; i < d; ++i)
                    acc += qd[i] * kr[i];
                z[t] = acc * sm;
                if (z[t] > zmax)
                    zmax = z[t];
            }
            double L = 0.0;
            for (int64_t t = 0; t < len; ++t) {
                z[t] = exp(z[t] - zmax);
                L += z[t];
            }
            double *o = out + (row * Hq + g) * d;
            for (int i = 0; i < d; ++i)
                o[i] = 0.0;
            for (int64_t t = 0; t < len; ++t) {
                const double *vr = V + ((cu_k[b] + t) * Hkv + h) * d;
                double w = z[t] / L;
                for (int i = 0; i < d; ++i)
                    o[i] += w * vr[i];
            }
        }
        free(z);
        free(qd);
    }
    return err ? -3 : 0;
}

/* ------------------------------------------------------------------ */
/* KV byte formula ([P3] s1.2): 2 * batch * seq_len * layers * kv_heads  */
/* * head_dim * bytes_per_element.  The INT8 per-group layout adds one   */
/* fp32 scale per group for K and for V (the pages do not print this     */
/* term; it follows from storing a scale per group, [P3] s2.3).          */
/* ------------------------------------------------------------------ */
ORC_API int64_t orc_kv_cache_bytes(int64_t batch, int64_t seq_len,
                                   int64_t layers, int64_t kv_heads,
                                   int64_t head_dim, int64_t elem_bytes)
{
    return 2 * batch * seq_len * layers * kv_heads * head_dim * elem_bytes;
}

ORC_API int64_t orc_kv_cache_bytes_int8_group(int64_t batch, int64_t seq_len,
                                              int64_t layers, int64_t kv_heads,
                                              int64_t head_dim, int64_t G)
{
    return orc_kv_cache_bytes(batch, seq_len, layers, kv_heads, head_dim, 1) +
           2 * batch * seq_len * layers * kv_heads * (head_dim / G) * 4;
}

ORC_API int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads used by the parallel loops from now on (for timing the oracle at
 * one thread and at all cores). */
ORC_API void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
