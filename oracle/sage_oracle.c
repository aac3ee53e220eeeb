/*
 * sage_oracle.c -- plain, slow CPU oracle for SageAttention-style quantized
 * attention.  TEST INFRASTRUCTURE ONLY: it is loaded by the tests, by the
 * package's smoke check and by the benchmark's CPU-baseline leg, never by the
 * library's product path.  It shares no code with the HIP kernels.
 *
 * Built with gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp, so every
 * float expression below rounds exactly once, in the written order.
 *
 * What it computes, and the passages it follows:
 *   - Online softmax: m_0 = -inf, d_0 = 0, m_i = max(m_{i-1}, a_i),
 *     d_i = d_{i-1} exp(m_{i-1}-m_i) + exp(a_i - m_i); result exp(a-m_n)/d_n
 *     (SageAttention review thread, reply to reviewer xY6z Q3).
 *   - FlashAttention tiling: rows of the score tile S_i^j are the queries of a
 *     Q tile, columns the keys of a K tile; one pass over K tiles per query
 *     (same reply).  Normalisation by diag(l)^-1 once, after the last K tile,
 *     with l^0 = 0 (reply to xY6z Q2).
 *   - Smoothing K, INT8 QK^T, per-block quantization granularity
 *     (SageAttention contributions, reply to reviewer wwcu W1; SageAttn-B, reply
 *     to xY6z W1-(2) and Q1).
 *   - P~ and V in FP8, smoothing Q for the 4-bit QK^T, two-level accumulation
 *     of P~V (SageAttention2 abstract, Jianfei Chen author page).
 *   - Microscaling FP4 attention (SageAttention3 abstract); the MX format is a
 *     fine-grained per-group quantization (TetraJet abstract, same author page).
 *   - 8-bit forward + backward for training (SageAttention3 abstract): the
 *     oracle gives the exact fp64 backward the GPU gradients are held to.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   mean over all N tokens per (b,h,channel) for smoothing; INT8 symmetric
 *   +-127 with delta = amax/127 and code = rne(x/delta) in fp32; FP8 = OCP
 *   E4M3FN (RNE, saturating at 448); P~ = E4M3(448 p); V per-channel FP8 scale;
 *   MXFP4 = OCP MX: E2M1 elements, 32-element blocks, E8M0 scale with
 *   e = floor(log2 amax) - 2; P~ in the 4-bit path gets a per-row per-K-tile
 *   fp32 scale sigma = 6 / max_tile(p) before MX quantization over 32-key groups;
 *   the row sum l accumulates the unquantized p; LSE is natural-log over the
 *   true (unsmoothed) scores.  Every P~ code is decided from the fp64 p; a
 *   weight whose p lies within a stated relative window of a rounding boundary
 *   has a second admissible code, and the simulation reports, per output, how
 *   far the other choice could move it (see p_window).  Non-finite inputs follow IEEE arithmetic through
 *   these steps: a NaN score makes its row's max and sum NaN (not a masked key),
 *   the E8M0 byte 0xFF is NaN (OCP MX), the P~V sum takes every key of the tile
 *   (0 * NaN = NaN), and INT8 codes clamp with fmaxf / fminf (NaN -> -127).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_API __attribute__((visibility("default")))

#ifdef _OPENMP
#include <omp.h>
#endif

/* Host threads the oracle's parallel loops use (n <= 0: the OpenMP default); returns the
 * count in effect.  Timing aid for the CPU baseline; no effect on any result. */
OR_API int or_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* Widening of the 16-bit input formats (exact).                       */
/* ------------------------------------------------------------------ */
static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static float f16_to_float(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return (float)(s ? -v : v);
}

/* dtype: 0 = bf16, 1 = fp16 */
OR_API void or_widen(const uint16_t *src, int dtype, float *dst, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        dst[i] = dtype == 0 ? bf16_to_float(src[i]) : f16_to_float(src[i]);
}

/* ------------------------------------------------------------------ */
/* Element codecs (OCP 8-bit FP and MX formats, INT8).                 */
/* ------------------------------------------------------------------ */

/* floor(log2 a) for finite a > 0, exact. */
static int floor_log2(double a)
{
    int e;
    frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1) */
    return e - 1;
}

/* E4M3FN decode: bias 7, 3 mantissa bits, subnormals, 0x7F/0xFF = NaN. */
OR_API double or_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);                  /* m/8 * 2^-6 */
    else
        v = ldexp((double)(8 + m), e - 10);        /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* E4M3FN encode: round to nearest, ties to even, saturate to +-448. */
OR_API uint8_t or_e4m3_encode(double x)
{
    uint8_t s = signbit(x) ? 0x80 : 0x00;
    if (isnan(x))
        return s | 0x7F;
    double a = fabs(x);
    if (a >= 448.0)
        return s | 0x7E;
    if (a == 0.0)
        return s;
    int E = floor_log2(a);
    if (E < -6)
        E = -6;                                    /* subnormal range shares 2^-6's quantum */
    double quantum = ldexp(1.0, E - 3);
    double n = rint(a / quantum);                  /* integer in [0, 16]; rint = RNE */
    double v = n * quantum;                        /* the rounded magnitude, <= 448 */
    if (v == 0.0)
        return s;
    int Ev = floor_log2(v);
    if (Ev < -6)
        return s | (uint8_t)(v / ldexp(1.0, -9));  /* subnormal: exponent field 0 */
    int mant = (int)(v / ldexp(1.0, Ev - 3)) - 8;
    return s | (uint8_t)(((Ev + 7) << 3) | mant);
}

/* IEEE binary16 decode: bias 15, 10 mantissa bits, subnormals, e = 31 inf / NaN. */
OR_API double or_f16_decode(uint16_t c)
{
    int s = c >> 15, e = (c >> 10) & 31, m = c & 1023;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -24);                 /* m/1024 * 2^-14 */
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return s ? -v : v;
}

/* IEEE binary16 encode: round to nearest, ties to even; magnitudes that round past the
 * largest finite value (65504) become infinity, as IEEE rounding does. */
OR_API uint16_t or_f16_encode(double x)
{
    uint16_t s = signbit(x) ? 0x8000 : 0x0000;
    if (isnan(x))
        return s | 0x7E00;
    double a = fabs(x);
    if (a == 0.0)
        return s;
    int E = floor_log2(a);
    if (E < -14)
        E = -14;                                   /* subnormal range shares 2^-14's quantum */
    double quantum = ldexp(1.0, E - 10);
    double v = rint(a / quantum) * quantum;        /* RNE to 11 significant bits */
    if (v >= 65536.0)
        return s | 0x7C00;                         /* overflow: infinity */
    if (v == 0.0)
        return s;
    int Ev = floor_log2(v);
    if (Ev < -14)
        return s | (uint16_t)(v / ldexp(1.0, -24));  /* subnormal: exponent field 0 */
    int mant = (int)(v / ldexp(1.0, Ev - 10)) - 1024;
    return s | (uint16_t)(((Ev + 15) << 10) | mant);
}

/* V as fp16 codes (the 16-bit P~V fallback): out[i] = fl16(v[i]). */
OR_API void or_quant_v_f16(const float *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = or_f16_encode((double)v[i]);
}

/* E2M1 decode: magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}. */
OR_API double or_e2m1_decode(uint8_t c)
{
    int e = (c >> 1) & 3, m = c & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (c & 8) ? -v : v;
}

/* E2M1 encode: round to nearest, ties to even, saturate to +-6. */
OR_API uint8_t or_e2m1_encode(double x)
{
    uint8_t s = signbit(x) ? 0x8 : 0x0;
    double a = fabs(x);
    if (isnan(x))
        return s | 0x7;                            /* no NaN in E2M1: saturate */
    if (a >= 6.0)
        return s | 0x7;
    int E = (a < 1.0) ? 0 : floor_log2(a);
    double quantum = ldexp(1.0, E - 1);
    double v = rint(a / quantum) * quantum;
    for (uint8_t c = 0; c < 8; c++)
        if (or_e2m1_decode(c) == v)
            return s | c;
    return s | 0x7;                                /* unreachable */
}

/* MX shared exponent of a block with amax a, for an element format whose
 * largest power of two is 2^emax: e = floor(log2 a) - emax, clamped to the
 * E8M0 range; a == 0 gives the byte 0.  Returns the E8M0 byte (e + 127). */
OR_API uint8_t or_mx_scale_byte(double amax, int emax)
{
    if (amax == 0.0)
        return 0;
    if (isnan(amax) || isinf(amax))
        return 0xFF;
    int e = floor_log2(amax) - emax;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return (uint8_t)(e + 127);
}

/* E8M0 byte -> 2^(b - 127); the byte 0xFF encodes NaN (OCP MX v1.0, the E8M0 scale format). */
static double e8m0_decode(uint8_t b)
{
    return b == 0xFF ? NAN : ldexp(1.0, (int)b - 127);
}

/* INT8 symmetric code with step delta (fp32): clamp(rne(fl32(x / delta)), -127, 127). */
OR_API int8_t or_int8_encode(float x, float delta)
{
    if (delta == 0.0f)
        return 0;
    float r = x / delta;                           /* one correctly rounded fp32 division */
    /* fmaxf / fminf return the non-NaN operand, so a NaN quotient (a NaN or infinite input
     * or step) clamps to -127 instead of reaching an undefined float -> int conversion */
    float n = fminf(fmaxf(rintf(r), -127.0f), 127.0f);
    return (int8_t)n;
}

/* ------------------------------------------------------------------ */
/* Prologue: statistics and codes for one (b,h) head.                  */
/* ------------------------------------------------------------------ */

/* mu[c] = fl32( (sum_t x[t,c]) / N ), the sum in fp64 in token order; an empty
 * sequence (N = 0) has nothing to smooth and gets mu = 0. */
static void channel_mean(const float *x, int N, int d, float *mu)
{
    for (int c = 0; c < d; c++) {
        if (N == 0) {
            mu[c] = 0.0f;
            continue;
        }
        double s = 0.0;
        for (int t = 0; t < N; t++)
            s += (double)x[(int64_t)t * d + c];
        mu[c] = (float)(s / (double)N);
    }
}

static float absmax(const float *x, int64_t n, int64_t stride)
{
    float a = 0.0f;
    for (int64_t i = 0; i < n; i++) {
        float v = fabsf(x[i * stride]);
        if (v > a || isnan(v))
            a = v;
    }
    return a;
}

/* INT8 codes per blk-token block over all d channels. */
static void quant_int8_blocks(const float *x, int N, int d, int blk, int8_t *codes, float *scales)
{
    int nb = (N + blk - 1) / blk;
    for (int b = 0; b < nb; b++) {
        int t0 = b * blk, t1 = t0 + blk < N ? t0 + blk : N;
        float a = absmax(x + (int64_t)t0 * d, (int64_t)(t1 - t0) * d, 1);
        float delta = a / 127.0f;
        scales[b] = delta;
        for (int64_t i = (int64_t)t0 * d; i < (int64_t)t1 * d; i++)
            codes[i] = or_int8_encode(x[i], delta);
    }
}

/* MX quantization of a group of n elements at stride `stride`, element format
 * E2M1 (emax 2) or E4M3 (emax 8).  Codes are stored one per byte. */
static void quant_mx_group(const float *x, int n, int64_t stride, int elem_fmt,
                           uint8_t *codes, int64_t cstride, uint8_t *scale_byte)
{
    int emax = elem_fmt == 4 ? 2 : 8;
    float a = absmax(x, n, stride);
    uint8_t sb = or_mx_scale_byte(a, emax);
    *scale_byte = sb;
    double inv = ldexp(1.0, -((int)sb - 127));     /* 2^-e, exact */
    for (int i = 0; i < n; i++) {
        double y = (sb == 0 && a == 0.0f) ? 0.0 * x[i * stride] : (double)x[i * stride] * inv;
        codes[i * cstride] = elem_fmt == 4 ? or_e2m1_encode(y) : or_e4m3_encode(y);
    }
}

/*
 * INT8-QK / FP8-PV prologue for BH heads: queries [BH,Nq,d], keys and values
 * [BH,Nk,d] fp32 (Nq = Nk for self-attention).
 *   mu_k [BH,d]; qc [BH,Nq,d], kc [BH,Nk,d] int8; qs [BH,nbq], ks [BH,nbk] fp32
 *   (nbq = ceil(Nq/qblk), nbk = ceil(Nk/kblk): a step per qblk query tokens and per
 *   kblk key tokens); vc [BH,Nk,d] E4M3 codes (token-major); vs [BH,d] fp32;
 *   corr [BH,Nq] fp64 = sm * q_i . mu_k (the per-row score shift removed by
 *   smoothing K).
 */
OR_API void or_quant_int8_fp8_x(const float *q, const float *k, const float *v,
                                int BH, int Nq, int Nk, int d, int qblk, int kblk, double sm,
                                float *mu_k, int8_t *qc, float *qs, int8_t *kc, float *ks,
                                uint8_t *vc, float *vs, double *corr)
{
    int nbq = (Nq + qblk - 1) / qblk, nbk = (Nk + kblk - 1) / kblk;
#pragma omp parallel for schedule(dynamic)
    for (int h = 0; h < BH; h++) {
        int64_t offq = (int64_t)h * Nq * d, offk = (int64_t)h * Nk * d;
        const float *Q = q + offq, *K = k + offk, *V = v + offk;
        float *mu = mu_k + (int64_t)h * d;
        channel_mean(K, Nk, d, mu);
        float *Ks = malloc(sizeof(float) * ((size_t)Nk * d + 1));
        for (int t = 0; t < Nk; t++)
            for (int c = 0; c < d; c++)
                Ks[(int64_t)t * d + c] = K[(int64_t)t * d + c] - mu[c];
        quant_int8_blocks(Q, Nq, d, qblk, qc + offq, qs + (int64_t)h * nbq);
        quant_int8_blocks(Ks, Nk, d, kblk, kc + offk, ks + (int64_t)h * nbk);
        for (int c = 0; c < d; c++) {
            float a = absmax(V + c, Nk, d);
            float delta = a / 448.0f;
            vs[(int64_t)h * d + c] = delta;
            for (int t = 0; t < Nk; t++) {
                float y = delta == 0.0f ? 0.0f : V[(int64_t)t * d + c] / delta;
                vc[offk + (int64_t)t * d + c] = or_e4m3_encode(y);
            }
        }
        for (int t = 0; t < Nq; t++) {
            double s = 0.0;
            for (int c = 0; c < d; c++)
                s += (double)Q[(int64_t)t * d + c] * (double)mu[c];
            corr[(int64_t)h * Nq + t] = sm * s;
        }
        free(Ks);
    }
}

OR_API void or_quant_int8_fp8(const float *q, const float *k, const float *v,
                              int BH, int N, int d, int blk, double sm,
                              float *mu_k, int8_t *qc, float *qs, int8_t *kc, float *ks,
                              uint8_t *vc, float *vs, double *corr)
{
    or_quant_int8_fp8_x(q, k, v, BH, N, N, d, blk, blk, sm, mu_k, qc, qs, kc, ks, vc, vs, corr);
}

/*
 * MXFP4-QK prologue.  Q and K are both smoothed by their channel means; the
 * smoothed rows are MX-quantized in 32-channel groups (E2M1 codes one per
 * byte, [BH,Nq,d] and [BH,Nk,d]; E8M0 bytes [BH,Nq,d/32] and [BH,Nk,d/32]).
 *   dS [BH,Nk] = fl32(sum_c mu_q[c] * Ks[t,c]) (fp64 sum in channel order):
 *       Q.Ks^T = Qs.Ks^T + 1 dS^T exactly, so dS is added back to every score.
 *   corr [BH,Nq] = sm * q_t . mu_k (fp64), added back to the LSE only.
 *   pv_fmt 3 (MXFP4): V codes [BH,Nk,d] E2M1 in 32-token groups per channel,
 *       E8M0 bytes ve [BH, ceil(Nk/32), d].
 *   pv_fmt 4 (MXFP8): the same grouping with E4M3 elements (emax 8).
 *   pv_fmt 2 (FP8): V codes E4M3 with per-channel fp32 scale vs [BH,d].
 *   qsb: Q is smoothed per block of qsb query tokens (0: one block, the whole sequence);
 *       mu_q is then [BH, nqb, d] and dS [BH, nqb, Nk] with nqb = ceil(Nq / qsb): the key
 *       term of query block b is mu_q[b] . Ks[t].
 */
OR_API void or_quant_mxfp4_x(const float *q, const float *k, const float *v,
                             int BH, int Nq, int Nk, int d, int pv_fmt, int qsb, double sm,
                             float *mu_q, float *mu_k,
                             uint8_t *qc, uint8_t *qe, uint8_t *kc, uint8_t *ke,
                             float *dS, double *corr,
                             uint8_t *vc, uint8_t *ve, float *vs)
{
    int ng = d / 32, nvg = (Nk + 31) / 32;
    int bq = qsb > 0 ? qsb : (Nq > 0 ? Nq : 1), nqb = (Nq + bq - 1) / bq;
    if (nqb < 1)
        nqb = 1;
#pragma omp parallel for schedule(dynamic)
    for (int h = 0; h < BH; h++) {
        int64_t offq = (int64_t)h * Nq * d, offk = (int64_t)h * Nk * d;
        const float *Q = q + offq, *K = k + offk, *V = v + offk;
        float *muq = mu_q + (int64_t)h * nqb * d, *muk = mu_k + (int64_t)h * d;
        for (int b = 0; b < nqb; b++) {
            int t0 = b * bq, n = Nq - t0 < bq ? Nq - t0 : bq;
            channel_mean(Q + (int64_t)t0 * d, n > 0 ? n : 0, d, muq + (int64_t)b * d);
        }
        channel_mean(K, Nk, d, muk);
        float *Qs = malloc(sizeof(float) * ((size_t)Nq * d + 1));
        float *Ks = malloc(sizeof(float) * ((size_t)Nk * d + 1));
        for (int t = 0; t < Nq; t++)
            for (int c = 0; c < d; c++)
                Qs[(int64_t)t * d + c] = Q[(int64_t)t * d + c] - muq[(int64_t)(t / bq) * d + c];
        for (int t = 0; t < Nk; t++)
            for (int c = 0; c < d; c++)
                Ks[(int64_t)t * d + c] = K[(int64_t)t * d + c] - muk[c];
        for (int t = 0; t < Nq; t++)
            for (int g = 0; g < ng; g++) {
                int64_t e0 = (int64_t)t * d + 32 * g;
                quant_mx_group(Qs + e0, 32, 1, 4, qc + offq + e0, 1, qe + ((int64_t)h * Nq + t) * ng + g);
            }
        for (int t = 0; t < Nk; t++)
            for (int g = 0; g < ng; g++) {
                int64_t e0 = (int64_t)t * d + 32 * g;
                quant_mx_group(Ks + e0, 32, 1, 4, kc + offk + e0, 1, ke + ((int64_t)h * Nk + t) * ng + g);
            }
        for (int b = 0; b < nqb; b++)
            for (int t = 0; t < Nk; t++) {
                double s = 0.0;
                for (int c = 0; c < d; c++)
                    s += (double)muq[(int64_t)b * d + c] * (double)Ks[(int64_t)t * d + c];
                dS[((int64_t)h * nqb + b) * Nk + t] = (float)s;
            }
        for (int t = 0; t < Nq; t++) {
            double cq = 0.0;
            for (int c = 0; c < d; c++)
                cq += (double)Q[(int64_t)t * d + c] * (double)muk[c];
            corr[(int64_t)h * Nq + t] = sm * cq;
        }
        if (pv_fmt == 3 || pv_fmt == 4) {
            for (int c = 0; c < d; c++)
                for (int g = 0; g < nvg; g++) {
                    int t0 = 32 * g, n = Nk - t0 < 32 ? Nk - t0 : 32;
                    quant_mx_group(V + (int64_t)t0 * d + c, n, d, pv_fmt == 3 ? 4 : 8,
                                   vc + offk + (int64_t)t0 * d + c, d, ve + ((int64_t)h * nvg + g) * d + c);
                }
        } else {
            for (int c = 0; c < d; c++) {
                float a = absmax(V + c, Nk, d);
                float delta = a / 448.0f;
                vs[(int64_t)h * d + c] = delta;
                for (int t = 0; t < Nk; t++) {
                    float y = delta == 0.0f ? 0.0f : V[(int64_t)t * d + c] / delta;
                    vc[offk + (int64_t)t * d + c] = or_e4m3_encode(y);
                }
            }
        }
        free(Qs);
        free(Ks);
    }
}

OR_API void or_quant_mxfp4(const float *q, const float *k, const float *v,
                           int BH, int N, int d, int pv_fmt, double sm,
                           float *mu_q, float *mu_k,
                           uint8_t *qc, uint8_t *qe, uint8_t *kc, uint8_t *ke,
                           float *dS, double *corr,
                           uint8_t *vc, uint8_t *ve, float *vs)
{
    or_quant_mxfp4_x(q, k, v, BH, N, N, d, pv_fmt, 0, sm, mu_q, mu_k, qc, qe, kc, ke, dS, corr, vc, ve, vs);
}

/* ------------------------------------------------------------------ */
/* The tiled forward (one query row at a time).                        */
/* ------------------------------------------------------------------ */

enum { QK_EXACT = 0, QK_INT8 = 1, QK_MXFP4 = 3 };
enum { PV_EXACT = 0, PV_FP8 = 2, PV_MXFP4 = 3, PV_MXFP8 = 4, PV_F16 = 5 };

typedef struct {
    int N, d, causal, tile;        /* N: keys (query rows are passed explicitly) */
    int qblk, kblk;                /* INT8: tokens per query / key step */
    double sm;
    int qk, pv;
    /* QK_EXACT: fp64 (smoothed) rows and an optional additive key term */
    const double *qx, *kx;
    /* QK_INT8 */
    const int8_t *qc, *kc;
    const float *qs, *ks;
    /* QK_MXFP4 */
    const uint8_t *q4, *qe, *k4, *ke;
    const float *dS;           /* additive score term [nqb][N] per query block and key (may be NULL) */
    int qsb;                   /* query tokens per dS block (0: one block) */
    const double *dSx;         /* same, fp64, exact mode */
    /* PV */
    const double *vx;          /* PV_EXACT */
    const uint8_t *vc;         /* PV_FP8, PV_MXFP4 or PV_MXFP8 codes */
    const float *vs;           /* PV_FP8 per-channel scale */
    const uint8_t *ve;         /* PV_MXFP4 / PV_MXFP8 E8M0 bytes [ceil(N/32), d] */
    const uint16_t *vh;        /* PV_F16 fp16 codes */
    const double *corr;        /* per-row LSE correction (may be NULL) */
    double *vdec;              /* vval of every (key, channel), decoded once per head by run_rows */
    double *q4d, *k4d;         /* QK_MXFP4: the E2M1 element values of q4 and k4, decoded likewise */
} head_t;

/* MXFP4 QK: the dot product of the decoded MX codes of query i and key j.  Each 32-channel
 * block sums to a multiple of 2^-2 times its scale pair, below 2^11 of it, so fp64 holds the
 * total exactly while the scale pairs of a row lie within 40 binades of each other. */
static double mx_dot(const head_t *H, int i, int j)
{
    int d = H->d, ng = d / 32;
    double s = 0.0;
    for (int g = 0; g < ng; g++) {
        double part = 0.0;
        for (int c = 32 * g; c < 32 * g + 32; c++)   /* or_e2m1_decode of q4 and k4, read from tables */
            part += H->q4d[(int64_t)i * d + c] * H->k4d[(int64_t)j * d + c];
        s += part * e8m0_decode(H->qe[(int64_t)i * ng + g]) * e8m0_decode(H->ke[(int64_t)j * ng + g]);
    }
    return s;
}

/* Unscaled score s_ij (sm not applied).  *mag receives the magnitude the score is built
 * from: |s| itself, or |Q_s K_s| + |dS| when the smoothing term dS is added to a dot product
 * (the two may cancel). */
static double score(const head_t *H, int i, int j, double *mag)
{
    int d = H->d;
    double s = 0.0;
    if (H->qk == QK_EXACT) {
        for (int c = 0; c < d; c++)
            s += H->qx[(int64_t)i * d + c] * H->kx[(int64_t)j * d + c];
        if (H->dSx)
            s += H->dSx[j];
        *mag = fabs(s);
    } else if (H->qk == QK_INT8) {
        int64_t acc = 0;
        for (int c = 0; c < d; c++)
            acc += (int64_t)H->qc[(int64_t)i * d + c] * (int64_t)H->kc[(int64_t)j * d + c];
        s = (double)H->qs[i / H->qblk] * (double)H->ks[j / H->kblk] * (double)acc;
        *mag = fabs(s);
    } else {
        s = mx_dot(H, i, j);
        double ds = H->dS ? (double)H->dS[(int64_t)(H->qsb ? i / H->qsb : 0) * H->N + j] : 0.0;
        *mag = fabs(s) + fabs(ds);
        s += ds;
    }
    return s;
}

/* Decoded V element (without the per-channel FP8 scale, which the epilogue applies).  run_rows
 * evaluates it once per (key, channel) into H->vdec, which the row loop reads. */
static double vval(const head_t *H, int j, int c)
{
    int64_t idx = (int64_t)j * H->d + c;
    if (H->pv == PV_EXACT)
        return H->vx[idx];
    if (H->pv == PV_FP8)
        return or_e4m3_decode(H->vc[idx]);
    if (H->pv == PV_F16)
        return or_f16_decode(H->vh[idx]);
    double e = e8m0_decode(H->ve[(int64_t)(j / 32) * H->d + c]);
    if (H->pv == PV_MXFP8)
        return or_e4m3_decode(H->vc[idx]) * e;
    return or_e2m1_decode(H->vc[idx]) * e;
}

/*
 * Admissible P~ codes.  A P~ code is a value that floating point decides: the code of 448 p
 * (FP8), of p (fp16) or of sigma p under an MX scale (MXFP4).  The pages fix no precision for
 * p, so the oracle decides every code from its fp64 p, and states for each weight how far a
 * correct evaluation in lower precision may move it.  An implementation that forms the exp
 * argument from binary32 quantities (the scale product, the running max, the score and the
 * smoothing term, each rounded a few times) and evaluates exp to a few ulps moves p by a
 * relative amount below
 *     eps = 2^-20 (8 + (|x| + |m| + |m_tile|) log2 e),
 * with x the scaled score (or, with a smoothing term, the sum of the magnitudes it is built
 * from) and m, m_tile the running and tile maxima, all in natural-log units: each binary32
 * rounding of a log2-domain quantity of size A costs at most 2^-24 A, and the bound keeps a
 * factor of about four over the sum of them.  Every code reachable from p (1 +- eps) is then
 * admissible; `dq` receives the width of that set in the code's own units (0 for almost every
 * weight: only values within eps of a rounding midpoint, of the E4M3 saturation point or of a
 * power of two that fixes an MX scale have a second admissible code).
 */
static double p_window(double xmag, double m, double mt)
{
    double a = fabs(xmag) + (isfinite(m) ? fabs(m) : 0.0) + (isfinite(mt) ? fabs(mt) : 0.0);
    return ldexp(8.0 + a * 1.4426950408889634, -20);
}

static double e4m3_round(double y) { return or_e4m3_decode(or_e4m3_encode(y)); }
static double f16_round(double y) { return or_f16_decode(or_f16_encode(y)); }

/* E2M1 value of y under the E8M0 byte sb (the MX element rule), in y's units. */
static double e2m1_round_scaled(double y, uint8_t sb)
{
    double s = ldexp(1.0, (int)sb - 127);
    return or_e2m1_decode(or_e2m1_encode(y / s)) * s;
}

/*
 * One query row of the tiled quantized forward.  o [d] and lse; slack [d] (may be NULL): for
 * each output channel, the largest change of o that a different choice among the admissible
 * P~ codes (see p_window) can make -- sum over weights with two admissible codes of
 * (width) |v| carried through the same rescales and normalisation as O.
 */
static void forward_row(const head_t *H, int i, double *o, double *lse, double *slack)
{
    int N = H->N, d = H->d, T = H->tile;
    double *O = calloc((size_t)d, sizeof(double));
    double *Sl = calloc((size_t)d, sizeof(double));
    double *acc = malloc(sizeof(double) * (size_t)d);
    double *x = malloc(sizeof(double) * (size_t)T);
    double *xm = malloc(sizeof(double) * (size_t)T);
    double *p = malloc(sizeof(double) * (size_t)T);
    double *pq = malloc(sizeof(double) * (size_t)T);
    double *dq = malloc(sizeof(double) * (size_t)T);
    double m = -INFINITY, l = 0.0;
    for (int j0 = 0; j0 < N; j0 += T) {
        if (H->causal && j0 > i)
            break;
        int n = N - j0 < T ? N - j0 : T;
        /* score tile row, masked entries -inf */
        double mt = -INFINITY;
        for (int jj = 0; jj < n; jj++) {
            int j = j0 + jj;
            double mag = 0.0;
            x[jj] = (H->causal && j > i) ? -INFINITY : H->sm * score(H, i, j, &mag);
            xm[jj] = H->sm * mag;
            if (x[jj] > mt || isnan(x[jj]))        /* a NaN score makes the row max NaN */
                mt = x[jj];
        }
        double mn = (m > mt || isnan(m)) ? m : mt;
        if (mn == -INFINITY)
            continue;
        double alpha = (m == -INFINITY) ? 0.0 : exp(m - mn);
        double psum = 0.0, pmax = 0.0;
        for (int jj = 0; jj < n; jj++) {
            p[jj] = (x[jj] == -INFINITY) ? 0.0 : exp(x[jj] - mn);
            psum += p[jj];
            if (p[jj] > pmax)
                pmax = p[jj];
        }
        l = alpha * l + psum;
        /* P~: quantize the tile row; dq = width of each weight's admissible set */
        double post = 1.0;
        for (int jj = 0; jj < n; jj++)
            dq[jj] = 0.0;
        if (H->pv == PV_EXACT) {
            for (int jj = 0; jj < n; jj++)
                pq[jj] = p[jj];
        } else if (H->pv == PV_FP8 || H->pv == PV_MXFP8 || H->pv == PV_F16) {
            /* FP8: static x448 scale, p <= 1 fills the E4M3 range; fp16: p itself */
            int f16 = H->pv == PV_F16;
            double s = f16 ? 1.0 : 448.0;
            for (int jj = 0; jj < n; jj++) {
                double y = s * p[jj];
                pq[jj] = f16 ? f16_round(y) : e4m3_round(y);
                if (p[jj] > 0.0) {
                    double e = p_window(xm[jj], mn, mt);
                    double lo = f16 ? f16_round(y * (1.0 - e)) : e4m3_round(y * (1.0 - e));
                    double hi = f16 ? f16_round(y * (1.0 + e)) : e4m3_round(y * (1.0 + e));
                    dq[jj] = hi - lo;
                }
            }
        } else if (pmax == 0.0) {
            for (int jj = 0; jj < n; jj++)
                pq[jj] = 0.0;
        } else {
            /* second-level fp32 scale sigma, then MX E2M1 over 32-key groups */
            float sigma = (float)(6.0 / pmax);
            float *pf = malloc(sizeof(float) * (size_t)n);
            uint8_t *codes = malloc((size_t)n);
            for (int jj = 0; jj < n; jj++)
                pf[jj] = (float)((double)sigma * p[jj]);
            for (int g0 = 0; g0 < n; g0 += 32) {
                int gn = n - g0 < 32 ? n - g0 : 32;
                uint8_t sb;
                quant_mx_group(pf + g0, gn, 1, 4, codes + g0, 1, &sb);
                /* admissible scales: those of the group max moved by its window */
                double a = 0.0, eg = 0.0;
                for (int jj = g0; jj < g0 + gn; jj++) {
                    double e = pf[jj] > 0.0f ? p_window(xm[jj], mn, mt) : 0.0;
                    if (fabs((double)pf[jj]) > a)
                        a = fabs((double)pf[jj]);
                    if (e > eg)
                        eg = e;
                }
                uint8_t sbs[2] = {or_mx_scale_byte(a * (1.0 - eg), 2), or_mx_scale_byte(a * (1.0 + eg), 2)};
                for (int jj = g0; jj < g0 + gn; jj++) {
                    pq[jj] = or_e2m1_decode(codes[jj]) * e8m0_decode(sb);
                    if (pf[jj] > 0.0f && a > 0.0) {
                        double e = p_window(xm[jj], mn, mt), lo = INFINITY, hi = -INFINITY;
                        for (int k = 0; k < 4; k++) {
                            double v = e2m1_round_scaled((double)pf[jj] * (k & 1 ? 1.0 + e : 1.0 - e), sbs[k >> 1]);
                            lo = v < lo ? v : lo;
                            hi = v > hi ? v : hi;
                        }
                        dq[jj] = hi - lo;
                    }
                }
            }
            post = 1.0 / (double)sigma;
            free(pf);
            free(codes);
        }
        /* first level: this tile's product; second level: the running O */
        for (int c = 0; c < d; c++)
            acc[c] = 0.0;
        /* every key of the tile, zero weights included: 0 * NaN = NaN, as in the matrix product */
        for (int jj = 0; jj < n; jj++)
            for (int c = 0; c < d; c++)
                acc[c] += pq[jj] * H->vdec[(int64_t)(j0 + jj) * d + c];
        for (int c = 0; c < d; c++)
            O[c] = alpha * O[c] + acc[c] * post;
        /* the slack rides through the same rescales as O */
        for (int c = 0; c < d; c++)
            Sl[c] = alpha * Sl[c];
        for (int jj = 0; jj < n; jj++)
            if (dq[jj] > 0.0)
                for (int c = 0; c < d; c++)
                    Sl[c] += dq[jj] * post * fabs(H->vdec[(int64_t)(j0 + jj) * d + c]);
        m = mn;
    }
    if (l == 0.0) {
        /* no visible key (an empty key sequence): zero output, LSE -inf */
        for (int c = 0; c < d; c++) {
            o[c] = 0.0;
            if (slack)
                slack[c] = 0.0;
        }
        *lse = -INFINITY;
    } else {
        for (int c = 0; c < d; c++) {
            /* FP8 P~: O and l both carry 448; FP8 V adds its channel step */
            double f = H->pv == PV_FP8 ? (double)H->vs[c] / (448.0 * l)
                       : H->pv == PV_MXFP8 ? 1.0 / (448.0 * l) : 1.0 / l;
            o[c] = O[c] * f;
            if (slack)
                slack[c] = Sl[c] * fabs(f);
        }
        *lse = m + log(l) + (H->corr ? H->corr[i] : 0.0);
    }
    free(O);
    free(Sl);
    free(acc);
    free(x);
    free(xm);
    free(p);
    free(pq);
    free(dq);
}

/* rows: the query rows to compute (shared by every head); out [BH,nrows,d], lse [BH,nrows],
 * slack [BH,nrows,d] or NULL. */
static void run_rows(const head_t *heads, int BH, const int *rows, int nrows, double *out, double *lse,
                     double *slack)
{
    int d = heads[0].d;
    head_t *hs = malloc(sizeof(head_t) * (size_t)(BH > 0 ? BH : 1));
    int nq = 0;
    for (int r = 0; r < nrows; r++)
        nq = rows[r] + 1 > nq ? rows[r] + 1 : nq;
    for (int h = 0; h < BH; h++) {
        hs[h] = heads[h];
        hs[h].vdec = malloc(sizeof(double) * ((size_t)hs[h].N * d + 1));
        hs[h].q4d = hs[h].k4d = NULL;
        if (hs[h].qk == QK_MXFP4) {
            hs[h].q4d = malloc(sizeof(double) * ((size_t)nq * d + 1));
            hs[h].k4d = malloc(sizeof(double) * ((size_t)hs[h].N * d + 1));
        }
    }
#pragma omp parallel for schedule(dynamic)
    for (int h = 0; h < BH; h++) {
        for (int j = 0; j < hs[h].N; j++)
            for (int c = 0; c < d; c++)
                hs[h].vdec[(int64_t)j * d + c] = vval(&hs[h], j, c);
        if (hs[h].qk == QK_MXFP4) {
            for (int64_t e = 0; e < (int64_t)nq * d; e++)
                hs[h].q4d[e] = or_e2m1_decode(hs[h].q4[e]);
            for (int64_t e = 0; e < (int64_t)hs[h].N * d; e++)
                hs[h].k4d[e] = or_e2m1_decode(hs[h].k4[e]);
        }
    }
#pragma omp parallel for schedule(dynamic) collapse(2)
    for (int h = 0; h < BH; h++)
        for (int r = 0; r < nrows; r++)
            forward_row(&hs[h], rows[r], out + ((int64_t)h * nrows + r) * d, lse + (int64_t)h * nrows + r,
                        slack ? slack + ((int64_t)h * nrows + r) * d : NULL);
    for (int h = 0; h < BH; h++) {
        free(hs[h].vdec);
        free(hs[h].q4d);
        free(hs[h].k4d);
    }
    free(hs);
}

/* Simulation of the INT8-QK / FP8-PV forward on codes from or_quant_int8_fp8_x
 * (queries [BH,Nq], keys [BH,Nk]). */
OR_API void or_attn_int8_fp8_x(const int8_t *qc, const float *qs, const int8_t *kc, const float *ks,
                               const uint8_t *vc, const float *vs, const double *corr,
                               int BH, int Nq, int Nk, int d, int qblk, int kblk, int tile, int causal, double sm,
                               const int *rows, int nrows, double *out, double *lse, double *slack)
{
    int nbq = (Nq + qblk - 1) / qblk, nbk = (Nk + kblk - 1) / kblk;
    head_t *H = calloc((size_t)BH, sizeof(head_t));
    for (int h = 0; h < BH; h++) {
        int64_t offq = (int64_t)h * Nq * d, offk = (int64_t)h * Nk * d;
        H[h] = (head_t){.N = Nk, .d = d, .causal = causal, .tile = tile, .qblk = qblk, .kblk = kblk, .sm = sm,
                        .qk = QK_INT8, .pv = PV_FP8,
                        .qc = qc + offq, .kc = kc + offk, .qs = qs + (int64_t)h * nbq, .ks = ks + (int64_t)h * nbk,
                        .vc = vc + offk, .vs = vs + (int64_t)h * d, .corr = corr + (int64_t)h * Nq};
    }
    run_rows(H, BH, rows, nrows, out, lse, slack);
    free(H);
}

/* The same with fp16 P~ and V (vh [BH,Nk,d] fp16 codes from or_quant_v_f16). */
OR_API void or_attn_int8_f16_x(const int8_t *qc, const float *qs, const int8_t *kc, const float *ks,
                               const uint16_t *vh, const double *corr,
                               int BH, int Nq, int Nk, int d, int qblk, int kblk, int tile, int causal, double sm,
                               const int *rows, int nrows, double *out, double *lse, double *slack)
{
    int nbq = (Nq + qblk - 1) / qblk, nbk = (Nk + kblk - 1) / kblk;
    head_t *H = calloc((size_t)BH, sizeof(head_t));
    for (int h = 0; h < BH; h++) {
        int64_t offq = (int64_t)h * Nq * d, offk = (int64_t)h * Nk * d;
        H[h] = (head_t){.N = Nk, .d = d, .causal = causal, .tile = tile, .qblk = qblk, .kblk = kblk, .sm = sm,
                        .qk = QK_INT8, .pv = PV_F16,
                        .qc = qc + offq, .kc = kc + offk, .qs = qs + (int64_t)h * nbq, .ks = ks + (int64_t)h * nbk,
                        .vh = vh + offk, .corr = corr + (int64_t)h * Nq};
    }
    run_rows(H, BH, rows, nrows, out, lse, slack);
    free(H);
}

OR_API void or_attn_int8_fp8(const int8_t *qc, const float *qs, const int8_t *kc, const float *ks,
                             const uint8_t *vc, const float *vs, const double *corr,
                             int BH, int N, int d, int blk, int tile, int causal, double sm,
                             const int *rows, int nrows, double *out, double *lse)
{
    or_attn_int8_fp8_x(qc, qs, kc, ks, vc, vs, corr, BH, N, N, d, blk, blk, tile, causal, sm, rows, nrows, out, lse,
                       NULL);
}

/* Simulation of the MXFP4-QK forward; pv_fmt 3 = MXFP4 P~ and V, 2 = FP8 P~ and V,
 * 4 = FP8 P~ with MXFP8 V.  Queries [BH,Nq], keys [BH,Nk]. */
OR_API void or_attn_mxfp4_x(const uint8_t *qc, const uint8_t *qe, const uint8_t *kc, const uint8_t *ke,
                            const float *dS, const double *corr,
                            const uint8_t *vc, const uint8_t *ve, const float *vs, int pv_fmt, int qsb,
                            int BH, int Nq, int Nk, int d, int tile, int causal, double sm,
                            const int *rows, int nrows, double *out, double *lse, double *slack)
{
    int ng = d / 32, nvg = (Nk + 31) / 32;
    int nqb = qsb > 0 ? (Nq + qsb - 1) / qsb : 1;
    if (nqb < 1)
        nqb = 1;
    head_t *H = calloc((size_t)BH, sizeof(head_t));
    for (int h = 0; h < BH; h++) {
        int64_t offq = (int64_t)h * Nq * d, offk = (int64_t)h * Nk * d;
        H[h] = (head_t){.N = Nk, .d = d, .causal = causal, .tile = tile, .sm = sm,
                        .qk = QK_MXFP4, .pv = pv_fmt == 3 ? PV_MXFP4 : pv_fmt == 4 ? PV_MXFP8 : PV_FP8,
                        .q4 = qc + offq, .qe = qe + (int64_t)h * Nq * ng, .k4 = kc + offk, .ke = ke + (int64_t)h * Nk * ng,
                        .dS = dS + (int64_t)h * nqb * Nk, .qsb = qsb, .corr = corr + (int64_t)h * Nq,
                        .vc = vc + offk};
        if (pv_fmt == 3 || pv_fmt == 4)
            H[h].ve = ve + (int64_t)h * nvg * d;
        else
            H[h].vs = vs + (int64_t)h * d;
    }
    run_rows(H, BH, rows, nrows, out, lse, slack);
    free(H);
}

OR_API void or_attn_mxfp4(const uint8_t *qc, const uint8_t *qe, const uint8_t *kc, const uint8_t *ke,
                          const float *dS, const double *corr,
                          const uint8_t *vc, const uint8_t *ve, const float *vs, int pv_fmt,
                          int BH, int N, int d, int tile, int causal, double sm,
                          const int *rows, int nrows, double *out, double *lse)
{
    or_attn_mxfp4_x(qc, qe, kc, ke, dS, corr, vc, ve, vs, pv_fmt, 0, BH, N, N, d, tile, causal, sm, rows, nrows,
                    out, lse, NULL);
}

/*
 * The same tiled forward with every codec replaced by the identity: smoothing
 * of K (and of Q when smooth_q) in fp64, the dS term and the LSE correction
 * kept.  In exact arithmetic it equals the two-pass softmax attention, which
 * is what pins the tile recurrence, the masking, the deferred normalisation
 * and the smoothing decomposition.
 */
OR_API void or_attn_tiled_exact(const float *q, const float *k, const float *v,
                                int BH, int N, int d, int tile, int causal, double sm, int smooth_q,
                                const int *rows, int nrows, double *out, double *lse)
{
    head_t *H = calloc((size_t)BH, sizeof(head_t));
    double **bufs = calloc((size_t)BH * 5, sizeof(double *));
    for (int h = 0; h < BH; h++) {
        int64_t off = (int64_t)h * N * d;
        double *qx = malloc(sizeof(double) * (size_t)N * d), *kx = malloc(sizeof(double) * (size_t)N * d);
        double *vx = malloc(sizeof(double) * (size_t)N * d), *dSx = calloc((size_t)N, sizeof(double));
        double *corr = calloc((size_t)N, sizeof(double));
        double *muq = calloc((size_t)d, sizeof(double)), *muk = calloc((size_t)d, sizeof(double));
        for (int t = 0; t < N; t++)
            for (int c = 0; c < d; c++) {
                muq[c] += q[off + (int64_t)t * d + c];
                muk[c] += k[off + (int64_t)t * d + c];
            }
        for (int c = 0; c < d; c++) {
            muq[c] = smooth_q ? muq[c] / N : 0.0;
            muk[c] /= N;
        }
        for (int t = 0; t < N; t++) {
            double cs = 0.0, ds = 0.0;
            for (int c = 0; c < d; c++) {
                int64_t i = (int64_t)t * d + c;
                qx[i] = q[off + i] - muq[c];
                kx[i] = k[off + i] - muk[c];
                vx[i] = v[off + i];
                cs += (double)q[off + i] * muk[c];
            }
            for (int c = 0; c < d; c++)
                ds += muq[c] * kx[(int64_t)t * d + c];
            corr[t] = sm * cs;
            dSx[t] = ds;
        }
        free(muq);
        free(muk);
        H[h] = (head_t){.N = N, .d = d, .causal = causal, .tile = tile, .sm = sm, .qk = QK_EXACT, .pv = PV_EXACT,
                        .qx = qx, .kx = kx, .vx = vx, .dSx = dSx, .corr = corr};
        bufs[h * 5 + 0] = qx;
        bufs[h * 5 + 1] = kx;
        bufs[h * 5 + 2] = vx;
        bufs[h * 5 + 3] = dSx;
        bufs[h * 5 + 4] = corr;
    }
    run_rows(H, BH, rows, nrows, out, lse, NULL);
    for (int i = 0; i < BH * 5; i++)
        free(bufs[i]);
    free(bufs);
    free(H);
}

/* ------------------------------------------------------------------ */
/* Exact fp64 attention (two-pass softmax) and its backward.           */
/* ------------------------------------------------------------------ */

/* One query row against N keys; causal masking is top-left aligned (key j is
 * visible to query i when j <= i).  No visible key: zero output, LSE -inf. */
static void ref_row(const float *Q, const float *K, const float *V, int N, int d, int causal, double sm,
                    int i, double *x, double *o, double *lse)
{
    int n = causal && i + 1 < N ? i + 1 : N;
    if (n == 0) {
        for (int c = 0; c < d; c++)
            o[c] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double mx = -INFINITY;
    for (int j = 0; j < n; j++) {
        double s = 0.0;
        for (int c = 0; c < d; c++)
            s += (double)Q[(int64_t)i * d + c] * (double)K[(int64_t)j * d + c];
        x[j] = sm * s;
        if (x[j] > mx)
            mx = x[j];
    }
    double l = 0.0;
    for (int j = 0; j < n; j++) {
        x[j] = exp(x[j] - mx);
        l += x[j];
    }
    /* o[c] = (sum_j x_j V[j,c]) / l, each channel's sum taken in key order */
    for (int c = 0; c < d; c++)
        o[c] = 0.0;
    for (int j = 0; j < n; j++)
        for (int c = 0; c < d; c++)
            o[c] += x[j] * (double)V[(int64_t)j * d + c];
    for (int c = 0; c < d; c++)
        o[c] = o[c] / l;
    *lse = mx + log(l);
}

/* O = softmax(sm Q K^T + mask) V and LSE, exact in fp64, for the listed query
 * rows; queries [BH,Nq,d], keys and values [BH,Nk,d]. */
OR_API void or_attn_ref_x(const float *q, const float *k, const float *v, int BH, int Nq, int Nk, int d,
                          int causal, double sm, const int *rows, int nrows, double *out, double *lse)
{
#pragma omp parallel for schedule(dynamic) collapse(2)
    for (int h = 0; h < BH; h++)
        for (int r = 0; r < nrows; r++) {
            int64_t offq = (int64_t)h * Nq * d, offk = (int64_t)h * Nk * d;
            double *x = malloc(sizeof(double) * ((size_t)Nk + 1));
            ref_row(q + offq, k + offk, v + offk, Nk, d, causal, sm, rows[r],
                    x, out + ((int64_t)h * nrows + r) * d, lse + (int64_t)h * nrows + r);
            free(x);
        }
}

OR_API void or_attn_ref(const float *q, const float *k, const float *v, int BH, int N, int d,
                        int causal, double sm, const int *rows, int nrows, double *out, double *lse)
{
    or_attn_ref_x(q, k, v, BH, N, N, d, causal, sm, rows, nrows, out, lse);
}

/*
 * Exact fp64 backward of O = softmax(sm Q K^T + mask) V for BH heads:
 *   P = softmax rows, D_i = sum_c dO_ic O_ic, dV = P^T dO, dP = dO V^T,
 *   dS = P o (dP - D), dQ = sm dS K, dK = sm dS^T Q.
 */
OR_API void or_attn_bwd_ref(const float *q, const float *k, const float *v, const float *dout,
                            int BH, int N, int d, int causal, double sm,
                            double *dq, double *dk, double *dv)
{
#pragma omp parallel for schedule(dynamic)
    for (int h = 0; h < BH; h++) {
        int64_t off = (int64_t)h * N * d;
        const float *Q = q + off, *K = k + off, *V = v + off, *dO = dout + off;
        double *dQ = dq + off, *dK = dk + off, *dV = dv + off;
        double *P = malloc(sizeof(double) * (size_t)N);
        double *dP = malloc(sizeof(double) * (size_t)N);
        double *o = malloc(sizeof(double) * (size_t)d);
        memset(dQ, 0, sizeof(double) * (size_t)N * d);
        memset(dK, 0, sizeof(double) * (size_t)N * d);
        memset(dV, 0, sizeof(double) * (size_t)N * d);
        for (int i = 0; i < N; i++) {
            int n = causal ? i + 1 : N;
            double lse;
            ref_row(Q, K, V, N, d, causal, sm, i, P, o, &lse);
            for (int j = 0; j < n; j++) {
                double s = 0.0;
                for (int c = 0; c < d; c++)
                    s += (double)Q[(int64_t)i * d + c] * (double)K[(int64_t)j * d + c];
                P[j] = exp(sm * s - lse);
            }
            double D = 0.0;
            for (int c = 0; c < d; c++)
                D += (double)dO[(int64_t)i * d + c] * o[c];
            for (int j = 0; j < n; j++) {
                double s = 0.0;
                for (int c = 0; c < d; c++)
                    s += (double)dO[(int64_t)i * d + c] * (double)V[(int64_t)j * d + c];
                dP[j] = s;
            }
            for (int j = 0; j < n; j++) {
                double dS = P[j] * (dP[j] - D);
                for (int c = 0; c < d; c++) {
                    dV[(int64_t)j * d + c] += P[j] * (double)dO[(int64_t)i * d + c];
                    dQ[(int64_t)i * d + c] += sm * dS * (double)K[(int64_t)j * d + c];
                    dK[(int64_t)j * d + c] += sm * dS * (double)Q[(int64_t)i * d + c];
                }
            }
        }
        free(P);
        free(dP);
        free(o);
    }
}
