/*
 * sanitize_main.c -- drives every exported function of sage_oracle.c on small inputs
 * (ragged lengths, one token, causal and not, every format pair, per-block Q smoothing,
 * NaN and infinite inputs) so that a build with AddressSanitizer and UndefinedBehavior-
 * Sanitizer can check the oracle's memory accesses and arithmetic.  TEST INFRASTRUCTURE:
 * built and run by the CPU test suite only.  Values are not checked here (the pin tests
 * do that); a sanitizer report or a crash fails the run.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

/* the oracle's exports (sage_oracle.c) */
void or_widen(const uint16_t *src, int dtype, float *dst, int64_t n);
double or_e4m3_decode(uint8_t c);
uint8_t or_e4m3_encode(double x);
double or_f16_decode(uint16_t c);
uint16_t or_f16_encode(double x);
double or_e2m1_decode(uint8_t c);
uint8_t or_e2m1_encode(double x);
uint8_t or_mx_scale_byte(double amax, int emax);
int8_t or_int8_encode(float x, float delta);
void or_quant_v_f16(const float *v, int64_t n, uint16_t *out);
void or_quant_int8_fp8_x(const float *q, const float *k, const float *v, int BH, int Nq, int Nk, int d, int qblk,
                         int kblk, double sm, float *mu_k, int8_t *qc, float *qs, int8_t *kc, float *ks,
                         uint8_t *vc, float *vs, double *corr);
void or_quant_mxfp4_x(const float *q, const float *k, const float *v, int BH, int Nq, int Nk, int d, int pv_fmt,
                      int qsb, double sm, float *mu_q, float *mu_k, uint8_t *qc, uint8_t *qe, uint8_t *kc,
                      uint8_t *ke, float *dS, double *corr, uint8_t *vc, uint8_t *ve, float *vs);
void or_attn_int8_fp8_x(const int8_t *qc, const float *qs, const int8_t *kc, const float *ks, const uint8_t *vc,
                        const float *vs, const double *corr, int BH, int Nq, int Nk, int d, int qblk, int kblk,
                        int tile, int causal, double sm, const int *rows, int nrows, double *out, double *lse,
                        double *slack);
void or_attn_int8_f16_x(const int8_t *qc, const float *qs, const int8_t *kc, const float *ks, const uint16_t *vh,
                        const double *corr, int BH, int Nq, int Nk, int d, int qblk, int kblk, int tile, int causal,
                        double sm, const int *rows, int nrows, double *out, double *lse, double *slack);
void or_attn_mxfp4_x(const uint8_t *qc, const uint8_t *qe, const uint8_t *kc, const uint8_t *ke, const float *dS,
                     const double *corr, const uint8_t *vc, const uint8_t *ve, const float *vs, int pv_fmt, int qsb,
                     int BH, int Nq, int Nk, int d, int tile, int causal, double sm, const int *rows, int nrows,
                     double *out, double *lse, double *slack);
void or_attn_tiled_exact(const float *q, const float *k, const float *v, int BH, int N, int d, int tile, int causal,
                         double sm, int smooth_q, const int *rows, int nrows, double *out, double *lse);
void or_attn_ref_x(const float *q, const float *k, const float *v, int BH, int Nq, int Nk, int d, int causal,
                   double sm, const int *rows, int nrows, double *out, double *lse);
void or_attn_bwd_ref(const float *q, const float *k, const float *v, const float *dout, int BH, int N, int d,
                     int causal, double sm, double *dq, double *dk, double *dv);

static uint64_t rs = 88172645463325252ull;
static float rnd(void)
{
    rs ^= rs << 13;
    rs ^= rs >> 7;
    rs ^= rs << 17;
    return (float)((double)(rs >> 11) / 9007199254740992.0 * 4.0 - 2.0);
}

static void *xm(size_t n) { return calloc(n ? n : 1, 1); }

static void run(int BH, int Nq, int Nk, int d, int causal, int bad)
{
    size_t eq = (size_t)BH * Nq * d, ek = (size_t)BH * Nk * d;
    float *q = xm(eq * 4), *k = xm(ek * 4), *v = xm(ek * 4);
    for (size_t i = 0; i < eq; i++)
        q[i] = rnd();
    for (size_t i = 0; i < ek; i++) {
        k[i] = rnd() + 3.0f;
        v[i] = rnd();
    }
    if (bad && eq > 5 && ek > 7) {
        q[3] = NAN;
        k[5] = INFINITY;
        v[7] = -INFINITY;
    }
    int nqb = (Nq + 127) / 128, nvg = (Nk + 31) / 32;
    int *rows = xm(sizeof(int) * (size_t)Nq);
    for (int i = 0; i < Nq; i++)
        rows[i] = i;
    double *out = xm(eq * 8), *lse = xm((size_t)BH * Nq * 8), *sl = xm(eq * 8), *corr = xm((size_t)BH * Nq * 8);
    float *mu_k = xm((size_t)BH * d * 4), *mu_q = xm((size_t)BH * (nqb + 1) * d * 4);
    int8_t *qc = xm(eq), *kc = xm(ek);
    float *qs = xm((size_t)BH * Nq * 4), *ks = xm((size_t)BH * Nk * 4), *vs = xm((size_t)BH * d * 4);
    uint8_t *vc = xm(ek), *q4 = xm(eq), *k4 = xm(ek), *qe = xm(eq / 32 + 1), *ke = xm(ek / 32 + 1);
    uint8_t *ve = xm((size_t)BH * nvg * d);
    uint16_t *vh = xm(ek * 2);
    float *dS = xm((size_t)BH * (nqb + 1) * Nk * 4);
    /* INT8 paths: 64-token steps and per-token / per-32-key steps */
    for (int fine = 0; fine < 2; fine++) {
        int qb = fine ? 1 : 64, kb = fine ? 32 : 64;
        or_quant_int8_fp8_x(q, k, v, BH, Nq, Nk, d, qb, kb, 0.125, mu_k, qc, qs, kc, ks, vc, vs, corr);
        or_quant_v_f16(v, (int64_t)ek, vh);
        or_attn_int8_fp8_x(qc, qs, kc, ks, vc, vs, corr, BH, Nq, Nk, d, qb, kb, 64, causal, 0.125, rows, Nq, out, lse,
                           sl);
        or_attn_int8_f16_x(qc, qs, kc, ks, vh, corr, BH, Nq, Nk, d, qb, kb, 64, causal, 0.125, rows, Nq, out, lse, sl);
    }
    /* MXFP4 QK with every P~V format, sequence and per-block Q smoothing */
    for (int pv = 2; pv <= 4; pv++)
        for (int qsb = 0; qsb <= 128; qsb += 128) {
            or_quant_mxfp4_x(q, k, v, BH, Nq, Nk, d, pv, qsb, 0.125, mu_q, mu_k, q4, qe, k4, ke, dS, corr, vc, ve, vs);
            or_attn_mxfp4_x(q4, qe, k4, ke, dS, corr, vc, ve, vs, pv, qsb, BH, Nq, Nk, d, 64, causal, 0.125, rows, Nq,
                            out, lse, sl);
        }
    or_attn_ref_x(q, k, v, BH, Nq, Nk, d, causal, 0.125, rows, Nq, out, lse);
    if (Nq == Nk) {
        or_attn_tiled_exact(q, k, v, BH, Nq, d, 64, causal, 0.125, 1, rows, Nq, out, lse);
        double *g = xm(eq * 8 * 3);
        or_attn_bwd_ref(q, k, v, q, BH, Nq, d, causal, 0.125, g, g + eq, g + 2 * eq);
        free(g);
    }
    free(q), free(k), free(v), free(rows), free(out), free(lse), free(sl), free(corr), free(mu_k), free(mu_q);
    free(qc), free(kc), free(qs), free(ks), free(vs), free(vc), free(q4), free(k4), free(qe), free(ke), free(ve);
    free(vh), free(dS);
}

int main(void)
{
    /* element codecs over every 16-bit pattern, widened both ways */
    for (uint32_t u = 0; u < 65536; u++) {
        uint16_t h = (uint16_t)u;
        float f[2];
        or_widen(&h, 0, &f[0], 1);
        or_widen(&h, 1, &f[1], 1);
        for (int t = 0; t < 2; t++) {
            or_e4m3_decode(or_e4m3_encode(f[t]));
            or_f16_decode(or_f16_encode(f[t]));
            or_e2m1_decode(or_e2m1_encode(f[t]));
            or_mx_scale_byte(fabs((double)f[t]), 2);
            or_int8_encode(f[t], 0.37f);
        }
    }
    int shapes[][5] = {{2, 130, 130, 64, 0}, {1, 1, 1, 64, 1}, {2, 70, 70, 128, 1}, {1, 40, 150, 64, 0},
                       {1, 150, 40, 64, 0}, {1, 129, 129, 64, 1}};
    for (unsigned s = 0; s < sizeof shapes / sizeof shapes[0]; s++)
        for (int bad = 0; bad < 2; bad++)
            run(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], shapes[s][4], bad);
    printf("oracle sanitizer run ok\n");
    return 0;
}
