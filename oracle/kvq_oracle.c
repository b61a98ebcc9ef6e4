/*
 * kvq_oracle.c -- plain, slow, obviously-correct CPU oracle for the compressed-KV path.
 *
 * TEST INFRASTRUCTURE ONLY (see kvq_oracle.h).  Build:
 *   gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared kvq_oracle.c -lm
 * Binary32 rounding is the C default (round-to-nearest-even); no expression below relies on FMA
 * contraction, and the build forbids it.
 *
 * Section map (pages cited by title and section):
 *   binary16 helpers ........ format of the "fp16 scale + fp16 zero" per group (quantcpp article,
 *                             KV compression claim of 6.4x = 32 bits / (4 + 32/32) bits).
 *   rotation ................ KVarN post, TL;DR: Walsh-Hadamard transform before quantizing;
 *                             TurboQuant row of the method table: random rotation.
 *   Sinkhorn ................ KVarN post, TL;DR: Sinkhorn variance balancing.
 *   uniform quantizer ....... quantcpp article, progressive table: 4-bit KV; groups of 32 along
 *                             the head dimension with fp16 scale/zero (reading of "6.4x").
 *   symmetric 8-bit ......... "q8_0": the 8-bit cache type of the KVarN post's comparison and the
 *                             "K = Q8" of the 2026 survey page's application rules (named, not
 *                             defined there: one fp16 scale per 32, codes in [-127, 127]).
 *   Lloyd-Max + turbo ....... TurboQuant row: per-coordinate optimal scalar quantizer after a
 *                             random rotation, 1-bit QJL on the residual for an unbiased inner
 *                             product.
 *   window .................. quantcpp article, progressive paragraph: the most recent 128
 *                             tokens stay FP32, everything else 4-bit.
 *   attention ............... plain softmax(q k^T * scale) v on the dequantized cache; the
 *                             prefix form serves the queries of a prefill chunk, each seeing
 *                             the tokens up to its own position (quantcpp article, v3.2 batched
 *                             prefill: the prompt is processed as whole chunks).
 */
#include "kvq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define D ORC_D
#define ORC_PI 3.14159265358979323846
#define GS ORC_GROUP
#define NG ORC_NGROUPS

/* ------------------------------------------------------------------------------------------ */
/* binary16 by integer manipulation                                                            */
/* ------------------------------------------------------------------------------------------ */

float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24); /* zero or subnormal: man * 2^-24 */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man | 0x400), ex - 25); /* (1024 + man) * 2^(ex - 15 - 10) */
    return (float)(sign ? -v : v);
}

/* Round-to-nearest-even binary32 -> binary16.  Every scaling below is by a power of two, so the
 * only rounding is the rint() (half-even under the default rounding mode). */
uint16_t orc_f32_to_f16_rn(float xf)
{
    double x = (double)xf;
    uint16_t s = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(a)) return 0x7e00;
    if (a >= 65520.0) return (uint16_t)(s | 0x7c00); /* halfway to 2^16 rounds to even = inf */
    if (a < ldexp(1.0, -14)) {                        /* subnormal range: units of 2^-24 */
        double m = rint(a * 16777216.0);               /* <= 1024; 1024 is the smallest normal */
        return (uint16_t)(s | (uint16_t)m);
    }
    int e;
    frexp(a, &e); /* a in [2^(e-1), 2^e) */
    int E = e - 1;
    double m = rint(ldexp(a, 10 - E)); /* in [1024, 2048] */
    if (m == 2048.0) {
        m = 1024.0;
        E += 1;
    }
    if (E > 15) return (uint16_t)(s | 0x7c00);
    return (uint16_t)(s | (uint16_t)(((E + 15) << 10) | ((int)m - 1024)));
}

/* Largest binary16 value <= x (x finite, |x| < 65504): round to nearest, then step down one
 * binary16 ulp if that overshot.  This is the zero-point rounding that keeps every value of a
 * group inside [z, z + L*s] (reading G2). */
uint16_t orc_f32_to_f16_rd(float x)
{
    uint16_t h = orc_f32_to_f16_rn(x);
    if (orc_f16_to_f32(h) > x) {
        if (h == 0x0000 || h == 0x8000)
            h = 0x8001; /* -(2^-24) */
        else if (h & 0x8000)
            h = (uint16_t)(h + 1); /* negative: larger magnitude */
        else
            h = (uint16_t)(h - 1); /* positive: smaller magnitude */
    }
    return h;
}

/* ------------------------------------------------------------------------------------------ */
/* rotation R(x) = c0 * H (d .* x), H the 128x128 Sylvester Hadamard matrix (entries +-1)      */
/* ------------------------------------------------------------------------------------------ */

/* c0 = 2^-3.5 rounded to binary32 (bits 0x3DB504F3). */
static float c0_f32(void)
{
    uint32_t bits = 0x3DB504F3u;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* Butterfly stages with span h = 1, 2, 4, ..., 64 in that order; each maps the pair
 * (t[i], t[i+h]), bit h of i clear, to (t[i] + t[i+h], t[i] - t[i+h]).  The final scaling by c0 is
 * one binary32 multiply per element. */
void orc_rotate_f32(const float* x, const float* signs, float* y)
{
    float t[D];
    for (int j = 0; j < D; j++) t[j] = (signs[j] < 0.0f) ? -x[j] : x[j];
    for (int h = 1; h < D; h <<= 1)
        for (int i = 0; i < D; i++)
            if (!(i & h)) {
                float a = t[i], b = t[i + h];
                t[i] = a + b;
                t[i + h] = a - b;
            }
    float c0 = c0_f32();
    for (int j = 0; j < D; j++) y[j] = t[j] * c0;
}

static void hadamard_f64(double* t)
{
    for (int h = 1; h < D; h <<= 1)
        for (int i = 0; i < D; i++)
            if (!(i & h)) {
                double a = t[i], b = t[i + h];
                t[i] = a + b;
                t[i + h] = a - b;
            }
}

void orc_rotate_f64(const double* x, const float* signs, double* y)
{
    double t[D];
    for (int j = 0; j < D; j++) t[j] = (double)signs[j] * x[j];
    hadamard_f64(t);
    double r = sqrt(128.0);
    for (int j = 0; j < D; j++) y[j] = t[j] / r;
}

/* R^-1 = R^T = d .* (H y) / sqrt(128): H is symmetric and H H = 128 I. */
void orc_unrotate_f64(const double* y, const float* signs, double* x)
{
    double t[D];
    for (int j = 0; j < D; j++) t[j] = y[j];
    hadamard_f64(t);
    double r = sqrt(128.0);
    for (int j = 0; j < D; j++) x[j] = (double)signs[j] * (t[j] / r);
}

/* ------------------------------------------------------------------------------------------ */
/* Sinkhorn variance balancing (reading C3)                                                    */
/* ------------------------------------------------------------------------------------------ */

/* X: n calibration tokens [n][128] in the original domain.  A = (double) R(X) (or X).  Each
 * iteration first divides every row by its population standard deviation, then every column by
 * its own, accumulating the column divisors in C.  Sums run sequentially in index order.  The
 * row divisors are discarded: per-token groups carry their own scale, and a future token's row
 * scale is unknown at append time.  Output c = fp32(C), inv_c = fp32(1 / (double) c). */
void orc_sinkhorn(const float* X, int n, const float* signs_or_null, int iters, float* c,
                  float* inv_c, double* A_out, double* C_out)
{
    double* A = (double*)malloc(sizeof(double) * (size_t)n * D);
    double C[D];
    float y[D];
    for (int t = 0; t < n; t++) {
        if (signs_or_null)
            orc_rotate_f32(X + (size_t)t * D, signs_or_null, y);
        else
            memcpy(y, X + (size_t)t * D, sizeof y);
        for (int j = 0; j < D; j++) A[(size_t)t * D + j] = (double)y[j];
    }
    for (int j = 0; j < D; j++) C[j] = 1.0;
    for (int it = 0; it < iters; it++) {
        for (int t = 0; t < n; t++) {
            double* row = A + (size_t)t * D;
            double s = 0.0;
            for (int j = 0; j < D; j++) s = s + row[j];
            double mean = s / 128.0;
            double v = 0.0;
            for (int j = 0; j < D; j++) {
                double dv = row[j] - mean;
                v = v + dv * dv;
            }
            double sd = sqrt(v / 128.0);
            if (sd < 1e-30) sd = 1e-30;
            for (int j = 0; j < D; j++) row[j] = row[j] / sd;
        }
        for (int j = 0; j < D; j++) {
            double s = 0.0;
            for (int t = 0; t < n; t++) s = s + A[(size_t)t * D + j];
            double mean = s / (double)n;
            double v = 0.0;
            for (int t = 0; t < n; t++) {
                double dv = A[(size_t)t * D + j] - mean;
                v = v + dv * dv;
            }
            double sd = sqrt(v / (double)n);
            if (sd < 1e-30) sd = 1e-30;
            for (int t = 0; t < n; t++) A[(size_t)t * D + j] = A[(size_t)t * D + j] / sd;
            C[j] = C[j] * sd;
        }
    }
    for (int j = 0; j < D; j++) {
        c[j] = (float)C[j];
        inv_c[j] = (float)(1.0 / (double)c[j]);
    }
    if (A_out) memcpy(A_out, A, sizeof(double) * (size_t)n * D);
    if (C_out) memcpy(C_out, C, sizeof C);
    free(A);
}

/* ------------------------------------------------------------------------------------------ */
/* uniform asymmetric b-bit quantizer for one group of 32 (reading C4)                          */
/* ------------------------------------------------------------------------------------------ */

void orc_quant_group(const float* y, int bits, uint8_t* codes, uint16_t* s16o, uint16_t* z16o)
{
    const int L = (1 << bits) - 1;
    float mn = y[0], mx = y[0];
    for (int i = 1; i < GS; i++) {
        if (y[i] < mn) mn = y[i];
        if (y[i] > mx) mx = y[i];
    }
    mn = mn + 0.0f; /* -0 -> +0 */
    mx = mx + 0.0f;
    uint16_t z16 = orc_f32_to_f16_rd(mn);
    float z = orc_f16_to_f32(z16);
    float s32 = (mx - z) / (float)L;
    uint16_t s16 = orc_f32_to_f16_rn(s32);
    float s = orc_f16_to_f32(s16);
    float inv = (s > 0.0f) ? 1.0f / s : 0.0f;
    for (int i = 0; i < GS; i++) {
        float d = y[i] - z;
        float u = d * inv;
        float r = rintf(u);
        if (r < 0.0f) r = 0.0f;
        if (r > (float)L) r = (float)L;
        codes[i] = (uint8_t)r;
    }
    *s16o = s16;
    *z16o = z16;
}

/* ------------------------------------------------------------------------------------------ */
/* symmetric 8-bit quantizer for one group of 32 ("q8_0"; see the header)                      */
/* ------------------------------------------------------------------------------------------ */

void orc_quant_group_sym8(const float* y, uint8_t* codes, uint16_t* d16o, uint16_t* z16o)
{
    float amax = 0.0f;
    for (int i = 0; i < GS; i++) {
        float a = fabsf(y[i]);
        if (a > amax) amax = a;
    }
    uint16_t d16 = orc_f32_to_f16_rn(amax / 127.0f);
    float d = orc_f16_to_f32(d16);
    float inv = (d > 0.0f) ? 1.0f / d : 0.0f;
    for (int i = 0; i < GS; i++) {
        float q = rintf(y[i] * inv);
        if (q < -127.0f) q = -127.0f;
        if (q > 127.0f) q = 127.0f;
        codes[i] = (uint8_t)((int)q + 128);
    }
    *d16o = d16;
    *z16o = orc_f32_to_f16_rn(-128.0f * d);
}

/* ------------------------------------------------------------------------------------------ */
/* Lloyd-Max 8-level quantizer of N(0,1), scaled to N(0,1/128) (reading C5)                    */
/* ------------------------------------------------------------------------------------------ */

static double phi(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * ORC_PI); }

/* Probability mass of N(0,1) on [a, b], 0 <= a < b <= inf, via erfc (accurate in the tails). */
static double mass(double a, double b)
{
    double eb = isinf(b) ? 0.0 : erfc(b / sqrt(2.0));
    return 0.5 * (erfc(a / sqrt(2.0)) - eb);
}

/* Lloyd's two conditions, iterated on the positive half line (the density is even, so the
 * optimal quantizer with an even number of levels is odd-symmetric with a threshold at 0):
 * thresholds are midpoints of neighbouring centroids, centroids are conditional means
 * (phi(a) - phi(b)) / mass(a, b).  `levels` = 2, 4, 8 or 16 (1- to 4-bit codes); the start is
 * the evenly spaced half line 2 (k + 1) / (levels / 2), k = 0 .. levels/2 - 1.  A coordinate of a
 * random rotation of a unit vector in `dim` dimensions is close to N(0, 1/dim), so the stored
 * centroids and thresholds are the N(0,1) ones divided by sqrt(dim). */
void orc_lloyd_max_dim(int levels, int dim, int iters, double* mu_star, float* mu, float* theta,
                       double* last_change)
{
    const int h = levels / 2;
    double m[8];
    for (int k = 0; k < h; k++) m[k] = 2.0 * (double)(k + 1) / (double)h;
    double change = 0.0;
    for (int it = 0; it < iters; it++) {
        double b[9];
        b[0] = 0.0;
        for (int k = 1; k < h; k++) b[k] = (m[k - 1] + m[k]) * 0.5;
        b[h] = INFINITY;
        change = 0.0;
        for (int k = 0; k < h; k++) {
            double pb = isinf(b[k + 1]) ? 0.0 : phi(b[k + 1]);
            double nm = (phi(b[k]) - pb) / mass(b[k], b[k + 1]);
            double dlt = fabs(nm - m[k]);
            if (dlt > change) change = dlt;
            m[k] = nm;
        }
    }
    double r = sqrt((double)dim);
    for (int k = 0; k < h; k++) {
        mu_star[h + k] = m[k];
        mu_star[h - 1 - k] = -m[k];
        float f = (float)(m[k] / r);
        mu[h + k] = f;
        mu[h - 1 - k] = -f;
    }
    theta[h - 1] = 0.0f;
    for (int k = 1; k < h; k++) {
        double t = (m[k - 1] + m[k]) * 0.5;
        float f = (float)(t / r);
        theta[h - 1 + k] = f;
        theta[h - 1 - k] = -f;
    }
    if (last_change) *last_change = change;
}

void orc_lloyd_max_levels(int levels, int iters, double* mu_star, float* mu, float* theta,
                          double* last_change)
{
    orc_lloyd_max_dim(levels, 128, iters, mu_star, mu, theta, last_change);
}

void orc_lloyd_max(int iters, double* mu_star, float* mu, float* theta, double* last_change)
{
    orc_lloyd_max_levels(8, iters, mu_star, mu, theta, last_change);
}

/* ------------------------------------------------------------------------------------------ */
/* TurboQuant token code (reading C5 / C6)                                                      */
/* ------------------------------------------------------------------------------------------ */

/* Pairwise sum of v[j]^2 in index order: level 1 adds (0,1), (2,3), ...; level 2 adds adjacent
 * pair sums; and so on up to one value.  Products and sums are binary32. */
float orc_tree_sum_sq(const float* v)
{
    float t[D];
    for (int j = 0; j < D; j++) t[j] = v[j] * v[j];
    for (int w = D / 2; w >= 1; w >>= 1)
        for (int i = 0; i < w; i++) t[i] = t[2 * i] + t[2 * i + 1];
    return t[0];
}

void orc_turbo_encode(const float* x, const orc_tables* tb, int with_qjl, float* rho_out,
                      uint8_t* codes, uint16_t* n16o, uint16_t* g16o, uint8_t* bits,
                      float* resid_out)
{
    orc_turbo_encode_bits(x, tb, 3, with_qjl, rho_out, codes, n16o, g16o, bits, resid_out);
}

void orc_turbo_encode_bits(const float* x, const orc_tables* tb, int code_bits, int with_qjl,
                           float* rho_out, uint8_t* codes, uint16_t* n16o, uint16_t* g16o,
                           uint8_t* bits, float* resid_out)
{
    const int n_thr = (1 << code_bits) - 1;
    float rho[D], r[D];
    orc_rotate_f32(x, tb->signs, rho);
    float nsq = orc_tree_sum_sq(rho);
    uint16_t n16 = orc_f32_to_f16_rn(sqrtf(nsq));
    float n = orc_f16_to_f32(n16);
    float inv = (n > 0.0f) ? 1.0f / n : 0.0f;
    for (int j = 0; j < D; j++) {
        float u = rho[j] * inv;
        int c = 0;
        for (int i = 0; i < n_thr; i++)
            if (u > tb->theta[i]) c++;
        codes[j] = (uint8_t)c;
        float p = n * tb->mu[c];
        r[j] = rho[j] - p;
    }
    uint16_t g16 = 0;
    if (with_qjl) {
        g16 = orc_f32_to_f16_rn(sqrtf(orc_tree_sum_sq(r)));
        for (int i = 0; i < D; i++) {
            float acc = 0.0f;
            for (int j = 0; j < D; j++) acc = fmaf(tb->S[i * D + j], r[j], acc);
            bits[i] = (acc >= 0.0f) ? 1 : 0; /* sign(0) = +1 */
        }
    } else if (bits) {
        memset(bits, 0, D);
    }
    *n16o = n16;
    *g16o = g16;
    if (rho_out) memcpy(rho_out, rho, sizeof rho);
    if (resid_out) memcpy(resid_out, r, sizeof r);
}

/* ------------------------------------------------------------------------------------------ */
/* outlier-channel split: fractional bit widths (reading R19)                                  */
/* ------------------------------------------------------------------------------------------ */
/*
 * TurboQuant reaches 2.5 and 3.5 bits per channel by splitting the channels into an outlier set
 * and the rest and running two independent instances of its quantizer, the outliers with one bit
 * more.  Reading R19 fixes the open parts: 64 outlier channels (the split that gives exactly
 * 2.5 = (64*3 + 64*2)/128 and 3.5 = (64*4 + 64*3)/128), chosen per (layer, kv head) from the
 * calibration tokens by energy; each subset is rotated by its own 64-point random-sign
 * Walsh-Hadamard transform, carries its own fp16 norm and is coded with the Lloyd-Max codebook
 * of N(0, 1/64).
 */

/* Butterflies of span h = 1, 2, ..., 32 in that order, then one binary32 multiply by 1/8. */
void orc_rotate64_f32(const float* x, const float* signs, float* y)
{
    float t[64];
    for (int j = 0; j < 64; j++) t[j] = (signs[j] < 0.0f) ? -x[j] : x[j];
    for (int h = 1; h < 64; h <<= 1)
        for (int i = 0; i < 64; i++)
            if (!(i & h)) {
                float a = t[i], b = t[i + h];
                t[i] = a + b;
                t[i + h] = a - b;
            }
    for (int j = 0; j < 64; j++) y[j] = t[j] * 0.125f;
}

/* Inverse: H64 H64 = 64 I, so R^-1 y = d .* (H64 y) / 8. */
void orc_unrotate64_f64(const double* y, const float* signs, double* x)
{
    double t[64];
    for (int j = 0; j < 64; j++) t[j] = y[j];
    for (int h = 1; h < 64; h <<= 1)
        for (int i = 0; i < 64; i++)
            if (!(i & h)) {
                double a = t[i], b = t[i + h];
                t[i] = a + b;
                t[i + h] = a - b;
            }
    for (int j = 0; j < 64; j++) x[j] = (double)signs[j] * (t[j] / 8.0);
}

/* Pairwise index-order sum of squares over 64 values (the 128-value tree cut to one half). */
float orc_tree_sum_sq64(const float* v)
{
    float t[64];
    for (int j = 0; j < 64; j++) t[j] = v[j] * v[j];
    for (int w = 32; w >= 1; w >>= 1)
        for (int i = 0; i < w; i++) t[i] = t[2 * i] + t[2 * i + 1];
    return t[0];
}

/* Energy of channel d = sum over the n tokens, in token order, of x[t][d]^2; a binary32 square
 * is exact in binary64, so only the running sum rounds.  The 64 channels of largest energy are
 * the outliers; of two channels with equal energy the one with the smaller index ranks first. */
void orc_select_outliers(const float* X, int n, int* perm)
{
    double e[D];
    int out[D];
    for (int d = 0; d < D; d++) {
        double acc = 0.0;
        for (int t = 0; t < n; t++) {
            double v = (double)X[(size_t)t * D + d];
            acc += v * v;
        }
        e[d] = acc;
    }
    for (int d = 0; d < D; d++) {
        int rank = 0;
        for (int i = 0; i < D; i++)
            if (e[i] > e[d] || (e[i] == e[d] && i < d)) rank++;
        out[d] = rank < D / 2;
    }
    int k = 0;
    for (int d = 0; d < D; d++)
        if (out[d]) perm[k++] = d;
    for (int d = 0; d < D; d++)
        if (!out[d]) perm[k++] = d;
}

/* Each subset h (positions 64h .. 64h+63, channels perm[.]): rho = R64(x_h) with signs
 * 64h .. 64h+63 of the tensor's sign vector; n_h = fp16(|rho|); code = number of thresholds of
 * the subset's codebook below rho / n_h (outliers: bits_o bits, the rest bits_o - 1).  rho (in
 * position order) goes to rho_out when that is not NULL. */
static void split_halves(const float* x, const orc_tables* tb, int bits_o, uint8_t* codes, uint16_t* n16,
                         float* rho_out)
{
    for (int h = 0; h < 2; h++) {
        float z[64], rho[64];
        for (int j = 0; j < 64; j++) z[j] = x[tb->perm[64 * h + j]];
        orc_rotate64_f32(z, tb->signs + 64 * h, rho);
        uint16_t nh = orc_f32_to_f16_rn(sqrtf(orc_tree_sum_sq64(rho)));
        float n = orc_f16_to_f32(nh);
        float inv = (n > 0.0f) ? 1.0f / n : 0.0f;
        const float* th = h ? tb->theta2 : tb->theta;
        const int n_thr = (1 << (h ? bits_o - 1 : bits_o)) - 1;
        for (int j = 0; j < 64; j++) {
            float u = rho[j] * inv;
            int c = 0;
            for (int i = 0; i < n_thr; i++)
                if (u > th[i]) c++;
            codes[64 * h + j] = (uint8_t)c;
        }
        n16[h] = nh;
        if (rho_out) memcpy(rho_out + 64 * h, rho, sizeof rho);
    }
}

void orc_split_encode(const float* x, const orc_tables* tb, int bits_o, uint8_t* codes, uint16_t* n16)
{
    split_halves(x, tb, bits_o, codes, n16, NULL);
}

/* Split TurboQuant key at b = 3 or 4 (reading R23): the MSE stage of the TurboQuant key code run
 * on the outlier split (outliers b - 1 bits, the rest b - 2, each half its own 64-point rotation,
 * norm and N(0, 1/64) codebook), then the 1-bit QJL sketch of the whole residual as for a
 * TurboQuant key: r = rho - n_h mu_h[code] in position order, gamma = fp16(|r|) (index-order tree
 * over the 128 positions), bit i = (sum_j S_ij r_j >= 0) with a sequential fma chain.  Budget:
 * (b - 1 + b - 2) / 2 + 1 = b - 0.5 bits per channel (2.5 or 3.5), plus three fp16 norms. */
void orc_split_qjl_encode(const float* x, const orc_tables* tb, int b, uint8_t* codes, uint16_t* n16,
                          uint16_t* g16o, uint8_t* bits)
{
    float rho[D], r[D];
    split_halves(x, tb, b - 1, codes, n16, rho);
    for (int j = 0; j < D; j++) {
        const int h = j >= 64;
        float n = orc_f16_to_f32(n16[h]);
        float p = n * (h ? tb->mu2 : tb->mu)[codes[j]];
        r[j] = rho[j] - p;
    }
    *g16o = orc_f32_to_f16_rn(sqrtf(orc_tree_sum_sq(r)));
    for (int i = 0; i < D; i++) {
        float acc = 0.0f;
        for (int j = 0; j < D; j++) acc = fmaf(tb->S[i * D + j], r[j], acc);
        bits[i] = (acc >= 0.0f) ? 1 : 0;
    }
}

/* The split domain of a query in binary64: position 64h + j = R64(q[perm[64h + .]])_j. */
void orc_split_rotate_f64(const double* q, const orc_tables* tb, double* y)
{
    for (int h = 0; h < 2; h++) {
        double t[64];
        for (int j = 0; j < 64; j++) {
            double v = q[tb->perm[64 * h + j]];
            t[j] = (tb->signs[64 * h + j] < 0.0f) ? -v : v;
        }
        for (int s = 1; s < 64; s <<= 1)
            for (int i = 0; i < 64; i++)
                if (!(i & s)) {
                    double a = t[i], c = t[i + s];
                    t[i] = a + c;
                    t[i + s] = a - c;
                }
        for (int j = 0; j < 64; j++) y[64 * h + j] = t[j] / 8.0;
    }
}

/* ------------------------------------------------------------------------------------------ */
/* plane layouts                                                                               */
/* ------------------------------------------------------------------------------------------ */
/*
 * Uniform K (token-major), blocks of 64 tokens.  Token t is stored at row
 *     64*(t/64) + 16*((t%64)%4) + (t%64)/4
 * of both the code plane and the meta plane.  4-bit row (64 B) = 16 little-endian u32 words;
 * word 4*kb + g (kb, g in 0..3) holds elements 32*g + 8*kb + i, i = 0..7, element i at bit
 * 16*(i%2) + 4*(i/2).  8-bit row (128 B) = 16 units of 8 B; unit 4*kb + g holds the same 8
 * elements, element i at byte i.  Meta row (16 B) = u16 scale[0..3], then u16 zero[0..3].
 *
 * Uniform planes of either tensor hold a whole number of 64-token blocks.
 *
 * Uniform 3-bit codes (reading of "3-bit group packing"; the pages print no layout) are kept as
 * three bit planes in exactly the byte layout of the TurboQuant 3-bit planes below (K: 48-byte
 * rows in the uniform K row order; V: 1536-byte blocks of 32 tokens), with the uniform meta
 * (16 B per token, K in row order, V in token order): 48 + 16 = 64 B per token-head.
 *
 * Uniform V (blocks of 32 tokens, head dimension outermost within 8-token lanes).  Token t:
 * block b = t/32, tau = t%32, kb = tau/8, i = tau%8; element d: n = d%16, N = d/16.
 * 4-bit block (2048 B): u32 word 8*(16*kb + n) + N, token i at bit 16*(i%2) + 4*(i/2).
 * 8-bit block (4096 B): 8-byte unit 8*(16*kb + n) + N, token i at byte i.
 * Meta: natural token order, 16 B per token as for K.
 *
 * Turbo planes store the 3-bit codes as three bit planes (bit k of every code) in
 * "half-interleaved" u32 words: value e (0..31) of a word sits at bit 16*(e%2) + e/2, so the
 * even-indexed values fill the low half and the odd-indexed values the high half.
 * Turbo K (TURBO_QJL or TURBO_MSE): rows in the same 64-token-block order as uniform K; a row is
 * 48 B: group g at byte 12*g holds words P0, P1, P2, where value e of Pk = bit k of the code of
 * channel 32g + e.  QJL plane (TURBO_QJL): 16 B per row, word w holds the sign bits of
 * projections 32w + e as values e.  Meta per row: u16 n, u16 gamma (TURBO_QJL) or u16 n
 * (TURBO_MSE).
 * Turbo V (TURBO_MSE, b = 3 or 4 bit planes): blocks of 32 tokens, 512*b B each.  Token t:
 * tau = t%32, octet o = tau/8, i = tau%8; channel d: n = d%16, N = d/16.  Bit k of the code of
 * (t, d) is in u32 word 2b*(16*o + n) + 2*k + N/4 of block t/32, at bit
 * 16*(i%2) + 4*(N%4) + i/2.  Meta: u16 n per token, natural order.
 * Split V (TURBO_SPLIT, outlier bits bo, the rest bo - 1, W = 2 bo - 1 words per (o, n)): blocks
 * of 32 tokens, 256 W B each; position j (channel perm[j]): n = j%16, N = j/16.  Bit k of the
 * code of (t, j) is in u32 word W*(16*o + n) + k (j < 64) or W*(16*o + n) + bo + k (j >= 64) of
 * block t/32, at bit 16*(i%2) + 4*(N%4) + i/2.  Meta: u16 n_outlier, u16 n_rest per token.
 * Split K (TURBO_SPLIT on the K tensor, b = 3 or 4, reading R23): rows in the uniform-K block
 * order; position group g (positions 32g .. 32g+31; groups 0, 1 the outliers with b - 1 planes,
 * groups 2, 3 the rest with b - 2) holds its planes as consecutive half-interleaved words, value
 * e of plane k at bit 16*(e%2) + e/2 of word k; group g starts at word g (b-1) for g < 2 and at
 * 2 (b-1) + (g-2) (b-2) otherwise: 4 (4b - 6) B per row (24 B at b = 3, 40 B at b = 4).  QJL
 * plane: 16 B per row as for TURBO_QJL.  Meta per row (8 B): u16 n_outlier, u16 n_rest,
 * u16 gamma, u16 0.
 * Every turbo plane holds a whole number of 64-token blocks.
 * Window ring: [W][128] fp32, token t at slot t % W.
 */

static int ceil_to(int x, int m) { return (x + m - 1) / m * m; }

static size_t k_row(int t) { return (size_t)(64 * (t / 64) + 16 * ((t % 64) % 4) + (t % 64) / 4); }

/* q8_0 planes use the 8-bit uniform byte layout */
static int uniform_layout(const orc_plane_cfg* pc) { return pc->scheme == ORC_UNIFORM || pc->scheme == ORC_Q8_0; }

static int split_k(const orc_plane_cfg* pc) { return pc->scheme == ORC_TURBO_SPLIT && pc->tensor == ORC_TENSOR_K; }

size_t orc_codes_bytes(const orc_plane_cfg* pc)
{
    if (split_k(pc)) return (size_t)ceil_to(pc->capacity, 64) * 4 * (4 * pc->bits - 6);
    if (pc->scheme == ORC_TURBO_SPLIT) return (size_t)ceil_to(pc->capacity, 64) * 8 * (2 * pc->bits - 1);
    if (!uniform_layout(pc)) return (size_t)ceil_to(pc->capacity, 64) * 16 * pc->bits; /* b bit planes */
    return (size_t)ceil_to(pc->capacity, 64) * 16 * pc->bits;
}

size_t orc_meta_bytes(const orc_plane_cfg* pc)
{
    if (split_k(pc)) return (size_t)ceil_to(pc->capacity, 64) * 8;
    if (pc->scheme == ORC_TURBO_QJL) return (size_t)ceil_to(pc->capacity, 64) * 4;
    if (pc->scheme == ORC_TURBO_MSE) return (size_t)ceil_to(pc->capacity, 64) * 2;
    if (pc->scheme == ORC_TURBO_SPLIT) return (size_t)ceil_to(pc->capacity, 64) * 4;
    return (size_t)ceil_to(pc->capacity, 64) * 16;
}

size_t orc_qjl_bytes(const orc_plane_cfg* pc)
{
    return (pc->scheme == ORC_TURBO_QJL || split_k(pc)) ? (size_t)ceil_to(pc->capacity, 64) * 16 : 0;
}

size_t orc_ring_floats(const orc_plane_cfg* pc) { return (size_t)pc->window * D; }

static void put_u16(uint8_t* p, uint16_t v)
{
    p[0] = (uint8_t)(v & 0xff);
    p[1] = (uint8_t)(v >> 8);
}
static uint16_t get_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Set 4-bit field `code` at bit position `bit` of the little-endian u32 at p. */
static void put_nibble(uint8_t* p, int bit, int code)
{
    int byte = bit / 8, sh = bit % 8;
    p[byte] = (uint8_t)((p[byte] & ~(0xf << sh)) | ((code & 0xf) << sh));
}
static int get_nibble(const uint8_t* p, int bit) { return (p[bit / 8] >> (bit % 8)) & 0xf; }

/* Single bits of the little-endian u32 at p. */
static void put_bit(uint8_t* p, int bit, int v)
{
    int byte = bit / 8, sh = bit % 8;
    p[byte] = (uint8_t)((p[byte] & ~(1 << sh)) | ((v & 1) << sh));
}
static int get_bit(const uint8_t* p, int bit) { return (p[bit / 8] >> (bit % 8)) & 1; }

/* Position of value e (0..31) inside a half-interleaved u32 word. */
static int ibit(int e) { return 16 * (e % 2) + e / 2; }

/* Turbo V: byte offset of the u32 word and bit position of bit k of (token t, channel d). */
static size_t tv_word(int t, int d, int k, int b)
{
    int tau = t % 32, o = tau / 8, n = d % 16, N = d / 16;
    return (size_t)(t / 32) * (size_t)(512 * b) + 4 * (size_t)(2 * b * (16 * o + n) + 2 * k + N / 4);
}
/* Split V: byte offset of the word holding bit k of (token t, position j); bo = outlier bits. */
static size_t ts_word(int t, int j, int k, int bo)
{
    int W = 2 * bo - 1, o = (t % 32) / 8, n = j % 16;
    return (size_t)(t / 32) * (size_t)(256 * W) + 4 * (size_t)(W * (16 * o + n) + (j < 64 ? k : bo + k));
}
static int tv_bit(int t, int d)
{
    int i = t % 8, N = d / 16;
    return 16 * (i % 2) + 4 * (N % 4) + i / 2;
}
/* Split K: byte offset (in the row) of plane k of position group g, and the planes of group g. */
static int sk_planes(int g, int b) { return g < 2 ? b - 1 : b - 2; }
static size_t sk_word(int g, int k, int b)
{
    return 4 * (size_t)((g < 2 ? g * (b - 1) : 2 * (b - 1) + (g - 2) * (b - 2)) + k);
}

static void pack_token(const orc_plane_cfg* pc, int t, const uint8_t* code, const uint16_t* s16,
                       const uint16_t* z16, uint16_t n16, uint16_t g16, const uint8_t* bits,
                       uint8_t* codes, uint8_t* meta, uint8_t* qjl)
{
    if (uniform_layout(pc) && pc->bits == 3) {
        /* 3-bit codes: the three bit planes of the TurboQuant 3-bit layout, uniform meta */
        if (pc->tensor == ORC_TENSOR_K) {
            size_t row = k_row(t);
            uint8_t* r = codes + row * 48;
            for (int j = 0; j < D; j++)
                for (int k = 0; k < 3; k++) put_bit(r + 12 * (j / 32) + 4 * k, ibit(j % 32), code[j] >> k);
            uint8_t* m = meta + row * 16;
            for (int g = 0; g < NG; g++) {
                put_u16(m + 2 * g, s16[g]);
                put_u16(m + 8 + 2 * g, z16[g]);
            }
        } else {
            for (int d = 0; d < D; d++)
                for (int k = 0; k < 3; k++) put_bit(codes + tv_word(t, d, k, 3), tv_bit(t, d), code[d] >> k);
            uint8_t* m = meta + (size_t)t * 16;
            for (int g = 0; g < NG; g++) {
                put_u16(m + 2 * g, s16[g]);
                put_u16(m + 8 + 2 * g, z16[g]);
            }
        }
        return;
    }
    if (uniform_layout(pc)) {
        if (pc->tensor == ORC_TENSOR_K) {
            size_t row = k_row(t);
            uint8_t* r = codes + row * (size_t)(16 * pc->bits);
            for (int j = 0; j < D; j++) {
                int g = j / 32, e = j % 32, kb = e / 8, i = e % 8;
                if (pc->bits == 4)
                    put_nibble(r + 4 * (4 * kb + g), 16 * (i % 2) + 4 * (i / 2), code[j]);
                else
                    r[8 * (4 * kb + g) + i] = code[j];
            }
            uint8_t* m = meta + row * 16;
            for (int g = 0; g < NG; g++) {
                put_u16(m + 2 * g, s16[g]);
                put_u16(m + 8 + 2 * g, z16[g]);
            }
        } else {
            int b = t / 32, tau = t % 32, kb = tau / 8, i = tau % 8;
            uint8_t* blk = codes + (size_t)b * (size_t)(512 * pc->bits);
            for (int d = 0; d < D; d++) {
                int n = d % 16, N = d / 16;
                int w = 8 * (16 * kb + n) + N;
                if (pc->bits == 4)
                    put_nibble(blk + 4 * w, 16 * (i % 2) + 4 * (i / 2), code[d]);
                else
                    blk[8 * w + i] = code[d];
            }
            uint8_t* m = meta + (size_t)t * 16;
            for (int g = 0; g < NG; g++) {
                put_u16(m + 2 * g, s16[g]);
                put_u16(m + 8 + 2 * g, z16[g]);
            }
        }
        return;
    }
    if (split_k(pc)) {
        size_t row = k_row(t);
        uint8_t* r = codes + row * (size_t)(4 * (4 * pc->bits - 6));
        for (int j = 0; j < D; j++) {
            int g = j / 32, e = j % 32;
            for (int k = 0; k < sk_planes(g, pc->bits); k++) put_bit(r + sk_word(g, k, pc->bits), ibit(e), code[j] >> k);
        }
        uint8_t* m = meta + row * 8;
        put_u16(m, s16[0]);
        put_u16(m + 2, s16[1]);
        put_u16(m + 4, g16);
        put_u16(m + 6, 0);
        uint8_t* q = qjl + row * 16;
        for (int i = 0; i < D; i++) put_bit(q + 4 * (i / 32), ibit(i % 32), bits[i]);
        return;
    }
    if (pc->scheme == ORC_TURBO_SPLIT) {
        for (int j = 0; j < D; j++) {
            int nb = (j < 64) ? pc->bits : pc->bits - 1;
            for (int k = 0; k < nb; k++) put_bit(codes + ts_word(t, j, k, pc->bits), tv_bit(t, j), code[j] >> k);
        }
        put_u16(meta + (size_t)t * 4, n16);
        put_u16(meta + (size_t)t * 4 + 2, g16);
        return;
    }
    if (pc->tensor == ORC_TENSOR_V) {
        for (int d = 0; d < D; d++)
            for (int k = 0; k < pc->bits; k++)
                put_bit(codes + tv_word(t, d, k, pc->bits), tv_bit(t, d), code[d] >> k);
        put_u16(meta + (size_t)t * 2, n16);
        return;
    }
    size_t row = k_row(t);
    uint8_t* r = codes + row * 48;
    for (int j = 0; j < D; j++) {
        int g = j / 32, e = j % 32;
        for (int k = 0; k < 3; k++) put_bit(r + 12 * g + 4 * k, ibit(e), code[j] >> k);
    }
    if (pc->scheme == ORC_TURBO_QJL) {
        put_u16(meta + row * 4, n16);
        put_u16(meta + row * 4 + 2, g16);
        uint8_t* q = qjl + row * 16;
        for (int i = 0; i < D; i++) put_bit(q + 4 * (i / 32), ibit(i % 32), bits[i]);
    } else {
        put_u16(meta + row * 2, n16);
    }
}

void orc_plane_read(const orc_plane_cfg* pc, const uint8_t* codes, const uint8_t* meta,
                    const uint8_t* qjl, int t, uint8_t* code, uint16_t* meta8, uint8_t* bits)
{
    if (uniform_layout(pc) && pc->bits == 3) {
        const uint8_t* m;
        if (pc->tensor == ORC_TENSOR_K) {
            size_t row = k_row(t);
            const uint8_t* r = codes + row * 48;
            for (int j = 0; j < D; j++) {
                int c = 0;
                for (int k = 0; k < 3; k++) c |= get_bit(r + 12 * (j / 32) + 4 * k, ibit(j % 32)) << k;
                code[j] = (uint8_t)c;
            }
            m = meta + row * 16;
        } else {
            for (int d = 0; d < D; d++) {
                int c = 0;
                for (int k = 0; k < 3; k++) c |= get_bit(codes + tv_word(t, d, k, 3), tv_bit(t, d)) << k;
                code[d] = (uint8_t)c;
            }
            m = meta + (size_t)t * 16;
        }
        for (int k = 0; k < 8; k++) meta8[k] = get_u16(m + 2 * k);
        return;
    }
    if (uniform_layout(pc)) {
        const uint8_t* m;
        if (pc->tensor == ORC_TENSOR_K) {
            size_t row = k_row(t);
            const uint8_t* r = codes + row * (size_t)(16 * pc->bits);
            for (int j = 0; j < D; j++) {
                int g = j / 32, e = j % 32, kb = e / 8, i = e % 8;
                if (pc->bits == 4)
                    code[j] = (uint8_t)get_nibble(r + 4 * (4 * kb + g), 16 * (i % 2) + 4 * (i / 2));
                else
                    code[j] = r[8 * (4 * kb + g) + i];
            }
            m = meta + row * 16;
        } else {
            int b = t / 32, tau = t % 32, kb = tau / 8, i = tau % 8;
            const uint8_t* blk = codes + (size_t)b * (size_t)(512 * pc->bits);
            for (int d = 0; d < D; d++) {
                int w = 8 * (16 * kb + d % 16) + d / 16;
                if (pc->bits == 4)
                    code[d] = (uint8_t)get_nibble(blk + 4 * w, 16 * (i % 2) + 4 * (i / 2));
                else
                    code[d] = blk[8 * w + i];
            }
            m = meta + (size_t)t * 16;
        }
        for (int k = 0; k < 8; k++) meta8[k] = get_u16(m + 2 * k);
        return;
    }
    for (int k = 0; k < 8; k++) meta8[k] = 0;
    if (split_k(pc)) {
        size_t row = k_row(t);
        const uint8_t* r = codes + row * (size_t)(4 * (4 * pc->bits - 6));
        for (int j = 0; j < D; j++) {
            int g = j / 32, e = j % 32, c = 0;
            for (int k = 0; k < sk_planes(g, pc->bits); k++) c |= get_bit(r + sk_word(g, k, pc->bits), ibit(e)) << k;
            code[j] = (uint8_t)c;
        }
        for (int k = 0; k < 3; k++) meta8[k] = get_u16(meta + row * 8 + 2 * k);
        if (bits)
            for (int i = 0; i < D; i++) bits[i] = (uint8_t)get_bit(qjl + row * 16 + 4 * (i / 32), ibit(i % 32));
        return;
    }
    if (pc->scheme == ORC_TURBO_SPLIT) {
        for (int j = 0; j < D; j++) {
            int nb = (j < 64) ? pc->bits : pc->bits - 1, c = 0;
            for (int k = 0; k < nb; k++) c |= get_bit(codes + ts_word(t, j, k, pc->bits), tv_bit(t, j)) << k;
            code[j] = (uint8_t)c;
        }
        meta8[0] = get_u16(meta + (size_t)t * 4);
        meta8[1] = get_u16(meta + (size_t)t * 4 + 2);
        return;
    }
    if (pc->tensor == ORC_TENSOR_V) {
        for (int d = 0; d < D; d++) {
            int c = 0;
            for (int k = 0; k < pc->bits; k++) c |= get_bit(codes + tv_word(t, d, k, pc->bits), tv_bit(t, d)) << k;
            code[d] = (uint8_t)c;
        }
        meta8[0] = get_u16(meta + (size_t)t * 2);
        return;
    }
    size_t row = k_row(t);
    const uint8_t* r = codes + row * 48;
    for (int j = 0; j < D; j++) {
        int g = j / 32, e = j % 32, c = 0;
        for (int k = 0; k < 3; k++) c |= get_bit(r + 12 * g + 4 * k, ibit(e)) << k;
        code[j] = (uint8_t)c;
    }
    if (pc->scheme == ORC_TURBO_QJL) {
        meta8[0] = get_u16(meta + row * 4);
        meta8[1] = get_u16(meta + row * 4 + 2);
        if (bits)
            for (int i = 0; i < D; i++) bits[i] = (uint8_t)get_bit(qjl + row * 16 + 4 * (i / 32), ibit(i % 32));
    } else {
        meta8[0] = get_u16(meta + row * 2);
    }
}

/* Append semantics (reading C7): every token is coded when it is appended; with W > 0 the
 * original binary32 values of token t also go to ring slot t % W, so after any sequence of
 * appends the ring holds the originals of the last min(n, W) tokens. */
void orc_plane_append(const orc_plane_cfg* pc, const orc_tables* tb, const float* X, int t0, int n,
                      uint8_t* codes, uint8_t* meta, uint8_t* qjl, float* ring)
{
    for (int k = 0; k < n; k++) {
        int t = t0 + k;
        const float* x = X + (size_t)k * D;
        uint8_t code[D], bits[D];
        uint16_t s16[NG] = {0}, z16[NG] = {0}, n16 = 0, g16 = 0;
        if (uniform_layout(pc)) {
            float y[D];
            if (pc->rotate)
                orc_rotate_f32(x, tb->signs, y);
            else
                memcpy(y, x, sizeof y);
            if (pc->sinkhorn)
                for (int j = 0; j < D; j++) y[j] = y[j] * tb->inv_c[j];
            for (int g = 0; g < NG; g++) {
                if (pc->scheme == ORC_Q8_0)
                    orc_quant_group_sym8(y + GS * g, code + GS * g, &s16[g], &z16[g]);
                else
                    orc_quant_group(y + GS * g, pc->bits, code + GS * g, &s16[g], &z16[g]);
            }
        } else if (split_k(pc)) {
            orc_split_qjl_encode(x, tb, pc->bits, code, s16, &g16, bits); /* s16[0..1] = n_O, n_R */
        } else if (pc->scheme == ORC_TURBO_SPLIT) {
            uint16_t nn[2];
            orc_split_encode(x, tb, pc->bits, code, nn);
            n16 = nn[0]; /* outlier subset */
            g16 = nn[1]; /* the rest */
        } else {
            orc_turbo_encode_bits(x, tb, pc->bits, pc->scheme == ORC_TURBO_QJL, NULL, code, &n16, &g16, bits,
                                  NULL);
        }
        pack_token(pc, t, code, s16, z16, n16, g16, bits, codes, meta, qjl);
        if (pc->window > 0) memcpy(ring + (size_t)(t % pc->window) * D, x, sizeof(float) * D);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* dequantization and attention                                                                */
/* ------------------------------------------------------------------------------------------ */

void orc_dequant_token(const orc_plane_cfg* pc, const orc_tables* tb, const uint8_t* codes,
                       const uint8_t* meta, int t, double* out)
{
    uint8_t code[D];
    uint16_t m8[8];
    double y[D];
    orc_plane_read(pc, codes, meta, NULL, t, code, m8, NULL);
    if (uniform_layout(pc)) {
        for (int j = 0; j < D; j++) {
            int g = j / GS;
            double s = orc_f16_to_f32(m8[g]), z = orc_f16_to_f32(m8[4 + g]);
            if (pc->scheme == ORC_Q8_0)
                y[j] = s * ((double)code[j] - 128.0); /* d q */
            else
                y[j] = z + s * (double)code[j]; /* exact in binary64 */
            if (pc->sinkhorn) y[j] = y[j] * (double)tb->c[j];
        }
        if (pc->rotate)
            orc_unrotate_f64(y, tb->signs, out);
        else
            memcpy(out, y, sizeof y);
        return;
    }
    if (pc->scheme == ORC_TURBO_SPLIT) {
        for (int h = 0; h < 2; h++) {
            double nh = orc_f16_to_f32(m8[h]), z[64];
            const float* mu = h ? tb->mu2 : tb->mu;
            for (int j = 0; j < 64; j++) y[64 * h + j] = nh * (double)mu[code[64 * h + j]];
            orc_unrotate64_f64(y + 64 * h, tb->signs + 64 * h, z);
            for (int j = 0; j < 64; j++) out[tb->perm[64 * h + j]] = z[j];
        }
        return;
    }
    double n = orc_f16_to_f32(m8[0]);
    for (int j = 0; j < D; j++) y[j] = n * (double)tb->mu[code[j]];
    orc_unrotate_f64(y, tb->signs, out);
}

/* <q, k_t> ~= n <rho_q, mu[code]> + gamma sqrt(pi/2)/128 sum_i sign_i (S rho_q)_i, where
 * rho_q = R(q) and sign_i = 2 bit_i - 1.  The second term is the QJL estimate of <rho_q, r> from
 * E[sign(s.r) (s.x)] = sqrt(2/pi) <x, r> / |r| for s ~ N(0, I). */
double orc_turbo_score(const orc_tables* tb, const uint8_t* codes, const uint8_t* meta,
                       const uint8_t* qjl, int t, const double* rho_q, const double* s_rho_q)
{
    orc_plane_cfg pc = {ORC_TURBO_QJL, 3, 1, 0, 0, ORC_TENSOR_K, t + 1};
    uint8_t code[D], bits[D];
    uint16_t m8[8];
    orc_plane_read(&pc, codes, meta, qjl, t, code, m8, bits);
    double n = orc_f16_to_f32(m8[0]), gam = orc_f16_to_f32(m8[1]);
    double a = 0.0, b = 0.0;
    for (int j = 0; j < D; j++) a += rho_q[j] * (double)tb->mu[code[j]];
    for (int i = 0; i < D; i++) b += (bits[i] ? 1.0 : -1.0) * s_rho_q[i];
    return n * a + gam * sqrt(ORC_PI / 2.0) / 128.0 * b;
}

/* Split K (reading R23): <q, k_t> ~= n_O <rho_q, mu_O[code]>_outliers + n_R <rho_q, mu_R[code]>_rest
 * + gamma sqrt(pi/2)/128 sum_i sign_i (S rho_q)_i, with rho_q the split domain of q
 * (orc_split_rotate_f64) and mu_O, mu_R = tb->mu, tb->mu2. */
double orc_split_score(const orc_plane_cfg* pc, const orc_tables* tb, const uint8_t* codes, const uint8_t* meta,
                       const uint8_t* qjl, int t, const double* rho_q, const double* s_rho_q)
{
    uint8_t code[D], bits[D];
    uint16_t m8[8];
    orc_plane_read(pc, codes, meta, qjl, t, code, m8, bits);
    double a[2] = {0.0, 0.0}, b = 0.0;
    for (int j = 0; j < D; j++) a[j >= 64] += rho_q[j] * (double)(j >= 64 ? tb->mu2 : tb->mu)[code[j]];
    for (int i = 0; i < D; i++) b += (bits[i] ? 1.0 : -1.0) * s_rho_q[i];
    return (double)orc_f16_to_f32(m8[0]) * a[0] + (double)orc_f16_to_f32(m8[1]) * a[1] +
           (double)orc_f16_to_f32(m8[2]) * sqrt(ORC_PI / 2.0) / 128.0 * b;
}

/* Attention of G query heads over the first n_vis tokens of a cache holding n tokens
 * (1 <= n_vis <= n).  Which tokens are read from the FP32 window depends on n (the cache as it
 * stands), not on n_vis: a query of a prefill chunk at position n_vis - 1 sees the same token
 * values as a decode query would, cut off at its own position (causal). */
void orc_attention_prefix(const orc_plane_cfg* kc, const orc_plane_cfg* vc,
                          const orc_tables* ktb, const orc_tables* vtb, const uint8_t* kcodes,
                          const uint8_t* kmeta, const uint8_t* kqjl, const float* kring,
                          const uint8_t* vcodes, const uint8_t* vmeta, const float* vring, int n,
                          int n_vis, int G, const float* q, double scale, double* out)
{
    if (n <= 0 || n_vis <= 0) {
        for (int i = 0; i < G * D; i++) out[i] = 0.0;
        return;
    }
    if (n_vis > n) n_vis = n;
    int W = kc->window;
    int nq = (W > 0 && n > W) ? n - W : (W > 0 ? 0 : n); /* tokens read from the codes */
    double* V = (double*)malloc(sizeof(double) * (size_t)n * D);
    double* K = NULL;
    const int ksplit = split_k(kc);
    if (kc->scheme != ORC_TURBO_QJL && !ksplit) K = (double*)malloc(sizeof(double) * (size_t)n * D);
    for (int t = 0; t < n; t++) {
        if (t >= nq) { /* FP32 window token */
            const float* kr = kring + (size_t)(t % W) * D;
            const float* vr = vring + (size_t)(t % W) * D;
            for (int j = 0; j < D; j++) {
                if (K) K[(size_t)t * D + j] = kr[j];
                V[(size_t)t * D + j] = vr[j];
            }
        } else {
            if (K) orc_dequant_token(kc, ktb, kcodes, kmeta, t, K + (size_t)t * D);
            orc_dequant_token(vc, vtb, vcodes, vmeta, t, V + (size_t)t * D);
        }
    }
    double* a = (double*)malloc(sizeof(double) * (size_t)n);
    for (int h = 0; h < G; h++) {
        const float* qh = q + (size_t)h * D;
        double qd[D], rq[D], srq[D];
        for (int j = 0; j < D; j++) qd[j] = qh[j];
        if (!K) {
            if (ksplit)
                orc_split_rotate_f64(qd, ktb, rq);
            else
                orc_rotate_f64(qd, ktb->signs, rq);
            for (int i = 0; i < D; i++) {
                double s = 0.0;
                for (int j = 0; j < D; j++) s += (double)ktb->S[i * D + j] * rq[j];
                srq[i] = s;
            }
        }
        double mx = -INFINITY;
        for (int t = 0; t < n_vis; t++) {
            double s;
            if (K || t >= nq) {
                s = 0.0;
                if (t >= nq) {
                    const float* kr = kring + (size_t)(t % W) * D;
                    for (int j = 0; j < D; j++) s += qd[j] * (double)kr[j];
                } else {
                    for (int j = 0; j < D; j++) s += qd[j] * K[(size_t)t * D + j];
                }
            } else if (ksplit) {
                s = orc_split_score(kc, ktb, kcodes, kmeta, kqjl, t, rq, srq);
            } else {
                s = orc_turbo_score(ktb, kcodes, kmeta, kqjl, t, rq, srq);
            }
            a[t] = scale * s;
            if (a[t] > mx) mx = a[t];
        }
        double l = 0.0;
        double o[D];
        for (int j = 0; j < D; j++) o[j] = 0.0;
        for (int t = 0; t < n_vis; t++) {
            double p = exp(a[t] - mx);
            l += p;
            for (int j = 0; j < D; j++) o[j] += p * V[(size_t)t * D + j];
        }
        for (int j = 0; j < D; j++) out[(size_t)h * D + j] = o[j] / l;
    }
    free(a);
    free(V);
    free(K);
}

/* Decode attention: every token of the cache is visible. */
void orc_attention(const orc_plane_cfg* kc, const orc_plane_cfg* vc, const orc_tables* ktb,
                   const orc_tables* vtb, const uint8_t* kcodes, const uint8_t* kmeta,
                   const uint8_t* kqjl, const float* kring, const uint8_t* vcodes,
                   const uint8_t* vmeta, const float* vring, int n, int G, const float* q,
                   double scale, double* out)
{
    orc_attention_prefix(kc, vc, ktb, vtb, kcodes, kmeta, kqjl, kring, vcodes, vmeta, vring, n, n,
                         G, q, scale, out);
}

/* ---- Seeded random tables --------------------------------------------------------------------
 * The pages draw a random-sign Walsh-Hadamard rotation (KVarN post, TL;DR; the TurboQuant row of
 * "LLM memory saving ... 2026", method comparison table) and a Gaussian projection for the QJL
 * sketch (same row) without naming a generator.  Reading: SplitMix64 (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014) used counter-style.  Its
 * generator adds the odd constant gamma to a 64-bit state and returns the state passed through
 * a fixed mixing function; so the (i + 1)-th output from state k is mix(k + (i + 1) gamma), and
 * every draw can be computed on its own.  Stream keys chain mix over the fields. */
static const uint64_t SM_GAMMA = 0x9E3779B97F4A7C15ull;

static uint64_t sm_mix(uint64_t z)
{
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

uint64_t orc_stream_key(uint64_t seed, int tag, int layer, int head, int tensor)
{
    uint64_t k = sm_mix(seed + SM_GAMMA * (uint64_t)(tag + 1));
    k = sm_mix(k + SM_GAMMA * (uint64_t)(layer + 1));
    k = sm_mix(k + SM_GAMMA * (uint64_t)(head + 1));
    return sm_mix(k + SM_GAMMA * (uint64_t)(tensor + 1));
}

uint64_t orc_stream_draw(uint64_t key, uint64_t i) { return sm_mix(key + SM_GAMMA * (i + 1)); }

double orc_box_muller(uint64_t x1, uint64_t x2)
{
    const double two_to_m53 = 1.0 / 9007199254740992.0; /* 2^-53 */
    double u1 = (double)((x1 >> 11) + 1) * two_to_m53;   /* (0, 1]: log never sees 0 */
    double u2 = (double)(x2 >> 11) * two_to_m53;         /* [0, 1) */
    double r = sqrt(-2.0 * log(u1));
    double c = cos(6.283185307179586 * u2);              /* 2 pi rounded to binary64 */
    return r * c;
}

void orc_derive_tables(uint64_t seed, int n_layers, int n_kv_heads, float* signs, float* S)
{
    if (signs) {
        for (int l = 0; l < n_layers; l++)
            for (int h = 0; h < n_kv_heads; h++)
                for (int t = 0; t < 2; t++) {
                    uint64_t key = orc_stream_key(seed, 1, l, h, t);
                    float* out = signs + (((size_t)l * n_kv_heads + h) * 2 + t) * D;
                    for (int j = 0; j < D; j++) out[j] = (orc_stream_draw(key, (uint64_t)j) >> 63) ? -1.0f : 1.0f;
                }
    }
    if (S) {
        uint64_t key = orc_stream_key(seed, 2, 0, 0, 0);
        for (int k = 0; k < D * D; k++)
            S[k] = (float)orc_box_muller(orc_stream_draw(key, 2 * (uint64_t)k), orc_stream_draw(key, 2 * (uint64_t)k + 1));
    }
}
