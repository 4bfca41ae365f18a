/*
 * nvfp4_oracle.c -- plain CPU reference of the NVFP4 hot path.
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
 * baseline load this; the HIP library never does, and the two share no code.
 *
 * Built with -O2 -ffp-contract=off on x86-64 (SSE arithmetic), so every float
 * expression below rounds once per operation, to nearest-even.
 *
 * What it follows:
 *  - NVFP4 element/scale format: 16 consecutive E2M1 values share one E4M3
 *    block scale (ARCQuant article on zizhi168.cn, section 1 "NVFP4 overview";
 *    also the abstract of "Replay the Curvature: Accurate and Scalable NVFP4
 *    Quantization for Large Language Model Inference").
 *  - E2M1 = 2 exponent bits (bias 1) and 1 mantissa bit; E4M3 = 4 exponent
 *    bits (bias 7) and 3 mantissa bits, relative step 2^-3 (ARCQuant article,
 *    section 4.2), in its finite-only form whose largest value is 448.
 *  - Two-stage residue quantization and the augmented tensor
 *    X_aug = [Q(X) | Q(R)] with one scale s_aug (ARCQuant article, section 3.1;
 *    the FP4 base plus FP4-quantized residue of the ResServe abstract).
 *  - The fused quantizer's steps: channel reorder, RMSNorm, main and residual
 *    quantization (ARCQuant article, section 3.2); outlier channels ranked by
 *    calibration absolute maximum (section 3.1); weights in the same channel
 *    order (section 6.3).
 * Readings where the pages are silent (all stated here and pinned by tests):
 *  - per-tensor FP32 scale S = amax / (6 * 448), S = 1 for an all-zero tensor;
 *  - block scale d = E4M3(a_b / (6 S)), element scale s = fl(d * S),
 *    q = fl(x * fl(1 / s)) (r = 0 when s = 0), code = E2M1(|q|) with the sign
 *    bit of x; every rounding is to nearest, ties to the even code, saturating;
 *  - the residue uses the FP32 dequantization fl(fl(e * d) * S);
 *  - RMSNorm sums squares in FP64 and rounds r to FP32;
 *  - the optional diagonal smoothing (abstract of "OSFP4: Joint Optimization of
 *    Diagonal Smoothing and Block Scales for NVFP4 Quantization": one diagonal
 *    matrix per linear projection, its inverse folded into the weight) multiplies
 *    each input channel by its entry in FP32 after RMSNorm, before the reorder.
 */
#include "nvfp4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ formats */

double or_e2m1_value(int code)
{
    int e = (code >> 1) & 3, m = code & 1;
    /* exponent bias 1; e == 0 is subnormal: m * 2^(1-1) * 0.5 */
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (code & 8) ? -mag : mag;
}

double or_e4m3_value(int byte)
{
    int e = (byte >> 3) & 15, m = byte & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;                 /* the only NaN pattern */
    mag = (e == 0) ? ldexp((double)m, -9)              /* subnormal m * 2^-6 / 8 */
                   : ldexp(1.0 + m / 8.0, e - 7);
    return (byte & 0x80) ? -mag : mag;
}

int or_e2m1_encode(float q)
{
    double a = fabs((double)q), best_d = INFINITY;
    int best = 0;
    /* Saturation: at or above the largest magnitude the nearest value is that
     * magnitude. Checked first because far above it the double distances below
     * would all round to the same number and tie. */
    if (a >= or_e2m1_value(7)) return 7 | (signbit(q) ? 8 : 0);
    for (int c = 0; c < 8; ++c) {
        double d = fabs(a - or_e2m1_value(c));
        if (d < best_d || (d == best_d && (c & 1) == 0)) { best_d = d; best = c; }
    }
    return best | (signbit(q) ? 8 : 0);
}

int or_e4m3_encode(float v)
{
    double a = (double)v, best_d = INFINITY;
    int best = 0;
    if (a >= or_e4m3_value(126)) return 126;           /* saturation, as above */
    for (int c = 0; c < 127; ++c) {                    /* all finite non-negative */
        double d = fabs(a - or_e4m3_value(c));
        if (d < best_d || (d == best_d && (c & 1) == 0)) { best_d = d; best = c; }
    }
    return best;
}

/* ------------------------------------------------------------- quantization */

float or_tensor_scale(const float *x, int64_t rows, int64_t K, int64_t ldx)
{
    float at = 0.0f;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(x[r * ldx + k]);
            if (a > at) at = a;
        }
    return at > 0.0f ? at / 2688.0f : 1.0f;
}

static int near_midpoint(float q)
{
    static const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
    double a = fabs((double)q);
    for (int i = 0; i < 7; ++i)
        if (fabs(a - mids[i]) <= mids[i] * ldexp(1.0, -20)) return 1;
    return 0;
}

int64_t or_quantize(const float *x, int64_t rows, int64_t K, int64_t ldx,
                    const float *static_S,
                    uint8_t *codes, int64_t ldc, uint8_t *scales, int64_t lds,
                    float *S_out)
{
    int64_t near = 0;
    float S = static_S ? *static_S : or_tensor_scale(x, rows, K, ldx);
    float t = 6.0f * S;
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * ldx;
        for (int64_t b = 0; b < K / 16; ++b) {
            float ab = 0.0f, sf, d, s, rcp;
            int db;
            for (int i = 0; i < 16; ++i) {
                float a = fabsf(xr[16 * b + i]);
                if (a > ab) ab = a;
            }
            sf = ab / t;
            db = or_e4m3_encode(sf);
            d = (float)or_e4m3_value(db);
            s = d * S;
            rcp = (s > 0.0f) ? 1.0f / s : 0.0f;
            scales[r * lds + b] = (uint8_t)db;
            for (int i = 0; i < 16; ++i) {
                float xv = xr[16 * b + i];
                float q = xv * rcp;
                int c = or_e2m1_encode(q) & 7;
                if (signbit(xv)) c |= 8;
                near += near_midpoint(q);
                int64_t k = 16 * b + i;
                uint8_t *byte = &codes[r * ldc + k / 2];
                if ((k & 1) == 0) *byte = (uint8_t)((*byte & 0xF0) | c);
                else              *byte = (uint8_t)((*byte & 0x0F) | (c << 4));
            }
        }
    }
    if (S_out) *S_out = S;
    return near;
}

static int code_at(const uint8_t *codes, int64_t ldc, int64_t r, int64_t k)
{
    uint8_t byte = codes[r * ldc + k / 2];
    return (k & 1) ? (byte >> 4) : (byte & 15);
}

void or_dequantize(const uint8_t *codes, int64_t ldc, const uint8_t *scales, int64_t lds,
                   float S, int64_t rows, int64_t K, double *out, int64_t ldo)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * ldo + k] = or_e2m1_value(code_at(codes, ldc, r, k)) *
                               or_e4m3_value(scales[r * lds + k / 16]) * (double)S;
}

void or_dequantize_f32(const uint8_t *codes, int64_t ldc, const uint8_t *scales, int64_t lds,
                       float S, int64_t rows, int64_t K, float *out, int64_t ldo)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k) {
            float ed = (float)(or_e2m1_value(code_at(codes, ldc, r, k)) *
                               or_e4m3_value(scales[r * lds + k / 16]));   /* exact */
            out[r * ldo + k] = ed * S;
        }
}

/* ------------------------------------------------------ RMSNorm and reorder */

void or_rmsnorm(const float *x, int64_t rows, int64_t K, int64_t ldx,
                const float *gamma, float eps, float *y, int64_t ldy)
{
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * ldx;
        double ss = 0.0;
        float rr;
        for (int64_t k = 0; k < K; ++k) ss += (double)xr[k] * (double)xr[k];
        rr = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
        for (int64_t k = 0; k < K; ++k) {
            float v = xr[k] * rr;
            y[r * ldy + k] = v * gamma[k];
        }
    }
}

void or_channel_absmax(const float *x, int64_t rows, int64_t K, int64_t ldx,
                       const float *gamma, float eps, float *v)
{
    float *y = (float *)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
    for (int64_t k = 0; k < K; ++k) v[k] = 0.0f;
    for (int64_t r = 0; r < rows; ++r) {
        if (gamma) or_rmsnorm(x + r * ldx, 1, K, ldx, gamma, eps, y, K);
        else memcpy(y, x + r * ldx, sizeof(float) * (size_t)K);
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(y[k]);
            if (a > v[k]) v[k] = a;
        }
    }
    free(y);
}

void or_perm_from_absmax(const float *v, int64_t K, int32_t *perm)
{
    /* insertion sort: descending v, ascending index among equal v */
    for (int64_t i = 0; i < K; ++i) perm[i] = (int32_t)i;
    for (int64_t i = 1; i < K; ++i) {
        int32_t p = perm[i];
        int64_t j = i - 1;
        while (j >= 0 && (v[perm[j]] < v[p] || (v[perm[j]] == v[p] && perm[j] > p))) {
            perm[j + 1] = perm[j];
            --j;
        }
        perm[j + 1] = p;
    }
}

int64_t or_quantize_aug(const float *x, int64_t rows, int64_t K_in, int64_t ldx,
                        const float *gamma, float eps, const float *smooth, const int32_t *perm,
                        int64_t S_cols, const float *static_S,
                        uint8_t *codes, int64_t ldc, uint8_t *scales, int64_t lds,
                        float *S_out)
{
    int64_t Ka = K_in + S_cols, near;
    float *y = (float *)malloc(sizeof(float) * (size_t)(rows * K_in + 1));
    float *xa = (float *)malloc(sizeof(float) * (size_t)(rows * Ka + 1));

    /* RMSNorm, then the diagonal smoothing multiply (one FP32 rounding per
     * element; its inverse belongs to the weight, OSFP4 abstract), then gather */
    if (gamma) or_rmsnorm(x, rows, K_in, ldx, gamma, eps, y, K_in);
    else for (int64_t r = 0; r < rows; ++r) memcpy(y + r * K_in, x + r * ldx, sizeof(float) * (size_t)K_in);
    if (smooth)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t k = 0; k < K_in; ++k) y[r * K_in + k] = y[r * K_in + k] * smooth[k];
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < K_in; ++j)
            xa[r * Ka + j] = y[r * K_in + (perm ? perm[j] : j)];

    if (S_cols > 0) {
        /* main stage on x', residue R = x' - deq32(Q(x')) on the first S_cols columns */
        int64_t ldm = (K_in + 1) / 2, ldms = K_in / 16 + 1;
        uint8_t *mc = (uint8_t *)calloc((size_t)(rows * ldm + 1), 1);
        uint8_t *ms = (uint8_t *)calloc((size_t)(rows * ldms + 1), 1);
        float *dq = (float *)malloc(sizeof(float) * (size_t)(rows * K_in + 1));
        float Sm;
        for (int64_t r = 0; r < rows; ++r)
            memcpy(y + r * K_in, xa + r * Ka, sizeof(float) * (size_t)K_in);
        or_quantize(y, rows, K_in, K_in, static_S, mc, ldm, ms, ldms, &Sm);
        or_dequantize_f32(mc, ldm, ms, ldms, Sm, rows, K_in, dq, K_in);
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t j = 0; j < S_cols; ++j)
                xa[r * Ka + K_in + j] = xa[r * Ka + j] - dq[r * K_in + j];
        free(mc); free(ms); free(dq);
    }
    /* X_aug quantized as one tensor */
    near = or_quantize(xa, rows, Ka, Ka, static_S, codes, ldc, scales, lds, S_out);
    free(y); free(xa);
    return near;
}

/* --------------------------------------------------------------------- GEMM */

static void decode_row(const uint8_t *codes, int64_t ldc, const uint8_t *scales, int64_t lds,
                       int64_t r, int64_t K, double *out)
{
    for (int64_t k = 0; k < K; ++k)
        out[k] = or_e2m1_value(code_at(codes, ldc, r, k)) * or_e4m3_value(scales[r * lds + k / 16]);
}

void or_gemm(const uint8_t *ac, int64_t ldac, const uint8_t *as, int64_t ldas, float Sa,
             const uint8_t *wc, int64_t ldwc, const uint8_t *ws, int64_t ldws, float Sw,
             int64_t M, int64_t N, int64_t K, double *y, int64_t ldy)
{
    double *a = (double *)malloc(sizeof(double) * (size_t)(M * K + 1));
    double *w = (double *)malloc(sizeof(double) * (size_t)(K + 1));
    double s = (double)Sa * (double)Sw;
    for (int64_t m = 0; m < M; ++m) decode_row(ac, ldac, as, ldas, m, K, a + m * K);
    for (int64_t n = 0; n < N; ++n) {
        decode_row(wc, ldwc, ws, ldws, n, K, w);
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            const double *am = a + m * K;
            for (int64_t k = 0; k < K; ++k) acc += am[k] * w[k];
            y[m * ldy + n] = acc * s;
        }
    }
    free(a); free(w);
}

void or_gemm_pairs(const uint8_t *ac, int64_t ldac, const uint8_t *as, int64_t ldas, float Sa,
                   const uint8_t *wc, int64_t ldwc, const uint8_t *ws, int64_t ldws, float Sw,
                   int64_t K, const int64_t *ms, const int64_t *ns, int64_t count, double *y)
{
    double *a = (double *)malloc(sizeof(double) * (size_t)(K + 1));
    double *w = (double *)malloc(sizeof(double) * (size_t)(K + 1));
    double s = (double)Sa * (double)Sw;
    for (int64_t i = 0; i < count; ++i) {
        double acc = 0.0;
        decode_row(ac, ldac, as, ldas, ms[i], K, a);
        decode_row(wc, ldwc, ws, ldws, ns[i], K, w);
        for (int64_t k = 0; k < K; ++k) acc += a[k] * w[k];
        y[i] = acc * s;
    }
    free(a); free(w);
}

/* 2*e(c) is an integer in [-12, 12] and d * 2^9 an integer below 2^18, so
 * e(c)*d = (2e)(512d) * 2^-10 exactly, and a product of two is an integer
 * multiple of 2^-20. */
static int64_t int_value(const uint8_t *codes, int64_t ldc, const uint8_t *scales, int64_t lds,
                         int64_t r, int64_t k)
{
    int64_t two_e = (int64_t)(2.0 * or_e2m1_value(code_at(codes, ldc, r, k)));
    int64_t d512 = (int64_t)(512.0 * or_e4m3_value(scales[r * lds + k / 16]));
    return two_e * d512;
}

int or_gemm_exact(const uint8_t *ac, int64_t ldac, const uint8_t *as, int64_t ldas, float Sa,
                  const uint8_t *wc, int64_t ldwc, const uint8_t *ws, int64_t ldws, float Sw,
                  int64_t M, int64_t N, int64_t K, double *y, int64_t ldy)
{
    const int64_t lim = (int64_t)1 << 62;
    double s = (double)Sa * (double)Sw;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t p = int_value(ac, ldac, as, ldas, m, k) * int_value(wc, ldwc, ws, ldws, n, k);
                if ((p > 0 && acc > lim - p) || (p < 0 && acc < -lim - p)) return -1;
                acc += p;
            }
            if (acc > ((int64_t)1 << 53) || acc < -((int64_t)1 << 53)) return -1;
            y[m * ldy + n] = ldexp((double)acc, -20) * s;
        }
    return 0;
}

/* ---------------------------------------------------------------- MXFP4
 * MXFP4: E2M1 elements (the element format of section 1 of the ARCQuant
 * article) sharing one power-of-two E8M0 scale per 32 consecutive elements
 * along K (the 32-element blocks and E8M0 scales of the MX formats, ARCQuant
 * article sections 2.2 and 4.2; MXFP4 is the second format of the ResServe
 * abstract). The pages give no scale rule; this follows the published MX
 * definition: shared exponent e = floor(log2(amax)) - 2 (2 = the exponent of
 * E2M1's largest value, 6 = 1.5 * 2^2), clamped to E8M0's range [-127, 127];
 * element q = x * 2^-e rounded to nearest E2M1 (ties even), saturating at 6,
 * sign of x. An all-zero block takes e = -127. There is no tensor scale. */

double or_e8m0_value(int byte)
{
    if (byte == 255) return NAN;
    return ldexp(1.0, byte - 127);
}

int or_mx_block_exponent(const float *v)
{
    float amax = 0.0f;
    int ex;
    for (int i = 0; i < 32; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) return -127;
    (void)frexp((double)amax, &ex);      /* amax = f 2^ex, f in [0.5, 1): floor(log2) = ex - 1 */
    ex = ex - 1 - 2;
    return ex < -127 ? -127 : (ex > 127 ? 127 : ex);
}

void or_mx_quantize(const float *x, int64_t rows, int64_t K, int64_t ldx,
                    uint8_t *codes, int64_t ldc, uint8_t *scales, int64_t lds)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < K / 32; ++b) {
            const float *v = x + r * ldx + 32 * b;
            int e = or_mx_block_exponent(v);
            scales[r * lds + b] = (uint8_t)(e + 127);
            for (int i = 0; i < 32; ++i) {
                double q = ldexp((double)v[i], -e);            /* exact */
                int c = or_e2m1_encode((float)q) & 7;          /* (float) exact: |q| < 8, >= 2^-22 or 0 */
                if (signbit(v[i])) c |= 8;
                int64_t k = 32 * b + i;
                uint8_t *byte = &codes[r * ldc + k / 2];
                if ((k & 1) == 0) *byte = (uint8_t)((*byte & 0xF0) | c);
                else              *byte = (uint8_t)((*byte & 0x0F) | (c << 4));
            }
        }
}

void or_mx_dequantize(const uint8_t *codes, int64_t ldc, const uint8_t *scales, int64_t lds,
                      int64_t rows, int64_t K, double *out, int64_t ldo)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * ldo + k] = or_e2m1_value(code_at(codes, ldc, r, k)) * or_e8m0_value(scales[r * lds + k / 32]);
}

/* X_aug = [Q(x) | Q(R)] in MXFP4, R = fl(x - deq(Q(x))) on columns [0, S_cols):
 * the two-stage residue of section 3.1 of the ARCQuant article in the MX format.
 * deq(Q(x)) = e(c) 2^e is exact in FP32 here, so R rounds once. Each 32-block
 * of R takes its own shared exponent (MX has no tensor-wide scale). */
void or_mx_quantize_aug(const float *x, int64_t rows, int64_t K, int64_t ldx, int64_t S_cols,
                        uint8_t *codes, int64_t ldc, uint8_t *scales, int64_t lds)
{
    float *res = (float *)malloc(sizeof(float) * (size_t)(rows * (S_cols > 0 ? S_cols : 1) + 1));
    or_mx_quantize(x, rows, K, ldx, codes, ldc, scales, lds);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < S_cols; ++k) {
            float deq = (float)(or_e2m1_value(code_at(codes, ldc, r, k)) * or_e8m0_value(scales[r * lds + k / 32]));
            res[r * S_cols + k] = x[r * ldx + k] - deq;
        }
    if (S_cols > 0) {
        /* the residue columns start at column K of the output rows */
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t b = 0; b < S_cols / 32; ++b) {
                const float *v = res + r * S_cols + 32 * b;
                int e = or_mx_block_exponent(v);
                scales[r * lds + K / 32 + b] = (uint8_t)(e + 127);
                for (int i = 0; i < 32; ++i) {
                    double q = ldexp((double)v[i], -e);
                    int c = or_e2m1_encode((float)q) & 7;
                    if (signbit(v[i])) c |= 8;
                    int64_t k = K + 32 * b + i;
                    uint8_t *byte = &codes[r * ldc + k / 2];
                    if ((k & 1) == 0) *byte = (uint8_t)((*byte & 0xF0) | c);
                    else              *byte = (uint8_t)((*byte & 0x0F) | (c << 4));
                }
            }
    }
    free(res);
}

/* y[m][n] = sum_k deq(a)[m][k] deq(w)[n][k] in FP64 (every product is exact). */
void or_mx_gemm(const uint8_t *ac, int64_t ldac, const uint8_t *as, int64_t ldas,
                const uint8_t *wc, int64_t ldwc, const uint8_t *ws, int64_t ldws,
                int64_t M, int64_t N, int64_t K, double *y, int64_t ldy)
{
    double *a = (double *)malloc(sizeof(double) * (size_t)(M * K + 1));
    double *w = (double *)malloc(sizeof(double) * (size_t)(K + 1));
    or_mx_dequantize(ac, ldac, as, ldas, M, K, a, K);
    for (int64_t n = 0; n < N; ++n) {
        or_mx_dequantize(wc + n * ldwc, ldwc, ws + n * ldws, ldws, 1, K, w, K);
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += a[m * K + k] * w[k];
            y[m * ldy + n] = acc;
        }
    }
    free(a); free(w);
}
