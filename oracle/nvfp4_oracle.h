/*
 * nvfp4_oracle.h -- plain CPU reference of the NVFP4 hot path (TEST INFRASTRUCTURE).
 *
 * This is the oracle that the HIP library is checked against. It is slow on
 * purpose: brute-force rounding, plain loops, FP64 accumulation. Only the
 * tests, the smoke check and the CPU-baseline leg of the bench may load it; the
 * product path (libnvfp4) never does and shares no code with it.
 *
 * All pointers are host pointers. Matrices are row-major with explicit leading
 * dimensions (in elements for float inputs, in bytes for codes and scales).
 *
 * Storage convention (a reading; the pages fix no layout):
 *   codes  [rows][ldc] bytes, byte j of a row = code(2j) | code(2j+1) << 4
 *   scales [rows][lds] bytes, E4M3 scale of block b = columns [16b, 16b+16)
 *   one FP32 tensor scale S per tensor.
 * A 4-bit code is sign(bit 3) | E2M1 magnitude index (bits 2..0).
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Format decoders (exact). */
double or_e2m1_value(int code);          /* 4-bit code -> value                   */
double or_e4m3_value(int byte);          /* 8-bit E4M3 byte -> value (NaN: 0x7F/0xFF) */

/* Brute-force round-to-nearest, ties to the even code, saturating at the
 * largest finite value. or_e2m1_encode returns the 4-bit code (sign from the
 * sign bit of q); or_e4m3_encode takes v >= 0 and returns the byte. */
int or_e2m1_encode(float q);
int or_e4m3_encode(float v);

/* Per-tensor scale: S = amax / 2688 (FP32 divide), S = 1 for an all-zero tensor. */
float or_tensor_scale(const float *x, int64_t rows, int64_t K, int64_t ldx);

/* NVFP4 quantization of a rows x K FP32 matrix (K % 16 == 0).
 * static_S: NULL = dynamic per-tensor scale, else use *static_S.
 * Returns the number of elements whose FP32 quotient x*(1/s) lies within
 * 2^-20 (relative) of an E2M1 rounding midpoint ("near-midpoint" count). */
int64_t or_quantize(const float *x, int64_t rows, int64_t K, int64_t ldx,
                    const float *static_S,
                    uint8_t *codes, int64_t ldc, uint8_t *scales, int64_t lds,
                    float *S_out);

/* Exact dequantization e(c) * d * S into FP64. */
void or_dequantize(const uint8_t *codes, int64_t ldc, const uint8_t *scales, int64_t lds,
                   float S, int64_t rows, int64_t K, double *out, int64_t ldo);

/* FP32 dequantization used for the residue: fl(fl(e(c)*d) * S). */
void or_dequantize_f32(const uint8_t *codes, int64_t ldc, const uint8_t *scales, int64_t lds,
                       float S, int64_t rows, int64_t K, float *out, int64_t ldo);

/* RMSNorm: y = fl(fl(x*r)*gamma), r = fl32(1 / sqrt(sum(x^2)/K + eps)), sum in FP64. */
void or_rmsnorm(const float *x, int64_t rows, int64_t K, int64_t ldx,
                const float *gamma, float eps, float *y, int64_t ldy);

/* Calibration statistic v[j] = max over rows of |RMSNorm(x)[:, j]| (|x| if gamma == NULL). */
void or_channel_absmax(const float *x, int64_t rows, int64_t K, int64_t ldx,
                       const float *gamma, float eps, float *v);

/* Channel order: channels sorted by v descending, ties by ascending index. */
void or_perm_from_absmax(const float *v, int64_t K, int32_t *perm);

/* Fused-quantizer reference: optional RMSNorm (gamma != NULL), optional diagonal
 * smoothing y[:, k] *= smooth[k] in FP32 (smooth != NULL), optional channel
 * gather x'[:, j] = y[:, perm[j]] (perm != NULL), then NVFP4 quantization of
 * X_aug = [x' | R] with R = fl(x' - deq32(Q(x'))) on columns [0, S_cols).
 * X_aug is quantized as one tensor (one tensor scale). Output has K_in + S_cols
 * columns. S_cols == 0 gives the plain quantization of x'. */
int64_t or_quantize_aug(const float *x, int64_t rows, int64_t K_in, int64_t ldx,
                        const float *gamma, float eps, const float *smooth, const int32_t *perm,
                        int64_t S_cols, const float *static_S,
                        uint8_t *codes, int64_t ldc, uint8_t *scales, int64_t lds,
                        float *S_out);

/* W4A4 product y[m][n] = Sa*Sw * sum_k deq(a)[m][k] * deq(w)[n][k], FP64 accumulate. */
void or_gemm(const uint8_t *ac, int64_t ldac, const uint8_t *as, int64_t ldas, float Sa,
             const uint8_t *wc, int64_t ldwc, const uint8_t *ws, int64_t ldws, float Sw,
             int64_t M, int64_t N, int64_t K, double *y, int64_t ldy);

/* The same product at selected (m, n) pairs only: y[i] for (ms[i], ns[i]). */
void or_gemm_pairs(const uint8_t *ac, int64_t ldac, const uint8_t *as, int64_t ldas, float Sa,
                   const uint8_t *wc, int64_t ldwc, const uint8_t *ws, int64_t ldws, float Sw,
                   int64_t K, const int64_t *ms, const int64_t *ns, int64_t count, double *y);

/* Exact-integer version of or_gemm: each product is an integer multiple of
 * 2^-20, summed in int64; returns 0, or -1 if a partial sum would overflow. */
int or_gemm_exact(const uint8_t *ac, int64_t ldac, const uint8_t *as, int64_t ldas, float Sa,
                  const uint8_t *wc, int64_t ldwc, const uint8_t *ws, int64_t ldws, float Sw,
                  int64_t M, int64_t N, int64_t K, double *y, int64_t ldy);

/* ---- MXFP4: E2M1 codes (same packing) with one E8M0 scale byte per 32 elements
 * along K (scales [rows][K/32], value 2^(byte - 127)); no tensor scale. */
double  or_e8m0_value(int byte);
int     or_mx_block_exponent(const float *v32);
void    or_mx_quantize(const float *x, int64_t rows, int64_t K, int64_t ldx,
                       uint8_t *codes, int64_t ldc, uint8_t *scales, int64_t lds);
void    or_mx_dequantize(const uint8_t *codes, int64_t ldc, const uint8_t *scales, int64_t lds,
                         int64_t rows, int64_t K, double *out, int64_t ldo);
void    or_mx_quantize_aug(const float *x, int64_t rows, int64_t K, int64_t ldx, int64_t S_cols,
                           uint8_t *codes, int64_t ldc, uint8_t *scales, int64_t lds);
void    or_mx_gemm(const uint8_t *ac, int64_t ldac, const uint8_t *as, int64_t ldas,
                   const uint8_t *wc, int64_t ldwc, const uint8_t *ws, int64_t ldws,
                   int64_t M, int64_t N, int64_t K, double *y, int64_t ldy);

#ifdef __cplusplus
}
#endif
#endif

