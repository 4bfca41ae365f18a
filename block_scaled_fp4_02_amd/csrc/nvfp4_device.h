// nvfp4_device.h -- scalar rounding helpers and FP4 decoding for gfx950.
//
// The rounding helpers reproduce, with integer arithmetic on the float bit
// pattern, round-to-nearest-even onto the E4M3 and E2M1 grids with saturation
// (the NVFP4 element/scale formats of the ARCQuant article, section 1). They
// are __host__ __device__ so that the same source can be checked on the CPU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

__host__ __device__ inline uint32_t f2u(float f) { union { float f; uint32_t u; } c; c.f = f; return c.u; }
__host__ __device__ inline float u2f(uint32_t u) { union { float f; uint32_t u; } c; c.u = u; return c.f; }

// E4M3 byte of sf >= 0 (finite): nearest of the 127 finite non-negative values,
// ties to the even code, everything >= 448 -> 448 (0x7E).
__host__ __device__ inline uint32_t e4m3_rne_sat(float sf) {
    if (sf >= 448.0f) return 0x7Eu;
    if (sf < 0.015625f) {                     // below 2^-6: subnormal grid, step 2^-9
        return (uint32_t)rintf(sf * 512.0f);  // exact scaling; 8 becomes 2^-6 = 0x08
    }
    uint32_t u = f2u(sf);
    uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);   // round mantissa to 3 bits, ties even
    uint32_t c = (r >> 20) - (120u << 3);           // exponent bias 127 -> 7
    return c > 0x7Eu ? 0x7Eu : c;
}

// Value of a non-negative E4M3 byte (0..0x7E) as float, exact.
__host__ __device__ inline float e4m3_to_float(uint32_t b) {
    uint32_t e = (b >> 3) & 15u, m = b & 7u;
    if (e == 0) return (float)m * 0.001953125f;     // m * 2^-9
    return u2f(((e + 120u) << 23) | (m << 20));
}

// E2M1 magnitude index (0..7) of a = |q|: nearest of {0,.5,1,1.5,2,3,4,6},
// ties to the even index, everything >= 6 -> 7.
__host__ __device__ inline uint32_t e2m1_rne_sat(float a) {
    if (a >= 6.0f) return 7u;
    if (a < 1.0f) return (uint32_t)rintf(a * 2.0f);  // 0, 0.5, 1.0 -> 0, 1, 2
    uint32_t u = f2u(a);
    uint32_t r = u + 0x1FFFFFu + ((u >> 22) & 1u);   // round mantissa to 1 bit, ties even
    uint32_t c = (r >> 22) - (126u << 1);            // exponent bias 127 -> 1
    return c > 7u ? 7u : c;
}

// Value e(code) of a 4-bit code, exact.
__host__ __device__ inline float e2m1_to_float(uint32_t c) {
    uint32_t e = (c >> 1) & 3u, m = c & 1u;
    float mag = (e == 0) ? 0.5f * (float)m : u2f(((e + 126u) << 23) | (m << 22));
    return (c & 8u) ? -mag : mag;
}

// 8 packed E2M1 codes (one dword, low nibble first) times an E4M3 block scale,
// as 8 f16 values e(c) * d. The hardware convert applies only the exponent of
// its f32 scale, so it produces e * 2^8 and the multiply by the f16 whose bits
// are (byte << 7) -- the E4M3 value times 2^-8, exact in f16 -- gives e * d.
// Both factors and the product are exact in f16 (<= 6 significant bits,
// 2^-10 <= |e d| <= 2688).
__device__ inline half8 decode8(uint32_t codes, half2v dd) {
    half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 0);
    half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 1);
    half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 2);
    half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 3);
    p0 *= dd; p1 *= dd; p2 *= dd; p3 *= dd;
    half8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    return r;
}

// f16 pair (d * 2^-8, d * 2^-8) from an E4M3 byte.
__device__ inline half2v scale_pair(uint32_t b) {
    uint32_t h = (b & 0x7Fu) << 7;
    uint32_t v = h | (h << 16);
    return __builtin_bit_cast(half2v, v);
}

// Quantize one block of 16 values against tensor scale S (t = 6 S, both FP32):
// returns the E4M3 byte, fills two dwords of packed codes (low nibble first)
// and sets d to the decoded block scale. FP32 order: sf = a_b / t,
// d = E4M3(sf), s = d * S, r = 1 / s (0 when s == 0), q = x * r.
// Callers compile with contraction off so each step rounds once.
__device__ inline uint32_t encode_block(const float *v, float S, float t, uint32_t *cw, float &d) {
    float ab = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ab = fmaxf(ab, fabsf(v[i]));
    const float sf = ab / t;
    const uint32_t db = e4m3_rne_sat(sf);
    d = e4m3_to_float(db);
    const float s = d * S;
    const float rcp = (s > 0.0f) ? 1.0f / s : 0.0f;
    // q = fl(x r) rounded onto E2M1 by v_cvt_scalef32_pk_fp4_f32 with scale 1: it
    // rounds to nearest with ties to the even code, saturates at 6 and keeps the
    // sign of zero -- the same rule as e2m1_rne_sat(|q|) | signbit, checked on
    // every finite bf16 pattern, every midpoint +-3 ulp and 4 M random floats.
    // Pair p of a dword goes to byte p: element 2p low nibble, 2p+1 high nibble.
    uint32_t w0 = 0, w1 = 0;
#define NVFP4_ENC(W, P, B) W = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(W, v[2 * (P)] * rcp, v[2 * (P) + 1] * rcp, 1.0f, B)
    NVFP4_ENC(w0, 0, 0); NVFP4_ENC(w0, 1, 1); NVFP4_ENC(w0, 2, 2); NVFP4_ENC(w0, 3, 3);
    NVFP4_ENC(w1, 4, 0); NVFP4_ENC(w1, 5, 1); NVFP4_ENC(w1, 6, 2); NVFP4_ENC(w1, 7, 3);
#undef NVFP4_ENC
    cw[0] = w0; cw[1] = w1;
    return db;
}

// Residue of a block: R = x - fl(fl(e d) S) for the 16 values and their codes.
// e(c) comes from v_cvt_scalef32_pk_f32_fp4 with scale 1 (exact).
__device__ inline void block_residue(const float *v, const uint32_t *cw, float d, float S, float *r) {
    typedef float float2v __attribute__((ext_vector_type(2)));
    float2v e[8];
    e[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[0], 1.0f, 0);
    e[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[0], 1.0f, 1);
    e[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[0], 1.0f, 2);
    e[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[0], 1.0f, 3);
    e[4] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[1], 1.0f, 0);
    e[5] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[1], 1.0f, 1);
    e[6] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[1], 1.0f, 2);
    e[7] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[1], 1.0f, 3);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float ed = e[i >> 1][i & 1] * d;
        const float deq = ed * S;
        r[i] = v[i] - deq;
    }
}

// 16 consecutive elements (bf16 when is_bf16, else f32) starting at element off.
__device__ inline void load16_any(const void *base, bool is_bf16, int64_t off, float *v) {
    if (is_bf16) {
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + off);
        const uint4 a = p[0], b = p[1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = u2f(w[i] << 16);
            v[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
        }
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 q = p[i];
            v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
        }
    }
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = f2u(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

}  // namespace nvfp4
