// attention.hip -- decode attention over an NVFP4 KV cache with FP4 residue
// compensation of its activation operands, for gfx950.
//
// The ResServe abstract applies the FP4 base + FP4-quantized residue of the
// linear layers also to decode attention. Read as scaled dot-product attention
// of one decode query per head over a cache stored like a weight (K as
// [H*T, D] rows with blocks along D, V transposed as [H*D, T] rows with blocks
// along T, one tensor scale each); the two activation operands of the step --
// the query q_h and the probabilities p_h -- are quantized with their residue
// columns (each its own tensor scale), exactly as in the residue product:
//   s_h = ([Q(q_h) | Q(R_q)] . [K_h | K_h]^T) / sqrt(D)
//   p_h = softmax(s_h)            (FP32: m = max s, e = exp(s - m), p = e / sum e)
//   o_h = [Q(p_h) | Q(R_p)] . [Vt_h | Vt_h]^T
// The residue columns meet the cache's own columns again, so the cache is read
// once and the two terms are added in registers ("combined on-chip").
//
// The residue columns meet the cache's own columns again, so each cache element
// is read once and multiplies the sum of the base and residue values of its
// operand element: (e_q d_q + e_r d_r) e_k d_k, the augmented product written
// per element ("combined on-chip").
//
// The step is HBM-bound (one query per head: nothing to share between tokens
// but the query), so it runs on the vector units: e(c) from the hardware
// convert, products accumulated by FMA per 16-block and scaled once by the
// block's E4M3 value. Two launches; the softmax needs the head's max and sum
// before any probability can be quantized (its tensor scale is 1 / sum):
//   attn_scores_kernel  (256 tokens, head), four waves: wave 0 quantizes q_h
//                       (+ residue) once for the workgroup; D / 32 lanes per token
//                       stream its K row (a 16-byte slice each, the query's slice
//                       in registers); each wave writes u = exp(s - m_w) for its 64
//                       tokens and its (m_w, sum of u), m_w the max of its scores.
//   attn_pv_kernel      (16 output dimensions, head): every workgroup folds the
//                       head's statistics into (m, l) (the same fixed order
//                       everywhere), forms p = u exp(m_w - m) / l (the softmax's
//                       exp(s - m) / l taken per 64-token group: one multiply per
//                       token), quantizes the head's probabilities (+ residue) into
//                       LDS, one block of 16 per thread, and streams its 16 Vt rows
//                       (a wave reads 1 KiB of one row per load); the slices'
//                       sums meet by cross-lane adds. The workgroup covers all
//                       tokens, so no partial outputs cross workgroups.
// Every thread issues its loads in the order their data is used, all before the
// first use: loads return in order, so waiting for the first does not wait for
// the cache stream behind it.
#include "internal.h"
#include "nvfp4_device.h"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {

constexpr int kST = 256;                       // scores threads: four waves of 64 tokens
constexpr int kPR = 16;                        // Vt rows (output dimensions) per PV workgroup
constexpr int kPT = 256;                       // PV threads: 2 x 128 slices of 32 tokens
constexpr int kTT = 4096;                      // tokens per LDS tile of probabilities

struct AArgs {
    const void *q; int qt; int64_t ldq;
    int64_t H, D, T;
    const uint8_t *k_codes; int64_t k_ldc;
    const uint8_t *k_scales; int64_t k_lds;
    const float *k_S;
    const uint8_t *v_codes; int64_t v_ldc;
    const uint8_t *v_scales; int64_t v_lds;
    const float *v_S;
    int comp;
    float *scores;                             // [H][T]: u = exp(s - m_w), m_w the max of the token's wave
    float *stats;                              // [H][NW][2]: a wave's max and sum of exp(s - max)
    float *out; int64_t ldo;
    int NW;                                    // waves (64 tokens each) per head
};

__device__ inline float warp_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ inline float warp_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// e(c) d of the 8 codes of one dword (low nibble first).
__device__ inline void decode8_f32(uint32_t w, float d, float *o) {
    typedef float float2v __attribute__((ext_vector_type(2)));
    const float2v e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const float2v e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const float2v e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const float2v e3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    o[0] = e0[0] * d; o[1] = e0[1] * d; o[2] = e1[0] * d; o[3] = e1[1] * d;
    o[4] = e2[0] * d; o[5] = e2[1] * d; o[6] = e3[0] * d; o[7] = e3[1] * d;
}

// acc + sum of x[i] e(c_i) over the 8 codes of one dword, by FMA.
__device__ inline float dot8(uint32_t w, const float *x, float acc) {
    typedef float float2v __attribute__((ext_vector_type(2)));
    const float2v e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const float2v e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const float2v e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const float2v e3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    acc = __builtin_fmaf(x[0], e0[0], acc); acc = __builtin_fmaf(x[1], e0[1], acc);
    acc = __builtin_fmaf(x[2], e1[0], acc); acc = __builtin_fmaf(x[3], e1[1], acc);
    acc = __builtin_fmaf(x[4], e2[0], acc); acc = __builtin_fmaf(x[5], e2[1], acc);
    acc = __builtin_fmaf(x[6], e3[0], acc); acc = __builtin_fmaf(x[7], e3[1], acc);
    return acc;
}

// Both E4M3 bytes of s2's low half as floats, exact: the OCP FP8 convert (scale 1).
__device__ inline float2 e4m3_pair(uint32_t s2) {
    typedef float float2v __attribute__((ext_vector_type(2)));
    const float2v d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s2, 1.0f, false);
    return make_float2(d[0], d[1]);
}

// sum of x[i] e(c_i) d over 32 codes (16 bytes) and their two E4M3 bytes.
__device__ inline float dot32(const uint4 c, uint32_t s2, const float *x) {
    const float2 d = e4m3_pair(s2);
    const float a0 = dot8(c.y, x + 8, dot8(c.x, x, 0.0f));
    const float a1 = dot8(c.w, x + 24, dot8(c.z, x + 16, 0.0f));
    return a0 * d.x + a1 * d.y;
}

// Quantize the 16 values of one block against S (and its residue when comp) and
// leave, per element, e(c) d + e(c_r) d_r (without S): the base plus the residue.
__device__ inline void quant_block_aug(const float *v, float S, bool comp, float *o) {
    uint32_t cw[2];
    float d;
    encode_block(v, S, 6.0f * S, cw, d);
    decode8_f32(cw[0], d, o);
    decode8_f32(cw[1], d, o + 8);
    if (!comp) return;
    float res[16];
    block_residue(v, cw, d, S, res);
    uint32_t rw[2];
    float dr, r[16];
    encode_block(res, S, 6.0f * S, rw, dr);
    decode8_f32(rw[0], dr, r);
    decode8_f32(rw[1], dr, r + 8);
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = o[i] + r[i];
}

// The same quantization with a block spread over an aligned group of four lanes
// (quarter j = lane & 3 holds elements 4 j .. 4 j + 3): every step and rounding
// of encode_block and block_residue per element, the block's absmax by two
// cross-lane maxima (a maximum does not round).
__device__ inline void enc4(const float *v, float S, float *ed, uint32_t &w, float &d) {
    typedef float float2v __attribute__((ext_vector_type(2)));
    float ab = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    ab = fmaxf(ab, __shfl_xor(ab, 1));
    ab = fmaxf(ab, __shfl_xor(ab, 2));
    const float sf = ab / (6.0f * S);
    d = e4m3_to_float(e4m3_rne_sat(sf));
    const float sc = d * S;
    const float rcp = (sc > 0.0f) ? 1.0f / sc : 0.0f;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0] * rcp, v[1] * rcp, 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2] * rcp, v[3] * rcp, 1.0f, 1);
    const float2v e01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const float2v e23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    ed[0] = e01[0] * d; ed[1] = e01[1] * d; ed[2] = e23[0] * d; ed[3] = e23[1] * d;
}
__device__ inline void quant4_aug(const float *v, float S, bool comp, float *o) {
    uint32_t w;
    float d;
    enc4(v, S, o, w, d);
    if (!comp) return;
    float r[4], er[4], dr;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = v[i] - o[i] * S;
    enc4(r, S, er, w, dr);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = o[i] + er[i];
}

// Four waves of 64 tokens per workgroup. Wave 0 quantizes q_h (four lanes per
// block) into LDS once for the workgroup; each wave then works alone. LPT lanes
// per token (D / 32 rounded up to a power of two): lane group g holds the
// query's dimensions 32 g .. 32 g + 31 and loads that 16-byte slice of its
// token's K row, so a wave reads 64 / LPT rows (1 KiB at D = 128) per load; the
// partial dot products meet by cross-lane adds. Statistics are per wave.
template <int XT, int LPT>
__global__ __launch_bounds__(kST) void attn_scores_kernel(AArgs a) {
    __shared__ __attribute__((aligned(16))) float qa[256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t h = blockIdx.y, w = (int64_t)blockIdx.x * (kST / 64) + wave;
    const int D = (int)a.D;
    constexpr int TPW = 64 / LPT;                // tokens per load
    const int g = lane % LPT, tl = lane / LPT;
    const bool gv = 32 * g < D;
    // the query first (used first: dimensions 4 lane .. 4 lane + 3, raw words;
    // lanes past D load dimension 0 and drop it), then the K slices
    constexpr int QB = XT == IN_BF16 ? 2 : 4;   // bytes per query element
    const bool qv = 4 * lane < D;
    uint32_t qw[QB];
    {
        const uint8_t *qp = static_cast<const uint8_t *>(a.q) + (h * a.ldq + (qv ? 4 * lane : 0)) * QB;
        if (XT == IN_BF16) {
            const uint2 t = *reinterpret_cast<const uint2 *>(qp);
            qw[0] = t.x; qw[1] = t.y;
        } else {
            const uint4 t = *reinterpret_cast<const uint4 *>(qp);
            qw[0] = t.x; qw[1] = t.y; qw[2] = t.z; qw[3] = t.w;
        }
    }
    const float kS = a.k_S[0];
    uint4 cw[LPT];
    uint32_t s2[LPT];
    int64_t tok[LPT];
#pragma unroll
    for (int it = 0; it < LPT; ++it) {
        tok[it] = 64 * w + TPW * it + tl;
        const bool ok = gv && tok[it] < a.T;
        const int64_t row = h * a.T + (ok ? tok[it] : 0);
        cw[it] = *reinterpret_cast<const uint4 *>(a.k_codes + row * a.k_ldc + (ok ? 16 * g : 0));
        s2[it] = *reinterpret_cast<const uint16_t *>(a.k_scales + row * a.k_lds + (ok ? 2 * g : 0));
    }
    __builtin_amdgcn_sched_barrier(0);         // every K load is out before q is used
    // q_h quantized as one tensor of D values (its residue against the same S)
    float am;
    {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float f = XT == IN_BF16 ? u2f(i & 1 ? qw[i >> 1] & 0xFFFF0000u : qw[i >> 1] << 16) : u2f(qw[i]);
            v[i] = qv ? f : 0.0f;
        }
        am = warp_max(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
        const float S = am > 0.0f ? am / 2688.0f : 1.0f;
        if (wave == 0) {
            float o[4];
            quant4_aug(v, S, a.comp != 0, o);
            if (qv) *reinterpret_cast<float4 *>(qa + 4 * lane) = make_float4(o[0], o[1], o[2], o[3]);
        }
    }
    const float S = am > 0.0f ? am / 2688.0f : 1.0f;
    __syncthreads();
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
        const float4 t = gv ? *reinterpret_cast<const float4 *>(qa + 32 * g + i) : make_float4(0, 0, 0, 0);
        x[i] = t.x; x[i + 1] = t.y; x[i + 2] = t.z; x[i + 3] = t.w;
    }
    const float scale = S * kS;
    const float inv = 1.0f / sqrtf((float)D);
    float mx = -INFINITY;
    float sv[LPT];
#pragma unroll
    for (int it = 0; it < LPT; ++it) {
        float sum = dot32(cw[it], s2[it], x);
#pragma unroll
        for (int o = 1; o < LPT; o <<= 1) sum += __shfl_xor(sum, o);
        const float sc = (sum * scale) * inv;
        const bool ok = tok[it] < a.T;
        sv[it] = ok ? sc : -INFINITY;
        mx = fmaxf(mx, sv[it]);
    }
    // the wave's max m_w and sum of u = exp(s - m_w) (every lane of a token holds its
    // score); u is what the P.V kernel needs of a token: p = u exp(m_w - m) / l
    mx = warp_max(mx);
    float e = 0.0f;
    if (g == 0) {
#pragma unroll
        for (int it = 0; it < LPT; ++it) {
            if (tok[it] < a.T) {
                const float u = expf(sv[it] - mx);
                a.scores[h * a.T + tok[it]] = u;
                e += u;
            }
        }
    }
    e = warp_sum(e);
    if (lane == 0 && w < a.NW) *reinterpret_cast<float2 *>(a.stats + (h * a.NW + w) * 2) = make_float2(mx, e);
}

// One workgroup per 16 output dimensions of a head, over all of its tokens.
// Thread t takes slice t % 128 (32 tokens) of rows 8 (t / 128) .. + 7 per tile of
// 4096 tokens, so the lanes of a wave read 64 consecutive 16-byte slices of one
// row per load; and block t of the tile's probabilities for the quantization.
// Workgroup i takes head i % H and dimension group i / H: workgroups go to the
// eight XCDs in turn by their index, so with H a multiple of 8 all groups of a
// head share one XCD and its L2 fetches the head's scores once (not once per XCD).
__global__ __launch_bounds__(kPT) void attn_pv_kernel(AArgs a) {
    __shared__ __attribute__((aligned(16))) float pa[kTT];
    __shared__ float red[kPT / 64][8];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t h = blockIdx.x % a.H, dg = blockIdx.x / a.H;
    const int sl = tid & 127;
    const int64_t row0 = h * a.D + dg * kPR + 8 * (tid >> 7);
    const float *st = a.stats + h * a.NW * 2;
    // loads in the order of use: the statistics (entries lane + 64 k of a batch of
    // 256), then the first tile's scores block and Vt slices
    auto stats_at = [&](int i0, float2 *e) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = i0 + 64 * k + lane;
            e[k] = *reinterpret_cast<const float2 *>(st + 2 * (i < a.NW ? i : 0));
        }
    };
    float sc[16], mw;                          // the block's u values and its wave's max
    uint4 cw[8];
    uint16_t s2[8];                            // widened where used (not ahead of the tile loop)
    auto tile_loads = [&](int64_t t0, int nt) {
        const int64_t b0 = t0 + (16 * tid < nt ? 16 * tid : 0);
        const float4 *sp = reinterpret_cast<const float4 *>(a.scores + h * a.T + b0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 t = sp[i];
            sc[4 * i] = t.x; sc[4 * i + 1] = t.y; sc[4 * i + 2] = t.z; sc[4 * i + 3] = t.w;
        }
        mw = st[2 * (b0 / 64)];
        asm volatile("" ::: "memory");          // keep the scores ahead of the Vt stream
        const int64_t tf = t0 + (32 * sl + 32 <= nt ? 32 * sl : 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            cw[i] = *reinterpret_cast<const uint4 *>(a.v_codes + (row0 + i) * a.v_ldc + tf / 2);
            s2[i] = *reinterpret_cast<const uint16_t *>(a.v_scales + (row0 + i) * a.v_lds + tf / 16);
        }
    };
    // the head's max and normalizer from the waves' statistics: every wave folds
    // them in the same fixed order (lane i takes entries i, i + 64, ...). Up to 256
    // entries (T <= 16384) they stay in registers from one batch of loads issued
    // ahead of the scores and the Vt stream; beyond, a loop folds them first.
    float2 e0[4];
    stats_at(0, e0);
    const float vS = a.v_S[0];
    float m = -INFINITY, l = 0.0f;
    if (a.NW > 256) {
        float mloc = -INFINITY;
        for (int i0 = 0; i0 < a.NW; i0 += 256) {
            float2 e[4];
            stats_at(i0, e);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (i0 + 64 * k + lane < a.NW) mloc = fmaxf(mloc, e[k].x);
        }
        m = warp_max(mloc);
        float lloc = 0.0f;
        for (int i0 = 0; i0 < a.NW; i0 += 256) {
            float2 e[4];
            stats_at(i0, e);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (i0 + 64 * k + lane < a.NW) lloc += e[k].y * expf(e[k].x - m);
        }
        l = warp_sum(lloc);
    }
    asm volatile("" ::: "memory");
    tile_loads(0, (int)(a.T < kTT ? a.T : kTT));
    if (a.NW <= 256) {
        float mloc = -INFINITY;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (64 * k + lane < a.NW) mloc = fmaxf(mloc, e0[k].x);
        m = warp_max(mloc);
        float lloc = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (64 * k + lane < a.NW) lloc += e0[k].y * expf(e0[k].x - m);
        l = warp_sum(lloc);
    }
    // p's tensor scale: max p = exp(0) / l
    const float pmax = 1.0f / l;
    const float Sp = pmax > 0.0f ? pmax / 2688.0f : 1.0f;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int64_t t0 = 0; t0 < a.T; t0 += kTT) {
        const int nt = (int)(a.T - t0 < kTT ? a.T - t0 : kTT);   // a multiple of 16
        if (t0 > 0) tile_loads(t0, nt);
        // this thread's block of 16 probabilities (+ residue) into LDS
        if (16 * tid < nt) {
            // p = exp(s - m) / l, evaluated as u exp(m_w - m) / l: the factor once per block
            const float cwl = expf(mw - m) / l;
            float p[16], o[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) p[i] = sc[i] * cwl;
            quant_block_aug(p, Sp, a.comp != 0, o);
#pragma unroll
            for (int i = 0; i < 16; i += 4)
                *reinterpret_cast<float4 *>(pa + 16 * tid + i) = make_float4(o[i], o[i + 1], o[i + 2], o[i + 3]);
        }
        __syncthreads();
        if (32 * sl + 32 <= nt) {
            float x[32];
#pragma unroll
            for (int i = 0; i < 32; i += 4) {
                const float4 t = *reinterpret_cast<const float4 *>(pa + 32 * sl + i);
                x[i] = t.x; x[i + 1] = t.y; x[i + 2] = t.z; x[i + 3] = t.w;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += dot32(cw[i], s2[i], x);
        } else if (32 * sl + 16 == nt) {
            // the tile ends with half a slice: 16 tokens, one scale byte
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; i += 4) {
                const float4 t = *reinterpret_cast<const float4 *>(pa + 32 * sl + i);
                x[i] = t.x; x[i + 1] = t.y; x[i + 2] = t.z; x[i + 3] = t.w;
            }
            const int64_t hc = (t0 + 32 * sl) / 2, hs = (t0 + 32 * sl) / 16;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint2 c = *reinterpret_cast<const uint2 *>(a.v_codes + (row0 + i) * a.v_ldc + hc);
                const float d = e4m3_to_float(a.v_scales[(row0 + i) * a.v_lds + hs]);
                acc[i] += dot8(c.y, x + 8, dot8(c.x, x, 0.0f)) * d;
            }
        }
        if (t0 + kTT < a.T) __syncthreads();    // the next tile overwrites pa
    }
    // the 128 slices of each row: across the wave, then the wave pair
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = warp_sum(acc[i]);
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) red[wave][i] = acc[i];
    }
    __syncthreads();
    if (tid < kPR) {
        const int hh = tid >> 3, i = tid & 7;
        const float o = red[2 * hh][i] + red[2 * hh + 1][i];
        a.out[h * a.ldo + dg * kPR + tid] = o * (Sp * vS);
    }
}

}  // namespace

size_t attention_workspace_bytes(int64_t H, int64_t D, int64_t T) {
    (void)D;
    const int64_t NW = (T + 63) / 64;
    auto up = [](size_t n) { return (n + 255) / 256 * 256; };
    return up((size_t)(H * T) * 4) + up((size_t)(H * NW * 2) * 4);
}

hipError_t launch_attention(const AttentionLaunch &g, hipStream_t st) {
    if (g.H == 0) return hipSuccess;
    AArgs a;
    a.q = g.q; a.qt = g.qt; a.ldq = g.ldq;
    a.H = g.H; a.D = g.D; a.T = g.T;
    a.k_codes = g.k_codes; a.k_ldc = g.k_ldc; a.k_scales = g.k_scales; a.k_lds = g.k_lds; a.k_S = g.k_S;
    a.v_codes = g.v_codes; a.v_ldc = g.v_ldc; a.v_scales = g.v_scales; a.v_lds = g.v_lds; a.v_S = g.v_S;
    a.comp = g.compensate;
    a.NW = (int)((g.T + 63) / 64);
    auto up = [](size_t n) { return (n + 255) / 256 * 256; };
    uint8_t *w = static_cast<uint8_t *>(g.scratch);
    a.scores = reinterpret_cast<float *>(w);
    w += up((size_t)(g.H * g.T) * 4);
    a.stats = reinterpret_cast<float *>(w);
    a.out = g.out; a.ldo = g.ldo;
    const dim3 sgrid((unsigned)((a.NW + kST / 64 - 1) / (kST / 64)), (unsigned)g.H);
#define AS(LPT)                                                                                    \
    do {                                                                                           \
        if (g.qt == IN_BF16) attn_scores_kernel<IN_BF16, LPT><<<sgrid, kST, 0, st>>>(a);           \
        else attn_scores_kernel<IN_F32, LPT><<<sgrid, kST, 0, st>>>(a);                            \
    } while (0)
    const int64_t nd = g.D / 32;               // 32-column slices per row: 1..8
    if (nd == 1) AS(1);
    else if (nd == 2) AS(2);
    else if (nd <= 4) AS(4);
    else AS(8);
#undef AS
    attn_pv_kernel<<<dim3((unsigned)(g.D / kPR * g.H)), kPT, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace nvfp4
