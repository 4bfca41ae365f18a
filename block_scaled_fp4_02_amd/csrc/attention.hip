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
// The step is HBM-bound (one query per head: nothing to share between tokens
// but the query), so it runs on the vector units with exact products
// (e(c) d from the hardware convert, times the E4M3 value) and FP32 sums:
//   attn_scores_kernel  (chunk of 256 tokens, head): quantizes q_h (+ residue)
//                       into LDS, one token per thread streams its K row, and
//                       writes s plus the chunk's (max, sum of exp);
//   attn_pv_kernel      (chunk, head): folds the chunks' statistics into the
//                       head's (m, l), quantizes its 256 probabilities (+ residue)
//                       into LDS, one output dimension per thread streams its
//                       Vt row segment, and writes an unscaled partial o;
//   attn_combine_kernel adds the partials in chunk order and applies S_p S_V.
#include "internal.h"
#include "nvfp4_device.h"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {

constexpr int kAT = 256;                       // threads per workgroup = tokens per chunk

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
    float *scores;                             // [H][T]
    float *stats;                              // [H][NC][2]: chunk max, chunk sum of exp(s - max)
    float *partial;                            // [H][NC][D]
    float *sp;                                 // [H]: S_p of each head
    float *out; int64_t ldo;
    int NC;
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

// Quantize the 16 values of one block against S (and its residue when comp)
// and leave e(c) d (without S) of the base and of the residue in b[16], r[16].
__device__ inline void quant_block(const float *v, float S, bool comp, float *b, float *r) {
    uint32_t cw[2];
    float d;
    encode_block(v, S, 6.0f * S, cw, d);
    decode8_f32(cw[0], d, b);
    decode8_f32(cw[1], d, b + 8);
    if (!comp) {
#pragma unroll
        for (int i = 0; i < 16; ++i) r[i] = 0.0f;
        return;
    }
    float res[16];
    block_residue(v, cw, d, S, res);
    uint32_t rw[2];
    float dr;
    encode_block(res, S, 6.0f * S, rw, dr);
    decode8_f32(rw[0], dr, r);
    decode8_f32(rw[1], dr, r + 8);
}

// 32 codes (16 bytes) and their two E4M3 bytes: e(c) d of the 32 values, by pairs.
__device__ inline void decode32(const uint4 c, uint32_t s2, float *o) {
    const float d0 = e4m3_to_float(s2 & 0xFFu), d1 = e4m3_to_float((s2 >> 8) & 0xFFu);
    decode8_f32(c.x, d0, o);
    decode8_f32(c.y, d0, o + 8);
    decode8_f32(c.z, d1, o + 16);
    decode8_f32(c.w, d1, o + 24);
}

template <int XT>
__global__ __launch_bounds__(kAT) void attn_scores_kernel(AArgs a) {
    __shared__ float qb[256], qr[256], red[kAT / 64];
    const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t h = blockIdx.y;
    const int D = (int)a.D, nb = D / 16;
    // q_h and its residue, quantized as one tensor of D values: lane b < nb owns block b
    float S = 1.0f;
    if (wave == 0) {
        float v[16];
        float m = 0.0f;
        if (lane < nb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int64_t off = h * a.ldq + 16 * lane + i;
                v[i] = XT == IN_BF16 ? u2f((uint32_t)static_cast<const uint16_t *>(a.q)[off] << 16)
                                     : static_cast<const float *>(a.q)[off];
                m = fmaxf(m, fabsf(v[i]));
            }
        }
        m = warp_max(m);
        S = m > 0.0f ? m / 2688.0f : 1.0f;
        if (lane < nb) {
            float b[16], r[16];
            quant_block(v, S, a.comp != 0, b, r);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                qb[16 * lane + i] = b[i];
                qr[16 * lane + i] = r[i];
            }
        }
        if (lane == 0) red[0] = S;
    }
    __syncthreads();
    S = red[0];
    const float scale = S * a.k_S[0];
    const float inv = 1.0f / sqrtf((float)D);
    __syncthreads();                           // red[] is reused below

    // one token per thread: s = (sum q_b e d + sum q_r e d) S_q S_K / sqrt(D)
    const int64_t t = (int64_t)c * kAT + tid;
    float s = -INFINITY;
    if (t < a.T) {
        const int64_t row = h * a.T + t;
        const uint8_t *cp = a.k_codes + row * a.k_ldc;
        const uint16_t *sp = reinterpret_cast<const uint16_t *>(a.k_scales + row * a.k_lds);
        float sb = 0.0f, sr = 0.0f;
        for (int k = 0; k < D; k += 32) {
            const uint4 cw = *reinterpret_cast<const uint4 *>(cp + k / 2);
            const uint32_t s2 = sp[k / 32];
            float kd[32];
            decode32(cw, s2, kd);
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                sb += qb[k + j] * kd[j];
                sr += qr[k + j] * kd[j];
            }
        }
        s = ((sb + sr) * scale) * inv;
        a.scores[h * a.T + t] = s;
    }
    // the chunk's max and sum of exp(s - max)
    float m = warp_max(s);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float e = t < a.T ? expf(s - m) : 0.0f;
    e = warp_sum(e);
    if (lane == 0) red[wave] = e;
    __syncthreads();
    if (tid == 0) {
        float* st = a.stats + (h * a.NC + c) * 2;
        st[0] = m;
        st[1] = (red[0] + red[1]) + (red[2] + red[3]);
    }
}

__global__ __launch_bounds__(kAT) void attn_pv_kernel(AArgs a) {
    __shared__ float pb[kAT], pr[kAT], sh[2];
    const int c = blockIdx.x, tid = threadIdx.x;
    const int64_t h = blockIdx.y;
    const int64_t t0 = (int64_t)c * kAT;
    const int nt = (int)(a.T - t0 < kAT ? a.T - t0 : kAT);   // a multiple of 16
    // the head's max and normalizer from the chunks' statistics, in chunk order
    if (tid == 0) {
        const float *st = a.stats + h * a.NC * 2;
        float m = -INFINITY;
        for (int i = 0; i < a.NC; ++i) m = fmaxf(m, st[2 * i]);
        float l = 0.0f;
        for (int i = 0; i < a.NC; ++i) l += st[2 * i + 1] * expf(st[2 * i] - m);
        sh[0] = m;
        sh[1] = l;
    }
    __syncthreads();
    const float m = sh[0], l = sh[1];
    // p's tensor scale: max p = exp(0) / l
    const float pmax = 1.0f / l;
    const float Sp = pmax > 0.0f ? pmax / 2688.0f : 1.0f;
    if (c == 0 && tid == 0) a.sp[h] = Sp;
    // thread b < nt / 16 quantizes the block of tokens t0 + 16 b ..
    if (tid < nt / 16) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = expf(a.scores[h * a.T + t0 + 16 * tid + i] - m) / l;
        float b[16], r[16];
        quant_block(v, Sp, a.comp != 0, b, r);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            pb[16 * tid + i] = b[i];
            pr[16 * tid + i] = r[i];
        }
    }
    __syncthreads();
    // one output dimension per thread over the chunk's tokens (Vt row h D + j)
    if (tid < a.D) {
        const int64_t row = h * a.D + tid;
        const uint8_t *cp = a.v_codes + row * a.v_ldc + t0 / 2;
        const uint16_t *sp = reinterpret_cast<const uint16_t *>(a.v_scales + row * a.v_lds + t0 / 16);
        float ob = 0.0f, orr = 0.0f;
        int k = 0;
        for (; k + 32 <= nt; k += 32) {
            const uint4 cw = *reinterpret_cast<const uint4 *>(cp + k / 2);
            const uint32_t s2 = sp[k / 32];
            float vd[32];
            decode32(cw, s2, vd);
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                ob += pb[k + j] * vd[j];
                orr += pr[k + j] * vd[j];
            }
        }
        if (k < nt) {                          // a last block of 16 tokens
            const uint2 cw = *reinterpret_cast<const uint2 *>(cp + k / 2);
            const float d = e4m3_to_float(a.v_scales[row * a.v_lds + (t0 + k) / 16]);
            float vd[16];
            decode8_f32(cw.x, d, vd);
            decode8_f32(cw.y, d, vd + 8);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                ob += pb[k + j] * vd[j];
                orr += pr[k + j] * vd[j];
            }
        }
        a.partial[(h * a.NC + c) * a.D + tid] = ob + orr;
    }
}

// o[h][j] = (sum over chunks, in order, of the partials) S_p S_V
__global__ __launch_bounds__(256) void attn_combine_kernel(AArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= a.H * a.D) return;
    const int64_t h = idx / a.D, j = idx - h * a.D;
    float s = 0.0f;
    for (int c = 0; c < a.NC; ++c) s += a.partial[(h * a.NC + c) * a.D + j];
    a.out[h * a.ldo + j] = s * (a.sp[h] * a.v_S[0]);
}

}  // namespace

size_t attention_workspace_bytes(int64_t H, int64_t D, int64_t T) {
    const int64_t NC = (T + kAT - 1) / kAT;
    auto up = [](size_t n) { return (n + 255) / 256 * 256; };
    return up((size_t)(H * T) * 4) + up((size_t)(H * NC * 2) * 4) + up((size_t)(H * NC * D) * 4) +
           up((size_t)H * 4);
}

hipError_t launch_attention(const AttentionLaunch &g, hipStream_t st) {
    if (g.H == 0) return hipSuccess;
    AArgs a;
    a.q = g.q; a.qt = g.qt; a.ldq = g.ldq;
    a.H = g.H; a.D = g.D; a.T = g.T;
    a.k_codes = g.k_codes; a.k_ldc = g.k_ldc; a.k_scales = g.k_scales; a.k_lds = g.k_lds; a.k_S = g.k_S;
    a.v_codes = g.v_codes; a.v_ldc = g.v_ldc; a.v_scales = g.v_scales; a.v_lds = g.v_lds; a.v_S = g.v_S;
    a.comp = g.compensate;
    a.NC = (int)((g.T + kAT - 1) / kAT);
    auto up = [](size_t n) { return (n + 255) / 256 * 256; };
    uint8_t *w = static_cast<uint8_t *>(g.scratch);
    a.scores = reinterpret_cast<float *>(w);
    w += up((size_t)(g.H * g.T) * 4);
    a.stats = reinterpret_cast<float *>(w);
    w += up((size_t)(g.H * a.NC * 2) * 4);
    a.partial = reinterpret_cast<float *>(w);
    w += up((size_t)(g.H * a.NC * g.D) * 4);
    a.sp = reinterpret_cast<float *>(w);
    a.out = g.out; a.ldo = g.ldo;
    const dim3 grid((unsigned)a.NC, (unsigned)g.H);
    if (g.qt == IN_BF16) attn_scores_kernel<IN_BF16><<<grid, kAT, 0, st>>>(a);
    else attn_scores_kernel<IN_F32><<<grid, kAT, 0, st>>>(a);
    attn_pv_kernel<<<grid, kAT, 0, st>>>(a);
    const int64_t n = g.H * g.D;
    attn_combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace nvfp4
