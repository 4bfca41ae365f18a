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
//   attn_scores_kernel  (chunk of 256 tokens, head): quantizes q_h (+ residue),
//                       D / 32 lanes per token stream its K row (a slice each,
//                       the query's slice in registers), and it writes s plus
//                       the chunk's (max, sum of exp);
//   attn_pv_kernel      (chunk, head): folds the chunks' statistics into the
//                       head's (m, l), quantizes its 256 probabilities (+ residue)
//                       into LDS, one output dimension per thread streams its
//                       Vt row segment and stores an unscaled partial o; the last
//                       workgroup of the head (a counter in the workspace header)
//                       adds the partials in chunk order and applies S_p S_V.
// Every thread issues all of its loads before it uses any (a loop with a load per
// step waited for each round trip in turn: 8.5 and 14.3 us per kernel).
#include "internal.h"
#include "nvfp4_device.h"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {

constexpr int kAT = 256;                       // threads per workgroup = tokens per chunk

template <typename T>
__device__ inline void st_dev(T *p, T v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <typename T>
__device__ inline T ld_dev(const T *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <typename T>
__device__ inline T add_dev(T *p, T v) { return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline void wait_own_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
    float *out; int64_t ldo;
    unsigned *cnt;                             // [H] arrival counters (workspace header), zero-kept
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

// LPT lanes per token (D / 32 rounded up to a power of two): lane group g holds
// the query's dimensions 32 g .. 32 g + 31 (base and residue, in registers) and
// loads that 16-byte slice of its token's K row, so LPT lanes read a row and a
// wave reads 64 / LPT rows (1 KiB at D = 128) per load; the partial dot products
// meet by cross-lane adds.
template <int XT, int LPT>
__global__ __launch_bounds__(kAT) void attn_scores_kernel(AArgs a) {
    __shared__ __attribute__((aligned(16))) float qb[256], qr[256];
    __shared__ float red[kAT / 64];
    const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t h = blockIdx.y;
    const int D = (int)a.D, nb = D / 16;
    constexpr int TPW = 64 / LPT;                // tokens per wave and load
    const int g = lane % LPT, tl = lane / LPT;
    const bool gv = 32 * g < D;
    // this lane's K slices of its LPT tokens, all loads first
    uint4 cw[LPT];
    uint32_t s2[LPT];
    int64_t tok[LPT];
#pragma unroll
    for (int it = 0; it < LPT; ++it) {
        tok[it] = (int64_t)c * kAT + 64 * wave + TPW * it + tl;
        const bool ok = gv && tok[it] < a.T;
        const int64_t row = h * a.T + (ok ? tok[it] : 0);
        cw[it] = *reinterpret_cast<const uint4 *>(a.k_codes + row * a.k_ldc + (ok ? 16 * g : 0));
        s2[it] = *reinterpret_cast<const uint16_t *>(a.k_scales + row * a.k_lds + (ok ? 2 * g : 0));
    }
    // q_h and its residue, quantized as one tensor of D values: lane b < nb of wave 0
    // owns block b
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
        const float S = m > 0.0f ? m / 2688.0f : 1.0f;
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
    const float scale = red[0] * a.k_S[0];
    const float inv = 1.0f / sqrtf((float)D);
    float q_b[32], q_r[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        q_b[i] = gv ? qb[32 * g + i] : 0.0f;
        q_r[i] = gv ? qr[32 * g + i] : 0.0f;
    }
    __syncthreads();                           // red[] is reused below

    float mx = -INFINITY;
    float sv[LPT];
#pragma unroll
    for (int it = 0; it < LPT; ++it) {
        float kd[32];
        decode32(cw[it], s2[it], kd);
        float sb = 0.0f, sr = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            sb += q_b[j] * kd[j];
            sr += q_r[j] * kd[j];
        }
        float sum = sb + sr;
#pragma unroll
        for (int o = 1; o < LPT; o <<= 1) sum += __shfl_xor(sum, o);
        const float sc = (sum * scale) * inv;
        const bool ok = tok[it] < a.T;
        if (ok && g == 0) a.scores[h * a.T + tok[it]] = sc;
        sv[it] = ok ? sc : -INFINITY;
        mx = fmaxf(mx, sv[it]);
    }
    // the chunk's max and sum of exp(s - max) (every lane of a token holds its score)
    mx = warp_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float e = 0.0f;
    if (g == 0) {
#pragma unroll
        for (int it = 0; it < LPT; ++it) e += tok[it] < a.T ? expf(sv[it] - m) : 0.0f;
    }
    e = warp_sum(e);
    if (lane == 0) red[wave] = e;
    __syncthreads();
    if (tid == 0) {
        float *st = a.stats + (h * a.NC + c) * 2;
        st[0] = m;
        st[1] = (red[0] + red[1]) + (red[2] + red[3]);
    }
}

__global__ __launch_bounds__(kAT) void attn_pv_kernel(AArgs a) {
    __shared__ float pb[kAT], pr[kAT], pv[kAT], sh[2];
    __shared__ int sh_last;
    const int c = blockIdx.x, tid = threadIdx.x;
    const int64_t h = blockIdx.y;
    const int64_t t0 = (int64_t)c * kAT;
    const int nt = (int)(a.T - t0 < kAT ? a.T - t0 : kAT);   // a multiple of 16
    // this thread's Vt row segment (dimension tid of head h), all loads first
    constexpr int NG = kAT / 32;
    const bool has_row = tid < a.D;
    const int64_t row = h * a.D + (has_row ? tid : 0);
    const uint8_t *cp = a.v_codes + row * a.v_ldc + t0 / 2;
    const uint16_t *sp2 = reinterpret_cast<const uint16_t *>(a.v_scales + row * a.v_lds + t0 / 16);
    uint4 cw[NG];
    uint32_t s2[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const bool ok = 32 * i + 32 <= nt;     // a whole group of 32 tokens (else its start, unused)
        cw[i] = *reinterpret_cast<const uint4 *>(cp + (ok ? 16 * i : 0));
        s2[i] = sp2[ok ? i : 0];
    }
    const float s_own = tid < nt ? a.scores[h * a.T + t0 + tid] : 0.0f;   // this thread's token
    const int g16 = nt & ~31;                  // a last block of 16 tokens starts here when nt % 32 == 16
    const uint2 tw = *reinterpret_cast<const uint2 *>(cp + (nt & 16 ? g16 / 2 : 0));
    const uint32_t ts = a.v_scales[row * a.v_lds + (t0 + (nt & 16 ? g16 : 0)) / 16];
    // the head's max and normalizer from the chunks' statistics: wave 0's lanes take
    // the chunks (the same fixed reduction in every workgroup of the head)
    if (tid < 64) {
        const float *st = a.stats + h * a.NC * 2;
        float mloc = -INFINITY;
        for (int i = tid; i < a.NC; i += 64) mloc = fmaxf(mloc, st[2 * i]);
        const float mh = warp_max(mloc);
        float lloc = 0.0f;
        for (int i = tid; i < a.NC; i += 64) lloc += st[2 * i + 1] * expf(st[2 * i] - mh);
        const float lh = warp_sum(lloc);
        if (tid == 0) {
            sh[0] = mh;
            sh[1] = lh;
        }
    }
    __syncthreads();
    const float m = sh[0], l = sh[1];
    // p's tensor scale: max p = exp(0) / l
    const float pmax = 1.0f / l;
    const float Sp = pmax > 0.0f ? pmax / 2688.0f : 1.0f;
    // every thread its token's probability, then thread b < nt / 16 quantizes the
    // block of tokens t0 + 16 b ..
    if (tid < nt) pv[tid] = expf(s_own - m) / l;
    __syncthreads();
    if (tid < nt / 16) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = pv[16 * tid + i];
        float b[16], r[16];
        quant_block(v, Sp, a.comp != 0, b, r);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            pb[16 * tid + i] = b[i];
            pr[16 * tid + i] = r[i];
        }
    }
    __syncthreads();
    // one output dimension per thread over the chunk's tokens
    float* part = a.partial + (h * a.NC + c) * a.D;
    if (has_row) {
        float ob = 0.0f, orr = 0.0f;
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            if (32 * i + 32 <= nt) {
                float vd[32];
                decode32(cw[i], s2[i], vd);
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    ob += pb[32 * i + j] * vd[j];
                    orr += pr[32 * i + j] * vd[j];
                }
            }
        }
        if (nt & 16) {
            const float d = e4m3_to_float(ts);
            float vd[16];
            decode8_f32(tw.x, d, vd);
            decode8_f32(tw.y, d, vd + 8);
            for (int j = 0; j < 16; ++j) {
                ob += pb[g16 + j] * vd[j];
                orr += pr[g16 + j] * vd[j];
            }
        }
        st_dev(part + tid, ob + orr);
    }
    // the last workgroup of the head adds the partials in chunk order (device-scope
    // stores, acknowledged before the arrival; device-scope loads after it)
    wait_own_stores();
    __syncthreads();
    if (tid == 0) sh_last = add_dev(&a.cnt[h], 1u) == (unsigned)a.NC - 1;
    __syncthreads();
    if (sh_last && has_row) {
        // sixteen device-scope loads in flight at a time, added in chunk order
        const float *src = a.partial + h * a.NC * a.D + tid;
        float s = 0.0f;
        for (int i0 = 0; i0 < a.NC; i0 += 16) {
            float v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) v[k] = i0 + k < a.NC ? ld_dev(src + (int64_t)(i0 + k) * a.D) : 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k)
                if (i0 + k < a.NC) s += v[k];
        }
        a.out[h * a.ldo + tid] = s * (Sp * a.v_S[0]);
    }
    if (sh_last && tid == 0) st_dev(&a.cnt[h], 0u);
}

}  // namespace

size_t attention_workspace_bytes(int64_t H, int64_t D, int64_t T) {
    const int64_t NC = (T + kAT - 1) / kAT;
    auto up = [](size_t n) { return (n + 255) / 256 * 256; };
    return up((size_t)(H * T) * 4) + up((size_t)(H * NC * 2) * 4) + up((size_t)(H * NC * D) * 4);
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
    a.out = g.out; a.ldo = g.ldo;
    a.cnt = g.counters;
    const dim3 grid((unsigned)a.NC, (unsigned)g.H);
#define AS(LPT)                                                                                    \
    do {                                                                                           \
        if (g.qt == IN_BF16) attn_scores_kernel<IN_BF16, LPT><<<grid, kAT, 0, st>>>(a);            \
        else attn_scores_kernel<IN_F32, LPT><<<grid, kAT, 0, st>>>(a);                             \
    } while (0)
    const int64_t nd = g.D / 32;               // 32-column slices per row: 1..8
    if (nd == 1) AS(1);
    else if (nd == 2) AS(2);
    else if (nd <= 4) AS(4);
    else AS(8);
#undef AS
    attn_pv_kernel<<<grid, kAT, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace nvfp4
