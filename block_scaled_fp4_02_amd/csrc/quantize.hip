// quantize.hip -- NVFP4 quantizer kernels for gfx950.
//
// Steps of the fused quantizer (ARCQuant article on zizhi168.cn, section 3.2:
// channel reorder, RMSNorm, main quantization and residual quantization in one
// kernel; ResServe abstract: FP4 base plus FP4-quantized residue):
//   amax pass    per-tensor |x| maximum (of the RMSNorm output when normalizing),
//                as one partial maximum per workgroup -- no atomics, so the
//                result does not depend on scheduling;
//   quant pass   every workgroup folds the partials into S, then quantizes
//                16-element blocks (two lanes per block without a reorder, one
//                thread per block group with it): block absmax, E4M3 block
//                scale, E2M1 codes, nibble packing, and the residue
//                R = x - fl(fl(e d) S) of columns below res_cols, quantized
//                against the same S and stored after column K_in;
//   one launch   decode-sized activations (the small quantizer) and mid-size
//                ones up to 16 M elements (the grid quantizer) keep X in
//                registers across one grid-wide arrival for amax(X) instead.
// All rounding follows the FP32 order of nvfp4.h; contraction into FMA is off
// so every product and difference rounds exactly once.
#include <algorithm>

#include "internal.h"
#include "nvfp4_device.h"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;

__device__ inline float bf16f(uint32_t h) { return u2f(h << 16); }

// 16 consecutive elements of a bf16 or f32 array as loaded (32 or 64 bytes).
template <int XT>
struct Raw16 {
    uint4 q[XT == IN_BF16 ? 2 : 4];
};

template <int XT>
__device__ inline void load_raw16(const void *base, int64_t off, Raw16<XT> &r) {
    const uint4 *p = XT == IN_BF16 ? reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + off)
                                   : reinterpret_cast<const uint4 *>(static_cast<const float *>(base) + off);
#pragma unroll
    for (int i = 0; i < (XT == IN_BF16 ? 2 : 4); ++i) r.q[i] = p[i];
}

template <int XT>
__device__ inline void raw16_to_f32(const Raw16<XT> &r, float *v) {
    if constexpr (XT == IN_BF16) {
        const uint32_t w[8] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w, r.q[1].x, r.q[1].y, r.q[1].z, r.q[1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = u2f(w[i] << 16);
            v[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[4 * i] = u2f(r.q[i].x); v[4 * i + 1] = u2f(r.q[i].y);
            v[4 * i + 2] = u2f(r.q[i].z); v[4 * i + 3] = u2f(r.q[i].w);
        }
    }
}

// 16 consecutive elements starting at element `off` of a bf16 or f32 array.
template <int XT>
__device__ inline void load16(const void *base, int64_t off, float *v) {
    Raw16<XT> r;
    load_raw16<XT>(base, off, r);
    raw16_to_f32<XT>(r, v);
}

__device__ inline void gamma16(const uint16_t *g, int64_t off, float *v) {
    const uint4 *p = reinterpret_cast<const uint4 *>(g + off);
    uint4 a = p[0], b = p[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = u2f(w[i] << 16);
        v[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
    }
}

// Diagonal smoothing (OSFP4 abstract: one diagonal matrix per linear projection,
// multiplied into the activation at run time; its inverse lives in the weight):
// v[i] *= s[off + i] for 16 consecutive input channels, one FP32 rounding each.
__device__ inline void smooth16(const float *s, int64_t off, float *v) {
    const float4 *p = reinterpret_cast<const float4 *>(s + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 q = p[i];
        v[4 * i] = v[4 * i] * q.x; v[4 * i + 1] = v[4 * i + 1] * q.y;
        v[4 * i + 2] = v[4 * i + 2] * q.z; v[4 * i + 3] = v[4 * i + 3] * q.w;
    }
}

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ inline double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Maximum over the workgroup (kThreads threads); result valid in every thread.
__device__ inline float block_max(float v, float *sh) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) sh[w] = v;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, sh[i]);
    return r;
}

__device__ inline double block_sum_d(double v, double *sh) {
    v = wave_sum_d(v);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) sh[w] = v;
    __syncthreads();
    double r = sh[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r += sh[i];
    return r;
}

// ---------------------------------------------------------------- amax pass

template <int XT>
__global__ __launch_bounds__(kThreads) void amax_plain_kernel(const void *x, int64_t rows, int64_t K,
                                                             int64_t ldx, const float *smooth, float *partials) {
    __shared__ float sh[kThreads / 64];
    const int64_t nb = K / 16, total = rows * nb;
    float m = 0.0f;
    for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < total;
         c += (int64_t)gridDim.x * kThreads) {
        const int64_t r = c / nb, b = c - r * nb;
        float v[16];
        load16<XT>(x, r * ldx + 16 * b, v);
        if (smooth) smooth16(smooth, 16 * b, v);
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
    }
    m = block_max(m, sh);
    if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// Row-parallel pass for RMSNorm: r = fl32(1 / sqrt(sum(x^2)/K + eps)) with the
// sum in FP64, then max |fl(fl(x r) gamma)| over the row.
template <int XT>
__device__ inline float row_rms_scale(const void *x, int64_t row, int64_t K, int64_t ldx, float eps,
                                      double *shd) {
    double ss = 0.0;
    for (int64_t b = threadIdx.x; b < K / 16; b += kThreads) {
        float v[16];
        load16<XT>(x, row * ldx + 16 * b, v);
#pragma unroll
        for (int i = 0; i < 16; ++i) ss += (double)v[i] * (double)v[i];
    }
    ss = block_sum_d(ss, shd);
    return (float)(1.0 / sqrt(ss / (double)K + (double)eps));
}

template <int XT>
__global__ __launch_bounds__(kThreads) void amax_rmsnorm_kernel(const void *x, int64_t rows, int64_t K,
                                                               int64_t ldx, const uint16_t *gamma,
                                                               float eps, const float *smooth, float *rscale,
                                                               float *partials) {
    __shared__ float sh[kThreads / 64];
    __shared__ double shd[kThreads / 64];
    float m = 0.0f;
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const float r = row_rms_scale<XT>(x, row, K, ldx, eps, shd);
        if (threadIdx.x == 0) rscale[row] = r;
        for (int64_t b = threadIdx.x; b < K / 16; b += kThreads) {
            float v[16], g[16];
            load16<XT>(x, row * ldx + 16 * b, v);
            gamma16(gamma, 16 * b, g);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float y = v[i] * r;
                v[i] = y * g[i];
            }
            if (smooth) smooth16(smooth, 16 * b, v);
#pragma unroll
            for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
        }
    }
    m = block_max(m, sh);
    if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// -------------------------------------------------------------- quant pass

struct QArgs {
    const void *x; int64_t rows, K_in, ldx;
    const uint16_t *gamma;
    const int32_t *perm;
    int64_t res_cols;
    const float *static_S;
    uint8_t *codes; int64_t ldc;
    uint8_t *scales; int64_t lds;
    float *S_out;
    const float *partials; int npart;
    const float *rscale;
    float eps;
    const float *smooth;                      // per input channel, or nullptr
};

__device__ inline float tensor_scale(const QArgs &a, float *sh) {
    if (a.static_S) return *a.static_S;
    float m = 0.0f;
    for (int i = threadIdx.x; i < a.npart; i += kThreads) m = fmaxf(m, a.partials[i]);
    m = block_max(m, sh);
    return m > 0.0f ? m / 2688.0f : 1.0f;
}

// Quantize `nb` (1..4) blocks of row `row` starting at column col0 from v[64].
__device__ inline void process_group(const QArgs &a, const float *v, int nb, int64_t row, int64_t col0,
                                     float S, float t) {
    uint32_t cw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t sw = 0;
    float dblk[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        if (b < nb) {
            const uint32_t db = encode_block(v + 16 * b, S, t, cw + 2 * b, dblk[b]);
            sw |= db << (8 * b);
        }
    }
    uint8_t *cp = a.codes + row * a.ldc + col0 / 2;
    uint8_t *sp = a.scales + row * a.lds + col0 / 16;
    if (nb == 4) {
        reinterpret_cast<uint4 *>(cp)[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
        reinterpret_cast<uint4 *>(cp)[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
        *reinterpret_cast<uint32_t *>(sp) = sw;
    } else {
        for (int b = 0; b < nb; ++b) {
            reinterpret_cast<uint2 *>(cp)[b] = make_uint2(cw[2 * b], cw[2 * b + 1]);
            sp[b] = (uint8_t)(sw >> (8 * b));
        }
    }
    if (col0 >= a.res_cols) return;
    // residue R = x - fl(fl(e d) S) on the columns below res_cols
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        if (b < nb && col0 + 16 * b < a.res_cols) {
            float rv[16];
            block_residue(v + 16 * b, cw + 2 * b, dblk[b], S, rv);
            uint32_t rc[2];
            float dr;
            const uint32_t rdb = encode_block(rv, S, t, rc, dr);
            const int64_t col = a.K_in + col0 + 16 * b;
            *reinterpret_cast<uint2 *>(a.codes + row * a.ldc + col / 2) = make_uint2(rc[0], rc[1]);
            a.scales[row * a.lds + col / 16] = (uint8_t)rdb;
        }
    }
}

// ------------------------------------------ large activations, lane pairs
// The flat quantizer (no reorder): two lanes per 16-element block, each loading
// 8 consecutive elements, so a wave's load is 1 KiB contiguous (32 blocks). The
// two lanes exchange their half maxima, then each encodes its own 8 codes (one
// dword) with the block's E4M3 scale -- the same FP32 steps as encode_block --
// and the even lane stores the scale byte. Grid-stride over blocks with two
// blocks per lane pair in flight.

template <int XT>
__device__ inline void load8(const void *base, int64_t off, float *v) {
    if constexpr (XT == IN_BF16) {
        const uint4 a = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + off);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = u2f(w[i] << 16);
            v[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
        }
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + off);
        const float4 q0 = p[0], q1 = p[1];
        v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w;
        v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
    }
}

__device__ inline void gamma8(const uint16_t *g, int64_t off, float *v) {
    const uint4 a = *reinterpret_cast<const uint4 *>(g + off);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = u2f(w[i] << 16);
        v[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
    }
}

__device__ inline void smooth8(const float *s, int64_t off, float *v) {
    const float4 *p = reinterpret_cast<const float4 *>(s + off);
    const float4 q0 = p[0], q1 = p[1];
    v[0] = v[0] * q0.x; v[1] = v[1] * q0.y; v[2] = v[2] * q0.z; v[3] = v[3] * q0.w;
    v[4] = v[4] * q1.x; v[5] = v[5] * q1.y; v[6] = v[6] * q1.z; v[7] = v[7] * q1.w;
}

// This lane's half of a block (the partner lane, lane ^ 1, holds the other half):
// returns the block's E4M3 byte, the 8 codes in cw (low nibble first) and d.
__device__ inline uint32_t encode_half(const float *v, float S, float t, uint32_t &cw, float &d) {
    float ab = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ab = fmaxf(ab, fabsf(v[i]));
    ab = fmaxf(ab, __shfl_xor(ab, 1));
    const float sf = ab / t;
    const uint32_t db = e4m3_rne_sat(sf);
    d = e4m3_to_float(db);
    const float s = d * S;
    const float rcp = (s > 0.0f) ? 1.0f / s : 0.0f;
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0] * rcp, v[1] * rcp, 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2] * rcp, v[3] * rcp, 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4] * rcp, v[5] * rcp, 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6] * rcp, v[7] * rcp, 1.0f, 3);
    cw = w;
    return db;
}

// Residue of this lane's half: R = x - fl(fl(e d) S), as block_residue.
__device__ inline void residue_half(const float *v, uint32_t cw, float d, float S, float *r) {
    typedef float float2v __attribute__((ext_vector_type(2)));
    float2v e[4];
    e[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0);
    e[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1);
    e[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2);
    e[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float ed = e[i >> 1][i & 1] * d;
        const float deq = ed * S;
        r[i] = v[i] - deq;
    }
}

template <int XT, bool NORM>
__global__ __launch_bounds__(kThreads) void quantize_pairs_kernel(QArgs a) {
    __shared__ float sh[kThreads / 64];
    const float S = tensor_scale(a, sh);
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.S_out = S;
    const float t = 6.0f * S;
    const int h = threadIdx.x & 1;
    const int64_t nb = a.K_in / 16, total = a.rows * nb;
    const int64_t stride = (int64_t)gridDim.x * (kThreads / 2);
    // block p of the flattened (row, block) order: load, RMSNorm / smoothing, encode, store
    auto where = [&](int64_t p, int64_t &row, int64_t &b) {
        row = p / nb;
        b = p - row * nb;
    };
    auto prep = [&](int64_t row, int64_t col, float *v) {
        if (NORM) {
            const float r = a.rscale[row];
            float g[8];
            gamma8(a.gamma, col, g);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float y = v[i] * r;
                v[i] = y * g[i];
            }
        }
        if (a.smooth) smooth8(a.smooth, col, v);
    };
    auto emit = [&](int64_t row, int64_t b, const float *v) {
        const int64_t col = 16 * b + 8 * h;
        uint32_t cw;
        float d;
        const uint32_t db = encode_half(v, S, t, cw, d);
        *reinterpret_cast<uint32_t *>(a.codes + row * a.ldc + col / 2) = cw;
        if (h == 0) a.scales[row * a.lds + b] = (uint8_t)db;
        if (16 * b < a.res_cols) {                 // the same for both lanes of the pair
            float rv[8];
            residue_half(v, cw, d, S, rv);
            uint32_t rc;
            float dr;
            const uint32_t rdb = encode_half(rv, S, t, rc, dr);
            const int64_t rcol = a.K_in + col;
            *reinterpret_cast<uint32_t *>(a.codes + row * a.ldc + rcol / 2) = rc;
            if (h == 0) a.scales[row * a.lds + rcol / 16] = (uint8_t)rdb;
        }
    };
    for (int64_t p = (int64_t)blockIdx.x * (kThreads / 2) + (threadIdx.x >> 1); p < total; p += 2 * stride) {
        const int64_t p1 = p + stride;
        const bool two = p1 < total;               // the same for both lanes of the pair
        int64_t r0, b0, r1 = 0, b1 = 0;
        where(p, r0, b0);
        float v0[8], v1[8];
        load8<XT>(a.x, r0 * a.ldx + 16 * b0 + 8 * h, v0);
        if (two) {
            where(p1, r1, b1);
            load8<XT>(a.x, r1 * a.ldx + 16 * b1 + 8 * h, v1);
        }
        prep(r0, 16 * b0 + 8 * h, v0);
        emit(r0, b0, v0);
        if (two) {
            prep(r1, 16 * b1 + 8 * h, v1);
            emit(r1, b1, v1);
        }
    }
}

// ------------------------------------------------- small activations, one launch
// Decode-sized activations (rows <= 32, no RMSNorm or reorder) in one launch of
// G <= 64 workgroups, a thread per 16-element block (up to kSmallPer each):
// partial maxima, one grid-wide arrival, then each workgroup encodes its blocks
// from registers.
//
// The arrival uses no read-modify-write (atomics on one word from many
// workgroups serialize in the memory system and cost microseconds): 64 slots
// of 8 bytes, each (partial maximum | epoch << 32). Between calls every slot
// holds the same epoch; workgroup b reads its own slot's epoch e at start,
// writes (partial, e + 1) into the slots l = b mod G, and waits until all 64
// slots carry e + 1, so the 64 partials it then holds are those of this call
// (slots l >= G repeat a real partial). The wait is bounded; a workgroup whose
// wait gives up recomputes amax(X) itself (same result), and it has still
// written its slots, so the epochs stay in step.
constexpr int kSmallPer = 2;                   // blocks per thread: 2 keeps the kernel's code small
                                               // (it alternates with the decode kernel in a call, and
                                               // 4 cost ~4 us per 15-call sweep in code fetches)
constexpr int kSmallMaxG = 64;
constexpr int64_t kRowsMaxK = 16384;           // row kernel: the row (f32) in LDS

template <typename T>
__device__ inline void st_dev(T *p, T v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <typename T>
__device__ inline T ld_dev(const T *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// The epoch half (the high 32 bits) of this workgroup's own slot as the call
// finds it, read by every thread at the start of the kernel, before the data.
// Nothing is computed from it until the arrival: arithmetic on a load inside a
// branch makes the compiler wait for that load there, and so does a 64-bit
// load whose unused half the register allocator hands out again; either way
// the data loads would start one memory round trip later.
__device__ inline unsigned slot_word(const unsigned long long *slot) {
    return ld_dev(reinterpret_cast<const unsigned *>(&slot[blockIdx.x]) + 1);
}

// This call's epoch: one past the one the slot carries.
__device__ inline unsigned slot_epoch(unsigned word) { return word + 1u; }

// Arrival of workgroup blockIdx.x < G <= 64 with partial m (after block_max:
// the same in every thread); `word` is slot_word() from the start of the
// kernel. Wave 0 writes the slots and waits; the grid maximum is returned in
// every thread, and *sh_ok says whether the wait completed (0: it gave up
// after `spin` polls, the caller recomputes).
__device__ inline float slot_max(unsigned long long *slot, int G, unsigned word, float m, unsigned spin,
                                 float *sh, int *sh_ok) {
    if (threadIdx.x < 64) {                    // wave 0: lane l owns slot l
        const int l = threadIdx.x;
        const unsigned ep = slot_epoch(word);
        if (l % G == (int)blockIdx.x) st_dev(&slot[l], (unsigned long long)ep << 32 | __float_as_uint(m));
        unsigned long long sv = ld_dev(&slot[l]);
        unsigned it = 0;
        int ok = 1;
        while (!__all((unsigned)(sv >> 32) == ep)) {
            if (++it > spin) { ok = 0; break; }
            __builtin_amdgcn_s_sleep(2);
            sv = ld_dev(&slot[l]);
        }
        const float pm = wave_max(__uint_as_float((unsigned)sv));
        if (l == 0) { *sh_ok = ok; sh[0] = pm; }
    }
    __syncthreads();
    return sh[0];
}

template <int XT>
__global__ __launch_bounds__(kThreads) void quantize_small_kernel(QArgs a, unsigned long long *slot, int G,
                                                                   unsigned spin) {
    __shared__ float sh[kThreads / 64];
    __shared__ int sh_ok;
    // NB <= kSmallMaxG * kThreads * kSmallPer blocks: block indices fit 32 bits
    const uint32_t KB = (uint32_t)(a.K_in / 16), NB = (uint32_t)a.rows * KB;
    const uint32_t b0 = blockIdx.x * NB / G, b1 = (blockIdx.x + 1) * NB / G;
    const bool arrive = !a.static_S && G > 1;
    const unsigned word = slot_word(slot);   // in flight beside the data loads
    // every block's load is issued before any is used (one memory round trip);
    // the raw words are converted after the branches, which then hold no use of them
    Raw16<XT> raw[kSmallPer];
#pragma unroll
    for (int t = 0; t < kSmallPer; ++t) {
        const uint32_t b = b0 + threadIdx.x + kThreads * t;
        if (b < b1) {
            const uint32_t row = b / KB, blk = b - row * KB;
            load_raw16<XT>(a.x, row * a.ldx + 16 * (int64_t)blk, raw[t]);
        } else {
#pragma unroll
            for (auto &q : raw[t].q) q = make_uint4(0, 0, 0, 0);
        }
    }
    float v[kSmallPer][16];
    float m = 0.0f;
#pragma unroll
    for (int t = 0; t < kSmallPer; ++t) {
        raw16_to_f32<XT>(raw[t], v[t]);
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[t][i]));
    }
    float S;
    if (a.static_S) {
        S = *a.static_S;
    } else {
        m = block_max(m, sh);
        if (arrive) {
            m = slot_max(slot, G, word, m, spin, sh, &sh_ok);   // the same in every thread
            if (!sh_ok) {
                float mm = 0.0f;                     // the wait gave up: all of X here
                for (uint32_t b = threadIdx.x; b < NB; b += kThreads) {
                    const uint32_t row = b / KB, blk = b - row * KB;
                    float w[16];
                    load16<XT>(a.x, row * a.ldx + 16 * (int64_t)blk, w);
#pragma unroll
                    for (int i = 0; i < 16; ++i) mm = fmaxf(mm, fabsf(w[i]));
                }
                m = block_max(mm, sh);
            }
        }
        S = m > 0.0f ? m / 2688.0f : 1.0f;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.S_out = S;
    const float t6 = 6.0f * S;
#pragma unroll
    for (int t = 0; t < kSmallPer; ++t) {
        const uint32_t b = b0 + threadIdx.x + kThreads * t;
        if (b < b1) {
            const int64_t row = b / KB, blk = b - row * KB;
            uint32_t cw[2];
            float d;
            const uint32_t db = encode_block(v[t], S, t6, cw, d);
            *reinterpret_cast<uint2 *>(a.codes + row * a.ldc + 8 * blk) = make_uint2(cw[0], cw[1]);
            a.scales[row * a.lds + blk] = (uint8_t)db;
            if (16 * blk < a.res_cols) {
                float rv[16];
                block_residue(v[t], cw, d, S, rv);
                uint32_t rc[2];
                float dr;
                const uint32_t rdb = encode_block(rv, S, t6, rc, dr);
                *reinterpret_cast<uint2 *>(a.codes + row * a.ldc + a.K_in / 2 + 8 * blk) = make_uint2(rc[0], rc[1]);
                a.scales[row * a.lds + KB + blk] = (uint8_t)rdb;
            }
        }
    }
}

// ------------------------------------------- mid-size activations, one launch
// Activations of up to kGridMaxG * kGridThreads * kGridPer 16-element blocks (16 M
// elements; bf16, no RMSNorm, reorder
// or smoothing; the smaller prefill activations) in one launch of G <= kGridMaxG
// workgroups of kGridThreads threads, at most one per CU, so that all of them are
// resident: each thread keeps its (up to kGridPer) blocks in registers as loaded,
// the workgroups' partial maxima meet in a grid-wide arrival on kGridMaxG slots
// (the small quantizer's epoch scheme, four slots per lane of wave 0), and every
// block is then encoded from its registers. X is read once, where the two-pass
// path reads it twice and launches twice. A workgroup whose wait gives up
// recomputes amax(X) from memory (same result), having written its slots, so
// the epochs stay in step.
constexpr int kGridThreads = 1024;
constexpr int kGridPer = 4;
constexpr int kGridMaxG = 256;
static_assert(kGridSlotsOffset + 8 * kGridMaxG <= kTileCntOffset, "grid slots overlap the tile counters");

__device__ inline float block_max_grid(float v, float *sh) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) sh[w] = v;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int i = 1; i < kGridThreads / 64; ++i) r = fmaxf(r, sh[i]);
    return r;
}

// Arrival of workgroup blockIdx.x < G <= kGridMaxG with partial m (the same in
// every thread): lane l of wave 0 owns slots l + 64 j; slot s carries the partial
// of workgroup s mod G.
__device__ inline float slot_max_grid(unsigned long long *slot, int G, unsigned word, float m,
                                      unsigned spin, float *sh, int *sh_ok) {
    if (threadIdx.x < 64) {
        const int l = threadIdx.x;
        const unsigned ep = slot_epoch(word);
        const unsigned long long mine = (unsigned long long)ep << 32 | __float_as_uint(m);
        unsigned long long sv[kGridMaxG / 64];
#pragma unroll
        for (int j = 0; j < kGridMaxG / 64; ++j)
            if ((l + 64 * j) % G == (int)blockIdx.x) st_dev(&slot[l + 64 * j], mine);
#pragma unroll
        for (int j = 0; j < kGridMaxG / 64; ++j) sv[j] = ld_dev(&slot[l + 64 * j]);
        auto arrived = [&]() {
            bool in = true;
#pragma unroll
            for (int j = 0; j < kGridMaxG / 64; ++j) in = in && (unsigned)(sv[j] >> 32) == ep;
            return __all(in);
        };
        unsigned it = 0;
        int ok = 1;
        while (!arrived()) {
            if (++it > spin) { ok = 0; break; }
            __builtin_amdgcn_s_sleep(2);
#pragma unroll
            for (int j = 0; j < kGridMaxG / 64; ++j) sv[j] = ld_dev(&slot[l + 64 * j]);
        }
        float pm = 0.0f;
#pragma unroll
        for (int j = 0; j < kGridMaxG / 64; ++j) pm = fmaxf(pm, __uint_as_float((unsigned)sv[j]));
        pm = wave_max(pm);
        if (l == 0) { *sh_ok = ok; sh[0] = pm; }
    }
    __syncthreads();
    return sh[0];
}

__global__ __launch_bounds__(kGridThreads) void quantize_grid_kernel(QArgs a, unsigned long long *slot, int G,
                                                                     unsigned spin) {
    __shared__ float sh[kGridThreads / 64];
    __shared__ int sh_ok;
    const uint32_t KB = (uint32_t)(a.K_in / 16);
    const int64_t NB = a.rows * (int64_t)KB;
    const int64_t b0 = (int64_t)blockIdx.x * NB / G, b1 = ((int64_t)blockIdx.x + 1) * NB / G;
    const bool arrive = !a.static_S && G > 1;
    const unsigned word = slot_word(slot);   // in flight beside the data loads
    // block b = b0 + tid + kGridThreads t of this thread: 16 bf16 (two 16-byte words each)
    uint4 raw[kGridPer][2];
#pragma unroll
    for (int t = 0; t < kGridPer; ++t) {
        const int64_t b = b0 + threadIdx.x + (int64_t)kGridThreads * t;
        if (b < b1) {
            const uint32_t row = (uint32_t)(b / KB), blk = (uint32_t)(b - (int64_t)row * KB);
            const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + row * a.ldx + 16 * (int64_t)blk);
            raw[t][0] = p[0];
            raw[t][1] = p[1];
        } else {
            raw[t][0] = make_uint4(0, 0, 0, 0);
            raw[t][1] = make_uint4(0, 0, 0, 0);
        }
    }
    // for finite values the order of |bf16| bit patterns is that of the magnitudes
    auto to_f32 = [](const uint4 *q, float *v) {
        const uint32_t w[8] = {q[0].x, q[0].y, q[0].z, q[0].w, q[1].x, q[1].y, q[1].z, q[1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = u2f(w[i] << 16);
            v[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
        }
    };
    float S;
    if (a.static_S) {
        S = *a.static_S;
    } else {
        float m = 0.0f;
#pragma unroll
        for (int t = 0; t < kGridPer; ++t) {
            float v[16];
            to_f32(raw[t], v);
#pragma unroll
            for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
        }
        m = block_max_grid(m, sh);
        if (arrive) {
            m = slot_max_grid(slot, G, word, m, spin, sh, &sh_ok);   // the same in every thread
            if (!sh_ok) {
                float mm = 0.0f;                     // the wait gave up: all of X here
                for (int64_t b = threadIdx.x; b < NB; b += kGridThreads) {
                    const uint32_t row = (uint32_t)(b / KB), blk = (uint32_t)(b - (int64_t)row * KB);
                    float w[16];
                    load16<IN_BF16>(a.x, row * a.ldx + 16 * (int64_t)blk, w);
#pragma unroll
                    for (int i = 0; i < 16; ++i) mm = fmaxf(mm, fabsf(w[i]));
                }
                m = block_max_grid(mm, sh);
            }
        }
        S = m > 0.0f ? m / 2688.0f : 1.0f;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.S_out = S;
    const float t6 = 6.0f * S;
#pragma unroll
    for (int t = 0; t < kGridPer; ++t) {
        const int64_t b = b0 + threadIdx.x + (int64_t)kGridThreads * t;
        if (b < b1) {
            const uint32_t row = (uint32_t)(b / KB), blk = (uint32_t)(b - (int64_t)row * KB);
            float v[16];
            to_f32(raw[t], v);
            uint32_t cw[2];
            float d;
            const uint32_t db = encode_block(v, S, t6, cw, d);
            *reinterpret_cast<uint2 *>(a.codes + row * a.ldc + 8 * (int64_t)blk) = make_uint2(cw[0], cw[1]);
            a.scales[row * a.lds + blk] = (uint8_t)db;
            if (16 * (int64_t)blk < a.res_cols) {
                float rv[16];
                block_residue(v, cw, d, S, rv);
                uint32_t rc[2];
                float dr;
                const uint32_t rdb = encode_block(rv, S, t6, rc, dr);
                *reinterpret_cast<uint2 *>(a.codes + row * a.ldc + a.K_in / 2 + 8 * (int64_t)blk) = make_uint2(rc[0], rc[1]);
                a.scales[row * a.lds + KB + blk] = (uint8_t)rdb;
            }
        }
    }
}

// ------------------------------------------- few rows with RMSNorm / reorder
// Rows <= 64 with RMSNorm and/or the calibration reorder, in one launch of one
// workgroup per row: the row, normalized, goes to LDS (the FP64 sum of squares
// in the order of row_rms_scale), its maximum meets the other rows' in the slot
// arrival, then each thread gathers a 16-column block through perm and encodes
// it (and its residue block below res_cols). A workgroup whose wait gives up
// recomputes every row's maximum itself (same values, same result).
// Column c sits at rowbuf[(c % 16) KB + c / 16]: a thread's 16 columns are 16
// rows of that table, so the lanes of a wave touch consecutive words.
template <int XT, bool NORM, bool PERM>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(QArgs a, unsigned long long *slot, unsigned spin) {
    extern __shared__ float rowbuf[];
    __shared__ float sh[kThreads / 64];
    __shared__ double shd[kThreads / 64];
    __shared__ int sh_ok;
    const int G = (int)gridDim.x;
    const int64_t row = blockIdx.x, K = a.K_in, KB = K / 16;
    const bool arrive = !a.static_S && G > 1;
    const unsigned word = slot_word(slot);   // in flight beside the data loads
    double ss = 0.0;
    float m = 0.0f;
    for (int64_t b = threadIdx.x; b < KB; b += kThreads) {
        float v[16];
        load16<XT>(a.x, row * a.ldx + 16 * b, v);
        if (NORM) {
#pragma unroll
            for (int i = 0; i < 16; ++i) ss += (double)v[i] * (double)v[i];
        } else if (a.smooth) {
            smooth16(a.smooth, 16 * b, v);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (!NORM) m = fmaxf(m, fabsf(v[i]));
            rowbuf[i * KB + b] = v[i];
        }
    }
    if (NORM) {
        ss = block_sum_d(ss, shd);
        const float r = (float)(1.0 / sqrt(ss / (double)K + (double)a.eps));
        for (int64_t b = threadIdx.x; b < KB; b += kThreads) {
            float g[16], y[16];
            gamma16(a.gamma, 16 * b, g);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float t = rowbuf[i * KB + b] * r;
                y[i] = t * g[i];
            }
            if (a.smooth) smooth16(a.smooth, 16 * b, y);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                rowbuf[i * KB + b] = y[i];
                m = fmaxf(m, fabsf(y[i]));
            }
        }
    }
    m = block_max(m, sh);                      // also: the row is complete in LDS
    float S;
    if (a.static_S) {
        S = *a.static_S;
    } else {
        if (arrive) {
            float mm = slot_max(slot, G, word, m, spin, sh, &sh_ok);
            if (!sh_ok) {                      // the wait gave up: every row here
                mm = 0.0f;
                for (int64_t rr = 0; rr < a.rows; ++rr) {
                    float rs = 1.0f;
                    if (NORM) rs = row_rms_scale<XT>(a.x, rr, K, a.ldx, a.eps, shd);
                    for (int64_t b = threadIdx.x; b < KB; b += kThreads) {
                        float v[16], g[16];
                        load16<XT>(a.x, rr * a.ldx + 16 * b, v);
                        if (NORM) {
                            gamma16(a.gamma, 16 * b, g);
#pragma unroll
                            for (int i = 0; i < 16; ++i) { const float t = v[i] * rs; v[i] = t * g[i]; }
                        }
                        if (a.smooth) smooth16(a.smooth, 16 * b, v);
#pragma unroll
                        for (int i = 0; i < 16; ++i) mm = fmaxf(mm, fabsf(v[i]));
                    }
                }
            }
            m = block_max(mm, sh);
        }
        S = m > 0.0f ? m / 2688.0f : 1.0f;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.S_out = S;
    const float t = 6.0f * S;
    for (int64_t b = threadIdx.x; b < KB; b += kThreads) {
        float v[16];
        if (PERM) {
            const int4 *pp = reinterpret_cast<const int4 *>(a.perm + 16 * b);
            const int4 p4[4] = {pp[0], pp[1], pp[2], pp[3]};
            const int32_t pi[16] = {p4[0].x, p4[0].y, p4[0].z, p4[0].w, p4[1].x, p4[1].y, p4[1].z, p4[1].w,
                                    p4[2].x, p4[2].y, p4[2].z, p4[2].w, p4[3].x, p4[3].y, p4[3].z, p4[3].w};
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                // indices outside [0, K) are clamped so a bad permutation cannot leave the row
                const int32_t c = pi[i] < 0 ? 0 : (pi[i] >= K ? (int32_t)(K - 1) : pi[i]);
                v[i] = rowbuf[(c & 15) * KB + (c >> 4)];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = rowbuf[i * KB + b];
        }
        process_group(a, v, 1, row, 16 * b, S, t);
    }
}

// Channel-gather variant: one workgroup per row stages the (normalized) row in
// LDS, then each thread gathers its 64 columns through perm.
template <int XT, bool NORM>
__global__ __launch_bounds__(kThreads) void quantize_perm_kernel(QArgs a) {
    extern __shared__ float rowbuf[];
    __shared__ float sh[kThreads / 64];
    const float S = tensor_scale(a, sh);
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.S_out = S;
    const float t = 6.0f * S;
    const int64_t ng = (a.K_in + 63) / 64;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const float r = NORM ? a.rscale[row] : 1.0f;
        for (int64_t b = threadIdx.x; b < a.K_in / 16; b += kThreads) {
            float v[16];
            load16<XT>(a.x, row * a.ldx + 16 * b, v);
            if (NORM) {
                float gm[16];
                gamma16(a.gamma, 16 * b, gm);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float y = v[i] * r;
                    v[i] = y * gm[i];
                }
            }
            if (a.smooth) smooth16(a.smooth, 16 * b, v);
#pragma unroll
            for (int i = 0; i < 16; ++i) rowbuf[16 * b + i] = v[i];
        }
        __syncthreads();
        for (int64_t gi = threadIdx.x; gi < ng; gi += kThreads) {
            const int64_t col0 = 64 * gi, rem = a.K_in - col0;
            const int nb = rem >= 64 ? 4 : (int)(rem / 16);
            float v[64];
#pragma unroll
            for (int i = 0; i < 64; ++i) {
                // indices outside [0, K_in) are clamped so a bad permutation cannot leave the row
                int32_t pi = (i < 16 * nb) ? a.perm[col0 + i] : 0;
                pi = pi < 0 ? 0 : (pi >= a.K_in ? (int32_t)(a.K_in - 1) : pi);
                v[i] = (i < 16 * nb) ? rowbuf[pi] : 0.0f;
            }
            process_group(a, v, nb, row, col0, S, t);
        }
        __syncthreads();
    }
}

// ------------------------------------------------------ calibration absmax

template <int XT>
__global__ __launch_bounds__(kThreads) void rms_scale_kernel(const void *x, int64_t rows, int64_t K,
                                                            int64_t ldx, float eps, float *rscale) {
    __shared__ double shd[kThreads / 64];
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const float r = row_rms_scale<XT>(x, row, K, ldx, eps, shd);
        if (threadIdx.x == 0) rscale[row] = r;
    }
}

// Column maxima: thread per group of 16 columns, loop over all rows.
template <int XT, bool NORM>
__global__ __launch_bounds__(kThreads) void channel_absmax_kernel(const void *x, int64_t rows, int64_t K,
                                                                 int64_t ldx, const uint16_t *gamma,
                                                                 const float *rscale, float *out) {
    const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (b >= K / 16) return;
    float m[16], g[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) { m[i] = 0.0f; g[i] = 1.0f; }
    if (NORM) gamma16(gamma, 16 * b, g);
    for (int64_t row = 0; row < rows; ++row) {
        float v[16];
        load16<XT>(x, row * ldx + 16 * b, v);
        const float r = NORM ? rscale[row] : 1.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float y = v[i];
            if (NORM) { y = y * r; y = y * g[i]; }
            m[i] = fmaxf(m[i], fabsf(y));
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) out[16 * b + i] = m[i];
}

int amax_grid(int64_t rows, int64_t K) {
    const int64_t chunks = rows * (K / 16);
    int64_t g = (chunks + kThreads * 4 - 1) / (kThreads * 4);
    if (g < 1) g = 1;
    if (g > kAmaxPartials) g = kAmaxPartials;
    return (int)g;
}

}  // namespace

// CUs of the current device (the grid quantizer launches at most one workgroup per CU).
static int grid_cus() {
    static int cus = 0;
    if (cus <= 0) {
        int dev = 0, c = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
            cus = c;
        else
            return 1;
    }
    return cus;
}

// A row staged in LDS takes K_in floats (up to 64 KiB): above 48 KiB of
// dynamic LDS the kernel's limit is raised first (gfx950 has 160 KiB per CU).
static hipError_t allow_lds(const void *fn, size_t lds) {
    if (lds <= 48 * 1024) return hipSuccess;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

hipError_t launch_quantize(const QuantLaunch &q, hipStream_t st) {
    const bool norm = q.gamma != nullptr, perm = q.perm != nullptr, smooth = q.smooth != nullptr;
    const int64_t nb = q.rows * (q.K_in / 16);
    if ((norm || perm || smooth) && q.slots && q.rows >= 1 && q.rows <= kSmallMaxG && q.K_in > 0 && q.K_in <= kRowsMaxK) {
        QArgs a;
        a.x = q.x; a.rows = q.rows; a.K_in = q.K_in; a.ldx = q.ldx;
        a.gamma = q.gamma; a.perm = q.perm; a.res_cols = q.res_cols; a.static_S = q.static_S;
        a.codes = q.codes; a.ldc = q.ldc; a.scales = q.scales; a.lds = q.lds; a.S_out = q.S_out;
        a.partials = q.partials; a.npart = 0; a.rscale = q.rscale; a.eps = q.eps; a.smooth = q.smooth;
        const size_t lds = (size_t)q.K_in * sizeof(float);
        const int g = (int)q.rows;
#define QR(XT, NM, PM)                                                                              \
    do {                                                                                            \
        const hipError_t e_ = allow_lds(reinterpret_cast<const void *>(&quantize_rows_kernel<XT, NM, PM>), lds); \
        if (e_ != hipSuccess) return e_;                                                            \
        quantize_rows_kernel<XT, NM, PM><<<g, kThreads, lds, st>>>(a, q.slots, q.spin);             \
    } while (0)
        if (q.xt == IN_BF16) {
            if (norm && perm) QR(IN_BF16, true, true); else if (norm) QR(IN_BF16, true, false);
            else if (perm) QR(IN_BF16, false, true); else QR(IN_BF16, false, false);
        } else {
            if (norm && perm) QR(IN_F32, true, true); else if (norm) QR(IN_F32, true, false);
            else if (perm) QR(IN_F32, false, true); else QR(IN_F32, false, false);
        }
#undef QR
        return hipGetLastError();
    }
    if (!norm && !perm && !smooth && q.slots && q.rows <= 32 && nb > 0 && nb <= (int64_t)kSmallMaxG * kThreads * kSmallPer) {
        int G = (int)((nb + kThreads - 1) / kThreads);
        if (G > kSmallMaxG) G = kSmallMaxG;
        QArgs a;
        a.x = q.x; a.rows = q.rows; a.K_in = q.K_in; a.ldx = q.ldx;
        a.gamma = nullptr; a.perm = nullptr; a.res_cols = q.res_cols; a.static_S = q.static_S;
        a.codes = q.codes; a.ldc = q.ldc; a.scales = q.scales; a.lds = q.lds; a.S_out = q.S_out;
        a.partials = q.partials; a.npart = 0; a.rscale = q.rscale; a.eps = q.eps; a.smooth = nullptr;
        if (q.xt == IN_BF16)
            quantize_small_kernel<IN_BF16><<<G, kThreads, 0, st>>>(a, q.slots, G, q.spin);
        else
            quantize_small_kernel<IN_F32><<<G, kThreads, 0, st>>>(a, q.slots, G, q.spin);
        return hipGetLastError();
    }
    if (!norm && !perm && !smooth && q.grid_slots && q.xt == IN_BF16 && nb > 0) {
        const int cus = grid_cus();
        const int64_t G = std::min<int64_t>(std::min<int64_t>(kGridMaxG, cus), (nb + kGridThreads - 1) / kGridThreads);
        if (G >= 1 && nb <= G * kGridThreads * kGridPer) {
            QArgs a;
            a.x = q.x; a.rows = q.rows; a.K_in = q.K_in; a.ldx = q.ldx;
            a.gamma = nullptr; a.perm = nullptr; a.res_cols = q.res_cols; a.static_S = q.static_S;
            a.codes = q.codes; a.ldc = q.ldc; a.scales = q.scales; a.lds = q.lds; a.S_out = q.S_out;
            a.partials = q.partials; a.npart = 0; a.rscale = q.rscale; a.eps = q.eps; a.smooth = nullptr;
            quantize_grid_kernel<<<(int)G, kGridThreads, 0, st>>>(a, q.grid_slots, (int)G, q.spin);
            return hipGetLastError();
        }
    }
    int npart = 0;
    if (!q.static_S) {
        if (norm) {
            npart = (int)(q.rows < kAmaxPartials ? q.rows : kAmaxPartials);
            if (npart < 1) npart = 1;
            if (q.xt == IN_BF16)
                amax_rmsnorm_kernel<IN_BF16><<<npart, kThreads, 0, st>>>(q.x, q.rows, q.K_in, q.ldx, q.gamma, q.eps, q.smooth, q.rscale, q.partials);
            else
                amax_rmsnorm_kernel<IN_F32><<<npart, kThreads, 0, st>>>(q.x, q.rows, q.K_in, q.ldx, q.gamma, q.eps, q.smooth, q.rscale, q.partials);
        } else {
            npart = amax_grid(q.rows, q.K_in);
            if (q.xt == IN_BF16)
                amax_plain_kernel<IN_BF16><<<npart, kThreads, 0, st>>>(q.x, q.rows, q.K_in, q.ldx, q.smooth, q.partials);
            else
                amax_plain_kernel<IN_F32><<<npart, kThreads, 0, st>>>(q.x, q.rows, q.K_in, q.ldx, q.smooth, q.partials);
        }
    } else if (norm) {
        const int g = (int)(q.rows < 4096 ? (q.rows > 0 ? q.rows : 1) : 4096);
        if (q.xt == IN_BF16)
            rms_scale_kernel<IN_BF16><<<g, kThreads, 0, st>>>(q.x, q.rows, q.K_in, q.ldx, q.eps, q.rscale);
        else
            rms_scale_kernel<IN_F32><<<g, kThreads, 0, st>>>(q.x, q.rows, q.K_in, q.ldx, q.eps, q.rscale);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    QArgs a;
    a.x = q.x; a.rows = q.rows; a.K_in = q.K_in; a.ldx = q.ldx;
    a.gamma = q.gamma; a.perm = q.perm; a.res_cols = q.res_cols; a.static_S = q.static_S;
    a.codes = q.codes; a.ldc = q.ldc; a.scales = q.scales; a.lds = q.lds; a.S_out = q.S_out;
    a.partials = q.partials; a.npart = npart; a.rscale = q.rscale; a.eps = q.eps; a.smooth = q.smooth;

    if (perm) {
        const int g = (int)(q.rows < 2048 ? (q.rows > 0 ? q.rows : 1) : 2048);
        const size_t lds = (size_t)q.K_in * sizeof(float);
#define QP(XT, NM)                                                                                  \
    do {                                                                                            \
        const hipError_t e_ = allow_lds(reinterpret_cast<const void *>(&quantize_perm_kernel<XT, NM>), lds); \
        if (e_ != hipSuccess) return e_;                                                            \
        quantize_perm_kernel<XT, NM><<<g, kThreads, lds, st>>>(a);                                  \
    } while (0)
        if (q.xt == IN_BF16) { if (norm) QP(IN_BF16, true); else QP(IN_BF16, false); }
        else { if (norm) QP(IN_F32, true); else QP(IN_F32, false); }
#undef QP
    } else {
        // two lanes per block, two blocks per lane pair in flight; up to 8 workgroups per CU
        const int64_t blocks = q.rows * (q.K_in / 16);
        int64_t g = (blocks + kThreads - 1) / kThreads;
        if (g > 2048) g = 2048;
        if (g < 1) g = 1;
#define QF(XT, NM) quantize_pairs_kernel<XT, NM><<<(int)g, kThreads, 0, st>>>(a)
        if (q.xt == IN_BF16) { if (norm) QF(IN_BF16, true); else QF(IN_BF16, false); }
        else { if (norm) QF(IN_F32, true); else QF(IN_F32, false); }
#undef QF
    }
    return hipGetLastError();
}

hipError_t launch_channel_absmax(const ChannelAbsmaxLaunch &c, hipStream_t st) {
    const bool norm = c.gamma != nullptr;
    if (norm) {
        const int g = (int)(c.rows < 4096 ? (c.rows > 0 ? c.rows : 1) : 4096);
        if (c.xt == IN_BF16)
            rms_scale_kernel<IN_BF16><<<g, kThreads, 0, st>>>(c.x, c.rows, c.K, c.ldx, c.eps, c.rscale);
        else
            rms_scale_kernel<IN_F32><<<g, kThreads, 0, st>>>(c.x, c.rows, c.K, c.ldx, c.eps, c.rscale);
    }
    const int g = (int)((c.K / 16 + kThreads - 1) / kThreads);
#define CA(XT, NM) channel_absmax_kernel<XT, NM><<<g > 0 ? g : 1, kThreads, 0, st>>>(c.x, c.rows, c.K, c.ldx, c.gamma, c.rscale, c.out)
    if (c.xt == IN_BF16) { if (norm) CA(IN_BF16, true); else CA(IN_BF16, false); }
    else { if (norm) CA(IN_F32, true); else CA(IN_F32, false); }
#undef CA
    return hipGetLastError();
}

}  // namespace nvfp4
