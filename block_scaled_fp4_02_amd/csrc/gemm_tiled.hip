// gemm_tiled.hip -- tiled W4A4 product for large M (prefill) on gfx950 matrix cores.
//
// Only here is the product a dense contraction, so only here is it tiled for
// MFMA. NVFP4's 16-element E4M3 block scales do not map onto CDNA4's scaled
// FP4 MFMA (E8M0 scales per 32 elements), and e(c)*d needs up to 6 significant
// bits, so each 16-element block is decoded to exact f16 e*d values in LDS and
// multiplied with v_mfma_f32_16x16x32_f16 (FP32 accumulation). The epilogue
// applies S_a S_w once and stores FP32 or BF16 (one write, no second pass).
//
// Residue columns (ARCQuant article, sections 3.1-3.2: one GEMM over K+S whose
// weight tail repeats the weight's first S columns) are handled by decoding the
// residue activation tile of the same K step and issuing a second set of MFMAs
// against the already-decoded weight tile, so the weights are read once.
//
// Tile: BM x BN output per workgroup of 4 waves (2 x 2), BK = 64 per step,
// LDS double-buffered; tiles are stored in MFMA operand order (each operand
// fetch is 1 KB contiguous per wave).
#include <type_traits>

#include "internal.h"
#include "lds_dma.h"
#include "nvfp4_device.h"

namespace nvfp4 {
namespace {

constexpr int BK = 64;

struct TArgs {
    const uint8_t *a_codes; int64_t a_ldc;
    const uint8_t *a_scales; int64_t a_lds;
    const float *a_S;
    const uint8_t *w_codes; int64_t w_ldc;
    const uint8_t *w_scales; int64_t w_lds;
    const float *w_S;
    int w_tiled;
    int64_t M, N, K, res_cols;
    void *y; int yt; int64_t ldy;
    int tiles_m, tiles_n;
    // split-K (tiled2 only): range p = blockIdx.y of P, kchunk k-steps each;
    // part != nullptr: unscaled fp32 partial tiles to part[p][M][N] instead of y
    int P; int64_t kchunk; float *part;
};

__device__ inline uint16_t f2bf(float f) {
    uint32_t u = f2u(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// 32 consecutive k of one row (codes + the two block scales), zero beyond kend.
struct RowChunk { uint4 c; uint32_t s; };

__device__ inline RowChunk load_chunk(const uint8_t *codes, int64_t ldc, const uint8_t *scales, int64_t lds,
                                      int64_t row, int64_t nrows, int64_t k, int64_t kend) {
    RowChunk rc;
    rc.c = make_uint4(0, 0, 0, 0);
    rc.s = 0;
    if (row < nrows) {
        const uint8_t *cp = codes + row * ldc + k / 2;
        const uint8_t *sp = scales + row * lds + k / 16;
        if (k + 32 <= kend) {
            rc.c = *reinterpret_cast<const uint4 *>(cp);
            rc.s = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
        } else if (k + 16 <= kend) {
            const uint2 h = *reinterpret_cast<const uint2 *>(cp);
            rc.c.x = h.x; rc.c.y = h.y;
            rc.s = sp[0];
        }
    }
    return rc;
}

// The same chunk of a tiled weight (16 x 512 items in decode lane order: the
// 32 columns at k of row n are lane 16 g + r, step i of item (n / 16, k / 512)).
__device__ inline RowChunk load_chunk_tiled(const uint8_t *codes, int64_t ldc, const uint8_t *scales, int64_t lds,
                                            int64_t row, int64_t nrows, int64_t k, int64_t kend) {
    RowChunk rc;
    rc.c = make_uint4(0, 0, 0, 0);
    rc.s = 0;
    if (row < nrows && k < kend) {                // tiled padding is zero: no half-chunk case
        const int64_t t = row >> 4, u = k >> 9;
        const int lane = (int)(16 * ((k >> 7) & 3) + (row & 15)), i = (int)((k >> 5) & 3);
        rc.c = *reinterpret_cast<const uint4 *>(codes + t * ldc + u * 4096 + 1024 * i + 16 * lane);
        const uint8_t *sp = scales + t * lds + u * 512 + 8 * lane + 2 * i;
        rc.s = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
    }
    return rc;
}

// Decode a chunk into 4 fragments (8 k each) and store them at LDS slots
// base + 16 q (q = 0..3): the lane (r16 + 16 q) of k-chunk `base`.
__device__ inline void store_chunk(half8 *lds, int slot, const RowChunk &rc) {
    const half2v d0 = scale_pair(rc.s & 0xFFu), d1 = scale_pair((rc.s >> 8) & 0xFFu);
    lds[slot + 0] = decode8(rc.c.x, d0);
    lds[slot + 16] = decode8(rc.c.y, d0);
    lds[slot + 32] = decode8(rc.c.z, d1);
    lds[slot + 48] = decode8(rc.c.w, d1);
}

template <int BM, int BN, bool RES>
__global__ __launch_bounds__(256) void tiled_kernel(TArgs a) {
    constexpr int RT = BM / 16, CT = BN / 16;               // 16-row tiles per operand
    constexpr int A_SLOTS = RT * 2 * 64, B_SLOTS = CT * 2 * 64;
    constexpr int STAGE = A_SLOTS * (RES ? 2 : 1) + B_SLOTS;
    constexpr int WRT = RT / 2, WCT = CT / 2;               // per-wave tiles (2 x 2 waves)
    extern __shared__ half8 lds[];                           // [2][STAGE]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // XCD-aware order: consecutive blocks go to different XCDs; regroup so that
    // blocks sharing a weight tile column land on the same XCD.
    const int nblk = a.tiles_m * a.tiles_n;
    int bid = blockIdx.x;
    if (nblk % 8 == 0) bid = (bid % 8) * (nblk / 8) + bid / 8;
    const int tn = bid / a.tiles_m, tm = bid % a.tiles_m;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    const int64_t ksteps = (a.K + BK - 1) / BK;
    const int64_t rsteps = RES ? (a.res_cols + BK - 1) / BK : 0;

    // loader mapping: thread -> (row, half) ; BM/BN rows x 2 halves
    constexpr int A_ITERS = (BM * 2 + 255) / 256, B_ITERS = (BN * 2 + 255) / 256;
    RowChunk ra[A_ITERS], rr[RES ? A_ITERS : 1], rb[B_ITERS];

    auto gload = [&](int64_t s) {
        const int64_t k = s * BK;
#pragma unroll
        for (int it = 0; it < A_ITERS; ++it) {
            const int idx = tid + 256 * it;
            const int r = idx >> 1, h = idx & 1;
            if (r < BM) {
                ra[it] = load_chunk(a.a_codes, a.a_ldc, a.a_scales, a.a_lds, m0 + r, a.M, k + 32 * h, a.K);
                if (RES) {
                    if (s < rsteps) {
                        RowChunk t = load_chunk(a.a_codes, a.a_ldc, a.a_scales, a.a_lds, m0 + r, a.M,
                                                a.K + k + 32 * h, a.K + a.res_cols);
                        rr[it] = t;
                    } else {
                        rr[it].c = make_uint4(0, 0, 0, 0); rr[it].s = 0;
                    }
                }
            }
        }
#pragma unroll
        for (int it = 0; it < B_ITERS; ++it) {
            const int idx = tid + 256 * it;
            const int r = idx >> 1, h = idx & 1;
            if (r < BN)
                rb[it] = a.w_tiled ? load_chunk_tiled(a.w_codes, a.w_ldc, a.w_scales, a.w_lds, n0 + r, a.N, k + 32 * h, a.K)
                                   : load_chunk(a.w_codes, a.w_ldc, a.w_scales, a.w_lds, n0 + r, a.N, k + 32 * h, a.K);
        }
    };
    auto lstore = [&](half8 *st) {
#pragma unroll
        for (int it = 0; it < A_ITERS; ++it) {
            const int idx = tid + 256 * it;
            const int r = idx >> 1, h = idx & 1;
            if (r < BM) {
                const int slot = ((r >> 4) * 2 + h) * 64 + (r & 15);
                store_chunk(st, slot, ra[it]);
                if (RES) store_chunk(st + A_SLOTS + B_SLOTS, slot, rr[it]);
            }
        }
#pragma unroll
        for (int it = 0; it < B_ITERS; ++it) {
            const int idx = tid + 256 * it;
            const int r = idx >> 1, h = idx & 1;
            if (r < BN) store_chunk(st + A_SLOTS, ((r >> 4) * 2 + h) * 64 + (r & 15), rb[it]);
        }
    };

    float4v acc[WRT][WCT];
#pragma unroll
    for (int i = 0; i < WRT; ++i)
#pragma unroll
        for (int j = 0; j < WCT; ++j) acc[i][j] = float4v{0, 0, 0, 0};

    gload(0);
    lstore(lds);
    __syncthreads();
    for (int64_t s = 0; s < ksteps; ++s) {
        half8 *cur = lds + (s & 1) * STAGE;
        half8 *nxt = lds + ((s + 1) & 1) * STAGE;
        if (s + 1 < ksteps) gload(s + 1);
        const bool res_step = RES && s < rsteps;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            half8 bf[WCT];
#pragma unroll
            for (int j = 0; j < WCT; ++j) bf[j] = cur[A_SLOTS + ((wn * WCT + j) * 2 + kc) * 64 + lane];
#pragma unroll
            for (int i = 0; i < WRT; ++i) {
                const half8 af = cur[((wm * WRT + i) * 2 + kc) * 64 + lane];
#pragma unroll
                for (int j = 0; j < WCT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[j], acc[i][j], 0, 0, 0);
            }
            if (res_step) {
#pragma unroll
                for (int i = 0; i < WRT; ++i) {
                    const half8 af = cur[A_SLOTS + B_SLOTS + ((wm * WRT + i) * 2 + kc) * 64 + lane];
#pragma unroll
                    for (int j = 0; j < WCT; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[j], acc[i][j], 0, 0, 0);
                }
            }
        }
        if (s + 1 < ksteps) lstore(nxt);
        __syncthreads();
    }

    const float scale = a.a_S[0] * a.w_S[0];
    const int g = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int i = 0; i < WRT; ++i) {
#pragma unroll
        for (int j = 0; j < WCT; ++j) {
            const int64_t n = n0 + (wn * WCT + j) * 16 + c16;
            if (n >= a.N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + (wm * WRT + i) * 16 + 4 * g + e;
                if (m < a.M) {
                    const float v = acc[i][j][e] * scale;
                    if (a.yt == 1) static_cast<float *>(a.y)[m * a.ldy + n] = v;
                    else static_cast<uint16_t *>(a.y)[m * a.ldy + n] = f2bf(v);
                }
            }
        }
    }
}

// Chunk loads for the large-tile product: the scale pair is one 2-byte load
// (k is a multiple of 32, so the pair is 2-byte aligned in both layouts).
__device__ inline RowChunk load_chunk2(const uint8_t *codes, int64_t ldc, const uint8_t *scales, int64_t lds,
                                       int64_t row, int64_t nrows, int64_t k, int64_t kend) {
    RowChunk rc;
    rc.c = make_uint4(0, 0, 0, 0);
    rc.s = 0;
    if (row < nrows) {
        const uint8_t *cp = codes + row * ldc + k / 2;
        const uint8_t *sp = scales + row * lds + k / 16;
        if (k + 32 <= kend) {
            rc.c = *reinterpret_cast<const uint4 *>(cp);
            rc.s = *reinterpret_cast<const uint16_t *>(sp);
        } else if (k + 16 <= kend) {
            const uint2 h = *reinterpret_cast<const uint2 *>(cp);
            rc.c.x = h.x; rc.c.y = h.y;
            rc.s = sp[0];
        }
    }
    return rc;
}

__device__ inline RowChunk load_chunk2_tiled(const uint8_t *codes, int64_t ldc, const uint8_t *scales, int64_t lds,
                                             int64_t row, int64_t nrows, int64_t k, int64_t kend) {
    RowChunk rc;
    rc.c = make_uint4(0, 0, 0, 0);
    rc.s = 0;
    if (row < nrows && k < kend) {                // tiled padding is zero: no half-chunk case
        const int64_t t = row >> 4, u = k >> 9;
        const int lane = (int)(16 * ((k >> 7) & 3) + (row & 15)), i = (int)((k >> 5) & 3);
        rc.c = *reinterpret_cast<const uint4 *>(codes + t * ldc + u * 4096 + 1024 * i + 16 * lane);
        rc.s = *reinterpret_cast<const uint16_t *>(scales + t * lds + u * 512 + 8 * lane + 2 * i);
    }
    return rc;
}

// Large tiles: BM x BN per workgroup of NW waves (2 along
// M x NW/2 along N), each wave a BM/2 x 2 BN/NW block of 16 x 16 tiles, so
// every fragment read from LDS feeds 4 to 8 MFMAs (against 4 for the 64 x 64
// wave tile above). 256 x 256 runs 8 waves (two per SIMD, 128 accumulator
// registers each), 128 x 128 runs 4 with two workgroups per CU. Two LDS
// stages; within a wave the stages overlap as a software pipeline, in source
// order:
//  * a 2-deep register queue: the global loads of step s + 2 go out at the
//    start of step s and are decoded during step s + 1;
//  * the decode and LDS stores of step s + 1 (into the other stage) are spread
//    over the MFMA groups of step s;
//  * A fragments are read from LDS four MFMA groups ahead, the second
//    k-chunk's B fragments during the last groups of the first.
// Residue columns (the augmented K + S product of the ARCQuant article,
// sections 3.1-3.2; selective compensation of prompts in the ResServe
// abstract) are further k-steps after the K / BK main ones: step K / BK + r
// multiplies the activation's columns K + BK r.. (the quantized residue) with
// the weight's columns BK r.. (the W_aug tail is W's own first S columns, read
// again, never materialized). They run through the same pipeline and split-K
// ranges; K must be a multiple of 32 so their chunks stay 16-byte aligned.
template <int BM, int BN, int NW, int WPE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void tiled2_kernel(TArgs a) {
    constexpr int NT = 64 * NW;                              // threads
    constexpr int RT = BM / 16, CT = BN / 16;
    constexpr int A_SLOTS = RT * 2 * 64, B_SLOTS = CT * 2 * 64;
    constexpr int STAGE = A_SLOTS + B_SLOTS;
    constexpr int WN = NW / 2;                               // waves: 2 along M x WN along N
    constexpr int WRT = RT / 2, WCT = CT / WN;
    constexpr int A_ITERS = BM * 2 / NT, B_ITERS = BN * 2 / NT, NCH = A_ITERS + B_ITERS;
    static_assert(A_ITERS * NT == BM * 2 && B_ITERS * NT == BN * 2, "whole chunks per thread");
    constexpr int NG = 2 * WRT, NU = 4 * NCH;                // MFMA groups and decode units per step
    extern __shared__ half8 lds[];                           // [2][STAGE]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int nblk = a.tiles_m * a.tiles_n;
    int bid = blockIdx.x;
    if (nblk % 8 == 0) bid = (bid % 8) * (nblk / 8) + bid / 8;
    const int tn = bid / a.tiles_m, tm = bid % a.tiles_m;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    // this workgroup's k-steps [s0, s0 + ksteps) of the main and residue steps
    // (split-K: range blockIdx.y)
    const int64_t kmain = (a.K + BK - 1) / BK;
    const int64_t kall = kmain + (a.res_cols + BK - 1) / BK;
    const int64_t s0 = (int64_t)blockIdx.y * a.kchunk;
    const int64_t ksteps = (s0 + a.kchunk < kall ? s0 + a.kchunk : kall) - s0;

    // chunk c of this thread: A chunks (c < A_ITERS), then B chunks; (row, half) of the tile
    auto crow = [&](int c) { return ((tid + NT * (c < A_ITERS ? c : c - A_ITERS)) >> 1); };
    auto chalf = [&](int c) { return (tid + NT * (c < A_ITERS ? c : c - A_ITERS)) & 1; };
    auto cslot = [&](int c) {
        const int r = crow(c), h = chalf(c);
        return (c < A_ITERS ? 0 : A_SLOTS) + ((r >> 4) * 2 + h) * 64 + (r & 15);
    };
    RowChunk rq0[NCH], rq1[NCH];
    auto gload = [&](int64_t s, RowChunk *q) {
        const bool res = s0 + s >= kmain;      // a residue step (wave-uniform)
        const int64_t kw = (res ? s0 + s - kmain : s0 + s) * BK;      // weight column
        const int64_t ka = res ? a.K + kw : kw;                        // activation column
        const int64_t wend = res ? a.res_cols : a.K, aend = res ? a.K + a.res_cols : a.K;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int r = crow(c), h = chalf(c);
            if (c < A_ITERS)
                q[c] = load_chunk2(a.a_codes, a.a_ldc, a.a_scales, a.a_lds, m0 + r, a.M, ka + 32 * h, aend);
            else
                q[c] = a.w_tiled ? load_chunk2_tiled(a.w_codes, a.w_ldc, a.w_scales, a.w_lds, n0 + r, a.N, kw + 32 * h, wend)
                                 : load_chunk2(a.w_codes, a.w_ldc, a.w_scales, a.w_lds, n0 + r, a.N, kw + 32 * h, wend);
        }
    };
    // decode unit u = fragment (u & 3) of chunk (u >> 2) into stage st
    auto unit = [&](half8 *st, const RowChunk *q, int u) {
        const int c = u >> 2, f = u & 3;
        const uint32_t sb = f < 2 ? (q[c].s & 0xFFu) : ((q[c].s >> 8) & 0xFFu);
        const uint32_t w = f == 0 ? q[c].c.x : f == 1 ? q[c].c.y : f == 2 ? q[c].c.z : q[c].c.w;
        st[cslot(c) + 16 * f] = decode8(w, scale_pair(sb));
    };

    float4v acc[WRT][WCT];
#pragma unroll
    for (int i = 0; i < WRT; ++i)
#pragma unroll
        for (int j = 0; j < WCT; ++j) acc[i][j] = float4v{0, 0, 0, 0};

    gload(0, rq0);
    if (ksteps > 1) gload(1, rq1);
#pragma unroll
    for (int u = 0; u < NU; ++u) unit(lds, rq0, u);
    __syncthreads();

    // step s (parity P): MFMAs on stage P; decode the queue entry of step s + 1
    // (rq[P ^ 1]) into stage P ^ 1; load step s + 2 into rq[P]
    auto step = [&](int64_t s, auto parity) {
        constexpr int P = decltype(parity)::value;
        RowChunk *qload = P == 0 ? rq0 : rq1;
        const RowChunk *qdec = P == 0 ? rq1 : rq0;
        const half8 *cur = lds + P * STAGE;
        half8 *nxt = lds + (P ^ 1) * STAGE;
        const bool dec = s + 1 < ksteps;
        if (s + 2 < ksteps) gload(s + 2, qload);
        // A fragments of the step's groups, read kPD groups ahead; B fragments of
        // the second k-chunk read during the last groups of the first
        constexpr int kPD = 4;
        auto aslot = [&](int gi) { return ((wm * WRT + gi % WRT) * 2 + gi / WRT) * 64 + lane; };
        half8 afr[NG];
        half8 bf[WCT], bn[WCT];
#pragma unroll
        for (int j = 0; j < WCT; ++j) bf[j] = cur[A_SLOTS + ((wn * WCT + j) * 2 + 0) * 64 + lane];
#pragma unroll
        for (int gi = 0; gi < kPD && gi < NG; ++gi) afr[gi] = cur[aslot(gi)];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const int kc = gi / WRT, i = gi % WRT;
            if (gi + kPD < NG) afr[gi + kPD] = cur[aslot(gi + kPD)];
            if (kc == 0 && i == (WRT > 2 ? WRT - 2 : 0)) {
#pragma unroll
                for (int j = 0; j < WCT; ++j) bn[j] = cur[A_SLOTS + ((wn * WCT + j) * 2 + 1) * 64 + lane];
            }
#pragma unroll
            for (int j = 0; j < WCT; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr[gi], kc == 0 ? bf[j] : bn[j], acc[i][j], 0, 0, 0);
            if (dec) {
#pragma unroll
                for (int u = gi * NU / NG; u < (gi + 1) * NU / NG; ++u) unit(nxt, qdec, u);
            }
        }
        __syncthreads();
    };
    for (int64_t s = 0; s < ksteps; s += 2) {
        step(s, std::integral_constant<int, 0>{});
        if (s + 1 < ksteps) step(s + 1, std::integral_constant<int, 1>{});
    }

    const int g = lane >> 4, c16 = lane & 15;
    if (a.part) {                              // split-K: the unscaled partial tile
        float *part = a.part + (int64_t)blockIdx.y * a.M * a.N;
#pragma unroll
        for (int i = 0; i < WRT; ++i)
#pragma unroll
            for (int j = 0; j < WCT; ++j) {
                const int64_t n = n0 + (wn * WCT + j) * 16 + c16;
                if (n >= a.N) continue;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t m = m0 + (wm * WRT + i) * 16 + 4 * g + e;
                    if (m < a.M) part[m * a.N + n] = acc[i][j][e];
                }
            }
        return;
    }
    const float scale = a.a_S[0] * a.w_S[0];
#pragma unroll
    for (int i = 0; i < WRT; ++i) {
#pragma unroll
        for (int j = 0; j < WCT; ++j) {
            const int64_t n = n0 + (wn * WCT + j) * 16 + c16;
            if (n >= a.N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + (wm * WRT + i) * 16 + 4 * g + e;
                if (m < a.M) {
                    const float v = acc[i][j][e] * scale;
                    if (a.yt == 1) static_cast<float *>(a.y)[m * a.ldy + n] = v;
                    else static_cast<uint16_t *>(a.y)[m * a.ldy + n] = f2bf(v);
                }
            }
        }
    }
}

// ------------------------------------------------- FP4 operands staged in LDS
// The large-M product with the operands kept in LDS as stored (FP4 codes and
// E4M3 bytes, a quarter of the f16 bytes) and decoded to f16 per fragment in
// registers, right before the MFMAs that use it.
//
// A step is 128 columns of K. Its codes and scale bytes go from memory into one
// of three LDS stages by direct-to-LDS loads (no staging registers): row r's
// 32-column chunk b (16 code bytes) at r * 64 + 16 p, its two E4M3 bytes
// zero-extended into the dword at r * 4 + p, p = b ^ f(r) with
// f(r) = ((r >> 1) ^ (r >> 2)) & 3, so that the fragment reads below (16 rows x
// one chunk per 16 lanes) hit every bank group. The loads of step s + 3 go out
// at the end of step s into the stage step s read; step s + 1's are waited for
// there. A chunk past the data is loaded from its row's start and then
// overwritten (zero codes and scales) by the thread that loaded it.
//
// 256 x 256 output tiles on 8 waves, two per SIMD (one's LDS reads and decode
// run under the other's MFMAs), each a 128 x 64 block: 8 x 4 accumulators of
// v_mfma_f32_16x16x32_f16. Per step a lane reads the 16 code bytes of chunk g
// (its lane group) of each of its 12 rows, and MFMA k-substep j takes their
// dword j: the MFMA's k-slot (g, e) is column 32 g + 8 j + e of the step, for
// both operands, so the four substeps cover the 128 columns once. Dwords 0-1
// take the chunk's first E4M3 byte, 2-3 its second. The decode is exact
// (decode8: e(c) d in f16), the accumulation FP32, as in the other kernels.
//
// Residue columns are further steps (activation columns K + kw.., weight
// columns kw..), as in tiled2_kernel. Tiled weights are read in place: a
// chunk's 16 bytes and two scale bytes sit at offsets that split into a
// per-lane part fixed for the kernel and a per-step part.
constexpr int PF_BM = 256, PF_BN = 256;
constexpr int PF_ACODE = PF_BM * 64, PF_BCODE = PF_BN * 64;          // code bytes per stage
constexpr int PF_ASC = PF_BM * 16, PF_BSC = PF_BN * 16;              // a dword per chunk
constexpr int PF_STAGE = PF_ACODE + PF_BCODE + PF_ASC + PF_BSC;       // 40 KiB
constexpr int PF_GROUP_M = 8;                                         // row tiles per group of the tile order

// 8 waves, 2 along M x 4 along N, two per SIMD. (Four waves of 128 x 128, one per
// SIMD with the whole register file, decode a third less but measured half as fast:
// nothing hides one wave's decode and LDS waits.)
constexpr int PF_NW = 8;

__global__ __launch_bounds__(64 * PF_NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fp4lds_kernel(TArgs a) {
    constexpr int NW = PF_NW, PF_NT = 64 * NW;
    constexpr int PF_CH = PF_BM * 4 / PF_NT;                          // chunks per thread and operand
    constexpr int PF_LOADS = 4 * PF_CH;                               // direct-to-LDS loads per thread and step
    constexpr int WN = NW / 2, CT = PF_BN / WN / 16;                  // waves along N, 16-column tiles per wave
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_pf[];   // [3][PF_STAGE]
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN, r16 = lane & 15, g = lane >> 4;
    // tile order: each XCD takes a contiguous range of tiles (workgroups are dealt
    // to the 8 XCDs round robin), walked in groups of PF_GROUP_M row tiles that
    // sweep the columns together and so share panels in that XCD's L2
    const int nblk = a.tiles_m * a.tiles_n;
    int bid = blockIdx.x;
    if (nblk % 8 == 0) bid = (bid % 8) * (nblk / 8) + bid / 8;
    const int in_group = PF_GROUP_M * a.tiles_n, first_m = (bid / in_group) * PF_GROUP_M;
    const int gsize = a.tiles_m - first_m < PF_GROUP_M ? a.tiles_m - first_m : PF_GROUP_M;
    const int tm = first_m + (bid % in_group) % gsize, tn = (bid % in_group) / gsize;
    const int64_t m0 = (int64_t)tm * PF_BM, n0 = (int64_t)tn * PF_BN;
    const int64_t kmain = (a.K + 127) / 128, kall = kmain + (a.res_cols + 127) / 128;
    const int64_t s0 = (int64_t)blockIdx.y * a.kchunk;
    const int64_t ksteps = (s0 + a.kchunk < kall ? s0 + a.kchunk : kall) - s0;

    // chunk i of this thread: c = PF_NT i + tid, row c / 4 of the tile, position
    // c % 4; it fetches the chunk that belongs there (the row's low four bits are
    // those of tid / 4 for every i)
    const int q4 = (lane & 3) ^ (((lane >> 3) ^ (lane >> 4)) & 3);
    const int gp = g ^ (((r16 >> 1) ^ (r16 >> 2)) & 3);     // position of chunk g in this lane's rows
    // per-lane byte offsets from the tile's first row (rows past the matrix repeat
    // its last row); 32 bits hold them (launcher-checked)
    const uint8_t *abase = a.a_codes + m0 * a.a_ldc, *asbase = a.a_scales + m0 * a.a_lds;
    const int64_t wrow0 = a.w_tiled ? n0 / 16 : n0;
    const uint8_t *wbase = a.w_codes + wrow0 * a.w_ldc, *wsbase = a.w_scales + wrow0 * a.w_lds;
    uint32_t ra[PF_CH], rsa[PF_CH], rb[PF_CH], rsb[PF_CH];
#pragma unroll
    for (int i = 0; i < PF_CH; ++i) {
        const int row = (PF_NT * i + tid) >> 2;
        const int64_t ma = m0 + row, nb = n0 + row;
        const int64_t la = (ma < a.M ? ma : a.M - 1) - m0, n = nb < a.N ? nb : a.N - 1;
        ra[i] = (uint32_t)(la * a.a_ldc);
        rsa[i] = (uint32_t)(la * a.a_lds);
        if (a.w_tiled) {          // 16 x 512 items: strip n / 16, lane 16 (k / 128 % 4) + n % 16, k / 32 % 4
            rb[i] = (uint32_t)((n / 16 - n0 / 16) * a.w_ldc + 16 * (n & 15) + 1024 * q4);
            rsb[i] = (uint32_t)((n / 16 - n0 / 16) * a.w_lds + 8 * (n & 15) + 2 * q4);
        } else {
            rb[i] = (uint32_t)((n - n0) * a.w_ldc + 16 * q4);
            rsb[i] = (uint32_t)((n - n0) * a.w_lds + 2 * q4);
        }
    }
    // step s of this range: weight columns kw.., activation columns ka.., and
    // whether this thread's chunk of the step holds data
    auto cols = [&](int64_t s, int64_t &kw, int64_t &ka, bool &ok) {
        const bool main = s0 + s < kmain;
        kw = (main ? s0 + s : s0 + s - kmain) * 128;
        ka = main ? kw : a.K + kw;
        ok = kw + 32 * q4 < (main ? a.K : a.res_cols);
    };
    auto dma = [&](int64_t s, uint8_t *st) {
        int64_t kw, ka;
        bool ok;
        cols(s, kw, ka, ok);
        const uint32_t ca = ok ? (uint32_t)(ka / 2 + 16 * q4) : 0u, sa = ok ? (uint32_t)(ka / 16 + 2 * q4) : 0u;
        uint32_t cw = 0, sw = 0;
        if (ok) {
            if (a.w_tiled) {
                cw = (uint32_t)((kw >> 9) * 4096 + 256 * ((kw >> 7) & 3));
                sw = (uint32_t)((kw >> 9) * 512 + 128 * ((kw >> 7) & 3));
            } else {
                cw = (uint32_t)(kw / 2);
                sw = (uint32_t)(kw / 16);
            }
        }
        const uint32_t sbase = lds_addr_of(st);
#pragma unroll
        for (int i = 0; i < PF_CH; ++i) {
            const uint32_t cbase = (uint32_t)(PF_NT * i + 64 * wave);   // first chunk of this wave's instruction
            dma16s(abase, ra[i] + ca, sbase + 16 * cbase);
            dma16s(wbase, rb[i] + cw, sbase + PF_ACODE + 16 * cbase);
            dma2s(asbase, rsa[i] + sa, sbase + PF_ACODE + PF_BCODE + 4 * cbase);
            dma2s(wsbase, rsb[i] + sw, sbase + PF_ACODE + PF_BCODE + PF_ASC + 4 * cbase);
        }
    };
    // after this thread's loads of step s have landed: chunks past the data become
    // zero codes and zero scales (the loads read the row's first bytes instead)
    auto fixup = [&](int64_t s, uint8_t *st) {
        int64_t kw, ka;
        bool ok;
        cols(s, kw, ka, ok);
        if (ok) return;
#pragma unroll
        for (int i = 0; i < PF_CH; ++i) {
            const int c = PF_NT * i + tid;
            *reinterpret_cast<uint4 *>(st + 16 * c) = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(st + PF_ACODE + 16 * c) = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint32_t *>(st + PF_ACODE + PF_BCODE + 4 * c) = 0u;
            *reinterpret_cast<uint32_t *>(st + PF_ACODE + PF_BCODE + PF_ASC + 4 * c) = 0u;
        }
    };

    float4v acc[8][CT];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < CT; ++j) acc[i][j] = float4v{0, 0, 0, 0};

    auto stage = [&](int64_t s) { return lds_pf + (int)(s % 3) * PF_STAGE; };
    // one step: this wave's 12 rows of codes and scales from LDS, then four
    // k-substeps of 32 MFMAs, each operand fragment decoded right before use
    auto compute = [&](const uint8_t *st) {
        uint4 ca[8], cb[CT];
        uint32_t sa[8], sb[CT];
#pragma unroll
        for (int j = 0; j < CT; ++j) {
            const int row = wn * 16 * CT + 16 * j + r16;
            cb[j] = *reinterpret_cast<const uint4 *>(st + PF_ACODE + row * 64 + 16 * gp);
            sb[j] = *reinterpret_cast<const uint32_t *>(st + PF_ACODE + PF_BCODE + PF_ASC + 4 * (row * 4 + gp));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = wm * 128 + 16 * i + r16;
            ca[i] = *reinterpret_cast<const uint4 *>(st + row * 64 + 16 * gp);
            sa[i] = *reinterpret_cast<const uint32_t *>(st + PF_ACODE + PF_BCODE + 4 * (row * 4 + gp));
        }
        auto word = [](const uint4 &v, int k) { return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w; };
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            half8 bf[CT];
#pragma unroll
            for (int j = 0; j < CT; ++j) bf[j] = decode8(word(cb[j], k), scale_pair(sb[j] >> (8 * (k >> 1))));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const half8 af = decode8(word(ca[i], k), scale_pair(sa[i] >> (8 * (k >> 1))));
#pragma unroll
                for (int j = 0; j < CT; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[j], acc[i][j], 0, 0, 0);
            }
        }
    };

    if (ksteps > 0) dma(0, stage(0));
    if (ksteps > 1) dma(1, stage(1));
    if (ksteps > 2) dma(2, stage(2));
    if (ksteps > 0) {
        if (ksteps > 2) DMA_WAIT_VM(2 * PF_LOADS); else if (ksteps > 1) DMA_WAIT_VM(PF_LOADS); else DMA_WAIT_VM(0);
        fixup(0, stage(0));
        DMA_WAIT_LGKM0();
        __builtin_amdgcn_s_barrier();
    }
    for (int64_t s = 0; s < ksteps; ++s) {
        compute(stage(s));
        if (s + 1 < ksteps) {
            // step s + 1's loads landed (step s + 2's may still be in flight), patched, visible;
            // past this barrier no wave reads stage s any more
            if (s + 2 < ksteps) DMA_WAIT_VM(PF_LOADS); else DMA_WAIT_VM(0);
            fixup(s + 1, stage(s + 1));
            DMA_WAIT_LGKM0();
            __builtin_amdgcn_s_barrier();
            if (s + 3 < ksteps) dma(s + 3, stage(s));
        }
    }

    // epilogue: fully unrolled per output kind (constant accumulator indices)
    float *part = a.part ? a.part + (int64_t)blockIdx.y * a.M * a.N : nullptr;
    const float scale = part ? 1.0f : a.a_S[0] * a.w_S[0];
    const int64_t mrow = m0 + wm * 128 + 4 * g, ncol = n0 + wn * 16 * CT + r16;
    auto store_all = [&](auto kind) {
        constexpr int KIND = decltype(kind)::value;   // 2: partial, 1: FP32, 0: BF16
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < CT; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t m = mrow + 16 * i + e, n = ncol + 16 * j;
                    if (m < a.M && n < a.N) {
                        if constexpr (KIND == 2) part[m * a.N + n] = acc[i][j][e];
                        else if constexpr (KIND == 1) static_cast<float *>(a.y)[m * a.ldy + n] = acc[i][j][e] * scale;
                        else static_cast<uint16_t *>(a.y)[m * a.ldy + n] = f2bf(acc[i][j][e] * scale);
                    }
                }
    };
    if (part) store_all(std::integral_constant<int, 2>{});
    else if (a.yt == 1) store_all(std::integral_constant<int, 1>{});
    else store_all(std::integral_constant<int, 0>{});
}

// Split-K combine: y[m][n] = S_a S_w sum_p part[p][m][n], in order p = 0, 1, ...
// (deterministic); one thread per element.
__global__ __launch_bounds__(256) void prefill_combine_kernel(const float *part, int P, int64_t M, int64_t N,
                                                              const float *a_S, const float *w_S, void *y, int yt,
                                                              int64_t ldy) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * N) return;
    const int64_t m = idx / N, n = idx - m * N;
    float s = 0.0f;
    for (int p = 0; p < P; ++p) s += part[(int64_t)p * M * N + idx];
    const float v = s * (a_S[0] * w_S[0]);
    if (yt == 1) static_cast<float *>(y)[m * ldy + n] = v;
    else static_cast<uint16_t *>(y)[m * ldy + n] = f2bf(v);
}

template <int BM, int BN, int NW, int WPE>
hipError_t run2(const TArgs &a0, hipStream_t st) {
    TArgs a = a0;
    a.tiles_m = (int)((a.M + BM - 1) / BM);
    a.tiles_n = (int)((a.N + BN - 1) / BN);
    constexpr int STAGE = (BM / 16) * 2 * 64 + (BN / 16) * 2 * 64;
    const size_t lds = 2 * (size_t)STAGE * sizeof(half8);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&tiled2_kernel<BM, BN, NW, WPE>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    tiled2_kernel<BM, BN, NW, WPE><<<dim3(a.tiles_m * a.tiles_n, a.P), 64 * NW, lds, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.part) return e;
    const int64_t total = a.M * a.N;
    prefill_combine_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(a.part, a.P, a.M, a.N, a.a_S, a.w_S, a.y,
                                                                            a.yt, a.ldy);
    return hipGetLastError();
}

template <int BM, int BN, bool RES>
hipError_t run(const TArgs &a0, hipStream_t st) {
    TArgs a = a0;
    a.tiles_m = (int)((a.M + BM - 1) / BM);
    a.tiles_n = (int)((a.N + BN - 1) / BN);
    constexpr int STAGE = (BM / 16) * 2 * 64 * (RES ? 2 : 1) + (BN / 16) * 2 * 64;
    const size_t lds = 2 * (size_t)STAGE * sizeof(half8);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&tiled_kernel<BM, BN, RES>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int blocks = a.tiles_m * a.tiles_n;
    tiled_kernel<BM, BN, RES><<<blocks, 256, lds, st>>>(a);
    return hipGetLastError();
}

// The pipelined large-tile kernel takes residue columns when K is a multiple of
// 32; otherwise (and at M <= 64) the 64 x 64-per-wave tile kernel does.
inline bool large_tiles(int64_t M, int64_t K, int64_t S) { return M > 64 && (S == 0 || K % 32 == 0); }

// Split-K ranges for the large-tile product: only when even 256 x 256 tiles
// leave most of the chip idle and K (+ S residue columns) is long; P ranges of
// at least 32 k-steps until the chip holds ~one workgroup per CU.
int prefill_splits(int64_t M, int64_t N, int64_t K, int64_t S) {
    if (!large_tiles(M, K, S)) return 1;
    const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t ksteps = (K + BK - 1) / BK + (S + BK - 1) / BK;
    if (tiles * 2 >= 192 || ksteps < 256) return 1;     // large enough for the unsplit plans
    int P = 1;
    while (P < 8 && tiles * P < 224 && ksteps / (2 * P) >= 32) P *= 2;
    return P;
}

// Split-K ranges of fp4lds_kernel: when its 256 x 256 tiles leave most CUs idle
// and the 128-column steps are many, P ranges of at least 16 steps until the
// chip holds about one workgroup per CU.
int fp4lds_splits(int64_t M, int64_t N, int64_t K, int64_t S) {
    if (M <= 64) return 1;
    const int64_t tiles = ((M + PF_BM - 1) / PF_BM) * ((N + PF_BN - 1) / PF_BN);
    const int64_t steps = (K + 127) / 128 + (S + 127) / 128;
    int P = 1;
    while (P < 8 && tiles * P < 192 && steps / (2 * P) >= 16) P *= 2;
    return P;
}

inline bool aligned_to(const void *p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

// fp4lds_kernel takes the long-K products: measured against tiled2_kernel at
// M = 512 / 2048 / 8192 (bf16 out, tiled weights), it is ahead at K = 28672,
// N = 8192 (0.39 / 0.47 / 0.48 of the f16 peak against 0.40 / 0.46 / 0.44) and
// behind at K = 8192, N = 28672 for M <= 2048 (0.35 / 0.36 against 0.38 / 0.40;
// level at M = 8192). Its other conditions: K and S multiples of 32 (whole
// 32-column chunks), code rows 16-byte aligned and scale rows 2-byte aligned,
// and a tile's rows within 32-bit offsets of its first row.
constexpr int64_t kFp4ldsMinK = 16384;

bool fp4lds_fits(const PrefillLaunch &g) {
    if (g.M <= 64 || g.K % 32 != 0 || g.res_cols % 32 != 0) return false;
    if (g.K + g.res_cols < kFp4ldsMinK) return false;
    if (!aligned_to(g.a_codes, 16) || g.a_ldc % 16 != 0 || !aligned_to(g.a_scales, 2) || g.a_lds % 2 != 0) return false;
    if (!aligned_to(g.w_codes, 16) || g.w_ldc % 16 != 0 || !aligned_to(g.w_scales, 2) || g.w_lds % 2 != 0) return false;
    const int64_t wrows = g.w_tiled ? PF_BN / 16 : PF_BN;
    const int64_t span_a = (int64_t)PF_BM * (g.a_ldc > g.a_lds ? g.a_ldc : g.a_lds);
    const int64_t span_w = wrows * (g.w_ldc > g.w_lds ? g.w_ldc : g.w_lds);
    return span_a < ((int64_t)1 << 32) && span_w < ((int64_t)1 << 32);
}

hipError_t run_fp4lds(const TArgs &a0, hipStream_t st, void *scratch, size_t scratch_bytes) {
    TArgs a = a0;
    a.tiles_m = (int)((a.M + PF_BM - 1) / PF_BM);
    a.tiles_n = (int)((a.N + PF_BN - 1) / PF_BN);
    const int P = fp4lds_splits(a.M, a.N, a.K, a.res_cols);
    const int64_t kall = (a.K + 127) / 128 + (a.res_cols + 127) / 128;
    a.P = P;
    a.kchunk = (kall + P - 1) / P;
    a.part = nullptr;
    if (P > 1) {
        if (!scratch || scratch_bytes < (size_t)P * (size_t)a.M * (size_t)a.N * sizeof(float))
            return hipErrorInvalidValue;
        a.part = static_cast<float *>(scratch);
    }
    const size_t lds = 3 * (size_t)PF_STAGE;
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&fp4lds_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    fp4lds_kernel<<<dim3((unsigned)(a.tiles_m * a.tiles_n), (unsigned)P), 64 * PF_NW, lds, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || P == 1) return e;
    const int64_t total = a.M * a.N;
    prefill_combine_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(a.part, P, a.M, a.N, a.a_S, a.w_S, a.y,
                                                                            a.yt, a.ldy);
    return hipGetLastError();
}

hipError_t launch_prefill_impl(const PrefillLaunch &g, hipStream_t st) {
    TArgs a;
    a.a_codes = g.a_codes; a.a_ldc = g.a_ldc; a.a_scales = g.a_scales; a.a_lds = g.a_lds; a.a_S = g.a_S;
    a.w_codes = g.w_codes; a.w_ldc = g.w_ldc; a.w_scales = g.w_scales; a.w_lds = g.w_lds; a.w_S = g.w_S;
    a.w_tiled = g.w_tiled;
    a.M = g.M; a.N = g.N; a.K = g.K; a.res_cols = g.res_cols;
    a.y = g.y; a.yt = g.yt; a.ldy = g.ldy;
    a.tiles_m = a.tiles_n = 0;
    const int64_t ktot = (g.K + BK - 1) / BK + (g.res_cols + BK - 1) / BK;
    a.P = 1; a.kchunk = ktot; a.part = nullptr;
    if (fp4lds_fits(g)) return run_fp4lds(a, st, g.scratch, g.scratch_bytes);
    if (!large_tiles(g.M, g.K, g.res_cols)) {
        if (g.res_cols > 0) {
            if (g.M <= 64) return run<64, 128, true>(a, st);
            return run<128, 128, true>(a, st);
        }
        return run<64, 128, false>(a, st);
    }
    const int P = prefill_splits(g.M, g.N, g.K, g.res_cols);
    if (P > 1) {
        if (!g.scratch || g.scratch_bytes < (size_t)P * (size_t)g.M * (size_t)g.N * sizeof(float))
            return hipErrorInvalidValue;
        a.P = P;
        a.kchunk = (ktot + P - 1) / P;
        a.part = static_cast<float *>(g.scratch);
        return run2<256, 256, 8, 2>(a, st);
    }
    // 256 x 256 tiles whenever they fill ~3/8 of the CUs or more: measured at
    // M = 512, K = 8192, N = 28672 (224 such tiles), they beat 128 x 128 tiles
    // at two workgroups per CU (0.34 vs 0.26 of peak) and 128 x 256 tiles on
    // four waves (0.19)
    const int64_t tn = (g.N + 255) / 256;
    if (((g.M + 255) / 256) * tn >= 96) return run2<256, 256, 8, 2>(a, st);
    return run2<128, 128, 4, 2>(a, st);             // 128 x 128 tiles, two workgroups per CU
}

}  // namespace

// covers whichever kernel the call's strides select
size_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t S) {
    const int P1 = prefill_splits(M, N, K, S);
    const int P2 = (K % 32 == 0 && S % 32 == 0 && K + S >= kFp4ldsMinK) ? fp4lds_splits(M, N, K, S) : 1;
    const int P = P1 > P2 ? P1 : P2;
    return P > 1 ? (size_t)P * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_prefill(const PrefillLaunch &g, hipStream_t st) { return launch_prefill_impl(g, st); }

}  // namespace nvfp4
