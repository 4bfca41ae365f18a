// gemm_skinny.hip -- decode-shaped W4A4 product (M <= 32) for gfx950.
//
// y[m][n] = S_a S_w sum_k e(a)d(a) e(w)d(w)   (ARCQuant article, section 3.1)
// plus, when residue columns are present, the residue part over the same
// weight columns (ARCQuant section 3.2 unified GEMM over K+S; ResServe
// abstract: the residue contribution is combined on chip, no extra output
// pass). Small-batch decode is bandwidth-bound (the ReSET kernel discussion on
// zingnex.cn, section "CUDA内核优化"): the weight is streamed once.
//
// Layout of the work:
//  * the K axis is cut into 512-column units; a workgroup (4 waves) owns a
//    range of U units and a set of 16-row weight tiles;
//  * the activation operand of that K range is decoded once into LDS as f16
//    e*d values (exact), laid out in the lane order of
//    v_mfma_f32_16x16x32_f16's A operand so each MFMA reads 1 KB contiguous;
//  * a wave owns whole tiles: per (tile, unit) it loads 4 x 16 B of codes per
//    lane (16 rows x 256 B) and 8 scale bytes, decodes them in registers into
//    B operands and issues 16 MFMAs per m-tile; residue columns reuse the
//    decoded B registers for a second MFMA against the residue A operand;
//  * the next (tile, unit) is loaded before the current one is computed.
//
// k order inside a unit: lane quarter g (lanes 16g..16g+15) owns bytes
// [64g, 64g+64) of each row segment, loaded as 4 x 16 B (i = 0..3); dword j of
// load i holds k = 128g + 32i + 8j + (0..7). MFMA (i, j) contracts exactly
// those k across the four quarters, and the A operand is stored the same way.
#include "internal.h"
#include "nvfp4_device.h"

namespace nvfp4 {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

struct SkArgs {
    const uint8_t *a_codes; int64_t a_ldc;
    const uint8_t *a_scales; int64_t a_lds;
    const float *a_S;
    const uint8_t *w_codes; int64_t w_ldc;
    const uint8_t *w_scales; int64_t w_lds;
    const float *w_S;
    int64_t M, N, K, res_cols;
    void *y; int yt; int64_t ldy;
    float *partials;
    int U;          // units per K range
    int P;          // number of K ranges
    int T;          // tiles per workgroup
    int64_t NT;     // tiles in N
};

struct WLoad {
    uint4 c[4];
    uint2 s;
};

__device__ inline uint16_t f2bf(float f) {
    uint32_t u = f2u(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Load one (tile row n, unit starting at column kb) slice of W for this lane.
__device__ inline void load_w(const SkArgs &a, int64_t n, int64_t kb, int g, WLoad &w) {
    const uint8_t *crow = a.w_codes + n * a.w_ldc;
    const uint8_t *srow = a.w_scales + n * a.w_lds;
    const int64_t k0 = kb + 128 * g;                 // first k of this lane's 128
    if (k0 + 128 <= a.K) {
        const uint4 *p = reinterpret_cast<const uint4 *>(crow + k0 / 2);
        w.c[0] = p[0]; w.c[1] = p[1]; w.c[2] = p[2]; w.c[3] = p[3];
        w.s = *reinterpret_cast<const uint2 *>(srow + k0 / 16);
    } else {
        uint32_t sc[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t ki = k0 + 32 * i;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (ki + 32 <= a.K) {
                v = *reinterpret_cast<const uint4 *>(crow + ki / 2);
            } else if (ki + 16 <= a.K) {
                const uint2 h = *reinterpret_cast<const uint2 *>(crow + ki / 2);
                v.x = h.x; v.y = h.y;
            }
            w.c[i] = v;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int64_t kk = ki + 16 * b;
                if (kk + 16 <= a.K) sc[(2 * i + b) >> 2] |= (uint32_t)srow[kk / 16] << (8 * ((2 * i + b) & 3));
            }
        }
        w.s = make_uint2(sc[0], sc[1]);
    }
}

template <int MT, bool RES>
__global__ __launch_bounds__(kThreads) void skinny_kernel(SkArgs a) {
    extern __shared__ half8 lds_a[];          // [U][16][MT][64] (+ residue copy)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int p = blockIdx.x % a.P;
    const int64_t q = blockIdx.x / a.P;
    const int64_t kbeg = (int64_t)p * a.U * 512;
    const int64_t kend = kbeg + (int64_t)a.U * 512 < a.K ? kbeg + (int64_t)a.U * 512 : a.K;
    const int units = (int)((kend - kbeg + 511) / 512);
    const int64_t rbeg = kbeg, rend = (RES ? (a.res_cols < kend ? a.res_cols : kend) : kbeg);
    const int res_units = RES ? (rend > rbeg ? (int)((rend - rbeg + 511) / 512) : 0) : 0;
    const int slots = a.U * 16 * MT * 64;

    // ---- decode the activation operand of this K range into LDS
    for (int s = threadIdx.x; s < (units + res_units) * 16 * MT * 64; s += kThreads) {
        const bool is_res = s >= units * 16 * MT * 64;
        const int s2 = is_res ? s - units * 16 * MT * 64 : s;
        const int l = s2 & 63, mt = (s2 >> 6) % MT, ij = ((s2 >> 6) / MT) & 15, u = ((s2 >> 6) / MT) >> 4;
        const int m = 16 * mt + (l & 15), gg = l >> 4, i = ij >> 2, j = ij & 3;
        const int64_t k = kbeg + 512 * u + 128 * gg + 32 * i + 8 * j;
        half8 v = {0, 0, 0, 0, 0, 0, 0, 0};
        const int64_t lim = is_res ? rend : kend;
        if (m < a.M && k < lim) {
            const int64_t kc = is_res ? a.K + k : k;
            const uint32_t cw = *reinterpret_cast<const uint32_t *>(a.a_codes + m * a.a_ldc + kc / 2);
            const uint32_t sb = a.a_scales[m * a.a_lds + kc / 16];
            v = decode8(cw, scale_pair(sb));
        }
        lds_a[(is_res ? slots : 0) + s2] = v;
    }
    __syncthreads();

    const float scale = a.a_S[0] * a.w_S[0];
    const int64_t t_end = (q + 1) * a.T < a.NT ? (q + 1) * a.T : a.NT;
    const int64_t t_first = q * a.T + wave;
    const int ntiles = t_first < t_end ? (int)((t_end - t_first + kWaves - 1) / kWaves) : 0;
    const int nitems = ntiles * units;
    if (nitems == 0) return;

    auto tile_row = [&](int it) -> int64_t {
        const int64_t t = t_first + (int64_t)(it / units) * kWaves;
        const int64_t n = 16 * t + r16;
        return n < a.N ? n : a.N - 1;
    };

    WLoad cur, nxt;
    load_w(a, tile_row(0), kbeg, g, cur);
    float4v acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = float4v{0, 0, 0, 0};

    for (int it = 0; it < nitems; ++it) {
        const int u = it % units;
        if (it + 1 < nitems) load_w(a, tile_row(it + 1), kbeg + 512 * ((it + 1) % units), g, nxt);
        const half8 *abase = lds_a + (size_t)u * 16 * MT * 64 + lane;
        const bool res_u = RES && u < res_units;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t sw = (i < 2) ? cur.s.x : cur.s.y;
            const half2v d0 = scale_pair((sw >> (16 * (i & 1))) & 0xFFu);
            const half2v d1 = scale_pair((sw >> (16 * (i & 1) + 8)) & 0xFFu);
            const uint32_t cws[4] = {cur.c[i].x, cur.c[i].y, cur.c[i].z, cur.c[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const half8 b = decode8(cws[j], j < 2 ? d0 : d1);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const half8 av = abase[(4 * i + j) * MT * 64 + mt * 64];
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b, acc[mt], 0, 0, 0);
                    if (res_u) {
                        const half8 ar = abase[slots + (4 * i + j) * MT * 64 + mt * 64];
                        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ar, b, acc[mt], 0, 0, 0);
                    }
                }
            }
        }
        if (u == units - 1) {
            // tile finished: lane holds rows m = 16 mt + 4 g + e of column n
            const int64_t t = t_first + (int64_t)(it / units) * kWaves;
            const int64_t n = 16 * t + r16;
            if (n < a.N) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t m = 16 * mt + 4 * g + e;
                        if (m < a.M) {
                            if (a.P == 1) {
                                const float v = acc[mt][e] * scale;
                                if (a.yt == 1) static_cast<float *>(a.y)[m * a.ldy + n] = v;
                                else static_cast<uint16_t *>(a.y)[m * a.ldy + n] = f2bf(v);
                            } else {
                                a.partials[((int64_t)p * a.M + m) * a.N + n] = acc[mt][e];
                            }
                        }
                    }
                    acc[mt] = float4v{0, 0, 0, 0};
                }
            }
        }
        cur = nxt;
    }
}

// y = S_a S_w * sum over K ranges of the partial sums (fixed order).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *partials, int P, int64_t M, int64_t N,
                                                           const float *aS, const float *wS,
                                                           void *y, int yt, int64_t ldy) {
    const float scale = aS[0] * wS[0];
    const int64_t total = M * N;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
        float s = 0.0f;
        for (int p = 0; p < P; ++p) s += partials[(int64_t)p * total + idx];
        const int64_t m = idx / N, n = idx - m * N;
        const float v = s * scale;
        if (yt == 1) static_cast<float *>(y)[m * ldy + n] = v;
        else static_cast<uint16_t *>(y)[m * ldy + n] = f2bf(v);
    }
}

struct Plan { int MT, U, P, T; int64_t NT; int wgs; size_t lds; };

Plan make_plan(int64_t M, int64_t N, int64_t K, int64_t res_cols) {
    Plan pl;
    pl.MT = M <= 16 ? 1 : 2;
    const bool res = res_cols > 0;
    const int umax = (pl.MT == 1 ? 4 : 2) / (res ? 2 : 1);
    pl.NT = (N + 15) / 16;
    pl.T = 4;
    const int64_t ku = (K + 511) / 512;
    int U = umax;
    for (; U > 1; U /= 2) {
        const int64_t P = (ku + U - 1) / U;
        if (P * ((pl.NT + pl.T - 1) / pl.T) >= 384) break;
    }
    if (U > ku) U = (int)ku;
    if (U < 1) U = 1;
    pl.U = U;
    pl.P = (int)((ku + U - 1) / U);
    pl.wgs = (int)(pl.P * ((pl.NT + pl.T - 1) / pl.T));
    pl.lds = (size_t)U * 16 * pl.MT * 64 * sizeof(half8) * (res ? 2 : 1);
    return pl;
}

}  // namespace

size_t skinny_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t res_cols) {
    const Plan pl = make_plan(M, N, K, res_cols);
    return pl.P > 1 ? (size_t)pl.P * M * N * sizeof(float) : 0;
}

hipError_t launch_skinny(const SkinnyLaunch &g, hipStream_t st) {
    const Plan pl = make_plan(g.M, g.N, g.K, g.res_cols);
    SkArgs a;
    a.a_codes = g.a_codes; a.a_ldc = g.a_ldc; a.a_scales = g.a_scales; a.a_lds = g.a_lds; a.a_S = g.a_S;
    a.w_codes = g.w_codes; a.w_ldc = g.w_ldc; a.w_scales = g.w_scales; a.w_lds = g.w_lds; a.w_S = g.w_S;
    a.M = g.M; a.N = g.N; a.K = g.K; a.res_cols = g.res_cols;
    a.y = g.y; a.yt = g.yt; a.ldy = g.ldy; a.partials = g.partials;
    a.U = pl.U; a.P = pl.P; a.T = pl.T; a.NT = pl.NT;
    if (pl.P > 1 && (g.partials == nullptr || g.partial_bytes < (size_t)pl.P * g.M * g.N * sizeof(float)))
        return hipErrorInvalidValue;
    const bool res = g.res_cols > 0;
#define SK(MT, R) skinny_kernel<MT, R><<<pl.wgs, kThreads, pl.lds, st>>>(a)
    if (pl.MT == 1) { if (res) SK(1, true); else SK(1, false); }
    else { if (res) SK(2, true); else SK(2, false); }
#undef SK
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || pl.P == 1) return e;
    int64_t blocks = (g.M * g.N + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    splitk_reduce_kernel<<<(int)blocks, 256, 0, st>>>(g.partials, pl.P, g.M, g.N, g.a_S, g.w_S, g.y, g.yt, g.ldy);
    return hipGetLastError();
}

}  // namespace nvfp4
