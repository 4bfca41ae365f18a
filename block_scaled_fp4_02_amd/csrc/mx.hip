// mx.hip -- MXFP4 quantizer and W4A4 products on gfx950's scaled FP4 matrix cores.
//
// MXFP4: E2M1 codes (the element format of the ARCQuant article, section 1)
// sharing one power-of-two E8M0 scale per 32 consecutive elements along K (the
// 32-element blocks and E8M0 scales of the MX formats, ARCQuant article,
// sections 2.2 and 4.2; MXFP4 is the second format of the ResServe abstract).
// Shared exponent e = floor(log2(block amax)) - 2, clamped to [-127, 127]
// (-127 for an all-zero block); codes = E2M1 round-to-nearest-even of
// x * 2^-e, saturating at 6, with the sign of x. No tensor scale.
//
// These blocks are exactly what v_mfma_scale_f32_16x16x128_f8f6f4 consumes:
// each lane hands it 32 consecutive FP4 values of one row (16 bytes of the
// canonical codes) and that block's E8M0 byte, so the products below load the
// operands straight from memory into the matrix core -- there is no decode.
// Residue columns (ARCQuant article, sections 3.1-3.2; ResServe abstract: the
// residue is kept in the same format) follow column K of the activation and
// meet the weight's first S columns again.
#include <type_traits>

#include "internal.h"
#include "lds_dma.h"
#include "nvfp4_device.h"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kQThreads = 256;

// E8M0 shared exponent of a block from its largest magnitude's bit pattern:
// floor(log2(amax)) is the unbiased exponent field for normal amax; zero and
// subnormal amax (below 2^-126) clamp to -127 anyway.
__device__ inline int mx_exponent(float amax) {
    const int f = (int)((f2u(amax) >> 23) & 0xFFu);
    if (f == 0) return -127;
    const int e = f - 127 - 2;
    return e < -127 ? -127 : e;                     // f <= 254, so e <= 125
}

// 2^-e as a float, e in [-127, 125]: the biased exponent 127 - e is in [2, 254].
__device__ inline float pow2_neg(int e) { return u2f((uint32_t)(127 - e) << 23); }

// Encode 32 values: returns the E8M0 byte, fills 4 dwords of codes (element
// 2j in the low nibble of byte j). q = x * 2^-e is exact.
__device__ inline uint32_t mx_encode32(const float *v, uint32_t *cw, int &e) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    e = mx_exponent(amax);
    const float r = pow2_neg(e);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t w = 0;
        // v_cvt_scalef32_pk_fp4_f32 with scale 1 rounds to nearest even onto
        // E2M1, saturates at 6 and keeps the sign of zero (the rule the NVFP4
        // encoder relies on, checked against the rounding helpers)
#define MX_ENC(P) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * d + 2 * (P)] * r, v[8 * d + 2 * (P) + 1] * r, 1.0f, P)
        MX_ENC(0); MX_ENC(1); MX_ENC(2); MX_ENC(3);
#undef MX_ENC
        cw[d] = w;
    }
    return (uint32_t)(e + 127);
}

// R = x - e(c) 2^e for a block (both terms exact in FP32; one rounding). For
// e = -127 the scale 2^-127 is the subnormal with mantissa bit 22 set.
__device__ inline void mx_residue32(const float *v, const uint32_t *cw, int e, float *r) {
    typedef float float2v __attribute__((ext_vector_type(2)));
    const float s = e > -127 ? u2f((uint32_t)(127 + e) << 23) : u2f(1u << 22);
    auto pair = [&](int d, int p, float2v ev) {
        const float d0 = ev[0] * s, d1 = ev[1] * s;
        r[8 * d + 2 * p] = v[8 * d + 2 * p] - d0;
        r[8 * d + 2 * p + 1] = v[8 * d + 2 * p + 1] - d1;
    };
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        pair(d, 0, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[d], 1.0f, 0));
        pair(d, 1, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[d], 1.0f, 1));
        pair(d, 2, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[d], 1.0f, 2));
        pair(d, 3, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[d], 1.0f, 3));
    }
}

template <int XT>
__device__ inline void load32(const void *x, int64_t off, float *v) {
    if constexpr (XT == IN_BF16) {
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + off);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 a = p[q];
            const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[8 * q + 2 * i] = u2f(w[i] << 16);
                v[8 * q + 2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
            }
        }
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + off);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float4 a = p[q];
            v[4 * q] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
        }
    }
}

struct MXQArgs {
    const void *x; int64_t rows, K, ldx, res;
    uint8_t *codes; int64_t ldc;
    uint8_t *scales; int64_t lds;
};

// One thread per 32-element block of the input; a block below the residue
// bound also encodes its residue block into column K + 32 b.
template <int XT>
__global__ __launch_bounds__(kQThreads) void mx_quantize_kernel(MXQArgs a) {
    const int64_t nb = a.K / 32, total = a.rows * nb;
    for (int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kQThreads) {
        const int64_t row = i / nb, b = i - row * nb;
        float v[32];
        load32<XT>(a.x, row * a.ldx + 32 * b, v);
        uint32_t cw[4];
        int e;
        const uint32_t sb = mx_encode32(v, cw, e);
        uint8_t *crow = a.codes + row * a.ldc;
        *reinterpret_cast<uint4 *>(crow + 16 * b) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
        a.scales[row * a.lds + b] = (uint8_t)sb;
        if (32 * b < a.res) {
            float r[32];
            mx_residue32(v, cw, e, r);
            uint32_t rc[4];
            int er;
            const uint32_t rb = mx_encode32(r, rc, er);
            *reinterpret_cast<uint4 *>(crow + a.K / 2 + 16 * b) = make_uint4(rc[0], rc[1], rc[2], rc[3]);
            a.scales[row * a.lds + a.K / 32 + b] = (uint8_t)rb;
        }
    }
}

// ------------------------------------------------------------ small M (<= 64)
// Each workgroup (4 waves) owns TW 16-row weight tiles; its 4 waves split the
// 128-column k-steps (main, then residue) into contiguous quarters, each wave
// multiplying all TW tiles by the MT 16-row activation tiles for its steps,
// with D steps of loads in flight. Per step a lane loads 16 bytes of codes and
// one scale byte per operand tile. The waves' partial tiles meet in LDS and are
// added in wave order (deterministic), then stored.
//
// Every step issues the same loads unconditionally -- a lane whose 32-block lies
// past the data reads its row's first bytes and masks them at use (codes 0,
// scale 127), a refill past the wave's last step reads its first step again --
// and the step loop is unrolled NS steps at a time, so the compiler counts the
// loads in flight exactly and never drains the ring early.
struct MXDArgs {
    const uint8_t *a_codes; int64_t a_ldc;
    const uint8_t *a_scales; int64_t a_lds;
    const uint8_t *w_codes; int64_t w_ldc;
    const uint8_t *w_scales; int64_t w_lds;
    int64_t M, N, K, res;
    void *y; int yt; int64_t ldy;
    int64_t NT;
    int w_tiled;                               // W in the tiled MX layout
};

template <int TW, int MT>
struct MXStep {
    uint4 b[TW], a[MT];
    uint32_t sb[TW], sa[MT];
    uint32_t mask;                             // ~0: the lane's block holds data; 0: masked
};

template <int TW, int MT, int D, int NS, bool TILED>
__global__ __launch_bounds__(256) void mx_small_kernel(MXDArgs a) {
    __shared__ float4v red[4][TW * MT][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int64_t t0 = (int64_t)blockIdx.x * TW;
    const int64_t kmain = (a.K + 127) / 128, ktot = kmain + (a.res + 127) / 128;
    const int64_t per = (ktot + 3) / 4;
    const int64_t sbeg = wave * per < ktot ? wave * per : ktot;
    const int64_t send = sbeg + per < ktot ? sbeg + per : ktot;
    const int nst = (int)(send - sbeg);

    // operand rows of this lane, clamped into the tensors (rows past M or N give
    // outputs that are never stored)
    const uint8_t *wrow_c[TW], *wrow_s[TW], *arow_c[MT], *arow_s[MT];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        if (TILED) {
            // tile t0 + t (clamped: tiles past N are never stored); this lane's
            // 16 bytes and E8M0 byte of every step sit at fixed offsets in it
            const int64_t tile = t0 + t < a.NT ? t0 + t : a.NT - 1;
            wrow_c[t] = a.w_codes + tile * a.w_ldc + 16 * lane;
            wrow_s[t] = a.w_scales + tile * a.w_lds + lane;
        } else {
            int64_t n = 16 * (t0 + t) + r16;
            n = n < a.N ? n : a.N - 1;
            wrow_c[t] = a.w_codes + n * a.w_ldc;
            wrow_s[t] = a.w_scales + n * a.w_lds;
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        int64_t m = 16 * mt + r16;
        m = m < a.M ? m : a.M - 1;
        arow_c[mt] = a.a_codes + m * a.a_ldc;
        arow_s[mt] = a.a_scales + m * a.a_lds;
    }
    // k-step s: weight columns kw.. and activation columns ka..; a lane's 32-block
    // is inside the data or not as a whole (K and S are multiples of 32)
    auto load = [&](int64_t s, MXStep<TW, MT> &st) {
        const bool main = s < kmain;
        const int64_t kw = (main ? s : s - kmain) * 128 + 32 * g;
        const int64_t ka = main ? kw : a.K + kw;
        const bool ok = kw < (main ? a.K : a.res);
        const int64_t cw = ok ? kw / 2 : 0, ca = ok ? ka / 2 : 0, bw = ok ? kw / 32 : 0, ba = ok ? ka / 32 : 0;
        st.mask = ok ? ~0u : 0u;
        // tiled: weight step sw = kw / 128 of the lane's tile, in lane order (steps
        // past the data read the tile's first step; the mask zeroes them)
        const int64_t sw = ok ? (kw - 32 * g) / 128 : 0;
        const int64_t tc = (sw >> 2) * 4096 + 1024 * (sw & 3), ts = (sw >> 2) * 256 + 64 * (sw & 3);
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            st.b[t] = *reinterpret_cast<const uint4 *>(wrow_c[t] + (TILED ? tc : cw));
            st.sb[t] = wrow_s[t][TILED ? ts : bw];
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            st.a[mt] = *reinterpret_cast<const uint4 *>(arow_c[mt] + ca);
            st.sa[mt] = arow_s[mt][ba];
        }
    };

    float4v acc[TW][MT];
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = float4v{0, 0, 0, 0};

    if (nst > 0) {
        MXStep<TW, MT> ring[D];
#pragma unroll
        for (int d = 0; d < D; ++d) load(sbeg + (d < nst ? d : 0), ring[d]);
        for (int j0 = 0; j0 < nst; j0 += NS) {
#pragma unroll
            for (int jj = 0; jj < NS; ++jj) {
                const int j = j0 + jj, d = jj % D;
                if (j < nst) {
                    const uint32_t mk = ring[d].mask;
                    const uint32_t unit = 127u & ~mk;          // masked blocks: scale 2^0, codes 0
#pragma unroll
                    for (int t = 0; t < TW; ++t) {
                        const v8i bv = {(int)(ring[d].b[t].x & mk), (int)(ring[d].b[t].y & mk),
                                        (int)(ring[d].b[t].z & mk), (int)(ring[d].b[t].w & mk), 0, 0, 0, 0};
                        const int sb = (int)((ring[d].sb[t] & mk) | unit);
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
                            const v8i av = {(int)(ring[d].a[mt].x & mk), (int)(ring[d].a[mt].y & mk),
                                            (int)(ring[d].a[mt].z & mk), (int)(ring[d].a[mt].w & mk), 0, 0, 0, 0};
                            acc[t][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                av, bv, acc[t][mt], 4, 4, 0, (int)((ring[d].sa[mt] & mk) | unit), 0, sb);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                // refill the slot: the step D ahead, or a spare load of the first step
                const int nx = j + D;
                load(sbeg + (nx < nst ? nx : 0), ring[d]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    // partial tiles of the 4 waves, added in wave order
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[wave][t * MT + mt][lane] = acc[t][mt];
    __syncthreads();
    for (int q = wave; q < TW * MT; q += 4) {
        const int t = q / MT, mt = q % MT;
        float4v s = red[0][q][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) s += red[w][q][lane];
        const int64_t n = 16 * (t0 + t) + r16;
        if (n >= a.N) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t m = 16 * mt + 4 * g + e;
            if (m < a.M) {
                if (a.yt == 1) static_cast<float *>(a.y)[m * a.ldy + n] = s[e];
                else static_cast<uint16_t *>(a.y)[m * a.ldy + n] = f32_to_bf16_rne(s[e]);
            }
        }
    }
}

// NS: the unrolled step count, at least a wave's quarter of the k-steps when it fits
template <int TW, int MT>
hipError_t run_small(const MXDArgs &a, hipStream_t st) {
    const int64_t G = (a.NT + TW - 1) / TW;
    const int64_t per = ((a.K + 127) / 128 + (a.res + 127) / 128 + 3) / 4;
#define MXS(NS, TL) mx_small_kernel<TW, MT, 4, NS, TL><<<dim3((unsigned)G), dim3(256), 0, st>>>(a)
    if (a.w_tiled) {
        if (per <= 8) MXS(8, true);
        else if (per <= 16) MXS(16, true);
        else MXS(32, true);
    } else {
        if (per <= 8) MXS(8, false);
        else if (per <= 16) MXS(16, false);
        else MXS(32, false);
    }
#undef MXS
    return hipGetLastError();
}

// ------------------------------------------------------------ large M (tiles)
// BM x BN = 256 x 256 output tiles, 16 x 16 MFMAs over 128-column steps.
// A step's codes and E8M0 bytes go from memory straight into LDS with gfx950's
// direct-to-LDS loads (global_load_lds_dwordx4 / _ubyte: no staging registers,
// no decode -- the matrix cores take them as stored): a row's 32-block b at
// row * 64 + 16 p, p its swizzled position (below); a scale byte lands as a
// zero-extended dword (the ubyte form writes lane l at base + 4 l), entry
// row * 4 + p.
// Three LDS stages: the loads of step s + 3 go out at the end of step s, into
// the stage step s - 1 read, and step s + 2's are waited for there. A
// 32-block past the data is loaded from its row's start and then overwritten in
// LDS by the thread that loaded it (codes 0, scale 127). Residue columns are
// further steps, as in the small-M kernel. Split-K writes FP32 partial tiles
// for a combine in fixed order.
constexpr int MX_BM = 256, MX_BN = 256;
constexpr int MX_ACODE = MX_BM * 64, MX_BCODE = MX_BN * 64;          // bytes per stage
constexpr int MX_ASC = MX_BM * 4 * 4, MX_BSC = MX_BN * 4 * 4;        // a dword per scale byte
constexpr int MX_STAGE = MX_ACODE + MX_BCODE + MX_ASC + MX_BSC;       // 40 KiB
constexpr int MX_GROUP_M = 8;                                         // row tiles per group of the tile order

struct MXTArgs {
    const uint8_t *a_codes; int64_t a_ldc;
    const uint8_t *a_scales; int64_t a_lds;
    const uint8_t *w_codes; int64_t w_ldc;
    const uint8_t *w_scales; int64_t w_lds;
    int64_t M, N, K, res;
    void *y; int yt; int64_t ldy;
    int tiles_m, tiles_n;
    int64_t kchunk;                            // k-steps per split-K range (blockIdx.y)
    float *part;                               // split-K partials [P][M][N], or nullptr
};

// 8 waves, two per SIMD (2 along M x 4 along N, 128 x 64 each, 128 accumulator
// registers): one wave's LDS reads and waits run under the other's MFMAs (a probe
// of back-to-back scaled FP4 MFMAs: 7.6 PF with one wave per SIMD, 8.9 PF with
// two). Per step a wave reads its 12 rows' chunks and scale bytes and issues 32
// MFMAs. (Four waves of 128 x 128, one per SIMD, with the fragments double-
// buffered in registers and the next step's reads placed between the MFMAs:
// 10% slower at prefill sizes.)
constexpr int MX8_NW = 8, MX8_NT = 64 * MX8_NW;
constexpr int MX8_CH = MX_BM * 4 / MX8_NT;                            // chunks per thread and operand (2)
constexpr int MX8_LOADS = 4 * MX8_CH;

__global__ __launch_bounds__(MX8_NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mx_tile8_kernel(MXTArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_m8[];   // [3][MX_STAGE]
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3, r16 = lane & 15, g = lane >> 4;
    const int nblk = a.tiles_m * a.tiles_n;
    int bid = blockIdx.x;
    if (nblk % 8 == 0) bid = (bid % 8) * (nblk / 8) + bid / 8;
    const int in_group = MX_GROUP_M * a.tiles_n, first_m = (bid / in_group) * MX_GROUP_M;
    const int gsize = a.tiles_m - first_m < MX_GROUP_M ? a.tiles_m - first_m : MX_GROUP_M;
    const int tm = first_m + (bid % in_group) % gsize, tn = (bid % in_group) / gsize;
    const int64_t m0 = (int64_t)tm * MX_BM, n0 = (int64_t)tn * MX_BN;
    const int64_t kmain = (a.K + 127) / 128, kall = kmain + (a.res + 127) / 128;
    const int64_t s0 = (int64_t)blockIdx.y * a.kchunk;
    const int64_t ksteps = (s0 + a.kchunk < kall ? s0 + a.kchunk : kall) - s0;
    // chunk i of this thread: c = MX8_NT i + tid, row c / 4, position c % 4 (the
    // row's low four bits are those of tid / 4 for every i)
    const int q4 = (lane & 3) ^ (((lane >> 3) ^ (lane >> 4)) & 3);
    const int gp = g ^ (((r16 >> 1) ^ (r16 >> 2)) & 3);
    const uint8_t *abase = a.a_codes + m0 * a.a_ldc, *wbase = a.w_codes + n0 * a.w_ldc;
    const uint8_t *asbase = a.a_scales + m0 * a.a_lds, *wsbase = a.w_scales + n0 * a.w_lds;
    uint32_t ra[MX8_CH], rb[MX8_CH], rsa[MX8_CH], rsb[MX8_CH];
#pragma unroll
    for (int i = 0; i < MX8_CH; ++i) {
        const int row = (MX8_NT * i + tid) >> 2;
        const int64_t ma = m0 + row, nb = n0 + row;
        const int64_t la = (ma < a.M ? ma : a.M - 1) - m0, lb = (nb < a.N ? nb : a.N - 1) - n0;
        ra[i] = (uint32_t)(la * a.a_ldc); rsa[i] = (uint32_t)(la * a.a_lds);
        rb[i] = (uint32_t)(lb * a.w_ldc); rsb[i] = (uint32_t)(lb * a.w_lds);
    }
    auto cols = [&](int64_t s, int64_t &kw, int64_t &ka, bool &ok) {
        const bool main = s0 + s < kmain;
        kw = (main ? s0 + s : s0 + s - kmain) * 128;
        ka = main ? kw : a.K + kw;
        ok = kw + 32 * q4 < (main ? a.K : a.res);
    };
    auto dma = [&](int64_t s, uint8_t *st) {
        int64_t kw, ka;
        bool ok;
        cols(s, kw, ka, ok);
        const uint32_t cw = ok ? (uint32_t)(kw / 2 + 16 * q4) : 0u, ca = ok ? (uint32_t)(ka / 2 + 16 * q4) : 0u;
        const uint32_t bw = ok ? (uint32_t)(kw / 32 + q4) : 0u, ba = ok ? (uint32_t)(ka / 32 + q4) : 0u;
        const uint32_t sbase = lds_addr_of(st);
#pragma unroll
        for (int i = 0; i < MX8_CH; ++i) {
            const uint32_t cbase = (uint32_t)(MX8_NT * i + 64 * wave);
            dma16s(abase, ra[i] + ca, sbase + 16 * cbase);
            dma16s(wbase, rb[i] + cw, sbase + MX_ACODE + 16 * cbase);
            dma1s(asbase, rsa[i] + ba, sbase + MX_ACODE + MX_BCODE + 4 * cbase);
            dma1s(wsbase, rsb[i] + bw, sbase + MX_ACODE + MX_BCODE + MX_ASC + 4 * cbase);
        }
    };
    // chunks past the data become zero codes with a unit scale (127)
    auto fixup = [&](int64_t s, uint8_t *st) {
        int64_t kw, ka;
        bool ok;
        cols(s, kw, ka, ok);
        if (ok) return;
#pragma unroll
        for (int i = 0; i < MX8_CH; ++i) {
            const int c = MX8_NT * i + tid;
            *reinterpret_cast<uint4 *>(st + 16 * c) = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(st + MX_ACODE + 16 * c) = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint32_t *>(st + MX_ACODE + MX_BCODE + 4 * c) = 127u;
            *reinterpret_cast<uint32_t *>(st + MX_ACODE + MX_BCODE + MX_ASC + 4 * c) = 127u;
        }
    };

    float4v acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = float4v{0, 0, 0, 0};
    auto stage = [&](int64_t s) { return lds_m8 + (int)(s % 3) * MX_STAGE; };
    auto compute = [&](const uint8_t *st) {
        v8i fa[8], fb[4];
        int sa[8], sb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = wn * 64 + 16 * j + r16;
            const uint4 v = *reinterpret_cast<const uint4 *>(st + MX_ACODE + row * 64 + 16 * gp);
            fb[j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            sb[j] = st[MX_ACODE + MX_BCODE + MX_ASC + 4 * (row * 4 + gp)];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = wm * 128 + 16 * i + r16;
            const uint4 v = *reinterpret_cast<const uint4 *>(st + row * 64 + 16 * gp);
            fa[i] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            sa[i] = st[MX_ACODE + MX_BCODE + 4 * (row * 4 + gp)];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], acc[i][j], 4, 4, 0, sa[i],
                                                                             0, sb[j]);
    };

    if (ksteps > 0) dma(0, stage(0));
    if (ksteps > 1) dma(1, stage(1));
    if (ksteps > 2) dma(2, stage(2));
    if (ksteps > 0) {
        if (ksteps > 2) DMA_WAIT_VM(2 * MX8_LOADS); else if (ksteps > 1) DMA_WAIT_VM(MX8_LOADS); else DMA_WAIT_VM(0);
        fixup(0, stage(0));
        DMA_WAIT_LGKM0();
        __builtin_amdgcn_s_barrier();
    }
    for (int64_t s = 0; s < ksteps; ++s) {
        compute(stage(s));
        if (s + 1 < ksteps) {
            // step s + 1's loads landed (step s + 2's may still be in flight), patched, visible;
            // past this barrier no wave reads stage s any more
            if (s + 2 < ksteps) DMA_WAIT_VM(MX8_LOADS); else DMA_WAIT_VM(0);
            fixup(s + 1, stage(s + 1));
            DMA_WAIT_LGKM0();
            __builtin_amdgcn_s_barrier();
            if (s + 3 < ksteps) dma(s + 3, stage(s));
        }
    }

    float *part = a.part ? a.part + (int64_t)blockIdx.y * a.M * a.N : nullptr;
    const int64_t mrow = m0 + wm * 128 + 4 * g, ncol = n0 + wn * 64 + r16;
    auto store_all = [&](auto kind) {
        constexpr int KIND = decltype(kind)::value;   // 2: partial, 1: FP32, 0: BF16
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t m = mrow + 16 * i + e, n = ncol + 16 * j;
                    if (m < a.M && n < a.N) {
                        if constexpr (KIND == 2) part[m * a.N + n] = acc[i][j][e];
                        else if constexpr (KIND == 1) static_cast<float *>(a.y)[m * a.ldy + n] = acc[i][j][e];
                        else static_cast<uint16_t *>(a.y)[m * a.ldy + n] = f32_to_bf16_rne(acc[i][j][e]);
                    }
                }
    };
    if (part) store_all(std::integral_constant<int, 2>{});
    else if (a.yt == 1) store_all(std::integral_constant<int, 1>{});
    else store_all(std::integral_constant<int, 0>{});
}

// y[m][n] = sum_p part[p][m][n] in order p = 0, 1, ... (deterministic).
__global__ __launch_bounds__(256) void mx_combine_kernel(const float *part, int P, int64_t M, int64_t N, void *y,
                                                         int yt, int64_t ldy) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * N) return;
    const int64_t m = idx / N, n = idx - m * N;
    float s = 0.0f;
    for (int p = 0; p < P; ++p) s += part[(int64_t)p * M * N + idx];
    if (yt == 1) static_cast<float *>(y)[m * ldy + n] = s;
    else static_cast<uint16_t *>(y)[m * ldy + n] = f32_to_bf16_rne(s);
}

// Split-K ranges of the tile kernel: when its 256 x 256 tiles leave most CUs idle
// and the steps are many, P ranges of at least 16 steps until ~one tile per CU.
int mx_splits(int64_t M, int64_t N, int64_t K, int64_t S) {
    if (M <= 64) return 1;
    const int64_t tiles = ((M + MX_BM - 1) / MX_BM) * ((N + MX_BN - 1) / MX_BN);
    const int64_t steps = (K + 127) / 128 + (S + 127) / 128;
    int P = 1;
    while (P < 8 && tiles * P < 192 && steps / (2 * P) >= 16) P *= 2;
    return P;
}

}  // namespace

hipError_t launch_mx_quantize(const MXQuantLaunch &q, hipStream_t st) {
    MXQArgs a;
    a.x = q.x; a.rows = q.rows; a.K = q.K; a.ldx = q.ldx; a.res = q.res_cols;
    a.codes = q.codes; a.ldc = q.ldc; a.scales = q.scales; a.lds = q.lds;
    const int64_t total = q.rows * (q.K / 32);
    if (total == 0) return hipSuccess;
    int64_t g = (total + kQThreads - 1) / kQThreads;
    if (g > 16384) g = 16384;
    if (q.xt == IN_BF16) mx_quantize_kernel<IN_BF16><<<(unsigned)g, kQThreads, 0, st>>>(a);
    else mx_quantize_kernel<IN_F32><<<(unsigned)g, kQThreads, 0, st>>>(a);
    return hipGetLastError();
}

size_t mx_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t S) {
    const int P = mx_splits(M, N, K, S);
    return P > 1 ? (size_t)P * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_mx_gemm(const MXGemmLaunch &g, hipStream_t st) {
    if (g.M < 1 || g.N < 1) return hipSuccess;
    MXDArgs a;
    a.a_codes = g.a_codes; a.a_ldc = g.a_ldc; a.a_scales = g.a_scales; a.a_lds = g.a_lds;
    a.w_codes = g.w_codes; a.w_ldc = g.w_ldc; a.w_scales = g.w_scales; a.w_lds = g.w_lds;
    a.M = g.M; a.N = g.N; a.K = g.K; a.res = g.res_cols;
    a.y = g.y; a.yt = g.yt; a.ldy = g.ldy;
    a.NT = (g.N + 15) / 16;
    a.w_tiled = g.w_tiled;
    // two tiles per workgroup (one activation load feeds both) once there are enough
    // tiles: from 512, or from 384 when M > 2 (measured on the N = 6144 sweep shape:
    // M = 16 9.1 -> 7.4 us, M = 1 5.7 -> 6.3 us; at N = 4096 the halved workgroup
    // count loses)
    const bool wide = a.NT >= 512 || (g.M > 2 && a.NT >= 384);
    if (g.M <= 16) return wide ? run_small<2, 1>(a, st) : run_small<1, 1>(a, st);
    if (g.M <= 32) return wide ? run_small<2, 2>(a, st) : run_small<1, 2>(a, st);
    if (g.M <= 64) return run_small<1, 4>(a, st);
    // larger M: 256 x 256 tiles on the matrix cores, split K when the tiles are few
    // the tile kernel addresses a tile's rows by 32-bit offsets from its first row
    int64_t stride = g.a_ldc > g.w_ldc ? g.a_ldc : g.w_ldc;
    stride = stride > g.a_lds ? stride : g.a_lds;
    stride = stride > g.w_lds ? stride : g.w_lds;
    if ((int64_t)MX_BM * stride >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
    MXTArgs t;
    t.a_codes = g.a_codes; t.a_ldc = g.a_ldc; t.a_scales = g.a_scales; t.a_lds = g.a_lds;
    t.w_codes = g.w_codes; t.w_ldc = g.w_ldc; t.w_scales = g.w_scales; t.w_lds = g.w_lds;
    t.M = g.M; t.N = g.N; t.K = g.K; t.res = g.res_cols;
    t.y = g.y; t.yt = g.yt; t.ldy = g.ldy;
    t.tiles_m = (int)((g.M + MX_BM - 1) / MX_BM);
    t.tiles_n = (int)((g.N + MX_BN - 1) / MX_BN);
    const int P = mx_splits(g.M, g.N, g.K, g.res_cols);
    const int64_t kall = (g.K + 127) / 128 + (g.res_cols + 127) / 128;
    t.kchunk = (kall + P - 1) / P;
    t.part = nullptr;
    if (P > 1) {
        if (!g.scratch || g.scratch_bytes < mx_workspace_bytes(g.M, g.N, g.K, g.res_cols)) return hipErrorInvalidValue;
        t.part = static_cast<float *>(g.scratch);
    }
    const size_t lds = 3 * (size_t)MX_STAGE;
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&mx_tile8_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    mx_tile8_kernel<<<dim3((unsigned)(t.tiles_m * t.tiles_n), (unsigned)P), MX8_NT, lds, st>>>(t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || P == 1) return e;
    const int64_t total = g.M * g.N;
    mx_combine_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(t.part, P, g.M, g.N, g.y, g.yt, g.ldy);
    return hipGetLastError();
}

}  // namespace nvfp4
