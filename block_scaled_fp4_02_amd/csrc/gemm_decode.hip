// gemm_decode.hip -- decode-shaped W4A4 product (M <= 32) in one launch, gfx950.
//
// y[m][n] = S_a S_w sum_k e(a)d(a) e(w)d(w)            (ARCQuant article, section 3.1)
// plus the residue columns of the augmented-K product (ARCQuant sections
// 3.1-3.2; ResServe abstract: the residue contribution is computed in the
// spare capacity of the narrow product and combined on chip).
//
// At small M the product is bound by streaming the packed weights once (the
// small-batch decode kernel discussion of the ReSET page on zingnex.cn,
// section "CUDA内核优化"). A call's whole weight (<= ~40 MB) fits in flight
// across the chip, so the kernel is built around issuing every weight load at
// once and doing everything else while those loads are in flight:
//
//  * a workgroup owns a K range of U 512-column units and T 16-row weight
//    tiles; it has four consumer waves and one producer wave;
//  * consumer waves issue the loads of their (tile, unit) items at once
//    (a ring of 4 items: 4 x 16 B codes + 8 B scales per lane each), wait at one
//    barrier for the activation operand, then decode each weight item in
//    registers (v_cvt_scalef32_pk_f16_fp4 + v_pk_mul_f16, exact) and issue 16
//    v_mfma_f32_16x16x32_f16 per item, refilling the ring; residue columns
//    reuse the decoded weight registers for a second MFMA;
//  * the producer wave has no weight loads in flight, so its waits are its own
//    (vmcnt is in order on gfx9): it quantizes the activations and writes the
//    K range's operand into LDS as exact f16 e*d values in A-operand lane order;
//  * with more than one K range, partial tiles go to the workspace through
//    device-coherent stores and the last workgroup of each tile group sums
//    them in fixed order (deterministic) and writes y.
//
// Activation quantization (raw activations in the call), chosen per shape:
//  LOCAL  X is small: every workgroup computes amax(X) itself and quantizes
//         its own K range -- no communication at all;
//  SYNC1  the grid agrees on amax(X) (each workgroup publishes the maximum of
//         1/G of X, one grid-wide wait), then each quantizes its own K range;
//  SYNC2  as SYNC1, then each workgroup quantizes 1/G of X's blocks into the
//         quantized-activation buffer and a second wait makes them visible.
// Cross-workgroup data moves through relaxed device-scope (sc1) loads and
// stores; a publisher waits for its own stores (s_waitcnt vmcnt(0)) and then
// counts. Grid-wide counters are hierarchical (16 sub-counters, then one top
// counter) because same-address device atomics serialize, and carry a call
// index in their upper half so they never need resetting. Every wait is
// bounded: past the spin limit a workgroup recomputes what it waited for from
// X itself (same arithmetic, same result), so no wait can hang.
#include <cstdio>
#include <cstdlib>

#include "internal.h"
#include "nvfp4_device.h"

namespace nvfp4 {
namespace {

constexpr int kCons = 4;                       // consumer waves
constexpr int kThreads = 64 * (kCons + 1);     // plus one producer wave
constexpr int kGroups = 16;                    // sub-counters per grid-wide wait
constexpr int kMaxItems = 8;                   // (tile, unit) items per consumer wave
constexpr size_t kTileCntOffset = 4096;        // header bytes before the tile counters
constexpr int64_t kMaxTileCounters = (int64_t)((kHeaderBytes - kTileCntOffset) / sizeof(unsigned));

enum Mode { MODE_PRE = 0, MODE_LOCAL = 1, MODE_SYNC1 = 2, MODE_SYNC2 = 3 };

struct DArgs {
    const void *x; int x_bf16; int64_t ldx;   // raw activations (modes LOCAL/SYNC1/SYNC2)
    const float *static_S;
    uint8_t *q_codes; int64_t q_ldc;          // quantized activations [M][K + res]
    uint8_t *q_scales; int64_t q_lds;
    float *q_S;
    const uint8_t *w_codes; int64_t w_ldc;
    const uint8_t *w_scales; int64_t w_lds;
    const float *w_S;
    int64_t M, N, K, res_cols;
    void *y; int yt; int64_t ldy;
    uint8_t *header;                          // zero-kept counters
    float *amax_slots;                        // G floats
    float *partials;                          // P x M x N floats
    int U, P, T, tw, G, mode;
    int64_t NT;
    unsigned spin_limit;
};

template <typename T>
__device__ inline void st_dev(T *p, T v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <typename T>
__device__ inline T ld_dev(const T *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <typename T>
__device__ inline T add_dev(T *p, T v) { return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

__device__ inline void wait_own_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// ------------------------------------------------------------ grid-wide wait
// Counter word: upper 32 bits = call index, lower = arrivals in this call.
struct Sync { unsigned long long *top, *sub; };

// Header bytes [1536 s, 1536 s + 64 (kGroups + 1)) belong to sync s (s = 0, 1):
// the top counter, then one 64-byte line per sub-counter.
constexpr size_t kSyncBytes = 1536;
static_assert(64 * (kGroups + 1) <= (int)kSyncBytes, "sub-counters overflow their sync's region");
static_assert(2 * kSyncBytes <= kTileCntOffset - 64, "sync regions overlap the timeout counter");

__device__ inline Sync sync_at(uint8_t *header, int s) {
    Sync y;
    y.top = reinterpret_cast<unsigned long long *>(header + kSyncBytes * s);
    y.sub = reinterpret_cast<unsigned long long *>(header + kSyncBytes * s + 64);
    return y;
}

// One lane per workgroup: count this workgroup in; returns the call index to wait past.
__device__ inline unsigned sync_arrive(Sync y, int G) {
    const int NG = G < kGroups ? G : kGroups;
    const int grp = (int)(blockIdx.x % NG);
    const unsigned members = (unsigned)((G - grp + NG - 1) / NG);
    const unsigned mine = (unsigned)(ld_dev(y.top) >> 32);   // cannot advance before we arrive
    unsigned long long *sc = y.sub + 8 * grp;                 // 64 bytes apart
    const unsigned long long old = add_dev(sc, 1ull);
    if ((unsigned)old + 1 == members) {
        add_dev(sc, (1ull << 32) - members);                  // next call, zero arrivals
        const unsigned long long ot = add_dev(y.top, 1ull);
        if ((unsigned)ot + 1 == (unsigned)NG) add_dev(y.top, (1ull << 32) - (unsigned long long)NG);
    }
    return mine;
}

// Header word counting waits that gave up (diagnostics; read by the host).
constexpr size_t kTimeoutCounterOffset = 4096 - 64;

__device__ inline bool sync_wait(Sync y, unsigned mine, unsigned limit, uint8_t *header) {
    unsigned it = 0;
    while ((unsigned)(ld_dev(y.top) >> 32) == mine) {
        if (++it > limit) {
            add_dev(reinterpret_cast<unsigned *>(header + kTimeoutCounterOffset), 1u);
            return false;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    return true;
}

// ------------------------------------------------------------ weight items
struct WLoad {
    uint4 c[4];
    uint2 s;
};

// Always the same five loads, so the compiler can count them (vmcnt) across the
// ring. Addresses past K are clamped to the row start: such weight lanes meet
// an activation operand that is exactly zero there, and any code/scale byte
// decodes to a finite f16, so they contribute 0. A 16 B load at a chunk start
// below K stays inside the row's padded stride (ld_codes is a multiple of 16
// and >= K/2), and so does an 8 B scale load at a unit start below K.
__device__ inline void load_w(const DArgs &a, int64_t n, int64_t kb, int g, WLoad &w) {
    const uint8_t *crow = a.w_codes + n * a.w_ldc;
    const uint8_t *srow = a.w_scales + n * a.w_lds;
    const int64_t k0 = kb + 128 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t ki = k0 + 32 * i;
        w.c[i] = *reinterpret_cast<const uint4 *>(crow + (ki < a.K ? ki / 2 : 0));
    }
    w.s = *reinterpret_cast<const uint2 *>(srow + (k0 < a.K ? k0 / 16 : 0));
}

// ------------------------------------------------------------ producer wave
// amax(X) over all rows and columns by one wave.
__device__ inline float wave_amax_x(const DArgs &a) {
    const int lane = threadIdx.x & 63;
    const int64_t KB = a.K / 16, NB = a.M * KB;
    float m = 0.0f;
    for (int64_t b = lane; b < NB; b += 64) {
        const int64_t row = b / KB, blk = b - row * KB;
        float v[16];
        load16_any(a.x, a.x_bf16, row * a.ldx + 16 * blk, v);
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
    }
    return wave_max(m);
}

__device__ inline float scale_of(float amax) { return amax > 0.0f ? amax / 2688.0f : 1.0f; }

// A 32-column chunk of one activation row as codes + 2 block scales.
struct Chunk { uint32_t c[4]; uint32_t s0, s1; };

// Quantize columns [k, k + 32) of row m from X (blocks beyond K stay zero);
// res selects the residue of those columns.
__device__ inline Chunk chunk_from_x(const DArgs &a, int64_t m, int64_t k, bool res, float S) {
    Chunk ch = {{0, 0, 0, 0}, 0, 0};
    const float t = 6.0f * S;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int64_t kb = k + 16 * b;
        if (kb + 16 <= a.K) {
            float v[16];
            load16_any(a.x, a.x_bf16, m * a.ldx + kb, v);
            uint32_t cw[2];
            float d;
            uint32_t db = encode_block(v, S, t, cw, d);
            if (res) {
                float r[16];
                block_residue(v, cw, d, S, r);
                db = encode_block(r, S, t, cw, d);
            }
            ch.c[2 * b] = cw[0];
            ch.c[2 * b + 1] = cw[1];
            if (b == 0) ch.s0 = db; else ch.s1 = db;
        }
    }
    return ch;
}

// The same chunk read from the quantized-activation buffer (column kc of the
// stored tensor; residue columns are stored after column K).
template <bool COHERENT>
__device__ inline Chunk chunk_from_q(const DArgs &a, int64_t m, int64_t kc, int64_t kend_cols) {
    Chunk ch = {{0, 0, 0, 0}, 0, 0};
    const uint8_t *cp = a.q_codes + m * a.q_ldc + kc / 2;
    const uint8_t *sp = a.q_scales + m * a.q_lds + kc / 16;
    if (kc + 32 <= kend_cols) {
        const unsigned long long *p = reinterpret_cast<const unsigned long long *>(cp);
        const unsigned long long lo = COHERENT ? ld_dev(p) : p[0];
        const unsigned long long hi = COHERENT ? ld_dev(p + 1) : p[1];
        ch.c[0] = (uint32_t)lo; ch.c[1] = (uint32_t)(lo >> 32);
        ch.c[2] = (uint32_t)hi; ch.c[3] = (uint32_t)(hi >> 32);
        ch.s0 = COHERENT ? ld_dev(sp) : sp[0];
        ch.s1 = COHERENT ? ld_dev(sp + 1) : sp[1];
    } else if (kc + 16 <= kend_cols) {
        const unsigned long long *p = reinterpret_cast<const unsigned long long *>(cp);
        const unsigned long long lo = COHERENT ? ld_dev(p) : p[0];
        ch.c[0] = (uint32_t)lo; ch.c[1] = (uint32_t)(lo >> 32);
        ch.s0 = COHERENT ? ld_dev(sp) : sp[0];
    }
    return ch;
}

__device__ inline void chunk_to_slots(half8 *lds, int base_slot, int stride, const Chunk &ch) {
    const half2v d0 = scale_pair(ch.s0), d1 = scale_pair(ch.s1);
#pragma unroll
    for (int j = 0; j < 4; ++j) lds[base_slot + j * stride] = decode8(ch.c[j], j < 2 ? d0 : d1);
}

// ---------------------------------------------------------------- kernel
template <int MT, bool RES>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void decode_kernel(DArgs a) {
    constexpr int kRing = MT == 1 ? 4 : 3;       // weight items in flight per consumer wave
    extern __shared__ half8 lds_a[];          // [U][16][MT][64] (+ residue copy)
    __shared__ float sh_S;
    __shared__ int sh_last;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int p = blockIdx.x % a.P;
    const int64_t q = blockIdx.x / a.P;
    const int64_t kbeg = (int64_t)p * a.U * 512;
    const int64_t kend = kbeg + (int64_t)a.U * 512 < a.K ? kbeg + (int64_t)a.U * 512 : a.K;
    const int units = (int)((kend - kbeg + 511) / 512);
    const int64_t rend = RES ? (a.res_cols < kend ? a.res_cols : kend) : kbeg;
    const int res_units = RES ? (rend > kbeg ? (int)((rend - kbeg + 511) / 512) : 0) : 0;
    const int slots = a.U * 16 * MT * 64;
    const int64_t t_lo = q * a.T, t_hi = (q + 1) * a.T < a.NT ? (q + 1) * a.T : a.NT;

    // consumer work: tiles t_lo + wave + kCons * j
    const int64_t t_first = t_lo + wave;
    const int ntiles = (wave < kCons && t_first < t_hi) ? (int)((t_hi - t_first + kCons - 1) / kCons) : 0;
    const int nitems = ntiles * units;
    auto item_row = [&](int it) -> int64_t {     // clamped into [0, N): loads never leave W
        const int64_t n = 16 * (t_first + (int64_t)(it / units) * kCons) + r16;
        return n < 0 ? 0 : (n < a.N ? n : a.N - 1);
    };

    // Loaded before the weight ring: vmcnt is in order, so anything loaded after
    // the ring and used early would wait for the whole ring.
    const float w_scale = a.w_S[0];
    WLoad ring[kRing];
    if (wave < kCons) {
        // ---- consumers: every weight load of the first items, right away
#pragma unroll
        for (int s = 0; s < kRing; ++s)
            if (s < nitems) load_w(a, item_row(s), kbeg + 512 * (s % units), g, ring[s]);
    } else {
        // ---- producer: activation operand of this K range into LDS
        float S = 0.0f;
        bool from_x = a.mode == MODE_LOCAL || a.mode == MODE_SYNC1;
        if (a.mode != MODE_PRE) {
            if (a.static_S) {
                S = *a.static_S;
            } else if (a.mode == MODE_LOCAL) {
                S = scale_of(wave_amax_x(a));
            } else {
                // publish the maximum of this workgroup's 1/G of X's blocks
                const int64_t KB = a.K / 16, NB = a.M * KB;
                const int64_t b0 = (int64_t)blockIdx.x * NB / a.G, b1 = ((int64_t)blockIdx.x + 1) * NB / a.G;
                float lmax = 0.0f;
                for (int64_t b = b0 + lane; b < b1; b += 64) {
                    const int64_t row = b / KB, blk = b - row * KB;
                    float v[16];
                    load16_any(a.x, a.x_bf16, row * a.ldx + 16 * blk, v);
#pragma unroll
                    for (int i = 0; i < 16; ++i) lmax = fmaxf(lmax, fabsf(v[i]));
                }
                lmax = wave_max(lmax);
                const Sync y0 = sync_at(a.header, 0);
                int ok = 1;
                if (lane == 0) {
                    st_dev(&a.amax_slots[blockIdx.x], lmax);
                    wait_own_stores();
                    ok = sync_wait(y0, sync_arrive(y0, a.G), a.spin_limit, a.header) ? 1 : 0;
                }
                ok = __shfl(ok, 0);
                if (ok) {
                    float m = 0.0f;
                    for (int i = lane; i < a.G; i += 64) m = fmaxf(m, ld_dev(&a.amax_slots[i]));
                    S = scale_of(wave_max(m));
                } else {
                    S = scale_of(wave_amax_x(a));
                }
            }
            if (blockIdx.x == 0 && lane == 0) *a.q_S = S;
            if (a.mode == MODE_SYNC2) {
                // quantize this workgroup's 1/G of X's blocks into the shared buffer
                const int64_t KB = a.K / 16, NB = a.M * KB;
                const int64_t b0 = (int64_t)blockIdx.x * NB / a.G, b1 = ((int64_t)blockIdx.x + 1) * NB / a.G;
                const float t = 6.0f * S;
                for (int64_t b = b0 + lane; b < b1; b += 64) {
                    const int64_t row = b / KB, blk = b - row * KB;
                    float v[16];
                    load16_any(a.x, a.x_bf16, row * a.ldx + 16 * blk, v);
                    uint32_t cw[2];
                    float d;
                    const uint32_t db = encode_block(v, S, t, cw, d);
                    unsigned long long *cp = reinterpret_cast<unsigned long long *>(a.q_codes + row * a.q_ldc + 8 * blk);
                    st_dev(cp, (unsigned long long)cw[0] | ((unsigned long long)cw[1] << 32));
                    st_dev(a.q_scales + row * a.q_lds + blk, (uint8_t)db);
                    if (RES && 16 * blk < a.res_cols) {
                        float r[16];
                        block_residue(v, cw, d, S, r);
                        uint32_t rc[2];
                        float dr;
                        const uint32_t rdb = encode_block(r, S, t, rc, dr);
                        unsigned long long *rp =
                            reinterpret_cast<unsigned long long *>(a.q_codes + row * a.q_ldc + 8 * (KB + blk));
                        st_dev(rp, (unsigned long long)rc[0] | ((unsigned long long)rc[1] << 32));
                        st_dev(a.q_scales + row * a.q_lds + KB + blk, (uint8_t)rdb);
                    }
                }
                wait_own_stores();
                const Sync y1 = sync_at(a.header, 1);
                int ok = 1;
                if (lane == 0) ok = sync_wait(y1, sync_arrive(y1, a.G), a.spin_limit, a.header) ? 1 : 0;
                from_x = __shfl(ok, 0) == 0;
            }
        }
        // The K range's operand: for each (unit u, sub-block i, m-tile mt) the 64
        // lanes take row 16 mt + (lane & 15) and quarter g = lane >> 4, i.e. the
        // 32 columns kbeg + 512 u + 128 g + 32 i, and write slots
        // ((u * 16 + 4 i + j) * MT + mt) * 64 + lane: consecutive lanes, consecutive
        // slots. Every slot of the range is written once (zero outside the data).
        const bool writer = from_x && q == 0 && a.mode != MODE_PRE;   // keeps the quantized buffer complete
        const int passes = (units + res_units) * 4 * MT;
        for (int w = 0; w < passes; ++w) {
            const bool is_res = w >= units * 4 * MT;
            const int w2 = is_res ? w - units * 4 * MT : w;
            const int mt = w2 % MT, i = (w2 / MT) & 3, u = (w2 / MT) >> 2;
            const int64_t row = r16 + 16 * mt;
            const int64_t kc = kbeg + 512 * u + 128 * g + 32 * i;
            Chunk ch = {{0, 0, 0, 0}, 0, 0};
            if (row < a.M && kc < (is_res ? rend : kend)) {
                if (from_x) {
                    ch = chunk_from_x(a, row, kc, is_res, S);
                    if (writer) {
                        const int64_t col = is_res ? a.K + kc : kc;
                        uint32_t *cp = reinterpret_cast<uint32_t *>(a.q_codes + row * a.q_ldc + col / 2);
                        if (kc + 32 <= a.K) {
                            cp[0] = ch.c[0]; cp[1] = ch.c[1]; cp[2] = ch.c[2]; cp[3] = ch.c[3];
                            a.q_scales[row * a.q_lds + col / 16] = (uint8_t)ch.s0;
                            a.q_scales[row * a.q_lds + col / 16 + 1] = (uint8_t)ch.s1;
                        } else {
                            cp[0] = ch.c[0]; cp[1] = ch.c[1];
                            a.q_scales[row * a.q_lds + col / 16] = (uint8_t)ch.s0;
                        }
                    }
                } else {
                    const int64_t col = is_res ? a.K + kc : kc;
                    const int64_t lim = is_res ? a.K + rend : kend;
                    ch = a.mode == MODE_PRE ? chunk_from_q<false>(a, row, col, lim)
                                            : chunk_from_q<true>(a, row, col, lim);
                }
            }
            chunk_to_slots(lds_a + (is_res ? slots : 0), ((u * 16 + 4 * i) * MT + mt) * 64 + lane, MT * 64, ch);
        }
        if (lane == 0) sh_S = a.mode == MODE_PRE ? a.q_S[0] : S;
    }
    __syncthreads();                           // activation operand ready

    // ---- consumers: decode weights, MFMA
    const float scale = sh_S * w_scale;
    if (wave < kCons && nitems > 0) {            // waves without tiles issue no loads at all
        float4v acc[MT], acc2[MT];                 // two MFMA chains: even / odd fragments
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) { acc[mt] = float4v{0, 0, 0, 0}; acc2[mt] = float4v{0, 0, 0, 0}; }
        // Fully unrolled over at most kMaxItems items (no loop back-edge): each slot
        // is consumed in place and refilled right after, always with the same five
        // loads (past the last item it re-reads the current one, a cache hit), so
        // the load stream is uniform and vmcnt is tracked exactly.
#pragma unroll
        for (int it = 0; it < kMaxItems; ++it) {
            const int s = it % kRing;
            {
                if (it < nitems) {
                    const int u = it % units;
                    const half8 *abase = lds_a + (size_t)u * 16 * MT * 64 + lane;
                    const bool res_u = RES && u < res_units;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t sw = (i < 2) ? ring[s].s.x : ring[s].s.y;
                        const half2v d0 = scale_pair((sw >> (16 * (i & 1))) & 0xFFu);
                        const half2v d1 = scale_pair((sw >> (16 * (i & 1) + 8)) & 0xFFu);
                        const uint32_t cws[4] = {ring[s].c[i].x, ring[s].c[i].y, ring[s].c[i].z, ring[s].c[i].w};
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const half8 b = decode8(cws[j], j < 2 ? d0 : d1);
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) {
                                float4v &ac = (j & 1) ? acc2[mt] : acc[mt];
                                ac = __builtin_amdgcn_mfma_f32_16x16x32_f16(abase[(4 * i + j) * MT * 64 + mt * 64], b,
                                                                            ac, 0, 0, 0);
                                if (res_u)
                                    ac = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                        abase[slots + (4 * i + j) * MT * 64 + mt * 64], b, ac, 0, 0, 0);
                            }
                        }
                    }
                    if (u == units - 1) {
                        // tile done: lane holds rows 16 mt + 4 g + e of column n
                        const int64_t n = 16 * (t_first + (int64_t)(it / units) * kCons) + r16;
                        if (n < a.N) {
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    const int64_t m = 16 * mt + 4 * g + e;
                                    const float tot = acc[mt][e] + acc2[mt][e];
                                    if (m < a.M) {
                                        if (a.P == 1) {
                                            const float v = tot * scale;
                                            if (a.yt == 1) static_cast<float *>(a.y)[m * a.ldy + n] = v;
                                            else static_cast<uint16_t *>(a.y)[m * a.ldy + n] = f32_to_bf16_rne(v);
                                        } else {
                                            st_dev(&a.partials[((int64_t)p * a.M + m) * a.N + n], tot);
                                        }
                                    }
                                }
                        }
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) { acc[mt] = float4v{0, 0, 0, 0}; acc2[mt] = float4v{0, 0, 0, 0}; }
                    }
                }
                if (it + kRing < kMaxItems) {
                    const int nx = it + kRing < nitems ? it + kRing : (it < nitems ? it : nitems - 1);
                    __builtin_amdgcn_sched_barrier(0);   // keep: consume slot s, then refill it
                    load_w(a, item_row(nx), kbeg + 512 * (nx % units), g, ring[s]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }

    // ---- split-K combine by the last workgroup of the tile group
    if (a.P > 1) {
        wait_own_stores();                     // this wave's partial tiles are visible
        __syncthreads();
        unsigned *tile_cnt = reinterpret_cast<unsigned *>(a.header + kTileCntOffset);
        if (threadIdx.x == 0) sh_last = add_dev(&tile_cnt[q], 1u) == (unsigned)a.P - 1;
        __syncthreads();
        if (sh_last) {
            const int64_t ncols = (t_hi - t_lo) * 16;   // multiple of 16: whole column pairs
            for (int64_t idx = threadIdx.x; idx < a.M * (ncols / 2); idx += kThreads) {
                const int64_t m = idx / (ncols / 2), n = 16 * t_lo + 2 * (idx - m * (ncols / 2));
                if (n >= a.N) continue;
                float s0 = 0.0f, s1 = 0.0f;
                for (int pp = 0; pp < a.P; ++pp) {
                    const float *src = &a.partials[((int64_t)pp * a.M + m) * a.N + n];
                    if (n + 1 < a.N && ((a.N & 1) == 0)) {
                        const unsigned long long v = ld_dev(reinterpret_cast<const unsigned long long *>(src));
                        s0 += u2f((uint32_t)v);
                        s1 += u2f((uint32_t)(v >> 32));
                    } else {
                        s0 += ld_dev(src);
                        if (n + 1 < a.N) s1 += ld_dev(src + 1);
                    }
                }
                for (int c = 0; c < 2 && n + c < a.N; ++c) {
                    const float v = (c ? s1 : s0) * scale;
                    if (a.yt == 1) static_cast<float *>(a.y)[m * a.ldy + n + c] = v;
                    else static_cast<uint16_t *>(a.y)[m * a.ldy + n + c] = f32_to_bf16_rne(v);
                }
            }
            if (threadIdx.x == 0) st_dev(&tile_cnt[q], 0u);
        }
    }
}

// ---------------------------------------------------------------- planning
struct Plan { int MT, U, P, T, tw, G, mode; int64_t NT, Q; size_t lds; };

int resident_capacity(const void *fn, size_t lds) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 1;                       // no device: plan conservatively
    int per = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, kThreads, lds) != hipSuccess || per < 1) per = 1;
    return per * cus;
}

const void *kernel_ptr(int MT, bool res) {
    if (MT == 1) return res ? reinterpret_cast<const void *>(&decode_kernel<1, true>)
                            : reinterpret_cast<const void *>(&decode_kernel<1, false>);
    return res ? reinterpret_cast<const void *>(&decode_kernel<2, true>)
               : reinterpret_cast<const void *>(&decode_kernel<2, false>);
}

Plan plan_for(int64_t M, int64_t N, int64_t K, int64_t res_cols, bool raw_x, bool norm_or_perm) {
    Plan pl;
    pl.MT = M <= 16 ? 1 : 2;
    const bool res = res_cols > 0;
    int umax = (pl.MT == 1 ? 4 : 2) / (res ? 2 : 1);
    if (umax < 1) umax = 1;
    const size_t lds_max = (size_t)umax * 16 * pl.MT * 64 * sizeof(half8) * (res ? 2 : 1);
    static int cap_cache[2][2] = {{0, 0}, {0, 0}};
    int &capc = cap_cache[pl.MT - 1][res ? 1 : 0];
    if (capc <= 1) capc = resident_capacity(kernel_ptr(pl.MT, res), lds_max);
    int cap = capc - capc / 8;
    if (const char *e = std::getenv("NVFP4_DECODE_MAX_GRID")) {      // tuning override
        const int v = std::atoi(e);
        if (v > 0 && v < cap) cap = v;
    }
    pl.NT = (N + 15) / 16;
    const int64_t ku = (K + 511) / 512 > 0 ? (K + 511) / 512 : 1;
    int bestU = 1, besttw = 1;
    double best = 1e30;
    for (int U = 1; U <= umax; U *= 2) {
        for (int tw = 1; tw <= 16; ++tw) {
            const int64_t P = (ku + U - 1) / U, Q = (pl.NT + kCons * tw - 1) / (kCons * tw);
            const int64_t G = P * Q;
            if (G > cap || Q > kMaxTileCounters) continue;
            const int items = tw * (int)(U < ku ? U : ku);
            if (items > kMaxItems) continue;
            const double cost = items + 0.15 * (double)P + (G < 192 ? 4.0 : 0.0);
            if (cost < best) { best = cost; bestU = U; besttw = tw; }
        }
    }
    pl.U = bestU > ku ? (int)ku : bestU;
    pl.tw = besttw;
    pl.T = kCons * pl.tw;
    pl.P = (int)((ku + pl.U - 1) / pl.U);
    pl.Q = (pl.NT + pl.T - 1) / pl.T;
    pl.G = (int)(pl.P * pl.Q);
    pl.lds = (size_t)pl.U * 16 * pl.MT * 64 * sizeof(half8) * (res ? 2 : 1);
    // activation handling
    const int64_t kc = (int64_t)pl.U * 512 < K ? (int64_t)pl.U * 512 : K;
    if (!raw_x || norm_or_perm) pl.mode = MODE_PRE;
    else if (M * kc <= 8192 && M * K <= 16384) pl.mode = MODE_LOCAL;
    else if (M * kc <= 8192) pl.mode = MODE_SYNC1;
    else pl.mode = MODE_SYNC2;
    if (std::getenv("NVFP4_DEBUG_PLAN"))
        std::fprintf(stderr, "[nvfp4] decode plan M=%lld N=%lld K=%lld S=%lld: MT=%d U=%d P=%d T=%d G=%d mode=%d "
                     "(resident capacity %d)\n", (long long)M, (long long)N, (long long)K, (long long)res_cols,
                     pl.MT, pl.U, pl.P, pl.T, pl.G, pl.mode, capc);
    return pl;
}

bool plan_ok(const Plan &pl) { return pl.Q <= kMaxTileCounters && pl.G >= 1; }

}  // namespace

size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t res_cols) {
    const Plan pl = plan_for(M, N, K, res_cols, true, false);
    const size_t part = pl.P > 1 ? (size_t)pl.P * M * N * sizeof(float) : 0;
    return part + ((size_t)pl.G * sizeof(float) + 255) / 256 * 256;
}

bool decode_can_fuse(int64_t M, int64_t N, int64_t K, int64_t res_cols) {
    return plan_ok(plan_for(M, N, K, res_cols, true, false));
}

hipError_t launch_decode(const DecodeLaunch &g, hipStream_t st) {
    const bool raw = g.x != nullptr;
    const Plan pl = plan_for(g.M, g.N, g.K, g.res_cols, raw, false);
    if (!plan_ok(pl)) return hipErrorInvalidValue;
    if (!g.header || !g.scratch || g.scratch_bytes < decode_workspace_bytes(g.M, g.N, g.K, g.res_cols))
        return hipErrorInvalidValue;
    DArgs a;
    a.x = g.x; a.x_bf16 = g.x_bf16; a.ldx = g.ldx; a.static_S = g.static_S;
    a.q_codes = g.q_codes; a.q_ldc = g.q_ldc; a.q_scales = g.q_scales; a.q_lds = g.q_lds; a.q_S = g.q_S;
    a.w_codes = g.w_codes; a.w_ldc = g.w_ldc; a.w_scales = g.w_scales; a.w_lds = g.w_lds; a.w_S = g.w_S;
    a.M = g.M; a.N = g.N; a.K = g.K; a.res_cols = g.res_cols;
    a.y = g.y; a.yt = g.yt; a.ldy = g.ldy;
    a.header = reinterpret_cast<uint8_t *>(g.header);
    a.amax_slots = static_cast<float *>(g.scratch);
    a.partials = reinterpret_cast<float *>(static_cast<uint8_t *>(g.scratch) +
                                           ((size_t)pl.G * sizeof(float) + 255) / 256 * 256);
    a.U = pl.U; a.P = pl.P; a.T = pl.T; a.tw = pl.tw; a.G = pl.G; a.mode = pl.mode; a.NT = pl.NT;
    a.spin_limit = g.spin_limit;
    void *args[] = {&a};
    return hipLaunchKernel(kernel_ptr(pl.MT, g.res_cols > 0), dim3(pl.G), dim3(kThreads), args, pl.lds, st);
}

}  // namespace nvfp4
