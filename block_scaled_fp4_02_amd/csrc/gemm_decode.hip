// gemm_decode.hip -- decode-shaped W4A4 product (M <= 64) in one launch, gfx950.
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
//    tiles; it has four consumer waves and four producer waves;
//  * producer waves issue their (small) activation loads first; after one
//    barrier (when producers hold more than one chunk per thread) the
//    consumer waves issue the loads of their first (tile, unit) items (a ring
//    of 4 items: 4 x 16 B codes + 8 B scales per lane each), so the
//    activation data is ahead of the weights in the CU's memory queue;
//  * producers write the K range's operand into LDS as exact f16 e*d values
//    in A-operand lane order; consumers then decode each weight item in
//    registers (v_cvt_scalef32_pk_f16_fp4 + v_pk_mul_f16, exact) and issue 16
//    v_mfma_f32_16x16x32_f16 per item as items land, refilling the ring;
//    residue columns reuse the decoded weight registers: their rows are
//    stacked under the activation rows (M <= 8, or M <= 16 when they cover at
//    least half of K; the same MFMAs) or else multiplied by a separate operand
//    copy in a second MFMA;
//  * with more than one K range, partial tiles go to the workspace through
//    device-coherent stores and the last workgroup of each tile group sums
//    them in fixed order (deterministic) and writes y.
//
// Activations: PRE reads an already quantized tensor; LOCAL (raw bf16 X with
// M K <= 32768) has every workgroup read all of X, take amax(X) itself and
// quantize its own K range -- no communication between workgroups. Larger raw
// activations are quantized by the quantize kernels first: a grid-wide wait
// inside a kernel that saturates HBM costs several microseconds, since every
// round trip queues behind the weight stream.
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <type_traits>
#include <unordered_map>

#include "internal.h"
#include "nvfp4_device.h"

namespace nvfp4 {
namespace {

constexpr int kCons = 4;                       // consumer waves: weights and MFMA
constexpr int kProd = 4;                       // producer waves: the activation operand
constexpr int kThreads = 64 * (kCons + kProd);
constexpr int kPThreads = 64 * kProd;
constexpr int kMaxItems = 8;                   // (tile, unit) items per consumer wave
constexpr int kPreItems = 2;                   // items each consumer issues before the operand barrier
constexpr int64_t kMaxTileCounters = kMaxCounters;
constexpr int64_t kLocalMaxElems = 32768;      // LOCAL: X read by every workgroup
constexpr int kLocalLoads = 4;                 // LOCAL: amax loads per lane and batch (K split over workgroups)
constexpr int kLocalChunks = 4;                // LOCAL: raw 32-column chunks per producer thread
constexpr int kPreChunks = 8;                  // PRE: quantized chunks per producer thread and batch
constexpr int kMaxP = 8;                       // split-K partials loaded at once by the combine

enum Mode { MODE_PRE = 0, MODE_LOCAL = 1 };

#ifdef NVFP4_TIMELINE
// Profiling builds only: per (workgroup, wave < 16, point) s_memrealtime stamps (100 MHz).
// Internal linkage: the kernel addresses it PC-relative, with no load of its address.
static __device__ unsigned long long g_timeline[1024 * 16 * 8];
#define TL(point) do { if ((threadIdx.x & 63) == 0 && blockIdx.x < 1024) \
    g_timeline[(blockIdx.x * 16 + (threadIdx.x >> 6)) * 8 + (point)] = __builtin_amdgcn_s_memrealtime(); } while (0)
#else
#define TL(point) do { } while (0)
#endif

struct DArgs {
    const void *x; int64_t ldx;               // raw bf16 activations (LOCAL)
    const float *static_S;
    uint8_t *q_codes; int64_t q_ldc;          // quantized activations [M][K + res]
    uint8_t *q_scales; int64_t q_lds;
    float *q_S;
    const uint8_t *w_codes; int64_t w_ldc;
    const uint8_t *w_scales; int64_t w_lds;
    const float *w_S;
    int64_t M, N, K, res_cols;
    void *y; int yt; int64_t ldy;
    uint8_t *header;                          // zero-kept tile counters
    float *partials;                          // P x M x N floats
    int U, P, T, tw, KW, G, mode;
    int Rr;                                   // operand rows per slot group (M, or 2 Mp when stacked)
    int Mp;                                   // stacked residue: residue row of m is Mp + m; else 0
    int ordered;                              // consumers issue their loads after the producers' (barrier)
    int64_t NT;
};

template <typename T>
__device__ inline void st_dev(T *p, T v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <typename T>
__device__ inline T ld_dev(const T *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <typename T>
__device__ inline T add_dev(T *p, T v) { return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

__device__ inline void wait_own_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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

// The same item from tiled weights: lane p's 4 x 16 B and 8 B are stored in
// lane order, so every load of the wave is one contiguous run (padding is zero).
__device__ inline void load_w_tiled(const DArgs &a, int64_t tile, int64_t unit, int lane, WLoad &w) {
    const uint8_t *c = a.w_codes + tile * a.w_ldc + unit * 4096 + 16 * lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) w.c[i] = *reinterpret_cast<const uint4 *>(c + 1024 * i);
    w.s = *reinterpret_cast<const uint2 *>(a.w_scales + tile * a.w_lds + unit * 512 + 8 * lane);
}

// ------------------------------------------------------------ activation operand
// The K range's operand lives in LDS as exact f16 values e*d in MFMA A-operand
// order: slot ((u * 16 + 4 i + j) * MT + mt) * 64 + 16 g + r holds row
// 16 mt + r, columns kbeg + 512 u + 128 g + 32 i + 8 j .. + 8 (u: 512-column
// unit, g: lane quarter, i: 32-column step, j: 8-column fragment). A "chunk" is
// 32 columns of one row, i.e. the four slots j = 0..3. The residue columns'
// operand is a second copy of the same layout, `slots` further on.

__device__ inline float scale_of(float amax) { return amax > 0.0f ? amax / 2688.0f : 1.0f; }

__device__ inline unsigned wave_max_u(unsigned v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (unsigned)__shfl_xor((int)v, o));
    return v;
}

// The workgroup's K range and its chunk counts.
// A load through the vector memory path: counted by vmcnt, in order with the
// weight loads, so it never holds up the scalar/LDS waits before the barriers
// (a scalar load of a value in HBM would: every lgkmcnt wait covers it).
__device__ inline float load_vmem(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Range {
    int64_t kbeg, kend, rend;   // columns [kbeg, kend); residue columns [kbeg, rend)
    int units, res_units;       // 512-column units of each
    int npm, npr;               // chunk positions per row (32 columns each)
};

// Operand layout (R rows per slot group): slot (((u * 4 + i) * 4 + j) * 4 + g) * R + rho
// holds operand row rho, columns kbeg + 512 u + 128 g + 32 i + 8 j .. + 8. The rows
// are the M activation rows (R = M), or -- residue columns with M <= 8 -- the M rows
// at 0.. and their residue rows at Mp.. (Mp = M rounded up to a power of two,
// R = 2 Mp): one 16-row MFMA then covers both, and output rows m and Mp + m are
// added when the tile is stored. This returns the slot of fragment j = 0 of the
// chunk of row rho starting at column kc; fragment j adds 4 R j.
__device__ inline int chunk_slot(int64_t kbeg, int R, int rho, int64_t kc) {
    const int off = (int)(kc - kbeg);
    const int u = off >> 9, w = (off >> 5) & 15;     // w = 4 g + i
    return ((u * 4 + (w & 3)) * 16 + (w >> 2)) * R + rho;
}

// Producer thread ptid takes operand row m = ptid % M and the chunk positions
// p0 + step t of the range (step = 256 / M, p0 = ptid / M): rows are fastest
// across a wave, so each load instruction covers consecutive columns of each
// row, and a thread's addresses need one division in all. Threads at or past
// M * step have no positions (p0 is set past every list).
struct PMap { int m, p0, step; };
__device__ inline PMap prod_map(int ptid, int M) {
    PMap r;
    r.step = kPThreads / M;
    r.m = ptid % M;
    r.p0 = ptid < M * r.step ? ptid / M : 1 << 20;
    return r;
}

// Chunk position pos of the range: 32 columns of one row; the npm main
// positions come first, then the npr residue positions. key = LDS slot of
// fragment j = 0, plus kV1 when the chunk's second 16-column block is inside
// the data; -1 past the list.
constexpr int kV1 = 1 << 30;
constexpr int kZS = 1 << 29;                   // key flag: the chunk lies past the data, store zeros
struct ChunkPos {
    int64_t col;   // stored column of the chunk start (residue columns follow column K)
    int key;
};

__device__ inline ChunkPos chunk_at(const DArgs &a, const Range &r, int m, int pos, int slots) {
    ChunkPos f;
    if (pos >= r.npm + r.npr) { f.col = 0; f.key = -1; return f; }
    const bool res = pos >= r.npm;
    const int lp = res ? pos - r.npm : pos;
    const int64_t kc = r.kbeg + 32 * (int64_t)lp;
    f.col = res ? a.K + kc : kc;
    // residue chunks: stacked rows Mp + m, or the second copy `slots` further on
    const int w = lp & 15;
    f.key = (((lp >> 4) * 4 + (w & 3)) * 16 + (w >> 2)) * a.Rr + (res && a.Mp ? a.Mp + m : m) +
            (res && !a.Mp ? slots : 0) + (kc + 16 < (res ? r.rend : r.kend) ? kV1 : 0);
    return f;
}

// A chunk of the quantized-activation buffer: 16 bytes of codes (low nibble =
// even column) and the two block scales.
struct QChunk { uint4 c; uint16_t s; int key; };   // s: the two block scales

// Every chunk starts at a multiple of 32 columns -- residue chunks at column
// K + kc, and the host sends residue columns here only when K is a multiple of
// 32 -- so a chunk is one 16-byte and one 2-byte load. Row-major rows hold at
// least as many bytes as their columns need, padded to multiples of 16 (codes)
// and 8 (scales), so both loads stay inside the row's pitch even where the
// second block lies past the data (those bytes are dropped when stored). Past
// the list it reads the row's start (dropped when stored).
__device__ inline QChunk qchunk_load(const uint8_t *crow, const uint8_t *srow, const ChunkPos &f) {
    QChunk q;
    q.key = f.key;
    q.c = *reinterpret_cast<const uint4 *>(crow + (f.col >> 1));
    q.s = *reinterpret_cast<const uint16_t *>(srow + (f.col >> 4));
    return q;
}

// Decode a chunk into its four fragments (j stride js = 4 R slots).
__device__ inline void qchunk_store(half8 *lds, int js, const QChunk &q) {
    if (q.key < 0) return;
    const bool v1 = q.key & kV1;
    const int slot = q.key & (kZS - 1);
    const uint32_t sv = (q.key & kZS) ? 0u : q.s;   // applied here, not at the load: no early wait
    const uint32_t s0 = sv & 0xFFu, s1 = sv >> 8;
    const half2v d0 = scale_pair(s0), d1 = scale_pair(v1 ? s1 : 0u);
    lds[slot] = decode8(q.c.x, d0);
    lds[slot + js] = decode8(q.c.y, d0);
    lds[slot + 2 * js] = decode8(v1 ? q.c.z : 0u, d1);
    lds[slot + 3 * js] = decode8(v1 ? q.c.w : 0u, d1);
}

// 32 bf16 activations of one row (a raw chunk); the second block is read only
// inside the data (else the first block again).
struct XChunk { uint4 w[4]; };

__device__ inline XChunk xchunk_load(const DArgs &a, int64_t m, int64_t kc, bool v1) {
    const uint16_t *row = static_cast<const uint16_t *>(a.x) + m * a.ldx;
    XChunk x;
    x.w[0] = *reinterpret_cast<const uint4 *>(row + kc);
    x.w[1] = *reinterpret_cast<const uint4 *>(row + kc + 8);
    x.w[2] = *reinterpret_cast<const uint4 *>(row + (v1 ? kc + 16 : kc));
    x.w[3] = *reinterpret_cast<const uint4 *>(row + (v1 ? kc + 24 : kc + 8));
    return x;
}

__device__ inline void bf16x16(const uint4 &p, const uint4 &q, float *v) {
    const uint32_t w[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = u2f(w[i] << 16);
        v[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
    }
}

// Quantize a raw chunk (row m, columns kc..) against S into its LDS slots and,
// for columns below the residue bound, the residue's slots; the writer also
// stores codes and scales into the quantized-activation buffer.
template <bool RES>
__device__ inline void xchunk_quantize(const DArgs &a, half8 *lds, int slots, int64_t kbeg, int64_t rend,
                                       int64_t m, int64_t kc, bool v1, const XChunk &x, float S, bool writer) {
    const float t = 6.0f * S;
    uint32_t mc[4] = {0, 0, 0, 0}, ms[2] = {0, 0}, rc[4] = {0, 0, 0, 0}, rs[2] = {0, 0};
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        if (b == 1 && !v1) break;
        float v[16];
        bf16x16(x.w[2 * b], x.w[2 * b + 1], v);
        uint32_t cw[2];
        float d;
        ms[b] = encode_block(v, S, t, cw, d);
        mc[2 * b] = cw[0];
        mc[2 * b + 1] = cw[1];
        if (RES && kc + 16 * b < rend) {
            block_residue(v, cw, d, S, v);          // element-wise, in place
            rs[b] = encode_block(v, S, t, cw, d);
            rc[2 * b] = cw[0];
            rc[2 * b + 1] = cw[1];
        }
    }
    const int js = 4 * a.Rr;
    const int slot = chunk_slot(kbeg, a.Rr, (int)m, kc);
    const int rslot = a.Mp ? chunk_slot(kbeg, a.Rr, a.Mp + (int)m, kc) : slots + slot;
    {
        const half2v d0 = scale_pair(ms[0]), d1 = scale_pair(ms[1]);
#pragma unroll
        for (int j = 0; j < 4; ++j) lds[slot + j * js] = decode8(mc[j], j < 2 ? d0 : d1);
    }
    const bool has_res = RES && kc < rend;
    if (has_res) {
        const half2v d0 = scale_pair(rs[0]), d1 = scale_pair(rs[1]);
#pragma unroll
        for (int j = 0; j < 4; ++j) lds[rslot + j * js] = decode8(rc[j], j < 2 ? d0 : d1);
    }
    if (writer) {
        uint8_t *crow = a.q_codes + m * a.q_ldc;
        uint8_t *srow = a.q_scales + m * a.q_lds;
        unsigned long long *cp = reinterpret_cast<unsigned long long *>(crow + kc / 2);
        cp[0] = (unsigned long long)mc[0] | ((unsigned long long)mc[1] << 32);
        srow[kc / 16] = (uint8_t)ms[0];
        if (v1) {
            cp[1] = (unsigned long long)mc[2] | ((unsigned long long)mc[3] << 32);
            srow[kc / 16 + 1] = (uint8_t)ms[1];
        }
        if (has_res) {
            unsigned long long *rp = reinterpret_cast<unsigned long long *>(crow + (a.K + kc) / 2);
            rp[0] = (unsigned long long)rc[0] | ((unsigned long long)rc[1] << 32);
            srow[(a.K + kc) / 16] = (uint8_t)rs[0];
            if (kc + 16 < rend) {
                rp[1] = (unsigned long long)rc[2] | ((unsigned long long)rc[3] << 32);
                srow[(a.K + kc) / 16 + 1] = (uint8_t)rs[1];
            }
        }
    }
}

// Zero the operand slots that no chunk writes: chunk positions past the data
// at the end of a ragged range, for the M activation rows and the residue rows
// (LDS only; producer waves). Padding rows between them are never read into a
// stored output row and stay as they are.
__device__ inline void zero_unwritten(half8 *lds, const DArgs &a, const Range &r, int slots) {
    const int ptid = (int)threadIdx.x - 64 * kCons;
    const int M = (int)a.M, R = a.Rr;
    const half8 z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int reg = 0; reg < 2; ++reg) {
        const int first = reg == 0 ? r.npm : r.npr;                     // first position past the data
        // stacked residue rows span every unit of the range; a separate copy only its own
        const int npos = (reg == 0 || a.Mp ? r.units : r.res_units) * 16;
        half8 *base = lds + (reg == 1 && !a.Mp ? slots : 0);
        const int row0 = reg == 1 && a.Mp ? a.Mp : 0;
        const int total = (npos - first) * 4 * M;                        // (position, j, row)
        for (int e = ptid; e < total; e += kPThreads) {
            const int m = e % M, rest = e / M, j = rest & 3, pos = first + (rest >> 2);
            const int u = pos >> 4, w = pos & 15;
            base[(((u * 4 + (w & 3)) * 4 + j) * 4 + (w >> 2)) * R + row0 + m] = z;
        }
    }
}

// ---------------------------------------------------------------- kernel
// STK: residue rows stacked under the activation rows (RES; M <= 8 in one row
// tile, or M = 9..16 as a second row tile); an instance of its own, so that its
// MFMA loop carries no residue branch.
template <int MT, bool RES, bool TILED, bool STK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void decode_kernel(DArgs a) {
    constexpr int kRing = MT == 1 ? 4 : 3;       // weight items in flight per consumer wave
    // Items issued before the operand barrier; the rest of the ring is issued
    // after it, so that computing on landed items overlaps the (throttled)
    // issue of later loads.
    constexpr int kPre = kPreItems < kRing ? kPreItems : kRing;
    extern __shared__ half8 lds_a[];          // operand [U][4 i][4 j][4 g][M] (+ residue copy); then tile sums
    __shared__ float sh_S, sh_wS;             // activation and weight tensor scales
    __shared__ float sh_part[kProd];
    __shared__ unsigned sh_cnt;
    __shared__ int sh_last;
    // wave index as a scalar: branches on it are uniform (barriers inside them stay per wave)
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r16 = lane & 15;
    const int M = (int)a.M;
    const int p = blockIdx.x % a.P;
    const int64_t q = blockIdx.x / a.P;
    Range rg;
    rg.kbeg = (int64_t)p * a.U * 512;
    rg.kend = rg.kbeg + (int64_t)a.U * 512 < a.K ? rg.kbeg + (int64_t)a.U * 512 : a.K;
    rg.units = (int)((rg.kend - rg.kbeg + 511) / 512);
    rg.rend = RES ? (a.res_cols < rg.kend ? a.res_cols : rg.kend) : rg.kbeg;
    if (rg.rend < rg.kbeg) rg.rend = rg.kbeg;
    rg.res_units = (int)((rg.rend - rg.kbeg + 511) / 512);
    rg.npm = (int)((rg.kend - rg.kbeg + 31) / 32);
    rg.npr = (int)((rg.rend - rg.kbeg + 31) / 32);
    const int64_t kbeg = rg.kbeg;
    const int units = rg.units, res_units = rg.res_units;
    const int R = a.Rr;                          // operand rows per slot group
    const int slots = a.U * 64 * R;              // operand slots of a full range; a residue copy follows
    const int64_t t_lo = q * a.T, t_hi = (q + 1) * a.T < a.NT ? (q + 1) * a.T : a.NT;

    // Consumer wave w takes tiles t_lo + w / KW + TW i_t (i_t < ntw) and units
    // w % KW + KW i_u (i_u < nuw) of the range: KW waves share each tile, each
    // summing its own units, and their parts are added in LDS at the end.
    // KW is 1, 2 or 4: shifts and masks instead of divisions (a 64-bit
    // division alone is ~130 scalar instructions ahead of the first load)
    const int KW = a.KW, kwl = KW >> 1, TW = kCons >> kwl;
    const int tg = wave >> kwl, uo = wave & (KW - 1);
    const int nt_wg = (int)(t_hi - t_lo);
    const int ntw = (wave < kCons && tg < nt_wg) ? (nt_wg - tg + TW - 1) >> (2 - kwl) : 0;
    const int nuw = (wave < kCons && uo < units) ? (units - uo + KW - 1) >> kwl : 0;
    const int nitems = ntw * nuw;
    // Item it = (tile i_t = it / nuw, unit i_u = it % nuw), it < kMaxItems (the
    // quotient by comparisons: no division); tiles and rows are clamped into
    // W, so loads never leave it.
    // spare: a ring slot past the wave's last item still takes the same five
    // loads (so vmcnt counts stay exact), every lane from W's first bytes: one
    // line per load, a cache hit after the first
    auto load_item = [&](int it, WLoad &w, bool spare) {
        int at = 0;
#pragma unroll
        for (int k = 1; k < kMaxItems; ++k) at += it >= k * nuw ? 1 : 0;
        const int bu = it - at * nuw;
        const int64_t t = t_lo + tg + (int64_t)TW * at;
        const int64_t ul = uo + (int64_t)KW * bu;
        if (TILED) {
            load_w_tiled(a, spare ? 0 : (t < a.NT ? t : a.NT - 1), spare ? 0 : kbeg / 512 + ul, spare ? 0 : lane, w);
        } else {
            const int64_t n = 16 * t + r16;
            load_w(a, spare ? 0 : (n < a.N ? n : a.N - 1), spare ? 0 : kbeg + 512 * ul, spare ? 0 : g, w);
        }
    };

    // The two kinds of wave meet at two workgroup barriers (the producers'
    // loads are out; the operand is complete); the producers' work sits in its
    // own branch so that it never shares registers with the consumers' loads in
    // flight.
    TL(0);
    WLoad ring[kRing];
    if (tid == 0) sh_cnt = 0;
    if (wave < kCons) {
        // Ordered launches wait until the producers' loads are out, so that the
        // operand lands ahead of the weight stream (LOCAL always: the barrier
        // also orders the counter reset above before the producers' arrivals).
        // Otherwise the producers' few loads race the consumers' first items.
        if (a.ordered) __syncthreads();
        if (nitems > 0) {
#pragma unroll
            for (int s = 0; s < kPre; ++s) load_item(s < nitems ? s : 0, ring[s], s >= nitems);
        }
        TL(1);
        __syncthreads();                       // operand complete
    } else {
        const int ptid = tid - 64 * kCons, pw = wave - kCons;
        if (a.mode == MODE_PRE) {
            // the thread's chunk positions of the quantized activations, kPreChunks
            // before the barrier; larger ranges take further batches after it
            const PMap pm = prod_map(ptid, M);
            const uint8_t *crow = a.q_codes + (int64_t)pm.m * a.q_ldc;
            const uint8_t *srow = a.q_scales + (int64_t)pm.m * a.q_lds;
            const int npos = rg.npm + rg.npr;
            // A wave whose first position (lane 0's) is past the list holds no chunk
            // and issues nothing; the others issue the whole batch back to back. The
            // two paths share no values (each meets the barrier itself), so nothing
            // loaded has to be settled where they join.
            float S = 0.0f, wS = 0.0f;
            // Chunk t of the thread is position p0 + step t. Without residue
            // columns and with step a multiple of 16 (M divides 16) its unit and
            // 32-column step advance by constants: the addresses and the LDS key
            // are affine in t and need no per-chunk branch (`affine`); otherwise
            // chunk_at places every position. The two forms are separate paths
            // around the whole batch loop, so no load is settled where they join.
            const int klen = (int)(rg.kend - rg.kbeg);
            const int w0 = pm.p0 & 15;
            const int key0 = (((pm.p0 >> 4) * 4 + (w0 & 3)) * 16 + (w0 >> 2)) * R + pm.m;
            const int dkey = (pm.step >> 4) * 64 * R;
            const int cbase = (int)(rg.kbeg >> 1), sbase = (int)(rg.kbeg >> 4);
            auto chunk = [&](int tt, auto affine) {
                if constexpr (decltype(affine)::value) {
                    const int pos = pm.p0 + pm.step * tt;
                    const bool ok = pos < rg.npm;
                    QChunk q;
                    q.c = *reinterpret_cast<const uint4 *>(crow + (ok ? cbase + 16 * pos : 0));
                    q.s = *reinterpret_cast<const uint16_t *>(srow + (ok ? sbase + 2 * pos : 0));
                    q.key = ok ? key0 + dkey * tt + (32 * pos + 16 < klen ? kV1 : 0) : -1;
                    return q;
                } else {
                    return qchunk_load(crow, srow, chunk_at(a, rg, pm.m, pm.p0 + pm.step * tt, slots));
                }
            };
            auto pre_body = [&](auto affine) {
                if (__builtin_amdgcn_readfirstlane(pm.p0) < npos) {
                    QChunk qc[kPreChunks];
#pragma unroll
                    for (int t = 0; t < kPreChunks; ++t) qc[t] = chunk(t, affine);
                    if (a.ordered) __syncthreads();    // loads out: consumers may issue theirs
                    // the two tensor scales (lane 0 of the first producer wave, which
                    // always holds chunks), after the batch is out
                    if (ptid == 0) { S = load_vmem(a.q_S); wS = load_vmem(a.w_S); }
                    zero_unwritten(lds_a, a, rg, slots);
#pragma unroll
                    for (int t = 0; t < kPreChunks; ++t) qchunk_store(lds_a, 4 * R, qc[t]);
                    for (int b = kPreChunks; pm.p0 + pm.step * b < npos; b += kPreChunks) {
#pragma unroll
                        for (int t = 0; t < kPreChunks; ++t) qc[t] = chunk(b + t, affine);
#pragma unroll
                        for (int t = 0; t < kPreChunks; ++t) qchunk_store(lds_a, 4 * R, qc[t]);
                    }
                } else {
                    if (a.ordered) __syncthreads();
                    zero_unwritten(lds_a, a, rg, slots);
                }
            };
            if (!RES && (pm.step & 15) == 0) pre_body(std::true_type{});
            else pre_body(std::false_type{});
            if (ptid == 0) { sh_S = S; sh_wS = wS; }
            TL(1);
            __syncthreads();                   // operand complete
        } else {
            // LOCAL: the thread's main chunk positions p0 + step t (t < kLocalChunks;
            // the plan makes them cover the range). When the range is all of K
            // (P == 1) they are all of X and give amax(X) directly; otherwise each
            // producer wave also reads its quarter of X for amax, in batches of
            // kLocalLoads loads per lane (the first before the barrier).
            const PMap pm = prod_map(ptid, M);
            const bool full = a.P == 1;
            // chunk slots of this wave that hold a chunk for some lane (wave-uniform);
            // a lane past its list in such a slot reads its row's start, which leaves
            // amax(X) unchanged; empty slots issue no loads and stay zero
            const int p0w = __builtin_amdgcn_readfirstlane(pm.p0);
            const int nt = p0w < rg.npm ? (rg.npm - p0w + pm.step - 1) / pm.step : 0;
            XChunk xc[kLocalChunks];
#pragma unroll
            for (int t = 0; t < kLocalChunks; ++t) {
                xc[t] = XChunk{};
                if (t < nt) {
                    const int pos = pm.p0 + pm.step * t;
                    const ChunkPos f = chunk_at(a, rg, pm.m, pos < rg.npm ? pos : 1 << 20, slots);
                    xc[t] = xchunk_load(a, pm.m, f.col, f.key >= 0 && (f.key & kV1));
                }
            }
            const float wS = ptid == 0 ? load_vmem(a.w_S) : 0.0f;   // behind the chunk loads
            // 16-byte units of X: M K / 8 <= 4096 here, so 32-bit indices
            const int NU = (int)(a.M * (a.K / 8));
            const int u0 = NU * pw / kProd, u1 = NU * (pw + 1) / kProd;
            const uint32_t KU = (uint32_t)(a.K / 8);
            const uint16_t *xb = static_cast<const uint16_t *>(a.x);
            auto amax_batch = [&](int base, uint4 *av) {
#pragma unroll
                for (int t = 0; t < kLocalLoads; ++t) {
                    const int idx = base + lane + 64 * t < u1 ? base + lane + 64 * t : u0;
                    const uint32_t row = (uint32_t)idx / KU, cu = (uint32_t)idx - row * KU;
                    av[t] = *reinterpret_cast<const uint4 *>(xb + (int64_t)row * a.ldx + 8 * (int64_t)cu);
                }
            };
            // for finite values the order of |bf16| bit patterns is that of the magnitudes
            auto bits_max = [](unsigned mx, const uint4 &v) {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) mx = max(mx, max(w[e] & 0x7FFFu, (w[e] >> 16) & 0x7FFFu));
                return mx;
            };
            uint4 av[kLocalLoads];
            if (!a.static_S && !full) amax_batch(u0, av);
            __syncthreads();                   // loads out: consumers may issue theirs
            zero_unwritten(lds_a, a, rg, slots);
            if (!a.static_S) {
                unsigned mx = 0;
                if (full) {
#pragma unroll
                    for (int t = 0; t < kLocalChunks; ++t)
#pragma unroll
                        for (int h = 0; h < 4; ++h) mx = bits_max(mx, xc[t].w[h]);
                } else {
#pragma unroll
                    for (int t = 0; t < kLocalLoads; ++t) mx = bits_max(mx, av[t]);
                    for (int base = u0 + 64 * kLocalLoads; base < u1; base += 64 * kLocalLoads) {
                        amax_batch(base, av);
#pragma unroll
                        for (int t = 0; t < kLocalLoads; ++t) mx = bits_max(mx, av[t]);
                    }
                }
                mx = wave_max_u(mx);
                if (lane == 0) {
                    sh_part[pw] = u2f(mx << 16);
                    __hip_atomic_fetch_add(&sh_cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
                }
                // the producers alone meet here: the consumers may still be issuing loads
                while (__hip_atomic_load(&sh_cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < (unsigned)kProd)
                    __builtin_amdgcn_s_sleep(1);
            }
            float S;
            if (a.static_S) {
                S = *a.static_S;
            } else {
                float m = 0.0f;
#pragma unroll
                for (int w = 0; w < kProd; ++w) m = fmaxf(m, sh_part[w]);
                S = scale_of(m);
            }
            if (blockIdx.x == 0 && ptid == 0) *a.q_S = S;
            if (ptid == 0) { sh_S = S; sh_wS = wS; }
#pragma unroll
            for (int t = 0; t < kLocalChunks; ++t) {
                const int pos = pm.p0 + pm.step * t;
                if (pos < rg.npm) {
                    const ChunkPos f = chunk_at(a, rg, pm.m, pos, slots);
                    xchunk_quantize<RES>(a, lds_a, slots, kbeg, rg.rend, pm.m, f.col, (f.key & kV1) != 0, xc[t], S,
                                         q == 0);
                }
            }
            TL(1);
            __syncthreads();                   // operand complete
        }
    }
    TL(2);

    // ---- consumers: decode weights, MFMA
    const float scale = sh_S * sh_wS;
    // Output tile t of this workgroup: lane holds rows 16 mt + 4 g + e of column
    // 16 t + r16; only rows < M are stored.
    auto store_tile = [&](int64_t t, const float4v *vin) {
        float4v v[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) v[mt] = vin[mt];
        if constexpr (STK && MT == 2) {
            // stacked residue, M = 9..16: the residue rows are the second row tile
            v[0] += v[MT - 1];
        } else if constexpr (STK) {
            // stacked residue (MT == 1): output row m += row Mp + m. Row 4 g + e sits
            // in lane group g, element e; Mp >= 4 puts the residue row in lane + 4 Mp.
            const int mp = a.Mp;
            float4v o;
            if (mp >= 4) {
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = __shfl(v[0][e], (lane + 4 * mp) & 63);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = e + mp < 4 ? v[0][(e + mp) & 3] : 0.0f;
            }
            v[0] += o;
        }
        const int64_t n = 16 * t + r16;
        if (n >= a.N) return;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = 16 * mt + 4 * g + e;
                if (m < a.M) {
                    if (a.P == 1) {
                        const float val = v[mt][e] * scale;
                        if (a.yt == 1) static_cast<float *>(a.y)[m * a.ldy + n] = val;
                        else static_cast<uint16_t *>(a.y)[m * a.ldy + n] = f32_to_bf16_rne(val);
                    } else {
                        st_dev(&a.partials[((int64_t)p * a.M + m) * a.N + n], v[mt][e]);
                    }
                }
            }
    };
    // A-operand rows 16 mt + r16 >= R read row R - 1 instead: the MFMA output
    // rows they feed are never stored.
    int arow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) arow[mt] = 16 * mt + r16 < R ? 16 * mt + r16 : R - 1;
    float4v ts0[MT], ts1[MT];                  // this wave's parts of its first two tiles (KW > 1)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) { ts0[mt] = float4v{0, 0, 0, 0}; ts1[mt] = float4v{0, 0, 0, 0}; }
    if (wave < kCons && nitems > 0) {            // waves without items issue no loads at all
        // independent MFMA chains: even / odd fragments, and (MT == 1; for MT == 2 the
        // registers are not there) the residue columns' own two
        constexpr bool kSepRes = RES && !STK && MT == 1;
        float4v acc[MT], acc2[MT], accr[1], accr2[1];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) { acc[mt] = float4v{0, 0, 0, 0}; acc2[mt] = float4v{0, 0, 0, 0}; }
#pragma unroll
        for (int mt = 0; mt < 1; ++mt) { accr[mt] = float4v{0, 0, 0, 0}; accr2[mt] = float4v{0, 0, 0, 0}; }
#pragma unroll
        for (int s = kPre; s < kRing; ++s) load_item(s < nitems ? s : 0, ring[s], s >= nitems);
        // Fully unrolled over NI = kMaxItems items (no loop back-edge): each slot
        // is consumed in place and refilled right after, always with the same
        // five loads (spare ones past the wave's last item), so vmcnt is tracked
        // exactly. One loop shape serves every plan: a second instance for plans
        // whose items fit the ring saved its spare loads but cost ~2 us at every
        // switch between the two instances in a sequence of calls (their code is
        // fetched again), more than it saved.
        auto run = [&](auto ni) {
            constexpr int NI = decltype(ni)::value;
            int at = 0, bu = 0;                    // tile and unit of the current item (wave-uniform)
#pragma unroll
            for (int it = 0; it < NI; ++it) {
                const int s = it % kRing;
                if (it < nitems) {
                    const int ul = uo + KW * bu;
                    const half8 *abase = lds_a + ul * 64 * R + g * R;
                    const bool res_u = RES && !STK && ul < res_units;   // a separate residue copy
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t sw = (i < 2) ? ring[s].s.x : ring[s].s.y;
                        const half2v d0 = scale_pair((sw >> (16 * (i & 1))) & 0xFFu);
                        const half2v d1 = scale_pair((sw >> (16 * (i & 1) + 8)) & 0xFFu);
                        const uint32_t cws[4] = {ring[s].c[i].x, ring[s].c[i].y, ring[s].c[i].z, ring[s].c[i].w};
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const half8 b = decode8(cws[j], j < 2 ? d0 : d1);
                            const int fo = (4 * i + j) * 4 * R;
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) {
                                float4v &ac = (j & 1) ? acc2[mt] : acc[mt];
                                ac = __builtin_amdgcn_mfma_f32_16x16x32_f16(abase[fo + arow[mt]], b, ac, 0, 0, 0);
                                if (RES && res_u) {
                                    float4v &ar = kSepRes ? ((j & 1) ? accr2[0] : accr[0]) : ac;
                                    ar = __builtin_amdgcn_mfma_f32_16x16x32_f16(abase[slots + fo + arow[mt]], b, ar,
                                                                                0, 0, 0);
                                }
                            }
                        }
                    }
                    if (bu == nuw - 1) {
                        // this wave's part of tile t_lo + tg + TW at is complete
                        float4v tot[MT];
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
                            tot[mt] = acc[mt] + acc2[mt];
                            if (kSepRes) tot[mt] += accr[0] + accr2[0];
                        }
                        if (KW == 1) {
                            store_tile(t_lo + tg + (int64_t)TW * at, tot);
                        } else if (at == 0) {
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) ts0[mt] = tot[mt];
                        } else {
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) ts1[mt] = tot[mt];
                        }
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) { acc[mt] = float4v{0, 0, 0, 0}; acc2[mt] = float4v{0, 0, 0, 0}; }
                        accr[0] = float4v{0, 0, 0, 0};
                        accr2[0] = float4v{0, 0, 0, 0};
                        bu = 0;
                        ++at;
                    } else {
                        ++bu;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);   // items stay in order (no hoisted decodes)
                if (it + kRing < NI) {
                    const bool spare = it + kRing >= nitems;
                    load_item(spare ? 0 : it + kRing, ring[s], spare);   // consume slot s, then refill it
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        run(std::integral_constant<int, kMaxItems>{});
    }

    // ---- tiles shared by KW waves: their parts are added in LDS, in wave order
    if (a.KW > 1) {
        __syncthreads();                       // every consumer is done with the operand
        float4v *red = reinterpret_cast<float4v *>(lds_a);   // [2 tiles][kCons][MT][64]
        if (wave < kCons && nitems > 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                red[((0 * kCons + wave) * MT + mt) * 64 + lane] = ts0[mt];
                if (ntw > 1) red[((1 * kCons + wave) * MT + mt) * 64 + lane] = ts1[mt];
            }
        }
        __syncthreads();
        if (wave < kCons && uo == 0) {
            for (int at = 0; at < ntw && at < 2; ++at) {
                float4v sum[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) sum[mt] = float4v{0, 0, 0, 0};
                for (int k = 0; k < KW && k < units; ++k) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) sum[mt] += red[((at * kCons + tg * KW + k) * MT + mt) * 64 + lane];
                }
                store_tile(t_lo + tg + (int64_t)TW * at, sum);
            }
        }
    }

    TL(3);
    // ---- split-K combine by the last workgroup of the tile group
    if (a.P > 1) {
        wait_own_stores();                     // this wave's partial tiles are visible
        __syncthreads();
        unsigned *tile_cnt = reinterpret_cast<unsigned *>(a.header + kTileCntOffset);
        if (threadIdx.x == 0) sh_last = add_dev(&tile_cnt[q], 1u) == (unsigned)a.P - 1;
        __syncthreads();
        if (sh_last) {
            const int64_t ncols = (t_hi - t_lo) * 16;   // multiple of 16: whole column pairs
            const bool pairs = (a.N & 1) == 0;
            for (int64_t idx = threadIdx.x; idx < a.M * (ncols / 2); idx += kThreads) {
                const int64_t m = idx / (ncols / 2), n = 16 * t_lo + 2 * (idx - m * (ncols / 2));
                if (n >= a.N) continue;
                float s0 = 0.0f, s1 = 0.0f;
                // kMaxP partials loaded at once, then added in order p = 0, 1, ...
                for (int p0 = 0; p0 < a.P; p0 += kMaxP) {
                    float v0[kMaxP], v1[kMaxP];
#pragma unroll
                    for (int k = 0; k < kMaxP; ++k) {
                        v0[k] = 0.0f;
                        v1[k] = 0.0f;
                        if (p0 + k < a.P) {
                            const float *src = &a.partials[((int64_t)(p0 + k) * a.M + m) * a.N + n];
                            if (pairs) {
                                const unsigned long long v = ld_dev(reinterpret_cast<const unsigned long long *>(src));
                                v0[k] = u2f((uint32_t)v);
                                v1[k] = u2f((uint32_t)(v >> 32));
                            } else {
                                v0[k] = ld_dev(src);
                                if (n + 1 < a.N) v1[k] = ld_dev(src + 1);
                            }
                        }
                    }
#pragma unroll
                    for (int k = 0; k < kMaxP; ++k)
                        if (p0 + k < a.P) { s0 += v0[k]; s1 += v1[k]; }
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
    TL(4);
}

// ---------------------------------------------------------------- M = 33..64
// Four row tiles take 64 rows x 1 KiB of operand per 512-column unit, so a
// whole K range does not fit in LDS. Here the operand streams through a window
// of two unit slots instead: a workgroup owns four 16-row weight tiles over all
// of K (no split-K across workgroups). Its eight consumer waves, two per SIMD,
// split each unit by 32-column step (wave w % 4) and weight-tile pair (w / 4),
// for all four row tiles, so each weight item is loaded and decoded once and each
// operand fragment read twice per CU (against a wave per weight tile: operand
// reads / 2, the M = 64 augmented call 35.4 -> 28.3 us with the deeper weight
// ring; eight waves instead of four one step each: 28.5 -> 28.0 us; eight producer
// waves instead of four, each two chunks of a unit: 27.7 -> 27.0 us); the waves'
// partial tiles are added in LDS in step order at the end; producers fill the slot of unit k + 2
// as soon as the consumers are done with unit k, one workgroup barrier per
// unit (weight loads run four units ahead, operand loads three). Residue columns (ARCQuant
// article, sections 3.1-3.2) are further
// "virtual units" after the K / 512 main ones: their operand is the residue
// rows, their weights W's first units again (read a second time: S / K more
// weight bytes, against twice the LDS for a second operand copy).
//
// Barriers: both kinds of wave pass exactly NV + 3 = KU + RU + 3 of them (the
// last two around the consumers' partial sums). The
// first: the producers' loads of units 0..2 are out, so the consumers' weight
// loads queue behind them (measured: the first units land ~1.9 us earlier, the
// M = 64 product 4% faster). Barrier 0: units 0 and 1 are in their slots.
// Barrier k >= 1: the consumers are done with unit k - 1, and the producers
// have stored unit k (k >= 2) into the slot unit k - 2 left. Consumers work on
// unit k between barriers k and k + 1.
constexpr int kWinProd = 8;                    // producer waves of the windowed kernel
constexpr int kWinPThreads = 64 * kWinProd;
constexpr int kWinChunks = 64 * 16 / kWinPThreads;   // operand chunks per producer thread and unit (64 x 16 in all)
constexpr int kWinRows = 64;                   // operand rows of a window slot: fixed, so every fragment
                                               // offset is an immediate of the LDS read

// A producer thread's chunks of a unit: rows m_i = ptid / 16 + (kWinPThreads /
// 16) i (i < kWinChunks), 32-column position p = ptid % 16 in every unit. Their row
// addresses and LDS keys are fixed; a unit only adds its byte offsets, so a
// chunk costs two address adds, its two loads and a few selects. Rows >= M
// read row 0 and are not stored (key -1); a position past the data (the last,
// partial unit) reads the unit's start and stores a zero chunk (scale 0).
//
// Row swizzle: in the slot group of position p = (32-column step s, lane
// quarter g), row m sits at row (m + g + 4 s) mod 64. The 16 lanes of a store
// phase hold one row at the 16 positions of a unit; unswizzled their slots lie
// 1 KiB apart, all in the same LDS banks (counters: a third of the kernel's
// cycles were bank conflicts); swizzled they are 16 consecutive slots. The
// consumers read row r of their fragments at (r + g + 4 s) mod 64, still 16
// consecutive slots per read phase.
struct WinRows {
    const uint8_t *c[kWinChunks], *s[kWinChunks];
    int key[kWinChunks];                       // LDS key of the chunk, -1 for rows >= M
    int p;
};

__device__ inline WinRows win_rows(const DArgs &a, int ptid) {
    WinRows w;
    w.p = ptid & 15;
#pragma unroll
    for (int i = 0; i < kWinChunks; ++i) {
        const int m = (ptid >> 4) + (kWinPThreads / 16) * i;
        const bool ok = m < a.M;
        w.c[i] = a.q_codes + (int64_t)(ok ? m : 0) * a.q_ldc + 16 * w.p;
        w.s[i] = a.q_scales + (int64_t)(ok ? m : 0) * a.q_lds + 2 * w.p;
        const int sw = (w.p >> 2) + 4 * (w.p & 3);
        w.key[i] = ok ? ((w.p & 3) * 16 + (w.p >> 2)) * kWinRows + ((m + sw) & (kWinRows - 1)) : -1;
    }
    return w;
}

template <bool RES>
__device__ inline void win_unit_load(const DArgs &a, const WinRows &w, int v, int KU, QChunk *q) {
    const bool resv = RES && v >= KU;
    const int u = resv ? v - KU : v;
    const int64_t lim = resv ? a.res_cols : a.K;
    const int64_t cend = lim < 512 * (int64_t)u + 512 ? lim : 512 * (int64_t)u + 512;
    const int64_t kc = 512 * (int64_t)u + 32 * w.p;               // operand column of the chunk
    const bool in = kc < cend, v1 = kc + 16 < cend;
    const int64_t coff = in ? (resv ? a.K / 2 : 0) + 256 * (int64_t)u : 0;
    const int64_t soff = in ? (resv ? a.K / 16 : 0) + 32 * (int64_t)u : 0;
#pragma unroll
    for (int i = 0; i < kWinChunks; ++i) {
        q[i].c = *reinterpret_cast<const uint4 *>(w.c[i] + coff);
        q[i].s = *reinterpret_cast<const uint16_t *>(w.s[i] + soff);
        q[i].key = w.key[i] < 0 ? -1 : w.key[i] + (v1 ? kV1 : 0) + (in ? 0 : kZS);
    }
}

// Eight consumer waves (two per SIMD, so that one's MFMAs run while the other
// decodes or waits) and eight producer waves: sixteen waves, 128 VGPRs each.
constexpr int kWinCons = 8;
constexpr int kWinTW = 4 * kCons / kWinCons;   // weight tiles per consumer wave
constexpr int kWinThreads = 64 * (kWinCons + kWinProd);

// A consumer's share of one unit: 32-column step iw of each of its weight tiles.
struct WStep {
    uint4 c[kWinTW];
    uint16_t s[kWinTW];                        // the step's two E4M3 bytes per tile
};

template <bool TILED, bool RES>
__global__ __launch_bounds__(kWinThreads) __attribute__((amdgpu_waves_per_eu(4)))   // 128 KiB of LDS: one per CU
void decode_win_kernel(DArgs a) {
    constexpr int R = kWinRows, SLOT = 64 * kWinRows;
    extern __shared__ half8 lds_a[];           // [2 slots][64 R]: rows >= M are never read
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r16 = lane & 15;
    const int M = (int)a.M;
    const int KU = (int)((a.K + 511) / 512), RU = RES ? (int)((a.res_cols + 511) / 512) : 0, NV = KU + RU;

    TL(0);
    if (wave < kWinCons) {
        // ---- consumer: 32-column step iw = wave % 4 of every (virtual) unit, for
        // weight tiles kWinTW (wave / 4) .. of the workgroup's four and all four row
        // tiles: each weight item is loaded and decoded once per workgroup and each
        // operand fragment read by 4 / kWinTW waves; the waves' partial tiles are added
        // in LDS at the end
        const int iw = wave & 3;
        const int64_t tb = 4 * (int64_t)blockIdx.x + kWinTW * (wave >> 2);
        int64_t tcl[kWinTW];                   // tiles clamped into W (tiles past it are not stored)
#pragma unroll
        for (int tt = 0; tt < kWinTW; ++tt) tcl[tt] = tb + tt < a.NT ? tb + tt : a.NT - 1;
        const float qS = load_vmem(a.q_S), wS = load_vmem(a.w_S);   // first: no wait holds a weight load on them
        auto issue = [&](int v, WStep &w) {
            const int64_t wu = v < KU ? v : v - KU;
#pragma unroll
            for (int tt = 0; tt < kWinTW; ++tt) {
                if (TILED) {
                    // step iw of the item is its own contiguous KiB; its two scale bytes
                    // sit at 2 iw in the lane's eight
                    w.c[tt] = *reinterpret_cast<const uint4 *>(a.w_codes + tcl[tt] * a.w_ldc + wu * 4096 +
                                                               1024 * iw + 16 * lane);
                    w.s[tt] = *reinterpret_cast<const uint16_t *>(a.w_scales + tcl[tt] * a.w_lds + wu * 512 +
                                                                   8 * lane + 2 * iw);
                } else {
                    const int64_t n0 = 16 * tcl[tt] + r16, n = n0 < a.N ? n0 : a.N - 1;
                    const int64_t ki = 512 * wu + 128 * g + 32 * iw;
                    w.c[tt] = *reinterpret_cast<const uint4 *>(a.w_codes + n * a.w_ldc + (ki < a.K ? ki / 2 : 0));
                    w.s[tt] = *reinterpret_cast<const uint16_t *>(a.w_scales + n * a.w_lds + (ki < a.K ? ki / 16 : 0));
                }
            }
        };
        int arow[4];                           // swizzled row of row tile mt in step iw
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            arow[mt] = ((16 * mt + r16 < M ? 16 * mt + r16 : M - 1) + g + 4 * iw) & (kWinRows - 1);
        float4v acc[kWinTW][4];                // [weight tile][row tile]
#pragma unroll
        for (int tt = 0; tt < kWinTW; ++tt)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) acc[tt][mt] = float4v{0, 0, 0, 0};
        WStep ring0, ring1, ring2, ring3;      // units v .. v + 3 in flight (v mod 4)
        __syncthreads();                       // the producers' first activation loads are out
        issue(0, ring0);
        if (NV > 1) issue(1, ring1);
        if (NV > 2) issue(2, ring2);
        if (NV > 3) issue(3, ring3);
        __syncthreads();                       // barrier 0: units 0 and 1 are in their slots
        TL(1);
        auto step = [&](int v, WStep &w) {
            const half8 *abase = lds_a + (v & 1) * SLOT + g * R;
            half2v d[kWinTW][2];
#pragma unroll
            for (int tt = 0; tt < kWinTW; ++tt) {
                d[tt][0] = scale_pair(w.s[tt] & 0xFFu);
                d[tt][1] = scale_pair((uint32_t)w.s[tt] >> 8);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                half8 b[kWinTW];
#pragma unroll
                for (int tt = 0; tt < kWinTW; ++tt) {
                    const uint32_t cw = j == 0 ? w.c[tt].x : j == 1 ? w.c[tt].y : j == 2 ? w.c[tt].z : w.c[tt].w;
                    b[tt] = decode8(cw, d[tt][j >> 1]);
                }
                const int fo = (4 * iw + j) * 4 * R;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const half8 av = abase[fo + arow[mt]];
#pragma unroll
                    for (int tt = 0; tt < kWinTW; ++tt)
                        acc[tt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b[tt], acc[tt][mt], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);   // one 8-column fragment's operands live at a time
            }
            if (v + 4 < NV) issue(v + 4, w);
            if (v + 1 < NV) __syncthreads();   // barrier v + 1: done with unit v
            if (v == 2) TL(2);
            if (v == 5) TL(3);
        };
        for (int v = 0; v < NV; v += 4) {
            step(v, ring0);
            if (v + 1 < NV) step(v + 1, ring1);
            if (v + 2 < NV) step(v + 2, ring2);
            if (v + 3 < NV) step(v + 3, ring3);
        }
        TL(4);
        // the waves' partial tiles, parked in the operand slots and added in step order:
        // tile t's parts are held by waves 4 (t / kWinTW) + iw, iw = 0..3, at index
        // (t % kWinTW) 4 + mt
        float4v *park = reinterpret_cast<float4v *>(lds_a);   // [wave][tt * 4 + mt][lane]: 64 KiB
        __syncthreads();                       // every wave is done with the operand
#pragma unroll
        for (int tt = 0; tt < kWinTW; ++tt)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) park[(wave * 4 * kWinTW + tt * 4 + mt) * 64 + lane] = acc[tt][mt];
        __syncthreads();
        const int tt = wave;                   // wave w < 4 sums and stores weight tile w
        const int64_t t4 = 4 * (int64_t)blockIdx.x + tt;
        const int64_t n = 16 * t4 + r16;
        const int pw0 = 4 * (tt / kWinTW), pi = (tt % kWinTW) * 4;
        if (wave < 4 && t4 < a.NT && n < a.N) {
            const float scale = qS * wS;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                float4v sum = park[(pw0 * 4 * kWinTW + pi + mt) * 64 + lane];
#pragma unroll
                for (int w2 = 1; w2 < 4; ++w2) sum += park[((pw0 + w2) * 4 * kWinTW + pi + mt) * 64 + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t row = 16 * mt + 4 * g + e;
                    if (row < a.M) {
                        const float val = sum[e] * scale;
                        if (a.yt == 1) static_cast<float *>(a.y)[row * a.ldy + n] = val;
                        else static_cast<uint16_t *>(a.y)[row * a.ldy + n] = f32_to_bf16_rne(val);
                    }
                }
            }
        }
    } else {
        // ---- producers: unit v's chunks (row c / 16, position c % 16) into slot v & 1,
        // from register set v mod 3; the loads of unit k + 2 go out while unit k is stored
        const int ptid = tid - 64 * kWinCons;
        QChunk q0[kWinChunks], q1[kWinChunks], q2[kWinChunks];
        const WinRows wr = win_rows(a, ptid);
        auto load_unit = [&](int v, QChunk *q) { win_unit_load<RES>(a, wr, v, KU, q); };
        auto store_unit = [&](int v, const QChunk *q) {
            half8 *dst = lds_a + (v & 1) * SLOT;
#pragma unroll
            for (int i = 0; i < kWinChunks; ++i) qchunk_store(dst, 4 * R, q[i]);
        };
        load_unit(0, q0);
        if (NV > 1) load_unit(1, q1);
        if (NV > 2) load_unit(2, q2);
        __syncthreads();                       // loads out: the consumers issue theirs behind them
        store_unit(0, q0);
        if (NV > 1) store_unit(1, q1);
        if (NV > 3) load_unit(3, q0);
        TL(5);
        __syncthreads();                       // barrier 0
        TL(6);
        auto pstep = [&](int k, QChunk *qs, QChunk *ql) {
            // barrier k: store unit k (k >= 2; its set qs = k mod 3), load unit k + 2 into ql
            // (set (k + 2) mod 3, whose unit k - 1 is stored)
            if (k >= 2) {
                store_unit(k, qs);
                if (k + 2 < NV) load_unit(k + 2, ql);
            }
            __syncthreads();
        };
        for (int k = 1; k < NV; k += 3) {      // k = 1 mod 3 at the top
            pstep(k, q1, q0);
            if (k + 1 < NV) pstep(k + 1, q2, q1);
            if (k + 2 < NV) pstep(k + 2, q0, q2);
        }
        __syncthreads();                       // the consumers' two barriers around their partial sums
        __syncthreads();
    }
}

// ---------------------------------------------------------------- planning
struct Plan { int MT, U, P, T, tw, KW, G, mode, Rr, Mp; bool ordered; int64_t NT, Q; size_t lds; };

constexpr size_t kLdsPerCu = 160 * 1024;       // gfx950
constexpr size_t kLdsStatic = 256;             // the kernel's own __shared__ words, rounded up

int cu_count() {
    static int cus = 0;
    if (cus <= 0) {
        int dev = 0, c = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
            cus = c;
        else
            return 256;                        // no device: plan for MI355X
    }
    return cus;
}

template <bool TILED>
const void *kernel_ptr_t(int MT, bool res, bool stk) {
    if (MT == 1) {
        if (!res) return reinterpret_cast<const void *>(&decode_kernel<1, false, TILED, false>);
        return stk ? reinterpret_cast<const void *>(&decode_kernel<1, true, TILED, true>)
                   : reinterpret_cast<const void *>(&decode_kernel<1, true, TILED, false>);
    }
    if (!res) return reinterpret_cast<const void *>(&decode_kernel<2, false, TILED, false>);
    return stk ? reinterpret_cast<const void *>(&decode_kernel<2, true, TILED, true>)
               : reinterpret_cast<const void *>(&decode_kernel<2, true, TILED, false>);
}

const void *kernel_ptr(int MT, bool res, bool tiled, bool stk) {
    return tiled ? kernel_ptr_t<true>(MT, res, stk) : kernel_ptr_t<false>(MT, res, stk);
}

// Work split of one call. A K range of U units (P ranges) costs its operand in
// LDS (U x 1 KiB per activation row, twice with residue columns); KW consumer
// waves share each tile (TW = 4 / KW tiles at a time, ntw per wave). The
// estimate charges each item (16 rows x 512 columns of W) its streaming time
// on the busiest CU -- a CU streams ~0.23 us per item with its loads in flight
// -- plus ~2 us for each further round of workgroups (a workgroup's start-up:
// arguments, operand, first items), plus ~1.5 us for a split-K combine, which
// costs three dependent round trips through the memory system.
Plan plan_compute(int64_t M, int64_t N, int64_t K, int64_t res_cols, bool raw_x, bool norm_or_perm, int ncu) {
    Plan pl;
    const bool res = res_cols > 0;
    // operand rows: residue rows stacked under the activation rows when M <= 8,
    // and as a second row tile for M = 9..16 when they cover at least half of K
    // (below that the stacked tile would multiply mostly zero rows)
    pl.Mp = 0;
    if (res && M <= 8) { pl.Mp = 1; while (pl.Mp < M) pl.Mp *= 2; }
    else if (res && M <= 16 && 2 * res_cols >= K) pl.Mp = 16;
    pl.MT = (M <= 16 && pl.Mp < 16) ? 1 : 2;
    pl.NT = (N + 15) / 16;
    const int64_t ku = (K + 511) / 512 > 0 ? (K + 511) / 512 : 1;
    pl.Rr = pl.Mp ? 2 * pl.Mp : (int)M;
    const int64_t op_rows = pl.Mp ? 2 * pl.Mp : (res ? 2 * M : M);   // rows of operand per unit
    double best = 1e30;
    int bU = 1, bKW = 1, bntw = 1;
    bool found = false;
    for (int64_t P0 = 1; P0 <= ku && P0 <= 64; ++P0) {
        const int64_t U = (ku + P0 - 1) / P0, P = (ku + U - 1) / U;
        if (P != P0) continue;                 // each split once
        const size_t lds_a = (size_t)U * 1024 * (size_t)op_rows;
        for (int KW = 1; KW <= kCons; KW *= 2) {
            const int TW = kCons / KW;
            const int64_t nuw = (U + KW - 1) / KW;
            for (int ntw = 1; ntw <= kMaxItems; ++ntw) {
                if (ntw * nuw > kMaxItems || (KW > 1 && ntw > 2)) break;
                const int64_t T = (int64_t)TW * ntw, Q = (pl.NT + T - 1) / T, G = P * Q;
                size_t lds = lds_a > (KW > 1 ? (size_t)8192 * pl.MT : 0) ? lds_a : (size_t)8192 * pl.MT;
                lds = (lds + 255) / 256 * 256;
                const int per_cu = lds + kLdsStatic <= kLdsPerCu / 2 ? 2 : (lds + kLdsStatic <= kLdsPerCu ? 1 : 0);
                if (per_cu == 0 || Q > kMaxTileCounters) continue;   // more than one round is allowed
                const double items_wg = (double)T * (double)U;
                // work of the busiest CU, and rounds of workgroups (per_cu of them fit a CU at once)
                const int64_t per_cu_wgs = (G + ncu - 1) / ncu, rounds = (G + ncu * per_cu - 1) / (ncu * per_cu);
                const double cost = 0.23 * items_wg * (double)per_cu_wgs + 2.0 * (double)(rounds - 1) +
                                    (P > 1 ? 1.5 + 0.1 * (double)P : 0.0) + (KW > 1 ? 0.1 : 0.0);
                if (cost < best) { best = cost; bU = (int)U; bKW = KW; bntw = ntw; found = true; }
            }
        }
    }
    if (!found) { bU = 1; bKW = 1; bntw = 1; }
    pl.U = bU > ku ? (int)ku : bU;
    pl.KW = bKW;
    pl.tw = bntw;
    pl.T = (kCons / pl.KW) * pl.tw;
    pl.P = (int)((ku + pl.U - 1) / pl.U);
    pl.Q = (pl.NT + pl.T - 1) / pl.T;
    pl.G = (int)(pl.P * pl.Q);
    {
        const size_t lds_a = (size_t)pl.U * 1024 * (size_t)op_rows;
        const size_t red = pl.KW > 1 ? (size_t)8192 * pl.MT : 0;
        pl.lds = ((lds_a > red ? lds_a : red) + 255) / 256 * 256;
    }
    // Raw activations are quantized in the kernel only when every workgroup can
    // read all of X and each producer thread holds at most kLocalChunks chunks.
    const int64_t kc = (int64_t)pl.U * 512 < K ? (int64_t)pl.U * 512 : K;
    const int64_t step = M > 0 ? kPThreads / M : 1;   // chunk positions per pass (prod_map)
    const int64_t per_thread = ((kc + 31) / 32 + step - 1) / step;
    // The quantization arithmetic of LOCAL runs on the four producer waves of
    // every workgroup; residue columns double it (a second block encoded per
    // block), so they count twice against the same bound.
    const int64_t local_work = per_thread * (res_cols > 0 ? 2 : 1);
    pl.mode = (raw_x && !norm_or_perm && local_work <= kLocalChunks && M * K <= kLocalMaxElems)
                  ? MODE_LOCAL : MODE_PRE;
    // PRE producers with more than one chunk per thread put enough loads in the
    // CU's queue that the operand lands late behind the consumers' first items;
    // then the consumers wait for them (measured: ordering wins from two chunks
    // per thread on, racing wins at one).
    const int64_t pre_per_thread = (((kc + 31) / 32) * (res_cols > 0 ? 2 : 1) + step - 1) / step;
    pl.ordered = pl.mode == MODE_LOCAL || pre_per_thread > 1;
    return pl;
}

// Plans are computed once per (shape, mode, CU count) and kept: a call asks for
// its plan up to three times (workspace size, fusion check, launch), and the
// search above walks a few hundred candidates. Thread-safe; the table is
// dropped wholesale if it ever holds 4096 shapes.
struct PlanKey {
    int64_t M, N, K, S;
    int flags, ncu;
    bool operator==(const PlanKey &o) const {
        return M == o.M && N == o.N && K == o.K && S == o.S && flags == o.flags && ncu == o.ncu;
    }
};
struct PlanKeyHash {
    size_t operator()(const PlanKey &k) const {
        uint64_t h = 1469598103934665603ull;
        for (uint64_t v : {(uint64_t)k.M, (uint64_t)k.N, (uint64_t)k.K, (uint64_t)k.S, (uint64_t)k.flags,
                           (uint64_t)k.ncu})
            h = (h ^ v) * 1099511628211ull;
        return (size_t)h;
    }
};

Plan plan_for(int64_t M, int64_t N, int64_t K, int64_t res_cols, bool raw_x, bool norm_or_perm) {
    static std::mutex mu;
    static std::unordered_map<PlanKey, Plan, PlanKeyHash> table;
    const int ncu = cu_count();
    const PlanKey key{M, N, K, res_cols, (raw_x ? 1 : 0) | (norm_or_perm ? 2 : 0), ncu};
    {
        std::lock_guard<std::mutex> lock(mu);
        const auto it = table.find(key);
        if (it != table.end()) return it->second;
    }
    const Plan pl = plan_compute(M, N, K, res_cols, raw_x, norm_or_perm, ncu);
    std::lock_guard<std::mutex> lock(mu);
    if (table.size() >= 4096) table.clear();
    table.emplace(key, pl);
    return pl;
}

bool plan_ok(const Plan &pl) { return pl.Q <= kMaxTileCounters && pl.G >= 1; }

}  // namespace

size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t res_cols) {
    if (M > 32) return 0;                      // the windowed kernel: no split-K
    const Plan pl = plan_for(M, N, K, res_cols, false, false);
    return pl.P > 1 ? (size_t)pl.P * M * N * sizeof(float) : 0;
}

bool decode_can_fuse(int64_t M, int64_t N, int64_t K, int64_t res_cols, bool x_bf16) {
    if (M > 32) return false;                  // the windowed kernel reads quantized activations
    const Plan pl = plan_for(M, N, K, res_cols, true, false);
    return x_bf16 && plan_ok(pl) && pl.mode == MODE_LOCAL;
}

#ifdef NVFP4_TIMELINE
extern "C" int nvfp4_debug_timeline(void *host, size_t bytes) {
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_timeline), bytes < sizeof(g_timeline) ? bytes : sizeof(g_timeline));
}
#endif

// M = 33..64: the windowed kernel, four weight tiles per workgroup over all of K
// (and the residue units), each of its eight consumer waves one 32-column step of
// every unit for two of them; quantized activations only.
hipError_t launch_decode_win(const DecodeLaunch &g, hipStream_t st) {
    if (g.x != nullptr || !g.header) return hipErrorInvalidValue;
    DArgs a{};
    a.q_codes = g.q_codes; a.q_ldc = g.q_ldc; a.q_scales = g.q_scales; a.q_lds = g.q_lds; a.q_S = g.q_S;
    a.w_codes = g.w_codes; a.w_ldc = g.w_ldc; a.w_scales = g.w_scales; a.w_lds = g.w_lds; a.w_S = g.w_S;
    a.M = g.M; a.N = g.N; a.K = g.K; a.res_cols = g.res_cols;
    a.y = g.y; a.yt = g.yt; a.ldy = g.ldy;
    a.header = reinterpret_cast<uint8_t *>(g.header);
    a.NT = (g.N + 15) / 16;
    a.Rr = (int)g.M;
    a.U = 1; a.P = 1; a.T = 4; a.tw = 1; a.KW = 1; a.G = (int)((a.NT + 3) / 4); a.mode = MODE_PRE; a.Mp = 0;
    const bool res = g.res_cols > 0, tiled = g.w_tiled != 0;
    const void *fn = tiled ? (res ? reinterpret_cast<const void *>(&decode_win_kernel<true, true>)
                                  : reinterpret_cast<const void *>(&decode_win_kernel<true, false>))
                           : (res ? reinterpret_cast<const void *>(&decode_win_kernel<false, true>)
                                  : reinterpret_cast<const void *>(&decode_win_kernel<false, false>));
    const size_t lds = 2 * 64 * (size_t)kWinRows * sizeof(half8);
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    void *args[] = {&a};
    return hipLaunchKernel(fn, dim3((unsigned)a.G), dim3(kWinThreads), args, lds, st);
}

hipError_t launch_decode(const DecodeLaunch &g, hipStream_t st) {
    const bool raw = g.x != nullptr;
    if (g.M < 1 || g.M > 64 || g.N < 1 || g.K < 1) return hipErrorInvalidValue;   // the kernels' row bound
    if (g.res_cols > 0 && g.K % 32 != 0) return hipErrorInvalidValue;          // residue chunks 16-byte aligned
    if (g.M > 32) return launch_decode_win(g, st);
    const Plan pl = plan_for(g.M, g.N, g.K, g.res_cols, raw, false);
    if (!plan_ok(pl) || (raw && pl.mode != MODE_LOCAL)) return hipErrorInvalidValue;
    if (!g.header || g.scratch_bytes < decode_workspace_bytes(g.M, g.N, g.K, g.res_cols) ||
        (pl.P > 1 && !g.scratch))
        return hipErrorInvalidValue;
    DArgs a;
    a.x = g.x; a.ldx = g.ldx; a.static_S = g.static_S;
    a.q_codes = g.q_codes; a.q_ldc = g.q_ldc; a.q_scales = g.q_scales; a.q_lds = g.q_lds; a.q_S = g.q_S;
    a.w_codes = g.w_codes; a.w_ldc = g.w_ldc; a.w_scales = g.w_scales; a.w_lds = g.w_lds; a.w_S = g.w_S;
    a.M = g.M; a.N = g.N; a.K = g.K; a.res_cols = g.res_cols;
    a.y = g.y; a.yt = g.yt; a.ldy = g.ldy;
    a.header = reinterpret_cast<uint8_t *>(g.header);
    a.partials = static_cast<float *>(g.scratch);
    a.U = pl.U; a.P = pl.P; a.T = pl.T; a.tw = pl.tw; a.KW = pl.KW; a.G = pl.G; a.mode = pl.mode; a.NT = pl.NT;
    a.Rr = pl.Rr; a.Mp = pl.Mp; a.ordered = pl.ordered ? 1 : 0;
    // stacking (Mp > 0) exists with residue columns only
    const void *fn = kernel_ptr(pl.MT, g.res_cols > 0, g.w_tiled != 0, pl.Mp > 0);
    if (pl.lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)pl.lds);
        if (e != hipSuccess) return e;
    }
    void *args[] = {&a};
    return hipLaunchKernel(fn, dim3(pl.G), dim3(kThreads), args, pl.lds, st);
}

}  // namespace nvfp4
