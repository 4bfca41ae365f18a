// api.hip -- extern "C" entry points of libnvfp4 (declared in include/nvfp4.h).
//
// Every argument is validated before anything is enqueued; on error the call
// returns a status and no output is touched. The library allocates nothing:
// scratch space comes from the caller's workspace, carved up here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/nvfp4.h"
#include "internal.h"
#include "nvfp4_device.h"

using namespace nvfp4;

namespace {

thread_local char g_last_error[256] = "";

nvfp4_status hip_fail(hipError_t e) {
    std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
    return NVFP4_ERR_HIP;
}

constexpr size_t kAlign = 256;
inline size_t up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The skinny (decode) path takes M up to this many rows; larger M is tiled, and
// so are products with residue columns when K is not a multiple of 32 (the
// decode kernels load the residue part in 16-byte chunks from column K).
constexpr int64_t kSkinnyMaxM = 64;
inline bool skinny_rows(int64_t M, int64_t K, int64_t S) {
    return K > 0 && M <= kSkinnyMaxM && (S == 0 || K % 32 == 0);
}

int64_t ldc_for(int64_t K) { return (int64_t)up((size_t)(K / 2), 16); }
int64_t lds_for(int64_t K) { return (int64_t)up((size_t)(K / 16), 8); }

size_t quant_ws(int64_t rows) {
    return up(kAmaxPartials * sizeof(float), kAlign) + up((size_t)std::max<int64_t>(rows, 1) * sizeof(float), kAlign);
}

size_t tensor_ws(int64_t rows, int64_t K) {
    return up((size_t)(rows * ldc_for(K)), kAlign) + up((size_t)(rows * lds_for(K)), kAlign) + kAlign;
}

size_t gemm_ws(int64_t M, int64_t N, int64_t K, int64_t S) {
    if (skinny_rows(M, K, S)) return up(decode_workspace_bytes(M, N, K, S), kAlign);
    return up(prefill_workspace_bytes(M, N, K, S), kAlign);
}

// Bound on the small quantizer's arrival wait, in polls of ~0.1 us (a few ms).
// NVFP4_SPIN_LIMIT overrides it from the host (0 = give up at once), so the
// recompute fallback can be exercised without any fault or hang.
unsigned spin_limit() {
    const char *e = std::getenv("NVFP4_SPIN_LIMIT");
    if (e && *e) return (unsigned)std::strtoul(e, nullptr, 10);
    return 1u << 16;
}

struct Carver {
    uint8_t *p; size_t left; bool ok = true;
    uint8_t *take(size_t n) {
        n = up(n, kAlign);
        if (n > left) { ok = false; return nullptr; }
        uint8_t *r = p; p += n; left -= n; return r;
    }
};

int elem_size(int xt) { return xt == NVFP4_BF16 ? 2 : 4; }

// A tensor with no elements may carry null code/scale pointers; its scale
// pointer is still required (the quantizer writes S = 1 for it).
// Tiled layout (weights only): strips of 16 rows, strides fixed by K.
int64_t tiled_ldc(int64_t K) { return (K + 511) / 512 * 4096; }
int64_t tiled_lds(int64_t K) { return (K + 511) / 512 * 512; }

nvfp4_status check_tensor(const nvfp4_tensor *t, int64_t rows, int64_t K, bool allow_tiled = false) {
    if (!t || !t->tensor_scale) return NVFP4_ERR_NULL;
    if (t->layout != NVFP4_LAYOUT_ROWMAJOR && t->layout != NVFP4_LAYOUT_TILED) return NVFP4_ERR_SHAPE;
    if (t->layout == NVFP4_LAYOUT_TILED && !allow_tiled) return NVFP4_ERR_UNSUPPORTED;
    if (t->rows != rows || t->K != K || rows < 0 || K < 0 || K % 16) return NVFP4_ERR_SHAPE;
    if (rows == 0 || K == 0) return aligned(t->tensor_scale, 4) ? NVFP4_OK : NVFP4_ERR_ALIGN;
    if (!t->codes || !t->scales) return NVFP4_ERR_NULL;
    if (t->layout == NVFP4_LAYOUT_TILED) {
        if (t->ld_codes != tiled_ldc(K) || t->ld_scales != tiled_lds(K)) return NVFP4_ERR_SHAPE;
        if (!aligned(t->codes, 16) || !aligned(t->scales, 8) || !aligned(t->tensor_scale, 4)) return NVFP4_ERR_ALIGN;
        return NVFP4_OK;
    }
    if (t->ld_codes < K / 2 || t->ld_scales < K / 16) return NVFP4_ERR_SHAPE;
    if (t->ld_codes % 16 || t->ld_scales % 8 || !aligned(t->codes, 16) || !aligned(t->scales, 8) ||
        !aligned(t->tensor_scale, 4))
        return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

nvfp4_status check_x(const void *x, int xt, int64_t rows, int64_t K, int64_t ldx) {
    if (xt != NVFP4_BF16 && xt != NVFP4_FP32) return NVFP4_ERR_DTYPE;
    if (rows < 0 || K < 0 || K % 16) return NVFP4_ERR_SHAPE;
    if (rows == 0 || K == 0) return NVFP4_OK;          // nothing is read
    if (!x) return NVFP4_ERR_NULL;
    if (ldx < K) return NVFP4_ERR_SHAPE;
    if (!aligned(x, 16) || (ldx * elem_size(xt)) % 16) return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

nvfp4_status check_opts(const nvfp4_quant_opts *o, int64_t K_in) {
    if (!o) return NVFP4_OK;
    if (o->residue_cols < 0 || o->residue_cols > K_in || o->residue_cols % 16) return NVFP4_ERR_SHAPE;
    if (o->gamma && !aligned(o->gamma, 16)) return NVFP4_ERR_ALIGN;
    if (o->perm && K_in > 32768) return NVFP4_ERR_UNSUPPORTED;   // the row staged in LDS (128 KiB)
    if (o->perm && !aligned(o->perm, 16)) return NVFP4_ERR_ALIGN;   // read as 16-byte vectors
    if (o->gamma && !(o->eps >= 0.0f)) return NVFP4_ERR_SHAPE;
    if (o->smooth && !aligned(o->smooth, 16)) return NVFP4_ERR_ALIGN;   // read as 16-byte vectors
    return NVFP4_OK;
}

#define CHECK(expr) do { nvfp4_status s_ = (expr); if (s_ != NVFP4_OK) return s_; } while (0)

// Enqueue the quantizer writing into `out` (validated by the caller).
nvfp4_status enqueue_quantize(const void *x, int xt, int64_t rows, int64_t K_in, int64_t ldx,
                              const nvfp4_quant_opts *opts, const nvfp4_tensor &out,
                              float *partials, float *rscale, unsigned *header, hipStream_t st) {
    QuantLaunch q;
    q.x = x; q.xt = xt; q.rows = rows; q.K_in = K_in; q.ldx = ldx;
    q.gamma = opts ? static_cast<const uint16_t *>(opts->gamma) : nullptr;
    q.eps = opts ? opts->eps : 0.0f;
    q.perm = opts ? opts->perm : nullptr;
    q.res_cols = opts ? opts->residue_cols : 0;
    q.static_S = opts ? opts->static_tensor_scale : nullptr;
    q.smooth = opts ? opts->smooth : nullptr;
    q.codes = out.codes; q.ldc = out.ld_codes; q.scales = out.scales; q.lds = out.ld_scales;
    q.S_out = out.tensor_scale;
    q.partials = partials; q.rscale = rscale;
    q.slots = reinterpret_cast<unsigned long long *>(header) + kSlotsOffset / 8;   // header bytes 512..1023
    q.grid_slots = reinterpret_cast<unsigned long long *>(header) + kGridSlotsOffset / 8;   // 1024..3071
    q.spin = spin_limit();
    hipError_t e = launch_quantize(q, st);
    return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

// Product on an already quantized activation tensor `a` (K + S columns).
nvfp4_status enqueue_gemm(const nvfp4_tensor &a, const nvfp4_tensor &w, int64_t M, int64_t K, int64_t S,
                          void *y, int yt, int64_t ldy, unsigned *header, uint8_t *scratch, size_t scratch_bytes,
                          hipStream_t st) {
    hipError_t e;
    if (skinny_rows(M, K, S)) {
        DecodeLaunch g{};
        g.x = nullptr;
        g.q_codes = a.codes; g.q_ldc = a.ld_codes; g.q_scales = a.scales; g.q_lds = a.ld_scales; g.q_S = a.tensor_scale;
        g.w_codes = w.codes; g.w_ldc = w.ld_codes; g.w_scales = w.scales; g.w_lds = w.ld_scales; g.w_S = w.tensor_scale;
        g.w_tiled = w.layout == NVFP4_LAYOUT_TILED;
        g.M = M; g.N = w.rows; g.K = K; g.res_cols = S;
        g.y = y; g.yt = yt; g.ldy = ldy;
        g.header = header; g.scratch = scratch; g.scratch_bytes = scratch_bytes;
        e = launch_decode(g, st);
    } else {
        PrefillLaunch g;
        g.a_codes = a.codes; g.a_ldc = a.ld_codes; g.a_scales = a.scales; g.a_lds = a.ld_scales; g.a_S = a.tensor_scale;
        g.w_codes = w.codes; g.w_ldc = w.ld_codes; g.w_scales = w.scales; g.w_lds = w.ld_scales; g.w_S = w.tensor_scale;
        g.w_tiled = w.layout == NVFP4_LAYOUT_TILED;
        g.M = M; g.N = w.rows; g.K = K; g.res_cols = S;
        g.y = y; g.yt = yt; g.ldy = ldy;
        g.scratch = scratch; g.scratch_bytes = scratch_bytes;
        e = launch_prefill(g, st);
    }
    return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

// Quantize-and-multiply in one launch (decode shapes, no RMSNorm or gather).
nvfp4_status enqueue_fused(const void *x, int xt, int64_t ldx, const float *static_S, const nvfp4_tensor &q,
                           const nvfp4_tensor &w, int64_t M, int64_t K, int64_t S, void *y, int yt, int64_t ldy,
                           unsigned *header, uint8_t *scratch, size_t scratch_bytes, hipStream_t st) {
    DecodeLaunch g{};
    (void)xt;                                   // decode_can_fuse admitted bf16 only
    g.x = x; g.ldx = ldx; g.static_S = static_S;
    g.q_codes = q.codes; g.q_ldc = q.ld_codes; g.q_scales = q.scales; g.q_lds = q.ld_scales; g.q_S = q.tensor_scale;
    g.w_codes = w.codes; g.w_ldc = w.ld_codes; g.w_scales = w.scales; g.w_lds = w.ld_scales; g.w_S = w.tensor_scale;
    g.w_tiled = w.layout == NVFP4_LAYOUT_TILED;
    g.M = M; g.N = w.rows; g.K = K; g.res_cols = S;
    g.y = y; g.yt = yt; g.ldy = ldy;
    g.header = header; g.scratch = scratch; g.scratch_bytes = scratch_bytes;
    const hipError_t e = launch_decode(g, st);
    return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

}  // namespace

extern "C" {

size_t nvfp4_workspace_size(int op, int64_t M, int64_t N, int64_t K, int64_t S) {
    if (M < 0 || N < 0 || K < 0 || S < 0) return 0;
    switch (op) {
        case 0: return kHeaderBytes + quant_ws(M);
        case 1: return kHeaderBytes + tensor_ws(M, K) + quant_ws(M) + gemm_ws(M, N, K, 0);
        case 2: return kHeaderBytes + tensor_ws(M, K + S) + quant_ws(M) + gemm_ws(M, N, K, S);
        case 3: return kHeaderBytes + up((size_t)std::max<int64_t>(M, 1) * sizeof(float), kAlign);
        case 4: return kHeaderBytes + mx_workspace_bytes(M, N, K, S);
        case 5: return K > 0 ? kHeaderBytes + attention_workspace_bytes(M, N, K) : kHeaderBytes;
        default: return 0;
    }
}

nvfp4_status nvfp4_quantize(const void *x, int xt, int64_t rows, int64_t K_in, int64_t ldx,
                            const nvfp4_quant_opts *opts, const nvfp4_tensor *out,
                            void *ws, size_t ws_bytes, void *stream) {
    CHECK(check_x(x, xt, rows, K_in, ldx));
    CHECK(check_opts(opts, K_in));
    const int64_t S = opts ? opts->residue_cols : 0;
    CHECK(check_tensor(out, rows, K_in + S));
    const size_t need = nvfp4_workspace_size(0, rows, 0, K_in, S);
    if (!ws || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
    Carver c{static_cast<uint8_t *>(ws) + kHeaderBytes, ws_bytes - kHeaderBytes};
    float *partials = reinterpret_cast<float *>(c.take(kAmaxPartials * sizeof(float)));
    float *rscale = reinterpret_cast<float *>(c.take((size_t)std::max<int64_t>(rows, 1) * sizeof(float)));
    if (!c.ok) return NVFP4_ERR_WORKSPACE;
    return enqueue_quantize(x, xt, rows, K_in, ldx, opts, *out, partials, rscale, static_cast<unsigned *>(ws),
                            static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Argument checks of nvfp4_gemm that do not involve the workspace.
nvfp4_status check_gemm(const nvfp4_tensor *a_q, const void *x, int xt, int64_t M, int64_t K, int64_t ldx,
                        const nvfp4_tensor *w, const void *y, int yt, int64_t ldy) {
    if (!w) return NVFP4_ERR_NULL;
    if (a_q == nullptr && x == nullptr && !(M == 0 || K == 0)) return NVFP4_ERR_NULL;
    if (a_q != nullptr && x != nullptr) return NVFP4_ERR_NULL;
    if (!y && M > 0 && w->rows > 0) return NVFP4_ERR_NULL;
    if (yt != NVFP4_BF16 && yt != NVFP4_FP32) return NVFP4_ERR_DTYPE;
    if (M < 0 || K < 0 || K % 16) return NVFP4_ERR_SHAPE;
    CHECK(check_tensor(w, w->rows, K, true));
    if (ldy < w->rows) return NVFP4_ERR_SHAPE;
    if (a_q) CHECK(check_tensor(a_q, M, K));
    else CHECK(check_x(x, xt, M, K, ldx));
    return NVFP4_OK;
}

// The product of nvfp4_gemm on a validated call and a large enough workspace.
nvfp4_status gemm_enqueue(const nvfp4_tensor *a_q, const void *x, int xt, int64_t M, int64_t K, int64_t ldx,
                          const nvfp4_tensor *w, void *y, int yt, int64_t ldy, void *ws, size_t ws_bytes,
                          hipStream_t st) {
    const int64_t N = w->rows;
    unsigned *header = static_cast<unsigned *>(ws);
    Carver c{static_cast<uint8_t *>(ws) + kHeaderBytes, ws_bytes - kHeaderBytes};
    nvfp4_tensor aq;
    if (a_q) {
        aq = *a_q;
    } else {
        aq.rows = M; aq.K = K; aq.ld_codes = ldc_for(K); aq.ld_scales = lds_for(K);
        aq.codes = c.take((size_t)std::max<int64_t>(M * aq.ld_codes, 1));
        aq.scales = c.take((size_t)std::max<int64_t>(M * aq.ld_scales, 1));
        aq.tensor_scale = reinterpret_cast<float *>(c.take(sizeof(float)));
    }
    float *partials = reinterpret_cast<float *>(c.take(kAmaxPartials * sizeof(float)));
    float *rscale = reinterpret_cast<float *>(c.take((size_t)std::max<int64_t>(M, 1) * sizeof(float)));
    const size_t sb = gemm_ws(M, N, K, 0);
    uint8_t *scratch = sb ? c.take(sb) : nullptr;
    if (!c.ok) return NVFP4_ERR_WORKSPACE;
    const bool skinny = skinny_rows(M, K, 0);
    if (!a_q && skinny && decode_can_fuse(M, N, K, 0, xt == NVFP4_BF16))
        return enqueue_fused(x, xt, ldx, nullptr, aq, *w, M, K, 0, y, yt, ldy, header, scratch, sb, st);
    if (!a_q) CHECK(enqueue_quantize(x, xt, M, K, ldx, nullptr, aq, partials, rscale, header, st));
    return enqueue_gemm(aq, *w, M, K, 0, y, yt, ldy, header, scratch, sb, st);
}

// ---- Workspace of nvfp4_gemm_noalloc: a static device array, one copy per GPU,
// held until the process ends. In host code the array's name is only a host-side
// stand-in: its device address (per device) comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is used.
__device__ __align__(256) static uint8_t g_static_scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

__global__ void zero_words_kernel(unsigned *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
struct StaticScratch {
    std::once_flag once;
    uint8_t *ptr = nullptr;
    hipError_t err = hipSuccess;
};
StaticScratch g_dev_scratch[kMaxDevices];

// This device's copy of the static scratch. The first call on a device takes its
// address and clears its counter header with a fill kernel on `st` (a kernel, so a
// caller's graph capture may hold it; the array also starts zeroed at load).
hipError_t static_scratch(hipStream_t st, uint8_t **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    StaticScratch &s = g_dev_scratch[dev];
    std::call_once(s.once, [&] {
        void *p = nullptr;
        s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(g_static_scratch));
        if (s.err != hipSuccess) return;
        s.ptr = static_cast<uint8_t *>(p);
        const int words = (int)(kHeaderBytes / sizeof(unsigned));
        hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, st,
                           reinterpret_cast<unsigned *>(s.ptr), words);
        s.err = hipGetLastError();
    });
    *out = s.ptr;
    return s.err;
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_gemm_noalloc(const nvfp4_tensor *a_q, const void *x, int xt,
                                int64_t M, int64_t K, int64_t ldx,
                                const nvfp4_tensor *w, void *y, int yt, int64_t ldy, void *stream) {
    CHECK(check_gemm(a_q, x, xt, M, K, ldx, w, y, yt, ldy));
    const size_t need = nvfp4_workspace_size(1, M, w->rows, K, 0);
    if (need > (size_t)NVFP4_NOALLOC_SCRATCH_BYTES) {
        std::snprintf(g_last_error, sizeof(g_last_error),
                      "nvfp4_gemm_noalloc: this product needs %zu bytes of scratch; the static scratch holds %zu",
                      need, (size_t)NVFP4_NOALLOC_SCRATCH_BYTES);
        return NVFP4_ERR_WORKSPACE;
    }
    if (M == 0 || w->rows == 0) return NVFP4_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t *ws = nullptr;
    const hipError_t e = static_scratch(st, &ws);
    if (e != hipSuccess) return hip_fail(e);
    return gemm_enqueue(a_q, x, xt, M, K, ldx, w, y, yt, ldy, ws, NVFP4_NOALLOC_SCRATCH_BYTES, st);
}

nvfp4_status nvfp4_gemm(const nvfp4_tensor *a_q, const void *x, int xt,
                        int64_t M, int64_t K, int64_t ldx,
                        const nvfp4_tensor *w, void *y, int yt, int64_t ldy,
                        void *ws, size_t ws_bytes, void *stream) {
    CHECK(check_gemm(a_q, x, xt, M, K, ldx, w, y, yt, ldy));
    const size_t need = nvfp4_workspace_size(1, M, w->rows, K, 0);
    if (!ws || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (M == 0 || w->rows == 0) return NVFP4_OK;
    return gemm_enqueue(a_q, x, xt, M, K, ldx, w, y, yt, ldy, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

nvfp4_status nvfp4_gemm_residue(const void *x, int xt, int64_t M, int64_t K, int64_t ldx,
                                const nvfp4_quant_opts *opts, const nvfp4_tensor *w,
                                void *y, int yt, int64_t ldy, const nvfp4_tensor *a_aug_out,
                                void *ws, size_t ws_bytes, void *stream) {
    if (!w) return NVFP4_ERR_NULL;
    if (!y && M > 0 && w->rows > 0) return NVFP4_ERR_NULL;
    if (yt != NVFP4_BF16 && yt != NVFP4_FP32) return NVFP4_ERR_DTYPE;
    CHECK(check_x(x, xt, M, K, ldx));
    CHECK(check_opts(opts, K));
    const int64_t S = opts ? opts->residue_cols : 0;
    CHECK(check_tensor(w, w->rows, K, true));
    const int64_t N = w->rows;
    if (ldy < N) return NVFP4_ERR_SHAPE;
    if (a_aug_out) CHECK(check_tensor(a_aug_out, M, K + S));
    const size_t need = nvfp4_workspace_size(2, M, N, K, S);
    if (!ws || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (M == 0) return NVFP4_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    unsigned *header = static_cast<unsigned *>(ws);
    Carver c{static_cast<uint8_t *>(ws) + kHeaderBytes, ws_bytes - kHeaderBytes};
    nvfp4_tensor aq;
    if (a_aug_out) {
        aq = *a_aug_out;
        c.take(tensor_ws(M, K + S) - kAlign);
    } else {
        aq.rows = M; aq.K = K + S; aq.ld_codes = ldc_for(K + S); aq.ld_scales = lds_for(K + S);
        aq.codes = c.take((size_t)std::max<int64_t>(M * aq.ld_codes, 1));
        aq.scales = c.take((size_t)std::max<int64_t>(M * aq.ld_scales, 1));
        aq.tensor_scale = reinterpret_cast<float *>(c.take(sizeof(float)));
    }
    float *partials = reinterpret_cast<float *>(c.take(kAmaxPartials * sizeof(float)));
    float *rscale = reinterpret_cast<float *>(c.take((size_t)std::max<int64_t>(M, 1) * sizeof(float)));
    const size_t sb = gemm_ws(M, N, K, S);
    uint8_t *scratch = sb ? c.take(sb) : nullptr;
    if (!c.ok) return NVFP4_ERR_WORKSPACE;
    const bool plain = !opts || (!opts->gamma && !opts->perm && !opts->smooth);
    const bool skinny = skinny_rows(M, K, S);
    if (N > 0 && plain && skinny && decode_can_fuse(M, N, K, S, xt == NVFP4_BF16))
        return enqueue_fused(x, xt, ldx, opts ? opts->static_tensor_scale : nullptr, aq, *w, M, K, S, y, yt, ldy,
                             header, scratch, sb, st);
    CHECK(enqueue_quantize(x, xt, M, K, ldx, opts, aq, partials, rscale, header, st));
    if (N == 0) return NVFP4_OK;
    return enqueue_gemm(aq, *w, M, K, S, y, yt, ldy, header, scratch, sb, st);
}

}  // extern "C"

namespace {

int64_t mx_tiled_ldc(int64_t K) { return (K + 511) / 512 * 4096; }
int64_t mx_tiled_lds(int64_t K) { return (K + 511) / 512 * 256; }

nvfp4_status check_mx(const nvfp4_mx_tensor *t, int64_t rows, int64_t K, bool allow_tiled = false) {
    if (!t) return NVFP4_ERR_NULL;
    if (t->layout != NVFP4_LAYOUT_ROWMAJOR && t->layout != NVFP4_LAYOUT_TILED) return NVFP4_ERR_SHAPE;
    if (t->layout == NVFP4_LAYOUT_TILED && !allow_tiled) return NVFP4_ERR_UNSUPPORTED;
    if (t->rows != rows || t->K != K || rows < 0 || K < 0 || K % 32) return NVFP4_ERR_SHAPE;
    if (rows == 0 || K == 0) return NVFP4_OK;
    if (!t->codes || !t->scales) return NVFP4_ERR_NULL;
    if (t->layout == NVFP4_LAYOUT_TILED) {
        if (t->ld_codes != mx_tiled_ldc(K) || t->ld_scales != mx_tiled_lds(K)) return NVFP4_ERR_SHAPE;
        if (!aligned(t->codes, 16)) return NVFP4_ERR_ALIGN;
        return NVFP4_OK;
    }
    if (t->ld_codes < K / 2 || t->ld_scales < K / 32) return NVFP4_ERR_SHAPE;
    if (t->ld_codes % 16 || !aligned(t->codes, 16)) return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_mx_quantize(const void *x, int xt, int64_t rows, int64_t K_in, int64_t ldx,
                               int64_t residue_cols, const nvfp4_mx_tensor *out, void *stream) {
    CHECK(check_x(x, xt, rows, K_in, ldx));
    if (K_in % 32 || residue_cols < 0 || residue_cols > K_in || residue_cols % 32) return NVFP4_ERR_SHAPE;
    CHECK(check_mx(out, rows, K_in + residue_cols));
    if (rows == 0 || K_in == 0) return NVFP4_OK;
    MXQuantLaunch q;
    q.x = x; q.xt = xt; q.rows = rows; q.K = K_in; q.ldx = ldx; q.res_cols = residue_cols;
    q.codes = out->codes; q.ldc = out->ld_codes; q.scales = out->scales; q.lds = out->ld_scales;
    const hipError_t e = launch_mx_quantize(q, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

nvfp4_status nvfp4_decode_attention(const void *q, int qt, int64_t H, int64_t D, int64_t ldq,
                                    const nvfp4_tensor *k_cache, const nvfp4_tensor *vt_cache, int64_t T,
                                    int compensate, float *out, int64_t ldo, void *ws, size_t ws_bytes,
                                    void *stream) {
    if (qt != NVFP4_BF16 && qt != NVFP4_FP32) return NVFP4_ERR_DTYPE;
    if (H < 0 || H > 65535 || D < 32 || D > 256 || D % 32 || T <= 0 || T % 16) return NVFP4_ERR_SHAPE;
    if (compensate != 0 && compensate != 1) return NVFP4_ERR_SHAPE;
    CHECK(check_tensor(k_cache, H * T, D));
    CHECK(check_tensor(vt_cache, H * D, T));
    if (H == 0) return NVFP4_OK;
    if (!q || !out) return NVFP4_ERR_NULL;
    if (ldq < D || ldo < D) return NVFP4_ERR_SHAPE;
    if (!aligned(q, 16) || (ldq * elem_size(qt)) % 16 || !aligned(out, 4)) return NVFP4_ERR_ALIGN;
    const size_t need = kHeaderBytes + attention_workspace_bytes(H, D, T);
    if (!ws || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
    AttentionLaunch g;
    g.q = q; g.qt = qt == NVFP4_BF16 ? IN_BF16 : IN_F32; g.ldq = ldq;
    g.H = H; g.D = D; g.T = T;
    g.k_codes = k_cache->codes; g.k_ldc = k_cache->ld_codes;
    g.k_scales = k_cache->scales; g.k_lds = k_cache->ld_scales; g.k_S = k_cache->tensor_scale;
    g.v_codes = vt_cache->codes; g.v_ldc = vt_cache->ld_codes;
    g.v_scales = vt_cache->scales; g.v_lds = vt_cache->ld_scales; g.v_S = vt_cache->tensor_scale;
    g.compensate = compensate;
    g.out = out; g.ldo = ldo;
    // scores and statistics after the header, which this call leaves untouched
    g.scratch = static_cast<uint8_t *>(ws) + kHeaderBytes;
    g.scratch_bytes = ws_bytes - kHeaderBytes;
    const hipError_t e = launch_attention(g, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

nvfp4_status nvfp4_mx_gemm(const nvfp4_mx_tensor *a, const nvfp4_mx_tensor *w, int64_t residue_cols,
                           void *y, int yt, int64_t ldy, void *ws, size_t ws_bytes, void *stream) {
    if (!a || !w) return NVFP4_ERR_NULL;
    if (yt != NVFP4_BF16 && yt != NVFP4_FP32) return NVFP4_ERR_DTYPE;
    const int64_t M = a->rows, N = w->rows, K = w->K, S = residue_cols;
    if (S < 0 || S > K || S % 32) return NVFP4_ERR_SHAPE;
    CHECK(check_mx(w, N, K, true));
    CHECK(check_mx(a, M, K + S));
    if (w->layout == NVFP4_LAYOUT_TILED && M > 64) return NVFP4_ERR_UNSUPPORTED;   // the tile kernel reads rows
    if (!y && M > 0 && N > 0) return NVFP4_ERR_NULL;
    if (ldy < N) return NVFP4_ERR_SHAPE;
    // the partials go after the header, which this product leaves untouched (the
    // workspace may be shared with the NVFP4 entry points and their counters)
    const size_t need = mx_workspace_bytes(M, N, K, S);
    if (need > 0 && (!ws || ws_bytes < kHeaderBytes + need)) return NVFP4_ERR_WORKSPACE;
    if (M == 0 || N == 0) return NVFP4_OK;
    MXGemmLaunch g;
    g.a_codes = a->codes; g.a_ldc = a->ld_codes; g.a_scales = a->scales; g.a_lds = a->ld_scales;
    g.w_codes = w->codes; g.w_ldc = w->ld_codes; g.w_scales = w->scales; g.w_lds = w->ld_scales;
    g.w_tiled = w->layout == NVFP4_LAYOUT_TILED;
    g.M = M; g.N = N; g.K = K; g.res_cols = S;
    g.y = y; g.yt = yt; g.ldy = ldy;
    g.scratch = need > 0 ? static_cast<uint8_t *>(ws) + kHeaderBytes : nullptr;
    g.scratch_bytes = need > 0 ? ws_bytes - kHeaderBytes : 0;
    const hipError_t e = launch_mx_gemm(g, static_cast<hipStream_t>(stream));   // K == 0 stores zeros
    return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

nvfp4_status nvfp4_mx_pack_tiled(const nvfp4_mx_tensor *src, const nvfp4_mx_tensor *dst, void *stream) {
    if (!src || !dst) return NVFP4_ERR_NULL;
    CHECK(check_mx(src, src->rows, src->K));
    if (dst->layout != NVFP4_LAYOUT_TILED) return NVFP4_ERR_SHAPE;
    CHECK(check_mx(dst, src->rows, src->K, true));
    if (src->rows > 0 && src->K > 0 && (src->codes == dst->codes || src->scales == dst->scales))
        return NVFP4_ERR_SHAPE;
    MXPackLaunch g;
    g.src_codes = src->codes; g.src_ldc = src->ld_codes; g.src_scales = src->scales; g.src_lds = src->ld_scales;
    g.dst_codes = dst->codes; g.dst_ldc = dst->ld_codes; g.dst_scales = dst->scales; g.dst_lds = dst->ld_scales;
    g.rows = src->rows; g.K = src->K;
    const hipError_t e = launch_mx_pack_tiled(g, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

nvfp4_status nvfp4_pack_tiled(const nvfp4_tensor *src, const nvfp4_tensor *dst, void *stream) {
    if (!src || !dst) return NVFP4_ERR_NULL;
    CHECK(check_tensor(src, src->rows, src->K));
    if (dst->layout != NVFP4_LAYOUT_TILED) return NVFP4_ERR_SHAPE;
    CHECK(check_tensor(dst, src->rows, src->K, true));
    if (src->tensor_scale == dst->tensor_scale && src->rows > 0 && src->K > 0) return NVFP4_ERR_SHAPE;
    PackLaunch g;
    g.src_codes = src->codes; g.src_ldc = src->ld_codes; g.src_scales = src->scales; g.src_lds = src->ld_scales;
    g.src_S = src->tensor_scale;
    g.dst_codes = dst->codes; g.dst_ldc = dst->ld_codes; g.dst_scales = dst->scales; g.dst_lds = dst->ld_scales;
    g.dst_S = dst->tensor_scale;
    g.rows = src->rows; g.K = src->K;
    const hipError_t e = launch_pack_tiled(g, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

nvfp4_status nvfp4_channel_absmax(const void *x, int xt, int64_t rows, int64_t K, int64_t ldx,
                                  const void *gamma, float eps, float *absmax_out,
                                  void *ws, size_t ws_bytes, void *stream) {
    CHECK(check_x(x, xt, rows, K, ldx));
    if (!absmax_out) return NVFP4_ERR_NULL;
    if (gamma && !aligned(gamma, 16)) return NVFP4_ERR_ALIGN;
    if (gamma && !(eps >= 0.0f)) return NVFP4_ERR_SHAPE;
    if (!ws || ws_bytes < nvfp4_workspace_size(3, rows, 0, K, 0)) return NVFP4_ERR_WORKSPACE;
    if (K == 0) return NVFP4_OK;
    ChannelAbsmaxLaunch cl;
    cl.x = x; cl.xt = xt; cl.rows = rows; cl.K = K; cl.ldx = ldx;
    cl.gamma = static_cast<const uint16_t *>(gamma); cl.eps = eps;
    cl.rscale = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + kHeaderBytes); cl.out = absmax_out;
    hipError_t e = launch_channel_absmax(cl, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : hip_fail(e);
}

nvfp4_status nvfp4_perm_from_absmax(const float *absmax_host, int64_t K, int32_t *perm_host) {
    if (K < 0) return NVFP4_ERR_SHAPE;
    if (K > 0 && (!absmax_host || !perm_host)) return NVFP4_ERR_NULL;
    std::vector<int32_t> idx((size_t)K);
    for (int64_t i = 0; i < K; ++i) idx[(size_t)i] = (int32_t)i;
    std::stable_sort(idx.begin(), idx.end(),
                     [&](int32_t a, int32_t b) { return absmax_host[a] > absmax_host[b]; });
    std::memcpy(perm_host, idx.data(), sizeof(int32_t) * (size_t)K);
    return NVFP4_OK;
}

const char *nvfp4_status_string(nvfp4_status s) {
    switch (s) {
        case NVFP4_OK: return "ok";
        case NVFP4_ERR_NULL: return "null pointer";
        case NVFP4_ERR_SHAPE: return "bad shape";
        case NVFP4_ERR_ALIGN: return "misaligned pointer or leading dimension";
        case NVFP4_ERR_DTYPE: return "bad dtype";
        case NVFP4_ERR_WORKSPACE: return "workspace too small";
        case NVFP4_ERR_UNSUPPORTED: return "unsupported";
        case NVFP4_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char *nvfp4_last_error(void) { return g_last_error; }
int nvfp4_version(void) { return 10300; }

int nvfp4_host_e4m3_encode(float v) { return (int)e4m3_rne_sat(v); }
int nvfp4_host_e2m1_encode(float q) { return (int)(e2m1_rne_sat(std::fabs(q)) | ((f2u(q) >> 31) << 3)); }

}  // extern "C"
