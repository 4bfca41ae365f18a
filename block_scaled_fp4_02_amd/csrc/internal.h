// internal.h -- host-side launch interfaces shared by the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

enum InType { IN_BF16 = 0, IN_F32 = 1 };

// Workspace carve-up for the quantizer: partial maxima and per-row RMSNorm factors.
constexpr int kAmaxPartials = 1024;          // upper bound on amax workgroups

struct QuantLaunch {
    const void *x; int xt; int64_t rows, K_in, ldx;
    const uint16_t *gamma; float eps;       // bf16 gamma or nullptr
    const int32_t *perm;                    // or nullptr
    int64_t res_cols;                       // residue columns appended at K_in
    const float *static_S;                  // or nullptr
    const float *smooth;                    // per input channel multiplier (FP32 [K_in]) or nullptr
    uint8_t *codes; int64_t ldc;
    uint8_t *scales; int64_t lds;
    float *S_out;
    // workspace
    float *partials;                        // kAmaxPartials floats
    float *rscale;                          // rows floats (RMSNorm factors)
    unsigned long long *slots;              // 64 arrival slots of the small quantizer (header), or nullptr
    unsigned long long *grid_slots;         // 256 arrival slots of the grid quantizer (header), or nullptr
    unsigned spin;                          // bound on the arrival wait (polls)
};

// Enqueue the amax pass (if the scale is dynamic) and the quantize pass.
hipError_t launch_quantize(const QuantLaunch &q, hipStream_t st);

struct ChannelAbsmaxLaunch {
    const void *x; int xt; int64_t rows, K, ldx;
    const uint16_t *gamma; float eps;
    float *rscale;                          // rows floats of scratch (only with gamma)
    float *out;                             // K floats
};
hipError_t launch_channel_absmax(const ChannelAbsmaxLaunch &c, hipStream_t st);

// Every workspace starts with a header of counters: the small quantizer's 64
// arrival slots (bytes 512..1023: partial maximum and epoch), the grid
// quantizer's 256 (bytes 1024..3071) and the decode product's split-K tile
// counters (from byte 4096). It must be zero before the
// first call on a workspace; calls keep it valid (counts return to zero, all
// slots advance to the same epoch), so it never needs clearing again.
constexpr size_t kHeaderBytes = 8192;
constexpr size_t kTileCntOffset = 4096;         // header bytes before the arrival counters
constexpr int64_t kMaxCounters = (int64_t)((kHeaderBytes - kTileCntOffset) / sizeof(unsigned));
constexpr size_t kSlotsOffset = 512;
constexpr size_t kGridSlotsOffset = 1024;

// Decode-shaped (M <= 64) product in one launch. With x != nullptr (bf16, and
// decode_can_fuse true) the raw activations are quantized inside the kernel and
// also stored into q_* (canonical NVFP4 layout, K + res_cols columns: the
// residue of columns [0, res_cols) after column K); with x == nullptr q_*
// already hold them.
struct DecodeLaunch {
    const void *x; int64_t ldx;
    const float *static_S;
    uint8_t *q_codes; int64_t q_ldc;
    uint8_t *q_scales; int64_t q_lds;
    float *q_S;
    const uint8_t *w_codes; int64_t w_ldc;  // row-major, or tiled (w_tiled: strip strides)
    const uint8_t *w_scales; int64_t w_lds;
    const float *w_S;
    int w_tiled;
    int64_t M, N, K, res_cols;
    void *y; int yt; int64_t ldy;
    unsigned *header;                       // kHeaderBytes, zero-kept
    void *scratch; size_t scratch_bytes;    // decode_workspace_bytes()
};
size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t res_cols);
bool decode_can_fuse(int64_t M, int64_t N, int64_t K, int64_t res_cols, bool x_bf16);
hipError_t launch_decode(const DecodeLaunch &g, hipStream_t st);

// Large-M matrix-core product over 128 x 128 (or 64 x 128) output tiles; the
// residue columns (res_cols > 0) follow column K in the activation tensor.
struct PrefillLaunch {
    const uint8_t *a_codes; int64_t a_ldc;
    const uint8_t *a_scales; int64_t a_lds;
    const float *a_S;
    const uint8_t *w_codes; int64_t w_ldc;  // row-major, or tiled (w_tiled)
    const uint8_t *w_scales; int64_t w_lds;
    const float *w_S;
    int w_tiled;
    int64_t M, N, K, res_cols;
    void *y; int yt; int64_t ldy;
    void *scratch; size_t scratch_bytes;    // split-K partials (prefill_workspace_bytes), or nullptr
};
// Workspace bytes of the prefill product: fp32 split-K partials when the plan
// splits K (long K, too few output tiles to fill the chip), else 0.
size_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t S);
hipError_t launch_prefill(const PrefillLaunch &g, hipStream_t st);

// Row-major -> tiled weight layout (16 x 512 items in decode lane order).
struct PackLaunch {
    const uint8_t *src_codes; int64_t src_ldc;
    const uint8_t *src_scales; int64_t src_lds;
    const float *src_S;
    uint8_t *dst_codes; int64_t dst_ldc;
    uint8_t *dst_scales; int64_t dst_lds;
    float *dst_S;
    int64_t rows, K;
};
hipError_t launch_pack_tiled(const PackLaunch &g, hipStream_t st);

// Row-major MXFP4 -> tiled MX layout (items of 16 rows x 512 columns).
struct MXPackLaunch {
    const uint8_t *src_codes; int64_t src_ldc;
    const uint8_t *src_scales; int64_t src_lds;
    uint8_t *dst_codes; int64_t dst_ldc;
    uint8_t *dst_scales; int64_t dst_lds;
    int64_t rows, K;
};
hipError_t launch_mx_pack_tiled(const MXPackLaunch &g, hipStream_t st);

// MXFP4 (E2M1 codes, one E8M0 byte per 32 elements along K, no tensor scale).
struct MXQuantLaunch {
    const void *x; int xt; int64_t rows, K, ldx;
    int64_t res_cols;                       // residue of columns [0, res_cols) after column K
    uint8_t *codes; int64_t ldc;
    uint8_t *scales; int64_t lds;
};
hipError_t launch_mx_quantize(const MXQuantLaunch &q, hipStream_t st);

// y = A W^T over the K (+ res_cols residue) columns: A is M x (K + res_cols),
// W is N x K; the residue columns meet W's first res_cols columns.
struct MXGemmLaunch {
    const uint8_t *a_codes; int64_t a_ldc;
    const uint8_t *a_scales; int64_t a_lds;
    const uint8_t *w_codes; int64_t w_ldc;
    const uint8_t *w_scales; int64_t w_lds;
    int w_tiled;                            // W in the tiled MX layout (M <= 64 only)
    int64_t M, N, K, res_cols;
    void *y; int yt; int64_t ldy;
    void *scratch; size_t scratch_bytes;    // mx_workspace_bytes()
};
size_t mx_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t S);
hipError_t launch_mx_gemm(const MXGemmLaunch &g, hipStream_t st);

// Decode attention over an NVFP4 KV cache with residue-compensated query and
// probabilities: K cache [H*T, D], V cache transposed [H*D, T] (row-major).
struct AttentionLaunch {
    const void *q; int qt; int64_t ldq;     // [H][D] bf16 or f32
    int64_t H, D, T;                        // H <= 65535, D % 32 == 0, D <= 256, T % 16 == 0, T > 0
    const uint8_t *k_codes; int64_t k_ldc;
    const uint8_t *k_scales; int64_t k_lds;
    const float *k_S;
    const uint8_t *v_codes; int64_t v_ldc;
    const uint8_t *v_scales; int64_t v_lds;
    const float *v_S;
    int compensate;
    float *out; int64_t ldo;                // [H][D] FP32
    void *scratch; size_t scratch_bytes;    // attention_workspace_bytes()
};
size_t attention_workspace_bytes(int64_t H, int64_t D, int64_t T);
hipError_t launch_attention(const AttentionLaunch &g, hipStream_t st);

}  // namespace nvfp4
