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
    uint8_t *codes; int64_t ldc;
    uint8_t *scales; int64_t lds;
    float *S_out;
    // workspace
    float *partials;                        // kAmaxPartials floats
    float *rscale;                          // rows floats (RMSNorm factors)
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

// Decode-shaped (small M) product; A is a canonical NVFP4 tensor whose first K
// columns are the main part and, when res_cols > 0, columns [K, K + res_cols)
// hold the residue of columns [0, res_cols).
struct SkinnyLaunch {
    const uint8_t *a_codes; int64_t a_ldc;
    const uint8_t *a_scales; int64_t a_lds;
    const float *a_S;
    const uint8_t *w_codes; int64_t w_ldc;
    const uint8_t *w_scales; int64_t w_lds;
    const float *w_S;
    int64_t M, N, K, res_cols;
    void *y; int yt; int64_t ldy;
    float *partials;                        // split-K partial sums (workspace)
    size_t partial_bytes;
};
size_t skinny_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t res_cols);
hipError_t launch_skinny(const SkinnyLaunch &g, hipStream_t st);

// Large-M tiled matrix-core product (no residue columns in this path unless
// res_cols > 0 is requested through the same tensor layout).
struct PrefillLaunch {
    const uint8_t *a_codes; int64_t a_ldc;
    const uint8_t *a_scales; int64_t a_lds;
    const float *a_S;
    const uint8_t *w_codes; int64_t w_ldc;
    const uint8_t *w_scales; int64_t w_lds;
    const float *w_S;
    int64_t M, N, K, res_cols;
    void *y; int yt; int64_t ldy;
};
hipError_t launch_prefill(const PrefillLaunch &g, hipStream_t st);

}  // namespace nvfp4
