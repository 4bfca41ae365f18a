// pack.hip -- row-major NVFP4 and MXFP4 weights -> the tiled layouts read by
// the decode products (items of 16 rows x 512 columns, stored in the lane order
// of their loads; zero codes and scales past the tensor). Byte permutations: no
// value changes.
#include "internal.h"

namespace nvfp4 {
namespace {

// One workgroup per item: 256 threads x 16 B of codes, 64 threads x 8 B of scales.
__global__ __launch_bounds__(256) void pack_tiled_kernel(PackLaunch g, int64_t KU) {
    const int64_t item = blockIdx.x, t = item / KU, u = item - t * KU;
    const int tid = threadIdx.x, i = tid >> 6, p = tid & 63, r = p & 15, gq = p >> 4;
    const int64_t n = 16 * t + r;
    const int64_t k = 512 * u + 128 * gq + 32 * i;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (n < g.rows && k < g.K) {
        const uint8_t *src = g.src_codes + n * g.src_ldc + k / 2;
        if (k + 32 <= g.K) {
            v = *reinterpret_cast<const uint4 *>(src);
        } else {                                         // 16 columns left
            const uint2 h = *reinterpret_cast<const uint2 *>(src);
            v.x = h.x; v.y = h.y;
        }
    }
    *reinterpret_cast<uint4 *>(g.dst_codes + t * g.dst_ldc + u * 4096 + 1024 * i + 16 * p) = v;
    if (tid < 64) {
        const int64_t b0 = 32 * u + 8 * gq;              // first block of this lane
        uint32_t w[2] = {0, 0};
        if (n < g.rows) {
#pragma unroll
            for (int b = 0; b < 8; ++b)
                if ((b0 + b) * 16 < g.K) w[b >> 2] |= (uint32_t)g.src_scales[n * g.src_lds + b0 + b] << (8 * (b & 3));
        }
        *reinterpret_cast<uint2 *>(g.dst_scales + t * g.dst_lds + u * 512 + 8 * p) = make_uint2(w[0], w[1]);
    }
    if (item == 0 && tid == 0) *g.dst_S = *g.src_S;
}

// One item (16 rows x 512 columns) per workgroup; thread (i, p) moves the 16
// code bytes and the E8M0 byte of row 16t + p % 16, step i, 32-column block p / 16.
__global__ __launch_bounds__(256) void mx_pack_tiled_kernel(MXPackLaunch g, int64_t KU) {
    const int64_t item = blockIdx.x, t = item / KU, u = item - t * KU;
    const int tid = threadIdx.x, i = tid >> 6, p = tid & 63, r = p & 15, gq = p >> 4;
    const int64_t n = 16 * t + r;
    const int64_t k = 512 * u + 128 * i + 32 * gq;   // a whole 32-column block: K % 32 == 0
    uint4 v = make_uint4(0, 0, 0, 0);
    uint8_t sb = 0;
    if (n < g.rows && k < g.K) {
        v = *reinterpret_cast<const uint4 *>(g.src_codes + n * g.src_ldc + k / 2);
        sb = g.src_scales[n * g.src_lds + k / 32];
    }
    *reinterpret_cast<uint4 *>(g.dst_codes + t * g.dst_ldc + u * 4096 + 1024 * i + 16 * p) = v;
    g.dst_scales[t * g.dst_lds + u * 256 + 64 * i + p] = sb;
}

}  // namespace

hipError_t launch_mx_pack_tiled(const MXPackLaunch &g, hipStream_t st) {
    const int64_t NT = (g.rows + 15) / 16, KU = (g.K + 511) / 512;
    if (NT * KU == 0) return hipSuccess;
    hipLaunchKernelGGL(mx_pack_tiled_kernel, dim3((unsigned)(NT * KU)), dim3(256), 0, st, g, KU);
    return hipGetLastError();
}

hipError_t launch_pack_tiled(const PackLaunch &g, hipStream_t st) {
    const int64_t NT = (g.rows + 15) / 16, KU = (g.K + 511) / 512;
    if (NT * KU == 0) {
        if (g.rows >= 0 && g.src_S != g.dst_S)
            return hipMemcpyAsync(g.dst_S, g.src_S, sizeof(float), hipMemcpyDeviceToDevice, st);
        return hipSuccess;
    }
    hipLaunchKernelGGL(pack_tiled_kernel, dim3((unsigned)(NT * KU)), dim3(256), 0, st, g, KU);
    return hipGetLastError();
}

}  // namespace nvfp4
