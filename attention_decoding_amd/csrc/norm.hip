// RMSNorm for the complete cross-decoder layer (gfx950):
//   x[t, :] = h[t, :] / sqrt(mean(h[t, :]^2) + eps) * g
// (plain pre-norm Transformer reading; the pages define only the GMU and the
// shared-cache cross-attention).  x feeds a weight-streaming product, so it is
// stored as a bf16 hi + lo pair (~16 significant bits).
//
// One workgroup per token row; the row and the gains are requested at once
// (8-byte pieces, four columns per thread per 1024-column chunk) and kept in
// registers for the scaling; the sum of squares in the fixed order of
// norm_order.hpp.
#include "device.hpp"
#include "launch.hpp"
#include "norm_order.hpp"

#include <math.h>

namespace sambay {

namespace {

__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const bf16_t *__restrict__ h,
                                                               const bf16_t *__restrict__ g, int d, float eps,
                                                               bf16_t *__restrict__ out_hi,
                                                               bf16_t *__restrict__ out_lo) {
    __shared__ float red[kNormThreads / 64];
    const size_t row = (size_t)blockIdx.x * d;
    const int nch = norm_chunks(d);
    u32x2 xs[kNormMaxChunks], gs[kNormMaxChunks];
#pragma unroll
    for (int c = 0; c < kNormMaxChunks; ++c) {
        const int n = kNormChunk * c + 4 * threadIdx.x;
        if (c < nch && n < d) {
            xs[c] = *reinterpret_cast<const u32x2 *>(h + row + n);
            gs[c] = *reinterpret_cast<const u32x2 *>(g + n);
        }
    }
    float tot = 0.f;
#pragma unroll
    for (int c = 0; c < kNormMaxChunks; ++c) {
        if (c >= nch) break;
        const int n = kNormChunk * c + 4 * threadIdx.x;
        tot += norm_chunk_sum(n < d ? norm_sq4(xs[c]) : 0.f, red);
    }
    const float r = norm_scale(tot, 1.f / (float)d, eps);
#pragma unroll
    for (int c = 0; c < kNormMaxChunks; ++c) {
        const int n = kNormChunk * c + 4 * threadIdx.x;
        if (c >= nch || n >= d) continue;
        u32x2 hi, lo;
        norm_apply4(xs[c], gs[c], r, hi, lo);
        *reinterpret_cast<u32x2 *>(out_hi + row + n) = hi;
        if (out_lo) *reinterpret_cast<u32x2 *>(out_lo + row + n) = lo;
    }
}

}  // namespace

hipError_t launch_rmsnorm(const bf16_t *h, const bf16_t *g, int rows, int d, float eps, bf16_t *out_hi,
                          bf16_t *out_lo, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    if (d % 4 != 0 || norm_chunks(d) > kNormMaxChunks) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(kNormThreads), 0, stream, h, g, d, eps, out_hi, out_lo);
    return hipGetLastError();
}

}  // namespace sambay
