// RMSNorm for the complete cross-decoder layer (gfx950):
//   x[t, :] = h[t, :] / sqrt(mean(h[t, :]^2) + eps) * g
// (plain pre-norm Transformer reading; the pages define only the GMU and the
// shared-cache cross-attention).  x feeds a weight-streaming product, so it is
// stored as a bf16 hi + lo pair (~16 significant bits).
//
// One workgroup per token row; 16-byte loads of h and g; the sum of squares is
// reduced in a fixed order (deterministic).  The row is re-read from L1/L2 for
// the scaling pass.
#include "device.hpp"
#include "launch.hpp"

#include <math.h>

namespace sambay {

namespace {

constexpr int kThreads = 256;

// Up to kMaxVec 8-element vectors of a row per thread (rows up to 8192).
constexpr int kMaxVec = 4;

__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(const bf16_t *__restrict__ h, const bf16_t *__restrict__ g,
                                                           int d, float eps, bf16_t *__restrict__ out_hi,
                                                           bf16_t *__restrict__ out_lo) {
    __shared__ float red[kThreads / 64];
    const size_t row = (size_t)blockIdx.x * d;
    const int nvec = d / 8;
    // The row and the gains are requested at once and kept in registers for
    // the scaling (one round trip to memory; same arithmetic order as a
    // strided loop over the vectors).
    u32x4 xs[kMaxVec], gs[kMaxVec];
#pragma unroll
    for (int i = 0; i < kMaxVec; ++i) {
        const int v = threadIdx.x + i * kThreads;
        if (v < nvec) {
            xs[i] = ld16(h + row + 8 * v);
            gs[i] = ld16(g + 8 * v);
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxVec; ++i) {
        const int v = threadIdx.x + i * kThreads;
        if (v < nvec) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = lo_bf16(xs[i][e]), b = hi_bf16(xs[i][e]);
                ss += a * a + b * b;
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) tot += red[w];
    const float r = 1.f / sqrtf(tot / (float)d + eps);
#pragma unroll
    for (int i = 0; i < kMaxVec; ++i) {
        const int v = threadIdx.x + i * kThreads;
        if (v >= nvec) break;
        const u32x4 x = xs[i], gv = gs[i];
        u32x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float y0 = lo_bf16(x[e]) * r * lo_bf16(gv[e]);
            const float y1 = hi_bf16(x[e]) * r * hi_bf16(gv[e]);
            const bf16_t h0 = f32_to_bf16(y0), h1 = f32_to_bf16(y1);
            hi[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lo[e] = pack_bf16x2(y0 - bf16_to_f32(h0), y1 - bf16_to_f32(h1));
        }
        *reinterpret_cast<u32x4 *>(out_hi + row + 8 * v) = hi;
        if (out_lo) *reinterpret_cast<u32x4 *>(out_lo + row + 8 * v) = lo;
    }
}

}  // namespace

hipError_t launch_rmsnorm(const bf16_t *h, const bf16_t *g, int rows, int d, float eps, bf16_t *out_hi,
                          bf16_t *out_lo, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    if (d % 8 != 0 || d > 8 * kThreads * kMaxVec) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(kThreads), 0, stream, h, g, d, eps, out_hi, out_lo);
    return hipGetLastError();
}

}  // namespace sambay
