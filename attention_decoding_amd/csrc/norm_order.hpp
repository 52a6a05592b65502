// The RMSNorm sum of squares in one fixed order, shared by every kernel that
// computes it, so that a norm computed in a residual product's finishing pass
// (then applied where the next product stages its operand) gives the same
// bits as the standalone RMSNorm kernel:
//  * the row's columns in chunks of 1024; in a chunk, thread i of 256 takes
//    columns 4i .. 4i + 3 and adds their squares in column order;
//  * the 64 lanes of a wave are summed by an xor butterfly, the four waves
//    of the chunk in wave order;
//  * the row's total adds the chunk sums in chunk order, from zero;
//  * r = rsqrt(total · (1 / d) + eps) by the hardware reciprocal square
//    root (v_rsq_f32, within 1 ulp), and x = (h · r) · g per column, stored
//    as a bf16 hi + lo pair.
#pragma once

#include "device.hpp"

namespace sambay {

constexpr int kNormChunk = 1024;
constexpr int kNormThreads = 256;
constexpr int kNormMaxChunks = 8;  // rows up to 8192 columns

// Per-token chunk sums are stored kNormStatsStride floats apart (16 or 32
// bytes: one or two copy lanes per token).
__host__ __device__ constexpr int norm_chunks(int d) { return (d + kNormChunk - 1) / kNormChunk; }
__host__ __device__ constexpr int norm_stats_stride(int d) { return norm_chunks(d) <= 4 ? 4 : 8; }

// The squares of four bf16 values (two packed pairs), added in column order.
__device__ __forceinline__ float norm_sq4(u32x2 v) {
    const float a = lo_bf16(v[0]), b = hi_bf16(v[0]), c = lo_bf16(v[1]), d = hi_bf16(v[1]);
    float s = a * a;
    s += b * b;
    s += c * c;
    s += d * d;
    return s;
}

// The chunk's sum over a workgroup of kNormThreads threads (every thread
// calls it; red: 4 floats of LDS, free again on return).
__device__ __forceinline__ float norm_chunk_sum(float ss, float *red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float c = ((red[0] + red[1]) + red[2]) + red[3];
    __syncthreads();
    return c;
}

__device__ __forceinline__ float norm_scale(float total, float inv_d, float eps) {
    return __builtin_amdgcn_rsqf(total * inv_d + eps);
}

// Four columns (two packed bf16 pairs of h and of the gain) normalised and
// split into bf16 hi + lo pairs: y = (h · r) · g rounded to fp32, hi = bf16(y),
// lo = bf16(y - hi).  No multiply-add contraction here: a fused
// (h · r) · g - hi would form lo from the unrounded product in some kernels
// and not in others.
__device__ __forceinline__ void norm_apply4(u32x2 x, u32x2 g, float r, u32x2 &hi, u32x2 &lo) {
#pragma clang fp contract(off)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const float y0 = lo_bf16(x[e]) * r * lo_bf16(g[e]);
        const float y1 = hi_bf16(x[e]) * r * hi_bf16(g[e]);
        const bf16_t h0 = f32_to_bf16(y0), h1 = f32_to_bf16(y1);
        hi[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lo[e] = pack_bf16x2(y0 - bf16_to_f32(h0), y1 - bf16_to_f32(h1));
    }
}

}  // namespace sambay
