// Measured-ceiling probes for benchmarks (not part of the method): a plain
// streaming read and a register-only MFMA loop.  Their rates say what this
// machine delivers to a kernel that does nothing else, beside the datasheet
// peaks (HBM 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s).
#include "sambay.h"

#include "device.hpp"
#include "launch.hpp"

using namespace sambay;

namespace {

constexpr int kReadThreads = 256, kReadInFlight = 8;

// Measured on MI355X: 256 workgroups saturate HBM on GB-sized buffers; reads
// of tens of MB finish sooner with ~1024 (more requests in flight at once).
int read_wgs(size_t bytes) { return bytes < ((size_t)256 << 20) ? 1024 : 256; }

// Grid-stride read: each workgroup reads 32 KB contiguous per step (eight 16-byte
// loads in flight per thread), the grid sweeps memory linearly.  Non-temporal
// loads: on MI355X they read a 4 GiB buffer at ~7.0-7.4 TB/s against
// ~6.2-6.4 TB/s for plain loads (256-4096 workgroups).
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4 *__restrict__ p, size_t n,
                                                                   unsigned *__restrict__ sink) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    const size_t stride = (size_t)gridDim.x * kReadThreads * kReadInFlight;
    for (size_t base = (size_t)blockIdx.x * kReadThreads * kReadInFlight + threadIdx.x; base < n; base += stride) {
        u32x4 v[kReadInFlight];
#pragma unroll
        for (int u = 0; u < kReadInFlight; ++u) {
            const size_t i = base + (size_t)u * kReadThreads;
            v[u] = i < n ? __builtin_nontemporal_load(p + i) : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kReadInFlight; ++u) acc ^= v[u];
    }
    // Never true for realistic data; keeps the loads live.
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u && threadIdx.x == 0) sink[0] = 1u;
}

constexpr int kMfmaWGs = 1024, kMfmaThreads = 256, kMfmaChains = 4;

__global__ __launch_bounds__(kMfmaThreads) void mfma_loop_kernel(int64_t iters, unsigned *__restrict__ sink) {
    u32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = pack_bf16x2(0.001f * threadIdx.x, 0.5f * i);
        b[i] = pack_bf16x2(0.25f * i, 0.002f * threadIdx.x);
    }
    f32x16 acc[kMfmaChains];
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
    for (int64_t it = 0; it < iters; ++it)
#pragma unroll
        for (int c = 0; c < kMfmaChains; ++c) acc[c] = mfma32x32x16(a, b, acc[c]);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) s += acc[c][0];
    if (s == 1234.5f && threadIdx.x == 0) sink[0] = 1u;
}

}  // namespace

extern "C" sb_status sb_probe_stream_read(const void *data, size_t bytes, void *sink, hipStream_t stream) {
    if (!data || !sink || bytes % 16 != 0 || ((uintptr_t)data & 15u) != 0) return SB_EINVAL;
    if (bytes == 0) return SB_OK;
    TimingScope ts(kTimeProbe, stream);
    hipLaunchKernelGGL(stream_read_kernel, dim3(read_wgs(bytes)), dim3(kReadThreads), 0, stream,
                       static_cast<const u32x4 *>(data), bytes / 16, static_cast<unsigned *>(sink));
    return hipGetLastError() == hipSuccess ? SB_OK : SB_EHIP;
}

extern "C" sb_status sb_probe_mfma(int64_t iters, void *sink, hipStream_t stream) {
    if (iters < 0 || !sink) return SB_EINVAL;
    TimingScope ts(kTimeProbe, stream);
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(kMfmaWGs), dim3(kMfmaThreads), 0, stream, iters,
                       static_cast<unsigned *>(sink));
    return hipGetLastError() == hipSuccess ? SB_OK : SB_EHIP;
}

extern "C" double sb_probe_mfma_flops(int64_t iters) {
    return (double)kMfmaWGs * (kMfmaThreads / 64) * kMfmaChains * (double)iters * 32768.0;
}
