// Cache append of the self-decoder's attention layers (gfx950).
//
// One decode step of a self-decoder attention layer stores the new token's
// key and value rows before its query attends (the Paper-Notes page on
// "Decoder-Hybrid-Decoder Architecture for Efficient Reasoning with Long
// Generation", section 整体框架: the final full-attention layer writes the
// one cache that the cross-decoder reads; section 消融实验: the other
// attention layers use a 256-position sliding window).  Sequence b's new
// token is at position p = pos[b]: with a full cache its rows go to position
// p, with a window of W slots to ring slot p mod W.  The kernel also writes
// the number of visible positions per sequence (p + 1, at most the cache's
// L or W slots; 0 for an inactive sequence, p < 0), which the attention
// kernels that follow on the same stream read as their lengths.
//
// Byte work: 2 x 256 B per (sequence, KV head) at D = 128, 16-byte stores.
#include "device.hpp"
#include "launch.hpp"

namespace sambay {

namespace {

constexpr int kPairsPerWG = 8;  // (sequence, KV head) pairs per workgroup: 32 threads each

__global__ __launch_bounds__(32 * kPairsPerWG) void kv_append_kernel(const bf16_t *__restrict__ k_new,
                                                                     const bf16_t *__restrict__ v_new,
                                                                     bf16_t *__restrict__ K, bf16_t *__restrict__ V,
                                                                     const int32_t *__restrict__ pos,
                                                                     int32_t *__restrict__ lens_out, int B, int Hkv,
                                                                     int L, int window) {
    const int pair = blockIdx.x * kPairsPerWG + (int)(threadIdx.x >> 5);
    if (pair >= B * Hkv) return;  // no barrier below
    const int b = pair / Hkv;
    const int p = pos[b];
    const int which = (threadIdx.x >> 4) & 1, c = threadIdx.x & 15;  // K or V row, 16-byte piece
    // A full cache has no slot for p >= L: nothing is stored and L positions
    // stay visible (the documented clamp; the host cannot see device values).
    if (p >= 0 && (window > 0 || p < L)) {
        const int slot = window > 0 ? p % window : p;
        const bf16_t *src = (which ? v_new : k_new) + (size_t)pair * kHeadDim + 8 * c;
        bf16_t *dst = (which ? V : K) + ((size_t)pair * L + slot) * kHeadDim + 8 * c;
        *reinterpret_cast<u32x4 *>(dst) = ld16(src);
    }
    if (lens_out && pair % Hkv == 0 && (threadIdx.x & 31) == 0)
        lens_out[b] = p < 0 ? 0 : min(p + 1, L);  // a window's cache has L == window slots
}

}  // namespace

hipError_t launch_kv_append(const bf16_t *k_new, const bf16_t *v_new, bf16_t *K, bf16_t *V, const int32_t *pos,
                            int32_t *lens_out, int B, int Hkv, int L, int window, hipStream_t stream) {
    const int pairs = B * Hkv;
    const unsigned wgs = (unsigned)((pairs + kPairsPerWG - 1) / kPairsPerWG);
    hipLaunchKernelGGL(kv_append_kernel, dim3(wgs), dim3(32 * kPairsPerWG), 0, stream, k_new, v_new, K, V, pos,
                       lens_out, B, Hkv, L, window);
    return hipGetLastError();
}

}  // namespace sambay
