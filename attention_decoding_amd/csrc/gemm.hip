// MFMA bf16 GEMM for GMU prefill (gfx950):
//   out[r, n] = epilogue( Σ_k X[r, k] · W[n, k] )   (both operands K-contiguous)
// The GMU (Paper-Notes reading notes on "Decoder-Hybrid-Decoder Architecture
// for Efficient Reasoning with Long Generation", section 关键设计) needs two:
//   H = M ⊙ SiLU(X W1^T)   — the SiLU·M Hadamard product fused in the epilogue,
//   Y = H W2^T.
//
// Design (compute-bound at prefill sizes):
//  * 128x128 output tile per workgroup, 4 waves in a 2x2 grid, each wave a
//    64x64 block of 4x4 16x16x32 MFMA tiles (fp32 accumulators in registers).
//  * K advances 64 at a time through a double-buffered LDS stage: global ->
//    registers for stage k+1 overlaps the MFMAs of stage k; one barrier per
//    stage.  16-byte chunks of each 128-byte LDS row are XOR-swizzled by
//    (row / 2) so the 16 lanes of an operand read hit 16 distinct bank groups.
//  * Workgroup ids are remapped so each XCD (ids round-robin over 8) works
//    on a contiguous band of tiles, grouped 8 row-tiles at a time, which keeps
//    the shared operand rows in that XCD's L2.
#include "device.hpp"
#include "launch.hpp"

#include <math.h>

namespace sambay {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

template <int EPI>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const bf16_t *__restrict__ X, const bf16_t *__restrict__ W,
                                                        int rows, int N, int K, bf16_t *__restrict__ out,
                                                        const bf16_t *__restrict__ aux) {
    __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * BK];
    __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * BK];

    // XCD-aware tile order.
    const int tiles_m = (rows + BM - 1) / BM, tiles_n = N / BN + (N % BN != 0);
    const int ntiles = tiles_m * tiles_n;
    int pid = blockIdx.x;
    if (ntiles % kXcds == 0) pid = (pid % kXcds) * (ntiles / kXcds) + pid / kXcds;
    const int group = pid / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int tm = first_m + (pid % (kGroupM * tiles_n)) % gsize;
    const int tn = (pid % (kGroupM * tiles_n)) / gsize;
    const int bm = tm * BM, bn = tn * BN;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4, col = lane & 15;
    const int wm = wave >> 1, wn = wave & 1;

    // Global loads: 4 chunks of 16 B per operand per thread; 8 threads per 128-byte row.
    const bf16_t *ga[4], *gb[4];
    int soff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = tid + kThreads * j;
        const int r = i >> 3, c = i & 7;
        ga[j] = X + (size_t)min(bm + r, rows - 1) * K + 8 * c;
        gb[j] = W + (size_t)min(bn + r, N - 1) * K + 8 * c;
        soff[j] = r * BK + 8 * swz(r, c);
    }

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    u32x4 ra[4], rb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ra[j] = ld16(ga[j]);
        rb[j] = ld16(gb[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<u32x4 *>(&sA[0][soff[j]]) = ra[j];
        *reinterpret_cast<u32x4 *>(&sB[0][soff[j]]) = rb[j];
    }
    __syncthreads();

    const int KT = K / BK;
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                ra[j] = ld16(ga[j] + (size_t)(kt + 1) * BK);
                rb[j] = ld16(gb[j] + (size_t)(kt + 1) * BK);
            }
        }
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
            u32x4 fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wm * 64 + 16 * i + col;
                fa[i] = *reinterpret_cast<const u32x4 *>(&sA[cur][r * BK + 8 * swz(r, 4 * kk + grp)]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wn * 64 + 16 * i + col;
                fb[i] = *reinterpret_cast<const u32x4 *>(&sB[cur][r * BK + 8 * swz(r, 4 * kk + grp)]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(fa[i], fb[j], acc[i][j]);
        }
        if (kt + 1 < KT) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                *reinterpret_cast<u32x4 *>(&sA[cur ^ 1][soff[j]]) = ra[j];
                *reinterpret_cast<u32x4 *>(&sB[cur ^ 1][soff[j]]) = rb[j];
            }
        }
        __syncthreads();
    }

    // acc[i][j][r]: row bm + 64·wm + 16·i + 4·grp + r, col bn + 64·wn + 16·j + col.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = bm + wm * 64 + 16 * i + 4 * grp + r;
            if (m >= rows) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = bn + wn * 64 + 16 * j + col;
                if (n >= N) continue;
                const size_t o = (size_t)m * N + n;
                float v = acc[i][j][r];
                if (EPI == EPI_GATE) v = bf16_to_f32(aux[o]) * (v / (1.f + expf(-v)));
                out[o] = f32_to_bf16(v);
            }
        }
}

}  // namespace

hipError_t launch_gemm(const bf16_t *X, const bf16_t *W, int rows, int N, int K, Epilogue epi, bf16_t *out,
                       const bf16_t *aux, hipStream_t stream) {
    const int tiles = ((rows + BM - 1) / BM) * ((N + BN - 1) / BN);
    TimingScope ts(kTimeGemm, stream);
    if (epi == EPI_GATE)
        hipLaunchKernelGGL(gemm_kernel<EPI_GATE>, dim3(tiles), dim3(kThreads), 0, stream, X, W, rows, N, K, out, aux);
    else
        hipLaunchKernelGGL(gemm_kernel<EPI_BF16>, dim3(tiles), dim3(kThreads), 0, stream, X, W, rows, N, K, out, aux);
    return hipGetLastError();
}

}  // namespace sambay
