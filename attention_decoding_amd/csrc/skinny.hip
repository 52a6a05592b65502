// Weight-streaming skinny products for decode (gfx950):
//   out[t, n] = epilogue( Σ_k X[t, k] · W[n, k] ),  t < T <= 64 tokens.
// Used for both GMU products of a decode step (Paper-Notes reading notes on
// "Decoder-Hybrid-Decoder Architecture for Efficient Reasoning with Long
// Generation", section 关键设计: Y = (M ⊙ SiLU(X W1^T)) W2) and for the
// cross-attention layer's query and output projections.
//
// Design (HBM-bound: every weight byte is read once per step, the tokens are
// few):
//  * The N weight rows are cut into ~256 equal row ranges, one workgroup each,
//    so every CU streams the same number of bytes.  Eight waves per
//    workgroup split the K dimension in 64-wide chunks; their 16x16x32 MFMA
//    partial tiles are summed through LDS in a fixed order (deterministic).
//  * A operand = 16 weight rows; MFMA k-step t of a chunk covers 32
//    contiguous K elements, lane group grp holding elements 8·grp .. 8·grp+7,
//    so each load instruction reads 64 contiguous bytes of 16 rows.  B operand
//    = 16 tokens of X with the same K assignment (X is small and L2-resident).
//    Tokens are padded to 16 per tile; rows past the range are zero operands.
//  * Epilogues are fused: fp32 store, bf16 store, the GMU gate
//    H = M ⊙ SiLU(acc) stored as bf16, or the residual add h = bf16(h + acc).
//  * For shapes whose row ranges would be too thin, K is also split across
//    workgroups; fp32 partials then go through a small finishing kernel.
#include "device.hpp"
#include "launch.hpp"

#include <math.h>
#include <stdlib.h>

namespace sambay {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 64;      // K per wave step: two MFMA k-steps
constexpr int kTargetWGs = 256;

template <int EPI>
__device__ __forceinline__ void apply_epilogue(float v, int t, int n, void *out, int ldo, const bf16_t *aux,
                                               int ldaux) {
    const size_t o = (size_t)t * ldo + n;
    if (EPI == EPI_F32) {
        reinterpret_cast<float *>(out)[o] = v;
    } else if (EPI == EPI_BF16) {
        reinterpret_cast<bf16_t *>(out)[o] = f32_to_bf16(v);
    } else if (EPI == EPI_GATE) {
        const float m = bf16_to_f32(aux[(size_t)t * ldaux + n]);
        const float silu = v / (1.f + expf(-v));
        reinterpret_cast<bf16_t *>(out)[o] = f32_to_bf16(m * silu);
    } else {
        bf16_t *h = reinterpret_cast<bf16_t *>(out);
        h[o] = f32_to_bf16(bf16_to_f32(h[o]) + v);
    }
}

// RT row tiles of 16, TB token tiles of 16, U chunks in flight per wave.
template <int RT, int TB, int U, int EPI>
__global__ __launch_bounds__(kThreads) void skinny_kernel(const bf16_t *__restrict__ X, int ldx,
                                                          const bf16_t *__restrict__ W, int T, int N, int K, int R,
                                                          int k_slice, void *out, int ldo,
                                                          const bf16_t *__restrict__ aux, int ldaux,
                                                          float *__restrict__ partials) {
    constexpr int TT = 16 * TB;
    __shared__ float red[kWaves][16 * RT][TT + 4];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
    const int n0 = blockIdx.x * R;
    const int kbeg = blockIdx.y * k_slice;
    const int nchunks = k_slice / kChunk;

    const bf16_t *wrow[RT];
    bool rvalid[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int rl = 16 * rt + col;
        rvalid[rt] = rl < R && n0 + rl < N;
        wrow[rt] = W + (size_t)(rvalid[rt] ? n0 + rl : 0) * K + kbeg + 8 * grp;
    }
    const bf16_t *xrow[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) xrow[tb] = X + (size_t)min(16 * tb + col, T - 1) * ldx + kbeg + 8 * grp;

    f32x4 acc[RT][TB];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[rt][tb] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Wave w owns chunks w, w + kWaves, w + 2·kWaves, ... (balanced); it keeps U
    // of them in flight: all weight loads of a group are issued before any MFMA.
    for (int j0 = 0; wave + kWaves * j0 < nchunks; j0 += U) {
        u32x4 wf[U][RT][2], xf[U][TB][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = wave + kWaves * (j0 + u);
            const bool live = c < nchunks;
            const int k = c * kChunk;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    wf[u][rt][t] = (live && rvalid[rt]) ? ld16(wrow[rt] + k + 32 * t) : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = wave + kWaves * (j0 + u);
            const bool live = c < nchunks;
            const int k = c * kChunk;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int t = 0; t < 2; ++t) xf[u][tb][t] = live ? ld16(xrow[tb] + k + 32 * t) : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb) acc[rt][tb] = mfma16x16x32(wf[u][rt][t], xf[u][tb][t], acc[rt][tb]);
    }

    // acc[rt][tb][r] = partial of row n0 + 16·rt + 4·grp + r, token 16·tb + col.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][16 * rt + 4 * grp + r][16 * tb + col] = acc[rt][tb][r];
    __syncthreads();

    const int total = R * T;
    for (int idx = threadIdx.x; idx < total; idx += kThreads) {
        const int t = idx / R, rl = idx % R, n = n0 + rl;
        if (n >= N) continue;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) v += red[w][rl][t];
        if (gridDim.y == 1)
            apply_epilogue<EPI>(v, t, n, out, ldo, aux, ldaux);
        else
            partials[((size_t)blockIdx.y * T + t) * N + n] = v;
    }
}

template <int EPI>
__global__ __launch_bounds__(256) void skinny_finish_kernel(const float *__restrict__ partials, int splits, int T,
                                                            int N, void *out, int ldo, const bf16_t *__restrict__ aux,
                                                            int ldaux) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)T * N) return;
    const int t = (int)(idx / N), n = (int)(idx % N);
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += partials[((size_t)s * T + t) * N + n];
    apply_epilogue<EPI>(v, t, n, out, ldo, aux, ldaux);
}

template <int RT, int TB, int EPI>
hipError_t launch3(const bf16_t *X, int ldx, const bf16_t *W, int T, int N, int K, void *out, int ldo,
                   const bf16_t *aux, int ldaux, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    // Chunks in flight per wave: operand registers U·8·(RT + TB) <= ~160.
    constexpr int U = 20 / (RT + TB) < 1 ? 1 : 20 / (RT + TB);
    const dim3 grid((N + p.rows_per_wg - 1) / p.rows_per_wg, p.k_splits);
    TimingScope ts(kTimeSkinny, stream);
    hipLaunchKernelGGL((skinny_kernel<RT, TB, U, EPI>), grid, dim3(kThreads), 0, stream, X, ldx, W, T, N, K,
                       p.rows_per_wg, p.k_slice, out, ldo, aux, ldaux, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.k_splits == 1) return e;
    const size_t total = (size_t)T * N;
    hipLaunchKernelGGL((skinny_finish_kernel<EPI>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       partials, p.k_splits, T, N, out, ldo, aux, ldaux);
    return hipGetLastError();
}

template <int RT, int TB>
hipError_t launch2(Epilogue epi, const bf16_t *X, int ldx, const bf16_t *W, int T, int N, int K, void *out, int ldo,
                   const bf16_t *aux, int ldaux, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    switch (epi) {
        case EPI_F32: return launch3<RT, TB, EPI_F32>(X, ldx, W, T, N, K, out, ldo, aux, ldaux, p, partials, stream);
        case EPI_BF16: return launch3<RT, TB, EPI_BF16>(X, ldx, W, T, N, K, out, ldo, aux, ldaux, p, partials, stream);
        case EPI_GATE: return launch3<RT, TB, EPI_GATE>(X, ldx, W, T, N, K, out, ldo, aux, ldaux, p, partials, stream);
        default: return launch3<RT, TB, EPI_RESID>(X, ldx, W, T, N, K, out, ldo, aux, ldaux, p, partials, stream);
    }
}

template <int RT>
hipError_t launch1(Epilogue epi, const bf16_t *X, int ldx, const bf16_t *W, int T, int N, int K, void *out, int ldo,
                   const bf16_t *aux, int ldaux, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    if (T <= 16) return launch2<RT, 1>(epi, X, ldx, W, T, N, K, out, ldo, aux, ldaux, p, partials, stream);
    if (T <= 32) return launch2<RT, 2>(epi, X, ldx, W, T, N, K, out, ldo, aux, ldaux, p, partials, stream);
    return launch2<RT, 4>(epi, X, ldx, W, T, N, K, out, ldo, aux, ldaux, p, partials, stream);
}

}  // namespace

SkinnyPlan skinny_plan(int T, int N, int K) {
    // Every workgroup re-reads X[:, its K slice] from L2, T·K·2 bytes without a
    // K split; splitting K across workgroups trades that for fp32 partials and
    // a finishing launch.  Measured: a 2-way split pays off above 16 tokens.
    int ks = T > 16 ? 2 : 1;
    const char *e = getenv("SAMBAY_SKINNY_KSPLIT");
    if (e && *e) ks = atoi(e);
    if (ks < 1) ks = 1;
    const int kc = K / kChunk;
    while (ks > 1 && kc % ks != 0) --ks;
    SkinnyPlan p;
    int R = (int)(((int64_t)N * ks + kTargetWGs - 1) / kTargetWGs);
    if (R > 64) R = 64;
    if (R < 1) R = 1;
    p.rows_per_wg = R;
    p.k_splits = ks;
    p.k_slice = K / ks;
    return p;
}

size_t skinny_partial_bytes(int T, int N, const SkinnyPlan &p) {
    return p.k_splits > 1 ? (size_t)p.k_splits * T * N * sizeof(float) : 0;
}

hipError_t launch_skinny(const bf16_t *X, int ldx, const bf16_t *W, int T, int N, int K, Epilogue epi, void *out,
                         int ldo, const bf16_t *aux, int ldaux, const SkinnyPlan &plan, float *partials,
                         hipStream_t stream) {
    const int R = plan.rows_per_wg;
    if (R <= 16) return launch1<1>(epi, X, ldx, W, T, N, K, out, ldo, aux, ldaux, plan, partials, stream);
    if (R <= 32) return launch1<2>(epi, X, ldx, W, T, N, K, out, ldo, aux, ldaux, plan, partials, stream);
    return launch1<4>(epi, X, ldx, W, T, N, K, out, ldo, aux, ldaux, plan, partials, stream);
}

}  // namespace sambay
