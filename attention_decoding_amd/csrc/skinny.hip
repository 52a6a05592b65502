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
//    For comparison, a plain 37.7 MB HBM read kernel takes ~7.2-7.7 us per
//    launch back to back on MI355X; one GMU product here takes ~9-12 us.
//  * A operand = 16 weight rows; MFMA k-step t of a chunk covers 32
//    contiguous K elements, lane group grp holding elements 8·grp .. 8·grp+7,
//    so each load instruction reads 64 contiguous bytes of 16 rows.  B operand
//    = 16 tokens of X with the same K assignment (X is small and L2-resident).
//    Tokens are padded to 16 per tile; rows past the range are zero operands.
//  * Epilogues are fused: fp32 store, bf16 store, the GMU gate
//    H = M ⊙ SiLU(acc) stored as a bf16 hi + lo pair, or the residual add
//    h = bf16(h + acc).  The complete layer's SwiGLU MLP streams its gate
//    and up weights in one pass (paired row tiles) and stores
//    SiLU(gate) ⊙ up as a bf16 hi + lo pair.  An X given as a hi + lo pair
//    (the gated H, the attention output o, a normalised input) is multiplied
//    as two MFMAs per operand, so rounding the intermediate to bf16 costs
//    ~16 significant bits instead of 8.
//  * One token: a VALU dot-product kernel (gemv_kernel) with row-contiguous
//    loads replaces the MFMA tile, whose 16 token slots would be 15/16 padding.
//  * When the token operand a workgroup must read is large (many tokens, a
//    hi + lo pair, long K), K is also split across workgroups so that each
//    takes ~48 rows and the grid stays at ~256 workgroups; fp32 partials then
//    go through a small finishing kernel (skinny_plan gives the measured rule).
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
__device__ __forceinline__ void apply_epilogue(float v, int t, int n, void *out, int ldo, bf16_t *out_lo,
                                               const bf16_t *aux, int ldaux) {
    const size_t o = (size_t)t * ldo + n;
    if (EPI == EPI_F32) {
        reinterpret_cast<float *>(out)[o] = v;
    } else if (EPI == EPI_BF16) {
        reinterpret_cast<bf16_t *>(out)[o] = f32_to_bf16(v);
    } else if (EPI == EPI_GATE) {
        const float m = bf16_to_f32(aux[(size_t)t * ldaux + n]);
        const float g = m * (v / (1.f + expf(-v)));
        const bf16_t hi = f32_to_bf16(g);
        reinterpret_cast<bf16_t *>(out)[o] = hi;
        if (out_lo) out_lo[o] = f32_to_bf16(g - bf16_to_f32(hi));
    } else {
        bf16_t *h = reinterpret_cast<bf16_t *>(out);
        h[o] = f32_to_bf16(bf16_to_f32(h[o]) + v);
    }
}

// The SwiGLU MLP's two products of the same input in one pass: u = SiLU(g) · v
// with g from W and v from W_b (same rows), stored as a bf16 hi + lo pair.
__device__ __forceinline__ void store_swiglu(float g, float v, int t, int n, void *out, int ldo, bf16_t *out_lo) {
    const size_t o = (size_t)t * ldo + n;
    const float u = (g / (1.f + expf(-g))) * v;
    const bf16_t hi = f32_to_bf16(u);
    reinterpret_cast<bf16_t *>(out)[o] = hi;
    if (out_lo) out_lo[o] = f32_to_bf16(u - bf16_to_f32(hi));
}

// RT row tiles of 16, TB token tiles of 16, U chunks in flight per wave; XLO:
// X arrives as a bf16 hi + lo pair (two MFMAs per operand pair).  DUAL: the
// first RT/2 row tiles come from W, the other RT/2 from W_b at the same rows
// (the SwiGLU gate and up products); partials then hold [slice][T][2N].
template <int RT, int TB, int U, int EPI, bool XLO, bool DUAL = false, int MINB = 1>
__global__ __launch_bounds__(kThreads, MINB) void skinny_kernel(const bf16_t *__restrict__ X,
                                                          const bf16_t *__restrict__ X_lo, int ldx,
                                                          const bf16_t *__restrict__ W,
                                                          const bf16_t *__restrict__ W_b, int T, int N, int K, int R,
                                                          int k_slice, void *out, int ldo, bf16_t *out_lo,
                                                          const bf16_t *__restrict__ aux, int ldaux,
                                                          float *__restrict__ partials) {
    constexpr int TT = 16 * TB;
    __shared__ float red[kWaves][16 * RT][TT + 4];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
    const int n0 = blockIdx.x * R;
    const int kbeg = blockIdx.y * k_slice;
    const int nchunks = k_slice / kChunk;

    constexpr int RH = DUAL ? RT / 2 : RT;  // row tiles per weight matrix
    static_assert(!DUAL || RT % 2 == 0, "dual products take row tiles in pairs");
    const bf16_t *wrow[RT];
    bool rvalid[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int rl = 16 * (rt % RH) + col;
        const bf16_t *Wm = (DUAL && rt >= RH) ? W_b : W;
        rvalid[rt] = rl < R && n0 + rl < N;
        wrow[rt] = Wm + (size_t)(rvalid[rt] ? n0 + rl : 0) * K + kbeg + 8 * grp;
    }
    size_t xoff[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) xoff[tb] = (size_t)min(16 * tb + col, T - 1) * ldx + kbeg + 8 * grp;

    f32x4 acc[RT][TB];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[rt][tb] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Wave w owns a contiguous run of ceil(nchunks / kWaves) chunks and keeps U
    // of them in flight: the (L2-resident) X loads of a group are issued first,
    // then all its weight loads, then the MFMAs.  (Strided chunk ownership and
    // weight-first ordering measured within 3%.)
    const int per_wave = (nchunks + kWaves - 1) / kWaves;
    auto chunk_of = [&](int j) { return wave * per_wave + j; };
    auto live_of = [&](int j) { return j < per_wave && wave * per_wave + j < nchunks; };
    for (int j0 = 0; live_of(j0); j0 += U) {
        u32x4 wf[U][RT][2], xf[U][TB][2], xl[XLO ? U : 1][TB][2];
        auto load_x = [&]() {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool live = live_of(j0 + u);
                const int k = chunk_of(j0 + u) * kChunk;
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        xf[u][tb][t] = live ? ld16(X + xoff[tb] + k + 32 * t) : (u32x4){0u, 0u, 0u, 0u};
                        if (XLO) xl[XLO ? u : 0][tb][t] = live ? ld16(X_lo + xoff[tb] + k + 32 * t) : (u32x4){0u, 0u, 0u, 0u};
                    }
            }
        };
        load_x();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool live = live_of(j0 + u);
            const int k = chunk_of(j0 + u) * kChunk;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    wf[u][rt][t] = (live && rvalid[rt]) ? ld16(wrow[rt] + k + 32 * t) : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb) {
                        acc[rt][tb] = mfma16x16x32(wf[u][rt][t], xf[u][tb][t], acc[rt][tb]);
                        if (XLO) acc[rt][tb] = mfma16x16x32(wf[u][rt][t], xl[XLO ? u : 0][tb][t], acc[rt][tb]);
                    }
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
        float v = 0.f, vb = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            v += red[w][rl][t];
            if (DUAL) vb += red[w][16 * RH + rl][t];
        }
        if (gridDim.y == 1) {
            if (DUAL)
                store_swiglu(v, vb, t, n, out, ldo, out_lo);
            else
                apply_epilogue<EPI>(v, t, n, out, ldo, out_lo, aux, ldaux);
        } else {
            const int np = DUAL ? 2 * N : N;
            partials[((size_t)blockIdx.y * T + t) * np + n] = v;
            if (DUAL) partials[((size_t)blockIdx.y * T + t) * np + N + n] = vb;
        }
    }
}

__global__ __launch_bounds__(256) void swiglu_finish_kernel(const float *__restrict__ partials, int splits, int T,
                                                            int N, void *out, int ldo, bf16_t *out_lo) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)T * N) return;
    const int t = (int)(idx / N), n = (int)(idx % N);
    float g = 0.f, v = 0.f;
    for (int s = 0; s < splits; ++s) {
        g += partials[((size_t)s * T + t) * 2 * N + n];
        v += partials[((size_t)s * T + t) * 2 * N + N + n];
    }
    store_swiglu(g, v, t, n, out, ldo, out_lo);
}

template <int EPI>
__global__ __launch_bounds__(256) void skinny_finish_kernel(const float *__restrict__ partials, int splits, int T,
                                                            int N, void *out, int ldo, bf16_t *out_lo,
                                                            const bf16_t *__restrict__ aux, int ldaux) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)T * N) return;
    const int t = (int)(idx / N), n = (int)(idx % N);
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += partials[((size_t)s * T + t) * N + n];
    apply_epilogue<EPI>(v, t, n, out, ldo, out_lo, aux, ldaux);
}

// K-split finishing of a residual product fused with the next sublayer's
// RMSNorm: one workgroup per token row sums the slices in slice order, stores
// h_new = bf16(h + Σ) and writes RMSNorm(h_new; g) as a bf16 hi + lo pair.
// The norm's loop structure and reduction order are those of the standalone
// RMSNorm kernel, so both give the same bits.
__global__ __launch_bounds__(256) void resid_norm_finish_kernel(const float *__restrict__ partials, int splits,
                                                                 int T, int N, bf16_t *__restrict__ h, int ldo,
                                                                 const bf16_t *__restrict__ g, float eps,
                                                                 bf16_t *__restrict__ xn, bf16_t *__restrict__ xn_lo) {
    __shared__ float red[4];
    const int t = blockIdx.x;
    bf16_t *hr = h + (size_t)t * ldo;
    const int nvec = N / 8;
    float ss = 0.f;
    for (int v = threadIdx.x; v < nvec; v += 256) {
        const int n = 8 * v;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        for (int sl = 0; sl < splits; ++sl) {
            const float *p = partials + ((size_t)sl * T + t) * N + n;
            const f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] += a[e];
                acc[4 + e] += b[e];
            }
        }
        const u32x4 hv = ld16(hr + n);
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bf16_t h0 = f32_to_bf16(lo_bf16(hv[e]) + acc[2 * e]);
            const bf16_t h1 = f32_to_bf16(hi_bf16(hv[e]) + acc[2 * e + 1]);
            o[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            const float a = bf16_to_f32(h0), b = bf16_to_f32(h1);
            ss += a * a + b * b;
        }
        *reinterpret_cast<u32x4 *>(hr + n) = o;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) tot += red[w];
    const float r = 1.f / sqrtf(tot / (float)N + eps);
    for (int v = threadIdx.x; v < nvec; v += 256) {
        const u32x4 x = ld16(hr + 8 * v), gv = ld16(g + 8 * v);  // this thread's own stores above
        u32x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float y0 = lo_bf16(x[e]) * r * lo_bf16(gv[e]);
            const float y1 = hi_bf16(x[e]) * r * hi_bf16(gv[e]);
            const bf16_t h0 = f32_to_bf16(y0), h1 = f32_to_bf16(y1);
            hi[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lo[e] = pack_bf16x2(y0 - bf16_to_f32(h0), y1 - bf16_to_f32(h1));
        }
        *reinterpret_cast<u32x4 *>(xn + (size_t)t * ldo + 8 * v) = hi;
        *reinterpret_cast<u32x4 *>(xn_lo + (size_t)t * ldo + 8 * v) = lo;
    }
}

// One-token products (batch-1 decode): a plain VALU dot product, lanes along
// K.  Each wave reads whole weight rows, 1 KB contiguous per load
// instruction (lane l holds elements 512·s + 8·l .. +7 of segment s), keeps
// the token row in registers, and reduces each row across the wave in a fixed
// order.  No token padding, no LDS.  Measured against the MFMA product at one
// token (3072/6144-wide, random data, weights from HBM): 8.3 vs 9.2 us
// (6144 x 3072) and 8.3 vs 10.4 us (3072 x 6144); at 4 tokens it is slower
// (register pressure), so it serves T == 1 only.
template <int KS, int RPW, int EPI, bool XLO>
__global__ __launch_bounds__(256) void gemv_kernel(const bf16_t *__restrict__ X, const bf16_t *__restrict__ X_lo,
                                                   const bf16_t *__restrict__ W, int N, void *out, bf16_t *out_lo,
                                                   const bf16_t *__restrict__ aux) {
    constexpr int K = KS * 512;
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6), nw = gridDim.x * 4;
    u32x4 xr[KS], xl[XLO ? KS : 1];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        xr[s] = ld16(X + s * 512 + 8 * lane);
        if (XLO) xl[XLO ? s : 0] = ld16(X_lo + s * 512 + 8 * lane);
    }
    for (int n0 = gw * RPW; n0 < N; n0 += nw * RPW) {
        u32x4 wr[RPW][KS];
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int s = 0; s < KS; ++s)
                wr[r][s] = n0 + r < N ? ld16(W + (size_t)(n0 + r) * K + s * 512 + 8 * lane) : (u32x4){0u, 0u, 0u, 0u};
        // The epilogue's own input (M for the gate, h for the residual add) is
        // fetched together with the weights so its latency overlaps theirs.
        float pre[RPW];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            pre[r] = 0.f;
            if ((EPI == EPI_GATE || EPI == EPI_RESID) && lane == 0 && n0 + r < N)
                pre[r] = bf16_to_f32(EPI == EPI_GATE ? aux[n0 + r] : reinterpret_cast<const bf16_t *>(out)[n0 + r]);
        }
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc += lo_bf16(wr[r][s][e]) * lo_bf16(xr[s][e]) + hi_bf16(wr[r][s][e]) * hi_bf16(xr[s][e]);
                    if (XLO)
                        acc += lo_bf16(wr[r][s][e]) * lo_bf16(xl[XLO ? s : 0][e]) +
                               hi_bf16(wr[r][s][e]) * hi_bf16(xl[XLO ? s : 0][e]);
                }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
            if (lane != 0 || n0 + r >= N) continue;
            const int n = n0 + r;
            if (EPI == EPI_F32) {
                reinterpret_cast<float *>(out)[n] = acc;
            } else if (EPI == EPI_BF16) {
                reinterpret_cast<bf16_t *>(out)[n] = f32_to_bf16(acc);
            } else if (EPI == EPI_GATE) {
                const float g = pre[r] * (acc / (1.f + expf(-acc)));
                const bf16_t hi = f32_to_bf16(g);
                reinterpret_cast<bf16_t *>(out)[n] = hi;
                if (out_lo) out_lo[n] = f32_to_bf16(g - bf16_to_f32(hi));
            } else {
                reinterpret_cast<bf16_t *>(out)[n] = f32_to_bf16(pre[r] + acc);
            }
        }
    }
}

template <int KS, int EPI, bool XLO>
hipError_t launch_gemv3(const SkinnyArgs &a, hipStream_t stream) {
    constexpr int RPW = KS >= 12 ? 1 : 2;  // rows in flight per wave (measured)
    // Up to 3072 waves (3 per SIMD): one wave per RPW rows, so that every
    // wave issues all its loads at once and none runs a second, dependent
    // round (the 6144 x 3072 gate product: 11.3 -> 10.7 us).  Larger
    // products and the hi + lo operand form keep 512 workgroups, which
    // measured faster for them (12288 x 3072: 15.6 vs 16.2 us; 3072 x 6144
    // with a hi + lo token: 11.6 vs 13.0 us).
    const int waves = (a.N + RPW - 1) / RPW;
    const int wgs = (!XLO && waves <= 3072) ? (waves + 3) / 4 : 512;
    TimingScope ts(kTimeSkinny, stream);
    hipLaunchKernelGGL((gemv_kernel<KS, RPW, EPI, XLO>), dim3(wgs), dim3(256), 0, stream, a.X, a.X_lo, a.W, a.N,
                       a.out, a.out_lo, a.aux);
    return hipGetLastError();
}

template <int KS, int EPI>
hipError_t launch_gemv2(const SkinnyArgs &a, hipStream_t stream) {
    return a.X_lo ? launch_gemv3<KS, EPI, true>(a, stream) : launch_gemv3<KS, EPI, false>(a, stream);
}

template <int KS>
hipError_t launch_gemv1(const SkinnyArgs &a, hipStream_t stream) {
    switch (a.epi) {
        case EPI_F32: return launch_gemv2<KS, EPI_F32>(a, stream);
        case EPI_BF16: return launch_gemv2<KS, EPI_BF16>(a, stream);
        case EPI_GATE: return launch_gemv2<KS, EPI_GATE>(a, stream);
        default: return launch_gemv2<KS, EPI_RESID>(a, stream);
    }
}

// The one-token path covers K in {3072, 6144, 8192} (contiguous rows, ld == N,
// ldx == K); anything else takes the MFMA product.
bool gemv_eligible(const SkinnyArgs &a) {
    if (a.T != 1 || a.epi == EPI_SWIGLU || a.ldo != a.N || a.ldx != a.K) return false;
    if ((a.epi == EPI_GATE) && a.ldaux != a.N) return false;
    return a.K == 3072 || a.K == 6144 || a.K == 8192;
}

hipError_t launch_gemv(const SkinnyArgs &a, hipStream_t stream) {
    switch (a.K) {
        case 3072: return launch_gemv1<6>(a, stream);
        case 6144: return launch_gemv1<12>(a, stream);
        default: return launch_gemv1<16>(a, stream);
    }
}

template <int RT, int TB, int EPI, bool XLO, bool DUAL = false>
hipError_t launch4(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    // Chunks in flight per wave: operand registers U·8·(RT + TB·(1 + XLO)) <= ~160.
    // The dual SwiGLU pass keeps one chunk in flight and two workgroups per
    // CU instead (at 32 tokens: 122 registers against 185, its 512
    // workgroups in one round instead of two; 34.9 -> ~30.5 us per 100.7 MB
    // launch, the whole-model decode step 10.19 -> 10.04 ms).
    constexpr int U0 = 20 / (RT + TB * (XLO ? 2 : 1)) < 1 ? 1 : 20 / (RT + TB * (XLO ? 2 : 1));
    constexpr int U = DUAL ? 1 : U0;
    constexpr int MINB = DUAL ? 2 : 1;
    const dim3 grid((a.N + p.rows_per_wg - 1) / p.rows_per_wg, p.k_splits);
    TimingScope ts(kTimeSkinny, stream);
    hipLaunchKernelGGL((skinny_kernel<RT, TB, U, EPI, XLO, DUAL, MINB>), grid, dim3(kThreads), 0, stream, a.X, a.X_lo, a.ldx,
                       a.W, a.W_b, a.T, a.N, a.K, p.rows_per_wg, p.k_slice, a.out, a.ldo, a.out_lo, a.aux, a.ldaux, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.k_splits == 1) return e;
    if (DUAL) {
        const size_t total = (size_t)a.T * a.N;
        hipLaunchKernelGGL(swiglu_finish_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, partials,
                           p.k_splits, a.T, a.N, a.out, a.ldo, a.out_lo);
        return hipGetLastError();
    }
    if (EPI == EPI_RESID && skinny_fuses_norm(a, p)) {
        hipLaunchKernelGGL(resid_norm_finish_kernel, dim3((unsigned)a.T), dim3(256), 0, stream, partials, p.k_splits,
                           a.T, a.N, static_cast<bf16_t *>(a.out), a.ldo, a.next_norm, a.eps, a.next_x,
                           a.next_x_lo);
        return hipGetLastError();
    }
    const size_t total = (size_t)a.T * a.N;
    hipLaunchKernelGGL((skinny_finish_kernel<EPI>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       partials, p.k_splits, a.T, a.N, a.out, a.ldo, a.out_lo, a.aux, a.ldaux);
    return hipGetLastError();
}

template <int RT, int TB, int EPI>
hipError_t launch3(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    if (EPI == EPI_SWIGLU) {  // always the dual gate + up pass
        if constexpr (RT % 2 == 0) {
            if (a.X_lo) return launch4<RT, TB, EPI, true, true>(a, p, partials, stream);
            return launch4<RT, TB, EPI, false, true>(a, p, partials, stream);
        }
        return hipErrorInvalidValue;
    }
    if (a.X_lo) return launch4<RT, TB, EPI, true>(a, p, partials, stream);
    return launch4<RT, TB, EPI, false>(a, p, partials, stream);
}

template <int RT, int TB>
hipError_t launch2(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    switch (a.epi) {
        case EPI_F32: return launch3<RT, TB, EPI_F32>(a, p, partials, stream);
        case EPI_BF16: return launch3<RT, TB, EPI_BF16>(a, p, partials, stream);
        case EPI_GATE: return launch3<RT, TB, EPI_GATE>(a, p, partials, stream);
        case EPI_SWIGLU: return launch3<RT, TB, EPI_SWIGLU>(a, p, partials, stream);
        default: return launch3<RT, TB, EPI_RESID>(a, p, partials, stream);
    }
}

template <int RT>
hipError_t launch1(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    if (a.T <= 16) return launch2<RT, 1>(a, p, partials, stream);
    if (a.T <= 32) return launch2<RT, 2>(a, p, partials, stream);
    return launch2<RT, 4>(a, p, partials, stream);
}

}  // namespace

SkinnyPlan skinny_plan(int T, int N, int K, bool xlo) {
    // Every workgroup reads the K slice of the token operand from L2: T·K·2
    // bytes without a K split (twice that for a hi + lo pair).  Measured on
    // MI355X (N, K in {3072, 6144}, 1-64 tokens, all epilogues): below ~190
    // KB per workgroup, one workgroup per CU over ceil(N/256) rows and no
    // split is fastest; above it, ~48 rows per workgroup with K split so that
    // the grid stays at ~256 workgroups wins by up to 30% (e.g. the 3072 x
    // 6144 product with a hi + lo operand at 32 tokens: 22.5 -> 18.6 us),
    // finishing pass included.
    const int64_t xbytes = (int64_t)T * K * 2 * (xlo ? 2 : 1);
    int ks = 1;
    if (xbytes >= (int64_t)192 * 1024) ks = (int)((256LL * 48 + N / 2) / N);
    // Short outputs (N < 768, e.g. the SSM layer's 224-row step/B/C
    // projection) would get dozens of splits whose finishing pass, one thread
    // per output summing every split, dominates (48 splits: 13.9 us of
    // finishing for a 6.9 us product); at most 8.
    if (N < 768 && ks > 8) ks = 8;
    const char *e = getenv("SAMBAY_SKINNY_KSPLIT");
    if (e && *e) ks = atoi(e);
    const int kc = K / kChunk;
    if (ks > kc) ks = kc;
    if (ks < 1) ks = 1;
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

size_t skinny_partial_bytes_max(int T, int N, int K) {
    const size_t a = skinny_partial_bytes(T, N, skinny_plan(T, N, K, false));
    const size_t b = skinny_partial_bytes(T, N, skinny_plan(T, N, K, true));
    return a > b ? a : b;
}

SkinnyPlan skinny_plan_dual(int T, int N, int K) {
    // The 2N weight rows are planned together (a 2-way K split above 16
    // tokens), then each workgroup takes R/2 output rows (R/2 rows of each
    // matrix).
    int ks = T > 16 ? 2 : 1;
    const int kc = K / kChunk;
    while (ks > 1 && kc % ks != 0) --ks;
    SkinnyPlan p;
    int R = (int)(((int64_t)2 * N * ks + kTargetWGs - 1) / kTargetWGs);
    if (R > 64) R = 64;
    p.rows_per_wg = R / 2 > 0 ? R / 2 : 1;
    p.k_splits = ks;
    p.k_slice = K / ks;
    return p;
}

size_t skinny_partial_bytes_dual(int T, int N, const SkinnyPlan &p) {
    return p.k_splits > 1 ? (size_t)p.k_splits * T * 2 * N * sizeof(float) : 0;
}

bool skinny_fuses_norm(const SkinnyArgs &a, const SkinnyPlan &p) {
    // SAMBAY_NO_NORM_FUSION=1 selects the separate RMSNorm launch instead (same bits).
    const char *env = getenv("SAMBAY_NO_NORM_FUSION");
    const bool off = env && *env && *env != '0';
    return !off && a.epi == EPI_RESID && p.k_splits > 1 && a.next_norm && a.next_x && a.next_x_lo &&
           a.ldo == a.N && a.N % 8 == 0;
}

size_t skinny_partial_bytes(int T, int N, const SkinnyPlan &p) {
    return p.k_splits > 1 ? (size_t)p.k_splits * T * N * sizeof(float) : 0;
}

hipError_t launch_skinny(const SkinnyArgs &a, const SkinnyPlan &plan, float *partials, hipStream_t stream) {
    const int R = plan.rows_per_wg;
    if (gemv_eligible(a) && plan.k_splits == 1) return launch_gemv(a, stream);
    if (a.epi == EPI_SWIGLU) {  // dual: row tiles in pairs, R <= 32 (skinny_plan_dual)
        if (!a.W_b || R > 32) return hipErrorInvalidValue;
        return R <= 16 ? launch1<2>(a, plan, partials, stream) : launch1<4>(a, plan, partials, stream);
    }
    if (R <= 16) return launch1<1>(a, plan, partials, stream);
    if (R <= 32) return launch1<2>(a, plan, partials, stream);
    if (R <= 48) return launch1<3>(a, plan, partials, stream);
    return launch1<4>(a, plan, partials, stream);
}

}  // namespace sambay
