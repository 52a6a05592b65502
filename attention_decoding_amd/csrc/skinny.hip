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
#include "norm_order.hpp"

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
        if (out_lo) out_lo[o] = split_lo(g, hi);
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
    if (out_lo) out_lo[o] = split_lo(u, hi);
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

// ---------------------------------------------------------------------------
// Weight streaming through LDS (decode products of 2-32 tokens).  Every
// workgroup (16 waves, one per CU) copies its whole block of weight rows
// [n0, n0 + R) x K-slice into LDS with direct global -> LDS copies of
// contiguous row segments (non-temporal policy), all issued at once; the
// token operand goes to registers underneath that latency.  Then each wave
// multiplies its own K part (16x16x32 MFMA: A = weight rows read from LDS,
// B = tokens) and the 16 partial tiles are summed through LDS in wave
// order (deterministic).  Measured on the memory side (37.7 MB, 256
// workgroups): 6.8-6.9 us, level with a plain streaming read of the same
// bytes, against 11-12 us for register loads in the MFMA operand layout
// (64 bytes of each of 16 rows per instruction) and 7.0-7.9 us with 8 waves
// or without the non-temporal policy.
constexpr int kStreamWaves = 16;
constexpr int kStreamThreads = 64 * kStreamWaves;
constexpr int kStreamCopyPolicy = 2;               // non-temporal
constexpr size_t kStreamLdsMax = 160 * 1024;

// Wave w's LDS region holds its R x KW block as R rows of CPR 16-byte
// chunks; global chunk g of row r sits in slot (g & ~(SW-1)) | ((g ^ r) &
// (SW-1)), SW the largest of 16, 8, 4 dividing CPR, so that the 16 rows of an
// MFMA operand read land in distinct banks (SW 16 and 8: conflict-free).
__host__ __device__ constexpr int stream_swizzle_width(int cpr) { return cpr % 16 == 0 ? 16 : (cpr % 8 == 0 ? 8 : 4); }

// KS: 32-wide k-steps per wave (K slice = 512·KS).  Rows past R or N read a
// valid row and are never stored; token slots past T read token T-1.
// XT: the token operand in the 16-token tiled layout; otiled (EPI_GATE): the
// output in that layout.
template <int RT, int TB, int KS, int EPI, bool XLO, bool XT>
__global__ __launch_bounds__(kStreamThreads) void stream_kernel(const bf16_t *__restrict__ X,
                                                                const bf16_t *__restrict__ X_lo, int ldx,
                                                                const bf16_t *__restrict__ W, int T, int N, int K,
                                                                int R, void *out, int ldo, bf16_t *out_lo,
                                                                const bf16_t *__restrict__ aux, int ldaux,
                                                                float *__restrict__ partials, int otiled) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int KW = KS * 32, CPR = KW / 8, SW = stream_swizzle_width(CPR), TT = 16 * TB;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
    const int n0 = blockIdx.x * R;
    // Wave w takes K part (w + blockIdx.x) % 16: neighbouring workgroups (on
    // the same XCD, which all read the same token rows from its L2) read
    // different lines of them at any moment.
    const int kpart = (wave + blockIdx.x) & (kStreamWaves - 1);
    const int kw0 = blockIdx.y * (KW * kStreamWaves) + kpart * KW;
    const int units = R * CPR, instr = (units + 63) / 64;
    unsigned char *wl = smem + (size_t)wave * instr * 1024;

    u32x4 xf[KS][TB], xl[XLO ? KS : 1][TB];
    const int ntiles = (T + 15) / 16;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const size_t xo = (size_t)min(16 * tb + col, T - 1) * ldx + kw0 + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            // Tiled: lane l's 16 bytes of k-step (kw0 / 32 + ks), token tile tb,
            // are bytes 16 l .. 16 l + 15 of one contiguous 1 KB block.
            const size_t xi = XT ? ((size_t)((kw0 >> 5) + ks) * ntiles + min(tb, ntiles - 1)) * 512 + lane * 8
                                 : xo + 32 * ks;
            xf[ks][tb] = ld16(X + xi);
            if (XLO) xl[XLO ? ks : 0][tb] = ld16(X_lo + xi);
        }
    }
    for (int i = 0; i < instr; ++i) {
        const int u = min(i * 64 + lane, units - 1), r = u / CPR, c = u % CPR;
        const int g = (c & ~(SW - 1)) | ((c ^ r) & (SW - 1));
        const int row = min(n0 + r, N - 1);
        __builtin_amdgcn_global_load_lds(W + (size_t)row * K + kw0 + 8 * g,
                                         (__attribute__((address_space(3))) void *)(wl + (size_t)i * 1024), 16, 0,
                                         kStreamCopyPolicy);
    }
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's copies and token loads have landed
    __builtin_amdgcn_wave_barrier();

    f32x4 acc[RT][TB];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[rt][tb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int r = min(16 * rt + col, R - 1), g = 4 * ks + grp;
            const int c = (g & ~(SW - 1)) | ((g ^ r) & (SW - 1));
            const u32x4 a = *reinterpret_cast<const u32x4 *>(wl + ((size_t)r * CPR + c) * 16);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                acc[rt][tb] = mfma16x16x32(a, xf[ks][tb], acc[rt][tb]);
                if (XLO) acc[rt][tb] = mfma16x16x32(a, xl[XLO ? ks : 0][tb], acc[rt][tb]);
            }
        }

    // acc[rt][tb][q] = partial of row 16·rt + 4·grp + q, token 16·tb + col.
    __syncthreads();  // every wave is done with its weights: the region becomes the reduction buffer
    float *red = reinterpret_cast<float *>(smem);
    constexpr int RS = TT + 4;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                red[(wave * 16 * RT + 16 * rt + 4 * grp + q) * RS + 16 * tb + col] = acc[rt][tb][q];
    __syncthreads();
    const int total = R * T;
    for (int idx = threadIdx.x; idx < total; idx += kStreamThreads) {
        const int t = idx / R, rl = idx % R, n = n0 + rl;
        if (n >= N) continue;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kStreamWaves; ++w) v += red[(w * 16 * RT + rl) * RS + t];
        if (gridDim.y > 1) {
            partials[((size_t)blockIdx.y * T + t) * N + n] = v;
        } else if (EPI == EPI_GATE && otiled) {
            const float m = bf16_to_f32(aux[(size_t)t * ldaux + n]);
            const float gv = m * (v / (1.f + expf(-v)));
            const bf16_t hi = f32_to_bf16(gv);
            const size_t o = tiled_index(t, n, ntiles);
            reinterpret_cast<bf16_t *>(out)[o] = hi;
            if (out_lo) out_lo[o] = split_lo(gv, hi);
        } else {
            apply_epilogue<EPI>(v, t, n, out, ldo, out_lo, aux, ldaux);
        }
    }
}

// ---------------------------------------------------------------------------
// Slab product (decode products of 17-64 tokens).  Every workgroup streams its
// weight bytes and, from L2, the token operand of its K range; measured on
// MI355X, one CU moves these at ~36-40 GB/s together, a token byte costing as
// much as a weight byte.  With 32 tokens as a hi + lo pair the whole token
// operand of a K = 3072 product is 393 KB, five times a workgroup's share of
// an 18.9 MB weight matrix.  So here a workgroup takes few columns and many
// rows: 128 x RTW weight rows by a K slab of 64 x KC columns (K split in
// K / (64 KC) slabs, fp32 partials summed by a finishing pass).  The token
// slab is copied into LDS once (direct global -> LDS copies) and read by all
// 8 waves; wave w streams its own 16 x RTW rows through a private ring of NS
// LDS stages of 16 rows x 64 columns (8 rows x 128 B per copy instruction,
// which streams at full rate; 16 rows x 64 B loses ~25%), NS - 1 stages
// ahead.  No wave waits for another after the token slab has landed, and
// each wave's accumulators hold finished partial rows (no reduction across
// waves).  The rows may come from up to three weight matrices stacked one
// after another (the SwiGLU gate and up pair; an attention layer's q, k and
// v), with one finishing pass for all of them.
constexpr int kSlabWaves = 8;
constexpr int kSlabThreads = 64 * kSlabWaves;
constexpr size_t kSlabLdsMax = 160 * 1024;
constexpr int kSlabMaxSplits = 16;  // K slabs (the finishing passes hold one partial per slab in registers)

__host__ __device__ constexpr size_t slab_token_bytes(int TB, int KC, bool xlo) {
    return (size_t)16 * TB * 64 * KC * 2 * (xlo ? 2 : 1);
}
// Ring stages per wave (2 KB each): what the token slab leaves of the LDS, at most 8.
__host__ __device__ constexpr int slab_stages(int TB, int KC, bool xlo) {
    return slab_token_bytes(TB, KC, xlo) >= kSlabLdsMax
               ? 0
               : ((kSlabLdsMax - slab_token_bytes(TB, KC, xlo)) / (kSlabWaves * 2048) > 8
                      ? 8
                      : (int)((kSlabLdsMax - slab_token_bytes(TB, KC, xlo)) / (kSlabWaves * 2048)));
}

// s_waitcnt vmcnt(n) for an n known after unrolling (the switch folds away).
__device__ __forceinline__ void slab_wait(int n) {
#define SLAB_WAIT_CASE(c) \
    case c: __builtin_amdgcn_s_waitcnt(0x3f70 | ((c) & 0xf) | (((c) >> 4) << 14)); break;
    switch (n) {
        SLAB_WAIT_CASE(0) SLAB_WAIT_CASE(2) SLAB_WAIT_CASE(4) SLAB_WAIT_CASE(6) SLAB_WAIT_CASE(8)
        SLAB_WAIT_CASE(10) SLAB_WAIT_CASE(12) SLAB_WAIT_CASE(14)
        default: __builtin_amdgcn_s_waitcnt(0x3f70); break;
    }
#undef SLAB_WAIT_CASE
}

__device__ __forceinline__ void slab_copy(const bf16_t *g, unsigned char *lds) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds, 16, 0, kStreamCopyPolicy);
}

// Rows [0, Na) of the Nrows come from W, rows [Na, Nb) from W_b (row
// n - Na), rows [Nb, Nrows) from W_c (row n - Nb): the SwiGLU pair (gate
// then up; Nb = Nrows) or a stacked product (the attention layer's q, k and
// v).  partials: fp32 [K / KR][T][Nrows].
// NORM: X is the residual stream h and the operand is RMSNorm(h; g): the
// h slab is copied in, together with the slab's gains and the tokens' chunk
// sums of squares (stats [T][stride], left by the residual product that
// wrote h), and turned into the bf16 hi + lo pair in LDS, with the
// arithmetic of norm_order.hpp (the same bits as the RMSNorm kernel).
template <int RTW, int TB, int KC, bool XLO, bool NORM = false>
__global__ __launch_bounds__(kSlabThreads) void slab_kernel(const bf16_t *__restrict__ X,
                                                            const bf16_t *__restrict__ X_lo, int ldx,
                                                            const bf16_t *__restrict__ W,
                                                            const bf16_t *__restrict__ W_b,
                                                            const bf16_t *__restrict__ W_c, int Na, int Nb, int Nrows,
                                                            int K,
                                                            int T, float *__restrict__ partials,
                                                            const bf16_t *__restrict__ norm_g,
                                                            const float *__restrict__ norm_stats, int stats_stride,
                                                            float eps) {
    static_assert(!NORM || XLO, "the normalised operand is a hi + lo pair");
    constexpr int KR = 64 * KC, CPR = KR / 8, T16 = 16 * TB;
    constexpr int NS = slab_stages(TB, KC, XLO);
    constexpr int S = RTW * KC;  // ring stages per wave
    constexpr size_t SLAB = slab_token_bytes(TB, KC, XLO);
    constexpr int NJ = (int)(SLAB / 1024);  // token copy instructions per workgroup
    constexpr int NJW = (NJ + kSlabWaves - 1) / kSlabWaves;
    static_assert(NS >= 3 && 2 * (NS - 1) <= 14, "ring depth");
    static_assert(CPR % 16 == 0 && SLAB % 1024 == 0, "slab rows of whole 16-chunk groups");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
    const int k0 = blockIdx.y * KR;
    const int row0 = blockIdx.x * (128 * RTW) + wave * 16 * RTW;  // this wave's first row
    unsigned char *ring = smem + SLAB + (size_t)wave * NS * 2048;

    // Token slab: row t (tokens past T repeat token T - 1), chunk g of the
    // slab's 64 KC columns at slot (g & ~15) | ((g ^ t) & 15); the lo half
    // after the hi half.  Copy instruction j fills slab bytes [1 KB j, 1 KB j + 1 KB).
    constexpr int NJC = NORM ? NJ / 2 : NJ;  // NORM: only the hi half is copied (h)
    constexpr int NJCW = (NJC + kSlabWaves - 1) / kSlabWaves;
    unsigned char *lo_half = smem + SLAB / 2;
#pragma unroll
    for (int jj = 0; jj < NJCW; ++jj) {
        const int j = min(wave + kSlabWaves * jj, NJC - 1);  // the last instruction may be repeated (same bytes)
        const int u = j * 64 + lane, part = u / (T16 * CPR), rem = u % (T16 * CPR), t = rem / CPR, slot = rem % CPR;
        const int g = (slot & ~15) | ((slot ^ t) & 15);
        slab_copy((part ? X_lo : X) + (size_t)min(t, T - 1) * ldx + k0 + 8 * g, smem + (size_t)j * 1024);
    }
    if (NORM) {
        // The gains of the slab's columns (lo half, bytes 0 .. 2 KB) and the
        // tokens' chunk sums (lo half, bytes 2 KB .. 4 KB), until the lo half
        // is written below.
        if (wave == 0) {
#pragma unroll
            for (int i = 0; i < (KR * 2 + 1023) / 1024; ++i)
                slab_copy(norm_g + k0 + 8 * min(64 * i + lane, CPR - 1), lo_half + 1024 * i);
        } else if (wave == 1) {
            const int per_tok = stats_stride / 4;  // 16-byte pieces per token
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int q = 64 * i + lane, tq = q / per_tok, pq = q % per_tok;
                if (i * 64 < T16 * per_tok)
                    slab_copy(reinterpret_cast<const bf16_t *>(norm_stats + (size_t)min(tq, T - 1) * stats_stride + 4 * pq),
                              lo_half + 2048 + 1024 * i);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // the token copies stay ahead of the ring's (the waits count them)
    // Ring stage s: this wave's row tile s % RTW, columns 64 (s / RTW) .. + 63
    // (row tiles fastest, so the token operands of a 64-column step are read
    // from LDS once for all of the wave's row tiles); row r's eight chunks at
    // r·128 + 16·(g ^ ((r >> 1) & 7)).
    auto issue = [&](int s) {
        const int rt = s % RTW, kc = s / RTW;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = 8 * i + (lane >> 3), g = (lane & 7) ^ ((r >> 1) & 7);
            const int row = min(row0 + 16 * rt + r, Nrows - 1);
            const bf16_t *src = row < Na   ? W + (size_t)row * K
                                : row < Nb ? W_b + (size_t)(row - Na) * K
                                           : W_c + (size_t)(row - Nb) * K;
            slab_copy(src + k0 + 64 * kc + 8 * g, ring + (size_t)(s % NS) * 2048 + i * 1024);
        }
    };
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < S) {
            issue(s);
            __builtin_amdgcn_sched_barrier(0);
        }
    slab_wait(2 * (NS - 1 < S ? NS - 1 : S));  // this wave's token copies have landed
    __builtin_amdgcn_s_barrier();               // ... and every wave's
    __builtin_amdgcn_sched_barrier(0);
    if (NORM) {
        // h -> RMSNorm(h; g) as hi (in place) + lo.  The gains and scales of
        // this thread's slots are read before any lo store (they live
        // there); every LDS read of a phase is issued before the first use.
        constexpr int SLOTS = T16 * CPR, PER = (SLOTS + kSlabThreads - 1) / kSlabThreads;
        const int nch = norm_chunks(K);
        const unsigned char *stb = lo_half + 2048;
        u32x4 gv[PER];
        f32x4 s0[PER], s1[PER];
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int j = min((int)threadIdx.x + kSlabThreads * m, SLOTS - 1), t = j / CPR, sl = j % CPR;
            const int g = (sl & ~15) | ((sl ^ t) & 15);
            gv[m] = *reinterpret_cast<const u32x4 *>(lo_half + 16 * g);
            // chunk sums 0-3 and 4-7 (with 4 per token the second read is the
            // next token's and unused)
            s0[m] = *reinterpret_cast<const f32x4 *>(stb + (size_t)t * stats_stride * 4);
            s1[m] = *reinterpret_cast<const f32x4 *>(stb + (size_t)t * stats_stride * 4 + 16);
        }
        float rv[PER];
        const float inv_k = 1.f / (float)K;
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            float tot = 0.f;
#pragma unroll
            for (int c = 0; c < kNormMaxChunks; ++c)
                if (c < nch) tot += c < 4 ? s0[m][c] : s1[m][c - 4];
            rv[m] = norm_scale(tot, inv_k, eps);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        u32x4 xv[PER];
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int j = min((int)threadIdx.x + kSlabThreads * m, SLOTS - 1);
            xv[m] = *reinterpret_cast<const u32x4 *>(smem + (size_t)(j / CPR) * KR * 2 + 16 * (j % CPR));
        }
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int j = (int)threadIdx.x + kSlabThreads * m;
            if (j >= SLOTS) break;
            const size_t off = (size_t)(j / CPR) * KR * 2 + 16 * (j % CPR);
            u32x2 h0, l0, h1, l1;
            norm_apply4((u32x2){xv[m][0], xv[m][1]}, (u32x2){gv[m][0], gv[m][1]}, rv[m], h0, l0);
            norm_apply4((u32x2){xv[m][2], xv[m][3]}, (u32x2){gv[m][2], gv[m][3]}, rv[m], h1, l1);
            *reinterpret_cast<u32x4 *>(smem + off) = (u32x4){h0[0], h0[1], h1[0], h1[1]};
            *reinterpret_cast<u32x4 *>(lo_half + off) = (u32x4){l0[0], l0[1], l1[0], l1[1]};
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the pair is in LDS before any wave reads it
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    }

    const int aslot = col * 128;                          // + 16 * (g ^ ((col >> 1) & 7))
    const unsigned char *bbase = smem + (size_t)col * KR * 2;  // token row col of tile 0
    f32x4 acc[RTW][TB];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[rt][tb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    u32x4 bh[2][TB], bl[2][XLO ? TB : 1];  // the current 64-column step's token operands
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int after = (NS - 2 < S - 1 - s) ? NS - 2 : S - 1 - s;
        slab_wait(2 * after);  // stage s has landed
        __builtin_amdgcn_wave_barrier();
        if (s + NS - 1 < S) issue(s + NS - 1);  // into the slot stage s - 1 used
        const unsigned char *st = ring + (size_t)(s % NS) * 2048 + aslot;
        const int rt = s % RTW, kc = s / RTW;
        if (rt == 0) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int g = 4 * (2 * kc + q) + grp;
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const int t = 16 * tb + col;
                    const size_t bo = (size_t)tb * 16 * KR * 2 + 16 * ((g & ~15) | ((g ^ t) & 15));
                    bh[q][tb] = *reinterpret_cast<const u32x4 *>(bbase + bo);
                    if (XLO) bl[q][XLO ? tb : 0] = *reinterpret_cast<const u32x4 *>(bbase + SLAB / 2 + bo);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(st + 16 * ((4 * q + grp) ^ ((col >> 1) & 7)));
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                acc[rt][tb] = mfma16x16x32(a, bh[q][tb], acc[rt][tb]);
                if (XLO) acc[rt][tb] = mfma16x16x32(a, bl[q][XLO ? tb : 0], acc[rt][tb]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // acc[rt][tb][e] = partial of row 16·rt + 4·grp + e of the wave's rows, token 16·tb + col.
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        const int grow = row0 + 16 * rt + 4 * grp;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int t = 16 * tb + col;
            if (t < T && grow < Nrows)
                *reinterpret_cast<f32x4 *>(partials + ((size_t)blockIdx.y * T + t) * Nrows + grow) = acc[rt][tb];
        }
    }
}

// Finishing passes of the slab product: four outputs per thread (16-byte
// partial loads), the slabs summed in slab order.
template <int EPI>
__global__ __launch_bounds__(256) void slab_finish_kernel(const float *__restrict__ partials, int ks, int T, int N,
                                                          void *out, int ldo, bf16_t *out_lo,
                                                          const bf16_t *__restrict__ aux, int ldaux) {
    const int n4 = N / 4;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)T * n4) return;
    const int t = (int)(idx / n4), n = 4 * (int)(idx % n4);
    // Every slab's partial is requested before the first is used (one round
    // trip to wherever the slab kernel's writes went, not one per slab).
    f32x4 pv[kSlabMaxSplits];
#pragma unroll
    for (int s = 0; s < kSlabMaxSplits; ++s)
        if (s < ks) pv[s] = *reinterpret_cast<const f32x4 *>(partials + ((size_t)s * T + t) * N + n);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSlabMaxSplits; ++s)
        if (s < ks) v += pv[s];
    const size_t o = (size_t)t * ldo + n;
    if (EPI == EPI_F32) {
        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + o) = v;
    } else if (EPI == EPI_BF16) {
        *reinterpret_cast<u32x2 *>(reinterpret_cast<bf16_t *>(out) + o) = (u32x2){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    } else if (EPI == EPI_GATE) {
        const u32x2 m = *reinterpret_cast<const u32x2 *>(aux + (size_t)t * ldaux + n);
        const float mm[4] = {lo_bf16(m[0]), hi_bf16(m[0]), lo_bf16(m[1]), hi_bf16(m[1])};
        bf16_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float g = mm[e] * (v[e] / (1.f + expf(-v[e])));
            hi[e] = f32_to_bf16(g);
            lo[e] = split_lo(g, hi[e]);
        }
        *reinterpret_cast<u32x2 *>(reinterpret_cast<bf16_t *>(out) + o) =
            (u32x2){(uint32_t)hi[0] | ((uint32_t)hi[1] << 16), (uint32_t)hi[2] | ((uint32_t)hi[3] << 16)};
        if (out_lo)
            *reinterpret_cast<u32x2 *>(out_lo + o) =
                (u32x2){(uint32_t)lo[0] | ((uint32_t)lo[1] << 16), (uint32_t)lo[2] | ((uint32_t)lo[3] << 16)};
    } else {
        bf16_t *h = reinterpret_cast<bf16_t *>(out);
        const u32x2 hv = *reinterpret_cast<const u32x2 *>(h + o);
        *reinterpret_cast<u32x2 *>(h + o) =
            (u32x2){(uint32_t)f32_to_bf16(lo_bf16(hv[0]) + v[0]) | ((uint32_t)f32_to_bf16(hi_bf16(hv[0]) + v[1]) << 16),
                    (uint32_t)f32_to_bf16(lo_bf16(hv[1]) + v[2]) | ((uint32_t)f32_to_bf16(hi_bf16(hv[1]) + v[3]) << 16)};
    }
}

// Stacked products (bf16 outputs): the slabs summed as above, output rows
// [0, na) into out, [na, nb) into out_b, [nb, N) into out_c (na and nb
// multiples of 4, so a thread's four outputs share one destination).
__global__ __launch_bounds__(256) void slab_stacked_finish_kernel(const float *__restrict__ partials, int ks, int T,
                                                                  int N, int na, int nb, bf16_t *__restrict__ out,
                                                                  int ldo, bf16_t *__restrict__ out_b, int ldo_b,
                                                                  bf16_t *__restrict__ out_c, int ldo_c) {
    const int n4 = N / 4;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)T * n4) return;
    const int t = (int)(idx / n4), n = 4 * (int)(idx % n4);
    f32x4 pv[kSlabMaxSplits];
#pragma unroll
    for (int s = 0; s < kSlabMaxSplits; ++s)
        if (s < ks) pv[s] = *reinterpret_cast<const f32x4 *>(partials + ((size_t)s * T + t) * N + n);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSlabMaxSplits; ++s)
        if (s < ks) v += pv[s];
    bf16_t *dst = n < na ? out + (size_t)t * ldo + n
                         : n < nb ? out_b + (size_t)t * ldo_b + (n - na) : out_c + (size_t)t * ldo_c + (n - nb);
    *reinterpret_cast<u32x2 *>(dst) = (u32x2){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// SwiGLU: partials [ks][T][2N], gate columns then up columns.
__global__ __launch_bounds__(256) void slab_swiglu_finish_kernel(const float *__restrict__ partials, int ks, int T,
                                                                 int N, bf16_t *__restrict__ out, int ldo,
                                                                 bf16_t *__restrict__ out_lo) {
    const int n4 = N / 4;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)T * n4) return;
    const int t = (int)(idx / n4), n = 4 * (int)(idx % n4);
    f32x4 pg[kSlabMaxSplits], pu[kSlabMaxSplits];
#pragma unroll
    for (int s = 0; s < kSlabMaxSplits; ++s)
        if (s < ks) {
            const float *p = partials + ((size_t)s * T + t) * 2 * N + n;
            pg[s] = *reinterpret_cast<const f32x4 *>(p);
            pu[s] = *reinterpret_cast<const f32x4 *>(p + N);
        }
    f32x4 g = {0.f, 0.f, 0.f, 0.f}, v = g;
#pragma unroll
    for (int s = 0; s < kSlabMaxSplits; ++s)
        if (s < ks) {
            g += pg[s];
            v += pu[s];
        }
    bf16_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float u = (g[e] / (1.f + expf(-g[e]))) * v[e];
        hi[e] = f32_to_bf16(u);
        lo[e] = split_lo(u, hi[e]);
    }
    const size_t o = (size_t)t * ldo + n;
    *reinterpret_cast<u32x2 *>(out + o) =
        (u32x2){(uint32_t)hi[0] | ((uint32_t)hi[1] << 16), (uint32_t)hi[2] | ((uint32_t)hi[3] << 16)};
    if (out_lo)
        *reinterpret_cast<u32x2 *>(out_lo + o) =
            (u32x2){(uint32_t)lo[0] | ((uint32_t)lo[1] << 16), (uint32_t)lo[2] | ((uint32_t)lo[3] << 16)};
}

// The residual finishing pass of the slab product that also leaves the next
// sublayer's RMSNorm statistics: one workgroup per (1024-column chunk, token
// row); h_new = bf16(h + Σ partials) as in slab_finish_kernel, and the
// chunk's sum of squares of h_new (order of norm_order.hpp) in
// stats[t · stride + chunk].
__global__ __launch_bounds__(kNormThreads) void slab_resid_stats_kernel(const float *__restrict__ partials, int ks,
                                                                        int T, int N, bf16_t *__restrict__ h, int ldo,
                                                                        float *__restrict__ stats, int stride) {
    __shared__ float red[kNormThreads / 64];
    const int c = blockIdx.x, t = blockIdx.y, n = kNormChunk * c + 4 * threadIdx.x;
    float ss = 0.f;
    if (n < N) {
        f32x4 pv[kSlabMaxSplits];
#pragma unroll
        for (int s = 0; s < kSlabMaxSplits; ++s)
            if (s < ks) pv[s] = *reinterpret_cast<const f32x4 *>(partials + ((size_t)s * T + t) * N + n);
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kSlabMaxSplits; ++s)
            if (s < ks) v += pv[s];
        bf16_t *hp = h + (size_t)t * ldo + n;
        const u32x2 hv = *reinterpret_cast<const u32x2 *>(hp);
        const u32x2 hn = {(uint32_t)f32_to_bf16(lo_bf16(hv[0]) + v[0]) | ((uint32_t)f32_to_bf16(hi_bf16(hv[0]) + v[1]) << 16),
                          (uint32_t)f32_to_bf16(lo_bf16(hv[1]) + v[2]) | ((uint32_t)f32_to_bf16(hi_bf16(hv[1]) + v[3]) << 16)};
        *reinterpret_cast<u32x2 *>(hp) = hn;
        ss = norm_sq4(hn);
    }
    const float cs = norm_chunk_sum(ss, red);
    if (threadIdx.x == 0) stats[(size_t)t * stride + c] = cs;
}

size_t stream_lds_bytes(int R, int KS, int RT, int TB) {
    const size_t units = (size_t)R * KS * 4, instr = (units + 63) / 64;
    const size_t copy = (size_t)kStreamWaves * instr * 1024;
    const size_t red = (size_t)kStreamWaves * 16 * RT * (16 * TB + 4) * sizeof(float);
    return copy > red ? copy : red;
}

__global__ __launch_bounds__(256) void swiglu_finish_kernel(const float *__restrict__ partials, int splits, int T,
                                                            int N, void *out, int ldo, bf16_t *out_lo) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)T * N) return;
    const int t = (int)(idx / N), n = (int)(idx % N);
    // The first 16 splits' partials are requested at once (one round trip).
    float pg[16], pu[16];
#pragma unroll
    for (int s = 0; s < 16; ++s)
        if (s < splits) {
            pg[s] = partials[((size_t)s * T + t) * 2 * N + n];
            pu[s] = partials[((size_t)s * T + t) * 2 * N + N + n];
        }
    float g = 0.f, v = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s)
        if (s < splits) g += pg[s], v += pu[s];
    for (int s = 16; s < splits; ++s) {
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
    // The first 16 splits' partials are requested at once (one round trip).
    float pv[16];
#pragma unroll
    for (int s = 0; s < 16; ++s)
        if (s < splits) pv[s] = partials[((size_t)s * T + t) * N + n];
    float v = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s)
        if (s < splits) v += pv[s];
    for (int s = 16; s < splits; ++s) v += partials[((size_t)s * T + t) * N + n];
    apply_epilogue<EPI>(v, t, n, out, ldo, out_lo, aux, ldaux);
}

// K-split finishing of a residual product fused with the next sublayer's
// RMSNorm: one workgroup per token row sums the slices in slice order, stores
// h_new = bf16(h + Σ) and writes RMSNorm(h_new; g) as a bf16 hi + lo pair,
// the sum of squares in the order of norm_order.hpp (the same bits as the
// standalone RMSNorm kernel).  Four columns per thread per 1024-column chunk.
__global__ __launch_bounds__(kNormThreads) void resid_norm_finish_kernel(
    const float *__restrict__ partials, int splits, int T, int N, bf16_t *__restrict__ h, int ldo,
    const bf16_t *__restrict__ g, float eps, bf16_t *__restrict__ xn, bf16_t *__restrict__ xn_lo) {
    __shared__ float red[kNormThreads / 64];
    const int t = blockIdx.x, nch = norm_chunks(N);
    bf16_t *hr = h + (size_t)t * ldo;
    u32x2 hn[kNormMaxChunks];
    float tot = 0.f;
#pragma unroll
    for (int c = 0; c < kNormMaxChunks; ++c) {
        if (c >= nch) break;
        const int n = kNormChunk * c + 4 * threadIdx.x;
        float ss = 0.f;
        if (n < N) {
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            for (int sl = 0; sl < splits; ++sl) v += *reinterpret_cast<const f32x4 *>(partials + ((size_t)sl * T + t) * N + n);
            const u32x2 hv = *reinterpret_cast<const u32x2 *>(hr + n);
            hn[c] = (u32x2){(uint32_t)f32_to_bf16(lo_bf16(hv[0]) + v[0]) | ((uint32_t)f32_to_bf16(hi_bf16(hv[0]) + v[1]) << 16),
                            (uint32_t)f32_to_bf16(lo_bf16(hv[1]) + v[2]) | ((uint32_t)f32_to_bf16(hi_bf16(hv[1]) + v[3]) << 16)};
            *reinterpret_cast<u32x2 *>(hr + n) = hn[c];
            ss = norm_sq4(hn[c]);
        }
        tot += norm_chunk_sum(ss, red);
    }
    const float r = norm_scale(tot, 1.f / (float)N, eps);
#pragma unroll
    for (int c = 0; c < kNormMaxChunks; ++c) {
        const int n = kNormChunk * c + 4 * threadIdx.x;
        if (c >= nch || n >= N) continue;
        u32x2 hi, lo;
        norm_apply4(hn[c], *reinterpret_cast<const u32x2 *>(g + n), r, hi, lo);
        *reinterpret_cast<u32x2 *>(xn + (size_t)t * ldo + n) = hi;
        *reinterpret_cast<u32x2 *>(xn_lo + (size_t)t * ldo + n) = lo;
    }
}

// One-token products (batch-1 decode): a plain VALU dot product, lanes along
// K.  Each wave reads one whole weight row, 1 KB contiguous per load
// instruction (lane l holds elements 512·s + 8·l .. +7 of segment s), with
// the non-temporal policy; the token row (and the epilogue's own input) is
// read by every wave from L2.  The code is straight-line: no loop and no
// branch sits between the loads, so all of a wave's loads are in flight
// together (a guarded load, or a loop over rows, made the compiler wait for
// the token row before issuing the weight loads, and for each row's loads
// before the next row's: 8.1-8.7 against 7.4 us for 37.7 MB).  Rows past N
// read row N-1 and store nothing.  Each row is reduced across the wave in a
// fixed order.  No token padding, no LDS.
template <int KS, int EPI, bool XLO>
__global__ __launch_bounds__(256) void gemv_kernel(const bf16_t *__restrict__ X, const bf16_t *__restrict__ X_lo,
                                                   const bf16_t *__restrict__ W, int N, void *out, bf16_t *out_lo,
                                                   const bf16_t *__restrict__ aux) {
    constexpr int K = KS * 512;
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nr = min(n, N - 1);
    u32x4 xr[KS], xl[XLO ? KS : 1], wr[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        xr[s] = ld16(X + s * 512 + 8 * lane);
        if (XLO) xl[XLO ? s : 0] = ld16(X_lo + s * 512 + 8 * lane);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) wr[s] = ld16_nt(W + (size_t)nr * K + s * 512 + 8 * lane);
    // The epilogue's own input (M for the gate, h for the residual add), fetched
    // with the weights so that its latency overlaps theirs.
    float pre = 0.f;
    if (EPI == EPI_GATE) pre = bf16_to_f32(aux[nr]);
    if (EPI == EPI_RESID) pre = bf16_to_f32(reinterpret_cast<const bf16_t *>(out)[nr]);
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc += lo_bf16(wr[s][e]) * lo_bf16(xr[s][e]) + hi_bf16(wr[s][e]) * hi_bf16(xr[s][e]);
            if (XLO)
                acc += lo_bf16(wr[s][e]) * lo_bf16(xl[XLO ? s : 0][e]) + hi_bf16(wr[s][e]) * hi_bf16(xl[XLO ? s : 0][e]);
        }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane != 0 || n >= N) return;
    if (EPI == EPI_F32) {
        reinterpret_cast<float *>(out)[n] = acc;
    } else if (EPI == EPI_BF16) {
        reinterpret_cast<bf16_t *>(out)[n] = f32_to_bf16(acc);
    } else if (EPI == EPI_GATE) {
        const float g = pre * (acc / (1.f + expf(-acc)));
        const bf16_t hi = f32_to_bf16(g);
        reinterpret_cast<bf16_t *>(out)[n] = hi;
        if (out_lo) out_lo[n] = split_lo(g, hi);
    } else {
        reinterpret_cast<bf16_t *>(out)[n] = f32_to_bf16(pre + acc);
    }
}

template <int KS, int EPI, bool XLO>
hipError_t launch_gemv3(const SkinnyArgs &a, hipStream_t stream) {
    // One wave per weight row, four per workgroup (measured against 2 and 4
    // rows per wave and 8 or 16 waves per workgroup on 6144 x 3072 and
    // 3072 x 6144: the single-row wave is fastest or level).
    const int wgs = (a.N + 3) / 4;
    TimingScope ts(kTimeSkinny, stream);
    hipLaunchKernelGGL((gemv_kernel<KS, EPI, XLO>), dim3(wgs), dim3(256), 0, stream, a.X, a.X_lo, a.W, a.N, a.out,
                       a.out_lo, a.aux);
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

// The finishing pass of a K-split product (fp32 partials [slice][T][N]).
template <int EPI>
hipError_t launch_finish(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    if (EPI == EPI_RESID && skinny_fuses_norm(a, p)) {
        hipLaunchKernelGGL(resid_norm_finish_kernel, dim3((unsigned)a.T), dim3(kNormThreads), 0, stream, partials, p.k_splits,
                           a.T, a.N, static_cast<bf16_t *>(a.out), a.ldo, a.next_norm, a.eps, a.next_x,
                           a.next_x_lo);
        return hipGetLastError();
    }
    const size_t total = (size_t)a.T * a.N;
    hipLaunchKernelGGL((skinny_finish_kernel<EPI>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       partials, p.k_splits, a.T, a.N, a.out, a.ldo, a.out_lo, a.aux, a.ldaux);
    return hipGetLastError();
}

template <int RT, int TB, int KS, int EPI, bool XLO, bool XT>
hipError_t launch_stream5(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    const size_t lds = stream_lds_bytes(p.rows_per_wg, KS, RT, TB);
    static const hipError_t attr = hipFuncSetAttribute((const void *)stream_kernel<RT, TB, KS, EPI, XLO, XT>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStreamLdsMax);
    if (attr != hipSuccess) return attr;
    const dim3 grid((a.N + p.rows_per_wg - 1) / p.rows_per_wg, p.k_splits);
    TimingScope ts(kTimeSkinny, stream);
    hipLaunchKernelGGL((stream_kernel<RT, TB, KS, EPI, XLO, XT>), grid, dim3(kStreamThreads), lds, stream, a.X, a.X_lo,
                       a.ldx, a.W, a.T, a.N, a.K, p.rows_per_wg, a.out, a.ldo, a.out_lo, a.aux, a.ldaux, partials,
                       a.out_tiled ? 1 : 0);
    return hipGetLastError();
}

template <int RT, int TB, int KS, int EPI, bool XLO>
hipError_t launch_stream4(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    {
        const hipError_t e0 = a.x_tiled ? launch_stream5<RT, TB, KS, EPI, XLO, true>(a, p, partials, stream)
                                        : launch_stream5<RT, TB, KS, EPI, XLO, false>(a, p, partials, stream);
        if (e0 != hipSuccess) return e0;
    }
    if (p.k_splits == 1) return hipSuccess;
    return launch_finish<EPI>(a, p, partials, stream);
}

template <int RT, int TB, int KS, int EPI>
hipError_t launch_stream3(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    if constexpr (KS * TB * 2 <= 24) {  // the hi + lo token operand doubles the token registers
        if (a.X_lo) return launch_stream4<RT, TB, KS, EPI, true>(a, p, partials, stream);
    }
    if constexpr (KS * TB <= 24) {
        if (!a.X_lo) return launch_stream4<RT, TB, KS, EPI, false>(a, p, partials, stream);
    }
    return hipErrorInvalidValue;  // never dispatched (stream_fit)
}

template <int RT, int TB, int KS>
hipError_t launch_stream2(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    switch (a.epi) {
        case EPI_F32: return launch_stream3<RT, TB, KS, EPI_F32>(a, p, partials, stream);
        case EPI_BF16: return launch_stream3<RT, TB, KS, EPI_BF16>(a, p, partials, stream);
        case EPI_GATE: return launch_stream3<RT, TB, KS, EPI_GATE>(a, p, partials, stream);
        default: return launch_stream3<RT, TB, KS, EPI_RESID>(a, p, partials, stream);
    }
}

// Shapes the LDS-streaming product takes: 2-32 tokens, no SwiGLU pairing, a K
// slice of 1536, 3072 or 6144 elements, at most 32 rows per workgroup, the
// token operand within 24 registers of 16 bytes per lane, the block within
// the LDS of one CU.
int stream_tb(int T) { return T <= 16 ? 1 : (T <= 32 ? 2 : 4); }

// The K steps per wave for which the LDS-streaming product takes a shape
// (0: it does not): a K slice of 1536, 3072 or 6144 elements, at most 32
// rows per workgroup, the token operand within 24 registers of 16 bytes per
// lane, the block within the LDS of one CU.
int stream_fit(int T, int R, int k_slice, bool xlo) {
    if (T < 2 || T > kSkinnyMaxTokens || R > 32 || k_slice % (32 * kStreamWaves) != 0) return 0;
    const int KS = k_slice / (32 * kStreamWaves);
    if (KS != 3 && KS != 6 && KS != 12) return 0;
    const int TB = stream_tb(T), RT = R <= 16 ? 1 : 2;
    if (KS * TB * (xlo ? 2 : 1) > 24) return 0;
    if (stream_lds_bytes(R, KS, RT, TB) > kStreamLdsMax) return 0;
    return KS;
}

int stream_ks(const SkinnyArgs &a, const SkinnyPlan &p) {
    if (a.epi == EPI_SWIGLU || a.ldx % 8 != 0 || a.K % 8 != 0) return 0;
    return stream_fit(a.T, p.rows_per_wg, p.k_slice, a.X_lo != nullptr);
}

template <int RT, int TB>
hipError_t launch_stream1(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream, int KS) {
    if (KS == 3) return launch_stream2<RT, TB, 3>(a, p, partials, stream);
    if (KS == 6) return launch_stream2<RT, TB, 6>(a, p, partials, stream);
    return launch_stream2<RT, TB, 12>(a, p, partials, stream);
}

template <int RT>
hipError_t launch_stream0(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream, int KS) {
    switch (stream_tb(a.T)) {
        case 1: return launch_stream1<RT, 1>(a, p, partials, stream, KS);
        case 2: return launch_stream1<RT, 2>(a, p, partials, stream, KS);
        default: return launch_stream1<RT, 4>(a, p, partials, stream, KS);
    }
}

hipError_t launch_stream(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream, int KS) {
    return p.rows_per_wg > 16 ? launch_stream0<2>(a, p, partials, stream, KS)
                              : launch_stream0<1>(a, p, partials, stream, KS);
}

template <int RTW, int TB, int KC, bool XLO, bool NORM = false>
hipError_t launch_slab4(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    const bool dual = a.epi == EPI_SWIGLU, stacked = a.na > 0;
    const int Nrows = dual ? 2 * a.N : a.N;
    // Row ranges of the weight sources: [0, na) W, [na, nb) W_b, [nb, Nrows) W_c.
    const int na = dual ? a.N : stacked ? a.na : a.N, nb = dual || !stacked ? Nrows : a.nb;
    const bf16_t *wb = dual || stacked ? a.W_b : a.W, *wc = stacked && a.W_c ? a.W_c : wb;
    const size_t lds = slab_token_bytes(TB, KC, XLO) + (size_t)kSlabWaves * slab_stages(TB, KC, XLO) * 2048;
    static const hipError_t attr = hipFuncSetAttribute((const void *)slab_kernel<RTW, TB, KC, XLO, NORM>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSlabLdsMax);
    if (attr != hipSuccess) return attr;
    const dim3 grid((Nrows + 128 * RTW - 1) / (128 * RTW), p.k_splits);
    {
        TimingScope ts(kTimeSkinny, stream);
        hipLaunchKernelGGL((slab_kernel<RTW, TB, KC, XLO, NORM>), grid, dim3(kSlabThreads), lds, stream, a.X, a.X_lo,
                           a.ldx, a.W, wb, wc, na, nb, Nrows, a.K, a.T, partials, a.norm_g, a.norm_stats,
                           norm_stats_stride(a.K), a.norm_eps);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.epi == EPI_RESID && a.stats_out) {
        hipLaunchKernelGGL(slab_resid_stats_kernel, dim3((unsigned)norm_chunks(a.N), (unsigned)a.T), dim3(kNormThreads),
                           0, stream, partials, p.k_splits, a.T, a.N, static_cast<bf16_t *>(a.out), a.ldo, a.stats_out,
                           norm_stats_stride(a.N));
        return hipGetLastError();
    }
    const unsigned blocks = (unsigned)(((size_t)a.T * (a.N / 4) + 255) / 256);
    if (stacked) {
        hipLaunchKernelGGL(slab_stacked_finish_kernel, dim3(blocks), dim3(256), 0, stream, partials, p.k_splits, a.T,
                           a.N, a.na, a.nb, static_cast<bf16_t *>(a.out), a.ldo, a.out_b, a.ldo_b, a.out_c, a.ldo_c);
        return hipGetLastError();
    }
    switch (a.epi) {
        case EPI_SWIGLU:
            hipLaunchKernelGGL(slab_swiglu_finish_kernel, dim3(blocks), dim3(256), 0, stream, partials, p.k_splits, a.T,
                               a.N, static_cast<bf16_t *>(a.out), a.ldo, a.out_lo);
            break;
        case EPI_F32:
            hipLaunchKernelGGL(slab_finish_kernel<EPI_F32>, dim3(blocks), dim3(256), 0, stream, partials, p.k_splits,
                               a.T, a.N, a.out, a.ldo, a.out_lo, a.aux, a.ldaux);
            break;
        case EPI_BF16:
            hipLaunchKernelGGL(slab_finish_kernel<EPI_BF16>, dim3(blocks), dim3(256), 0, stream, partials, p.k_splits,
                               a.T, a.N, a.out, a.ldo, a.out_lo, a.aux, a.ldaux);
            break;
        case EPI_GATE:
            hipLaunchKernelGGL(slab_finish_kernel<EPI_GATE>, dim3(blocks), dim3(256), 0, stream, partials, p.k_splits,
                               a.T, a.N, a.out, a.ldo, a.out_lo, a.aux, a.ldaux);
            break;
        default:
            hipLaunchKernelGGL(slab_finish_kernel<EPI_RESID>, dim3(blocks), dim3(256), 0, stream, partials, p.k_splits,
                               a.T, a.N, a.out, a.ldo, a.out_lo, a.aux, a.ldaux);
            break;
    }
    return hipGetLastError();
}

template <int RTW, int TB, int KC>
hipError_t launch_slab3(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    if (a.norm_g) {
        if constexpr (slab_stages(TB, KC, true) >= 3) return launch_slab4<RTW, TB, KC, true, true>(a, p, partials, stream);
        return hipErrorInvalidValue;
    }
    if (a.X_lo) {
        if constexpr (slab_stages(TB, KC, true) >= 3) return launch_slab4<RTW, TB, KC, true>(a, p, partials, stream);
        return hipErrorInvalidValue;
    }
    return launch_slab4<RTW, TB, KC, false>(a, p, partials, stream);
}

template <int TB>
hipError_t launch_slab2(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    const int kc = p.k_slice / 64;
    if (p.slab_rtw == 1 && kc == 6) return launch_slab3<1, TB, 6>(a, p, partials, stream);
    if (p.slab_rtw == 2 && kc == 6) return launch_slab3<2, TB, 6>(a, p, partials, stream);
    if (p.slab_rtw == 2 && kc == 8) return launch_slab3<2, TB, 8>(a, p, partials, stream);
    if (p.slab_rtw == 2 && kc == 12) return launch_slab3<2, TB, 12>(a, p, partials, stream);
    if (p.slab_rtw == 1 && kc == 12) return launch_slab3<1, TB, 12>(a, p, partials, stream);
    return hipErrorInvalidValue;
}

// The slab shapes (rows per wave in 16-row tiles, K slab in 64-column chunks)
// the plan chooses from.
struct SlabShape {
    int rtw, kc;
};
constexpr SlabShape kSlabShapes[] = {{1, 6}, {2, 6}, {2, 8}, {2, 12}, {1, 12}};

bool slab_fits(int T, int Nrows, int K, int ldx, bool x_tiled, const SkinnyPlan &p) {
    return T > 16 && T <= kSkinnyMaxTokens && Nrows % 4 == 0 && !x_tiled && ldx % 8 == 0 && p.k_splits >= 2 &&
           p.k_splits <= kSlabMaxSplits &&
           (int64_t)p.k_slice * p.k_splits == K;
}

hipError_t launch_slab(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    const bool dual = a.epi == EPI_SWIGLU;
    if (a.out_tiled || (dual && !a.W_b) || !slab_fits(a.T, dual ? 2 * a.N : a.N, a.K, a.ldx, a.x_tiled, p) ||
        a.N % 4 != 0 || a.ldo % 4 != 0 || (a.epi == EPI_GATE && a.ldaux % 4 != 0))
        return hipErrorInvalidValue;
    if (a.norm_g && (a.X_lo || !a.norm_stats || a.K % 4 != 0 || norm_chunks(a.K) > kNormMaxChunks))
        return hipErrorInvalidValue;
    if (a.stats_out && (a.epi != EPI_RESID || norm_chunks(a.N) > kNormMaxChunks)) return hipErrorInvalidValue;
    if (a.na > 0 && (a.epi != EPI_BF16 || a.na % 4 != 0 || a.nb % 4 != 0 || a.nb < a.na || a.nb > a.N || !a.W_b ||
                     !a.out_b || a.ldo_b % 4 != 0 || (a.nb < a.N && (!a.W_c || !a.out_c || a.ldo_c % 4 != 0))))
        return hipErrorInvalidValue;
    return stream_tb(a.T) == 2 ? launch_slab2<2>(a, p, partials, stream) : launch_slab2<4>(a, p, partials, stream);
}

// The slab plan of least modelled time: per workgroup, its weights, its token
// slab (16-token tiles, hi + lo) and its partial rows at ~38 GB/s per CU (in
// rounds of 256 workgroups), against all weights at ~6 TB/s, plus the
// partials written and read again at ~6 TB/s.  Taken above 16 tokens for a
// hi + lo token operand and for any operand above 32 tokens: a plain bf16
// operand at 17-32 tokens measured faster in the LDS-streaming product (the
// 32-token GMU: 23.7 us against 26.3 us with the slab product taking its
// K = 6144 output product, the hidden then no longer in the tiled layout);
// none for outputs whose rows are not a multiple of 4.  SAMBAY_NO_SLAB=1
// turns it off.
bool slab_plan(int T, int Nrows, int K, bool xlo, SkinnyPlan &p) {
    static const bool off = [] {
        const char *e = getenv("SAMBAY_NO_SLAB");
        return e && *e && *e != '0';
    }();
    if (off || T <= 16 || (!xlo && T <= 32) || T > kSkinnyMaxTokens || Nrows % 4 != 0) return false;
    const int TB = stream_tb(T);
    double best = 1e30;
    for (const SlabShape &sh : kSlabShapes) {
        const int KR = 64 * sh.kc;
        if (K % KR != 0 || K / KR < 2 || K / KR > kSlabMaxSplits || slab_stages(TB, sh.kc, xlo) < 3) continue;
        const int ks = K / KR, R = 128 * sh.rtw;
        const double wgs = (double)((Nrows + R - 1) / R) * ks, rounds = (double)(int)((wgs + kTargetWGs - 1) / kTargetWGs);
        const double per_wg = (double)R * KR * 2 + 16.0 * TB * KR * 2 * (xlo ? 2 : 1) + (double)T * R * 4;
        // (Bounding a CU's rate by the bytes its ring keeps in flight too
        // picked deeper rings with twice the slabs: slower everywhere, e.g.
        // the 64-token GMU 32.0 -> 40.5 us.)
        const double t_cu = rounds * per_wg / 38e3, t_hbm = (double)Nrows * K * 2 / 6e6;
        const double t = (t_cu > t_hbm ? t_cu : t_hbm) + 2.0 * ks * T * Nrows * 4 / 6e6;
        if (t < best) {
            best = t;
            p.rows_per_wg = R;
            p.k_splits = ks;
            p.k_slice = KR;
            p.slab_rtw = sh.rtw;
        }
    }
    return best < 1e30;
}

template <int RT, int TB, int EPI, bool XLO, bool DUAL = false>
hipError_t launch4(const SkinnyArgs &a, const SkinnyPlan &p, float *partials, hipStream_t stream) {
    // Chunks in flight per wave: operand registers U·8·(RT + TB·(1 + XLO)) <= ~160.
    // The dual SwiGLU pass keeps one chunk in flight and two workgroups per
    // CU instead.  That was measured at 32 tokens (122 registers against
    // 185, its 512 workgroups in one round instead of two; 34.9 -> ~30.5 us
    // per 100.7 MB launch), where the slab product has since taken over;
    // here it serves 2-16 tokens (one token tile).  Measured there too: the
    // 16-layer complete step at 4 / 8 / 16 tokens (2,048 cached positions)
    // 1.122 / 1.205 / 1.434 ms against 1.142 / 1.232 / 1.472 ms with the
    // chunks in flight and one workgroup per CU of the other products.
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
    return launch_finish<EPI>(a, p, partials, stream);
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

bool slab_norm_ok(int T, int Nrows, int K) {
    SkinnyPlan p;
    return !norm_fusion_off() && K % 4 == 0 && norm_chunks(K) <= kNormMaxChunks && slab_plan(T, Nrows, K, true, p);
}

SkinnyPlan skinny_plan(int T, int N, int K, bool xlo) {
    // The LDS-streaming product (2-64 tokens) first: the smallest K split
    // (1, 2, 4) at which it takes the shape, about 256 workgroups.
    static const bool no_stream = [] {
        const char *e = getenv("SAMBAY_NO_STREAM");
        return e && *e && *e != '0';
    }();
    {
        SkinnyPlan p;
        if (slab_plan(T, N, K, xlo, p)) return p;
    }
    if (T >= 2 && !no_stream) {
        for (int ks = 1; ks <= 4; ks *= 2) {
            if (K % ks != 0) break;
            const int R = (int)(((int64_t)N * ks + kTargetWGs - 1) / kTargetWGs);
            if (stream_fit(T, R, K / ks, xlo)) {
                SkinnyPlan p;
                p.rows_per_wg = R;
                p.k_splits = ks;
                p.k_slice = K / ks;
                return p;
            }
        }
    }
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
    // Over both operand kinds and every token group up to T (the products of a
    // batch run in groups of at most T tokens, the last one smaller, and the
    // plan's K split is chosen per group).
    size_t m = 0;
    for (int t = 1; t <= T; ++t)
        for (int xlo = 0; xlo < 2; ++xlo) {
            const size_t b = skinny_partial_bytes(t, N, skinny_plan(t, N, K, xlo != 0));
            if (b > m) m = b;
        }
    return m;
}

SkinnyPlan skinny_plan_dual(int T, int N, int K) {
    {
        SkinnyPlan p;  // the pair's token operand is a hi + lo pair in the layer stack
        if (slab_plan(T, 2 * N, K, true, p)) return p;
    }
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

bool norm_fusion_off() {
    // SAMBAY_NO_NORM_FUSION=1 selects the separate RMSNorm launch instead (same bits).
    const char *env = getenv("SAMBAY_NO_NORM_FUSION");
    return env && *env && *env != '0';
}

bool skinny_fuses_norm(const SkinnyArgs &a, const SkinnyPlan &p) {
    return !norm_fusion_off() && a.epi == EPI_RESID && p.k_splits > 1 && p.slab_rtw == 0 && a.next_norm && a.next_x && a.next_x_lo &&
           a.ldo == a.N && a.N % 4 == 0 && norm_chunks(a.N) <= kNormMaxChunks;
}

size_t skinny_partial_bytes(int T, int N, const SkinnyPlan &p) {
    return p.k_splits > 1 ? (size_t)p.k_splits * T * N * sizeof(float) : 0;
}

bool skinny_tiles(const SkinnyArgs &a, const SkinnyPlan &plan) {
    if (plan.slab_rtw > 0) return false;
    return !(gemv_eligible(a) && plan.k_splits == 1) && stream_ks(a, plan) != 0;
}

hipError_t launch_skinny(const SkinnyArgs &a, const SkinnyPlan &plan, float *partials, hipStream_t stream) {
    const int R = plan.rows_per_wg;
    // The tiled token layout exists only in the LDS-streaming product; a
    // tiled output only from its unsplit gate epilogue.
    if ((a.x_tiled || a.out_tiled) && !skinny_tiles(a, plan)) return hipErrorInvalidValue;
    if (a.out_tiled && (a.epi != EPI_GATE || plan.k_splits != 1)) return hipErrorInvalidValue;
    if (plan.slab_rtw > 0) return launch_slab(a, plan, partials, stream);
    // The deferred norm and the stacked products exist only in the slab product.
    if (a.norm_g || a.stats_out || a.na > 0) return hipErrorInvalidValue;
    if (gemv_eligible(a) && plan.k_splits == 1) return launch_gemv(a, stream);
    if (const int ks = stream_ks(a, plan)) return launch_stream(a, plan, partials, stream, ks);
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
