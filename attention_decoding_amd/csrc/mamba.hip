// SSM decode step of the self-decoder (gfx950): the Mamba layer whose
// token-mixing output M every GMU layer of the cross-decoder reuses (the
// Paper-Notes page on "Decoder-Hybrid-Decoder Architecture for Efficient
// Reasoning with Long Generation", sections 关键设计 and 整体框架; Mamba with
// per-channel decay, section 消融实验).  One step for T <= 64 sequences:
//
//   [xi | z] = W_in x                        weight-streaming product (fp32 out)
//   u = SiLU(conv(window of xi)), shift       mamba_conv_kernel (this file)
//   [δ | B | C] = W_x u                       weight-streaming product, u as a bf16 hi + lo pair
//   Δ = softplus(W_dt δ + dt_bias)            \
//   s <- exp(Δ·A)·s + Δ·B·u, M = C·s + D·u     > mamba_scan_kernel (this file)
//   g = M ⊙ SiLU(z)                           /  (g as a bf16 hi + lo pair)
//   y = W_out g                               weight-streaming product (bf16 out)
//
// HBM-bound: the four weight matrices (W_in and W_out dominate: 3/4 of
// 151 MB at d_model 3072) are each streamed once per step, and the fp32 SSM
// state is read and written once (T·d_inner·N·4 B each way).  The two
// kernels here are elementwise over (token, channel): the convolution keeps
// its window in fp32 and shifts it in place; the scan kernel stages the
// workgroup's 64 rows of W_dt in LDS (the step projection, fused here
// rather than streamed as a separate product) and reads δ, B, C of its
// token as wave-uniform values.
#include "device.hpp"
#include "launch.hpp"

#include <math.h>

namespace sambay {

namespace {

constexpr int kConvThreads = 256;
constexpr int kScanChannels = 64;  // channels per workgroup (one per lane)
constexpr int kScanWaves = 4;      // tokens per workgroup (one per wave) from 4 tokens up
constexpr int kMaxStates = 64;

__device__ __forceinline__ float silu(float v) { return v / (1.f + expf(-v)); }

__device__ __forceinline__ void store_pair(bf16_t *hi, bf16_t *lo, size_t i, float v) {
    const bf16_t h = f32_to_bf16(v);
    hi[i] = h;
    lo[i] = f32_to_bf16(v - bf16_to_f32(h));
}

// One thread per (token, channel): u = SiLU(conv_b + Σ_k conv_w[k]·window[k]),
// window = the K-1 stored inputs (oldest first) then the new xi; the stored
// window shifts by one.
__global__ __launch_bounds__(kConvThreads) void mamba_conv_kernel(const float *__restrict__ xz, int ldxz,
                                                                  float *__restrict__ conv_state,
                                                                  const float *__restrict__ conv_w,
                                                                  const float *__restrict__ conv_b,
                                                                  float *__restrict__ u, bf16_t *__restrict__ u_hi,
                                                                  bf16_t *__restrict__ u_lo, int T, int d_inner,
                                                                  int K) {
    const size_t idx = (size_t)blockIdx.x * kConvThreads + threadIdx.x;
    if (idx >= (size_t)T * d_inner) return;
    const int t = (int)(idx / d_inner), c = (int)(idx % d_inner);
    const float xi = xz[(size_t)t * ldxz + c];
    float *st = conv_state + idx * (K - 1);
    const float *wc = conv_w + (size_t)c * K;
    float acc = conv_b[c];
    float prev[kMaxConv];
#pragma unroll
    for (int k = 0; k < kMaxConv - 1; ++k)
        if (k < K - 1) {
            prev[k] = st[k];
            acc += wc[k] * prev[k];
        }
    acc += wc[K - 1] * xi;
#pragma unroll
    for (int k = 0; k < kMaxConv - 2; ++k)
        if (k < K - 2) st[k] = prev[k + 1];
    if (K > 1) st[K - 2] = xi;
    const float v = silu(acc);
    u[idx] = v;
    store_pair(u_hi, u_lo, idx, v);
}

// Workgroup = 64 channels (lane) x TW tokens (wave).  The tokens' δ | B | C
// rows are staged in LDS (read as broadcasts).  With TW = 4 the workgroup's
// 64 rows of W_dt are staged too, transposed to [pair of ranks][channel] so
// that the lanes' reads of one rank pair hit consecutive banks (each row
// serves 4 tokens); with TW = 1 (one token, no reuse) each lane reads its
// own row from memory.  Every staging load of a thread is issued before its
// first LDS store.  Then Δ from the row and δ; the NS states of (token,
// channel) are updated in registers and written back; M (bf16) and
// g = M·SiLU(z) (bf16 hi + lo).
template <int NS, int TW>
__global__ __launch_bounds__(64 * TW) void mamba_scan_kernel(
    const float *__restrict__ xz, int ldxz, const float *__restrict__ u, const float *__restrict__ xdbl, int P, int R,
    const bf16_t *__restrict__ W_dt, const float *__restrict__ dt_bias, const float *__restrict__ A_log,
    const float *__restrict__ Dp, float *__restrict__ ssm_state, bf16_t *__restrict__ M_out, bf16_t *__restrict__ g_hi,
    bf16_t *__restrict__ g_lo, int T, int d_inner) {
    constexpr int kMaxP = kMaxDtRank + 2 * kMaxStates;
    constexpr int kThreads = 64 * TW;
    __shared__ uint32_t wdt[TW > 1 ? kMaxDtRank / 2 : 1][kScanChannels];
    __shared__ float a2s[TW > 1 ? NS : 1][kScanChannels];  // A·log2(e) = -exp(A_log)·log2(e), [state][channel]
    __shared__ float xds[TW][kMaxP];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c0 = blockIdx.x * kScanChannels, t0 = blockIdx.y * TW;
    const int nchunk = R / 8;  // 8 ranks (16 bytes) per chunk
    {
        constexpr int kX = (TW * kMaxP + kThreads - 1) / kThreads;
        float xv[kX];
#pragma unroll
        for (int k = 0; k < kX; ++k) {
            const int i = threadIdx.x + k * kThreads, tt = i / P, j = i - tt * P;
            xv[k] = i < TW * P && t0 + tt < T ? xdbl[(size_t)(t0 + tt) * P + j] : 0.f;
        }
        if (TW > 1) {
            constexpr int kW = kMaxDtRank / 8 / TW;  // chunks per lane: chunk j = wave + TW·k of row lane
            u32x4 wv[kW];
            const bf16_t *row = W_dt + (size_t)(c0 + lane) * R;
#pragma unroll
            for (int k = 0; k < kW; ++k) {
                const int j = wave + TW * k;
                wv[k] = j < nchunk && c0 + lane < d_inner ? ld16(row + 8 * j) : (u32x4){0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int k = 0; k < kW; ++k) {
                const int j = wave + TW * k;
                if (j < nchunk)
#pragma unroll
                    for (int e = 0; e < 4; ++e) wdt[4 * j + e][lane] = wv[k][e];
            }
            // The decay rates, once per workgroup: wave w takes states w, w + TW, ...
            if (c0 + lane < d_inner)
                for (int n = wave; n < NS; n += TW) a2s[n][lane] = -expf(A_log[(size_t)(c0 + lane) * NS + n]) * kLog2e;
        }
#pragma unroll
        for (int k = 0; k < kX; ++k) {
            const int i = threadIdx.x + k * kThreads, tt = i / P, j = i - tt * P;
            if (i < TW * P) xds[tt][j] = xv[k];
        }
    }
    __syncthreads();
    const int c = c0 + lane, t = t0 + wave;
    if (c >= d_inner || t >= T) return;  // no barrier below

    const float *xd = xds[wave];  // δ [R] | B [NS] | C [NS]
    float a = dt_bias[c];
    if (TW > 1) {
        for (int r = 0; r < R / 2; ++r) {
            const uint32_t w = wdt[r][lane];
            a += lo_bf16(w) * xd[2 * r];
            a += hi_bf16(w) * xd[2 * r + 1];
        }
    } else {
        const bf16_t *row = W_dt + (size_t)c * R;
        for (int j0 = 0; j0 < nchunk; j0 += 8) {  // 8 chunks in flight
            u32x4 v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = j0 + k < nchunk ? ld16(row + 8 * (j0 + k)) : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (j0 + k < nchunk)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a += lo_bf16(v[k][e]) * xd[8 * (j0 + k) + 2 * e];
                        a += hi_bf16(v[k][e]) * xd[8 * (j0 + k) + 2 * e + 1];
                    }
        }
    }
    const float dlt = a > 20.f ? a : log1pf(expf(a));  // softplus
    const size_t tc = (size_t)t * d_inner + c;
    const float uu = u[tc];
    float s[NS];
    const f32x4 *sp = reinterpret_cast<const f32x4 *>(ssm_state + tc * NS);
#pragma unroll
    for (int q = 0; q < NS / 4; ++q) {
        const f32x4 v = sp[q];
        s[4 * q] = v[0];
        s[4 * q + 1] = v[1];
        s[4 * q + 2] = v[2];
        s[4 * q + 3] = v[3];
    }
    const float du = dlt * uu;
    float m = 0.f;
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        const float a2 = TW > 1 ? a2s[n][lane] : -expf(A_log[(size_t)c * NS + n]) * kLog2e;
        s[n] = exp2_fast(dlt * a2) * s[n] + du * xd[R + n];  // exp(Δ·A) as 2^(Δ·A·log2 e)
        m += xd[R + NS + n] * s[n];
    }
    f32x4 *so = reinterpret_cast<f32x4 *>(ssm_state + tc * NS);
#pragma unroll
    for (int q = 0; q < NS / 4; ++q) so[q] = (f32x4){s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
    m += Dp[c] * uu;
    M_out[tc] = f32_to_bf16(m);
    store_pair(g_hi, g_lo, tc, m * silu(xz[(size_t)t * ldxz + d_inner + c]));
}

}  // namespace

hipError_t launch_mamba_conv(const float *xz, int ldxz, float *conv_state, const float *conv_w, const float *conv_b,
                             float *u, bf16_t *u_hi, bf16_t *u_lo, int T, int d_inner, int K, hipStream_t stream) {
    const size_t n = (size_t)T * d_inner;
    hipLaunchKernelGGL(mamba_conv_kernel, dim3((unsigned)((n + kConvThreads - 1) / kConvThreads)), dim3(kConvThreads),
                       0, stream, xz, ldxz, conv_state, conv_w, conv_b, u, u_hi, u_lo, T, d_inner, K);
    return hipGetLastError();
}

hipError_t launch_mamba_scan(const float *xz, int ldxz, const float *u, const float *xdbl, int P, int R,
                             const bf16_t *W_dt, const float *dt_bias, const float *A_log, const float *Dp,
                             float *ssm_state, bf16_t *M_out, bf16_t *g_hi, bf16_t *g_lo, int T, int d_inner, int NS,
                             hipStream_t stream) {
    // Four tokens per workgroup share its staged W_dt rows; below four tokens
    // one wave per workgroup reads its rows directly.
    const int TW = T >= kScanWaves ? kScanWaves : 1;
    const dim3 grid((unsigned)((d_inner + kScanChannels - 1) / kScanChannels), (unsigned)((T + TW - 1) / TW));
#define SB_SCAN(N_, TW_)                                                                                             \
    hipLaunchKernelGGL((mamba_scan_kernel<N_, TW_>), grid, dim3(64 * TW_), 0, stream, xz, ldxz, u, xdbl, P, R, W_dt, \
                       dt_bias, A_log, Dp, ssm_state, M_out, g_hi, g_lo, T, d_inner)
#define SB_SCAN_TW(N_)                    \
    if (TW == kScanWaves) SB_SCAN(N_, 4); \
    else SB_SCAN(N_, 1);
    switch (NS) {
        case 8: SB_SCAN_TW(8); break;
        case 16: SB_SCAN_TW(16); break;
        case 32: SB_SCAN_TW(32); break;
        case 64: SB_SCAN_TW(64); break;
        default: return hipErrorInvalidValue;
    }
#undef SB_SCAN_TW
#undef SB_SCAN
    return hipGetLastError();
}

}  // namespace sambay
