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
#include <stdlib.h>

namespace sambay {

namespace {

constexpr int kConvThreads = 256;
constexpr int kScanChannels = 64;  // channels per workgroup (one per lane)
constexpr int kScanWaves = 4;      // tokens per workgroup (one per wave) from 4 tokens up,
constexpr int kScanWavesWide = 8;  // ... and from 8 tokens up
constexpr int kMaxStates = 64;

__device__ __forceinline__ float silu(float v) { return v / (1.f + expf(-v)); }

__device__ __forceinline__ void store_pair(bf16_t *hi, bf16_t *lo, size_t i, float v) {
    const bf16_t h = f32_to_bf16(v);
    hi[i] = h;
    lo[i] = split_lo(v, h);
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
// own row from memory.  A thread's state, input and gate are loaded first,
// so that their latency overlaps the staging and the step projection (every
// workgroup is resident at once and runs the same phases); every staging
// load of a thread is issued before its first LDS store.  Then Δ from the
// row and δ; the NS states of (token, channel) are updated in registers and
// written back; M (bf16) and g = M·SiLU(z) (bf16 hi + lo).
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
    const int c = c0 + lane, t = t0 + wave;
    // Every global load first, with indices clamped to valid elements instead
    // of conditions (threads past the last channel or token store nothing).
    const int cc = min(c, d_inner - 1);
    const size_t tc = (size_t)min(t, T - 1) * d_inner + cc;
    f32x4 sv[NS / 4], alv[TW > 1 ? 1 : NS / 4];
    {
        const f32x4 *sp = reinterpret_cast<const f32x4 *>(ssm_state + tc * NS);
#pragma unroll
        for (int q = 0; q < NS / 4; ++q) sv[q] = sp[q];
        if (TW == 1) {
            const f32x4 *ap = reinterpret_cast<const f32x4 *>(A_log + (size_t)cc * NS);
#pragma unroll
            for (int q = 0; q < NS / 4; ++q) alv[q] = ap[q];
        }
    }
    const float uu = u[tc];
    const float zz = xz[(size_t)min(t, T - 1) * ldxz + d_inner + cc];
    const float dtb = dt_bias[cc], dpc = Dp[cc];
    {
        constexpr int kX = (TW * kMaxP + kThreads - 1) / kThreads;
        float xv[kX];
#pragma unroll
        for (int k = 0; k < kX; ++k) {
            const int i = threadIdx.x + k * kThreads, tt = i / P, j = i - tt * P;
            xv[k] = xdbl[(size_t)min(t0 + tt, T - 1) * P + j];
        }
        if (TW > 1) {
            constexpr int kW = kMaxDtRank / 8 / TW;  // chunks per lane: chunk j = wave + TW·k of row lane
            constexpr int kA = (NS + TW - 1) / TW;   // decay rates per lane: state wave + TW·k of channel lane
            u32x4 wv[kW];
            float al[kA];
            const bf16_t *row = W_dt + (size_t)cc * R;
#pragma unroll
            for (int k = 0; k < kW; ++k) wv[k] = ld16(row + 8 * min(wave + TW * k, nchunk - 1));
#pragma unroll
            for (int k = 0; k < kA; ++k) al[k] = A_log[(size_t)cc * NS + min(wave + TW * k, NS - 1)];
#pragma unroll
            for (int k = 0; k < kW; ++k) {
                const int j = wave + TW * k;
                if (j < nchunk)
#pragma unroll
                    for (int e = 0; e < 4; ++e) wdt[4 * j + e][lane] = wv[k][e];
            }
#pragma unroll
            for (int k = 0; k < kA; ++k)
                if (wave + TW * k < NS) a2s[wave + TW * k][lane] = -expf(al[k]) * kLog2e;
        }
#pragma unroll
        for (int k = 0; k < kX; ++k) {
            const int i = threadIdx.x + k * kThreads, tt = i / P, j = i - tt * P;
            if (i < TW * P) xds[tt][j] = xv[k];
        }
    }
    __syncthreads();
    if (c >= d_inner || t >= T) return;  // no barrier below

    const float *xd = xds[wave];  // δ [R] | B [NS] | C [NS]
    float a = dtb;
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
            for (int k = 0; k < 8; ++k) v[k] = ld16(row + 8 * min(j0 + k, nchunk - 1));
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
    float s[NS];
#pragma unroll
    for (int q = 0; q < NS / 4; ++q) {
        const f32x4 v = sv[q];
        s[4 * q] = v[0];
        s[4 * q + 1] = v[1];
        s[4 * q + 2] = v[2];
        s[4 * q + 3] = v[3];
    }
    const float du = dlt * uu;
    float m = 0.f;
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        const float a2 = TW > 1 ? a2s[n][lane] : -expf(alv[TW > 1 ? 0 : n / 4][n % 4]) * kLog2e;
        s[n] = exp2_fast(dlt * a2) * s[n] + du * xd[R + n];  // exp(Δ·A) as 2^(Δ·A·log2 e)
        m += xd[R + NS + n] * s[n];
    }
    f32x4 *so = reinterpret_cast<f32x4 *>(ssm_state + tc * NS);
#pragma unroll
    for (int q = 0; q < NS / 4; ++q) so[q] = (f32x4){s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
    m += dpc * uu;
    M_out[tc] = f32_to_bf16(m);
    store_pair(g_hi, g_lo, tc, m * silu(zz));
}

// ------------------------------------------------------------------ prefill
// The same layer over T prompt tokens: the projections are MFMA GEMMs over
// all B·T rows (bf16 operands), the convolution and the scan run over the
// sequence.

// Grid (blocks of 8·256 channels, token blocks of kConvRun, b): each thread
// runs the convolution over kConvRun consecutive tokens of 8 adjacent
// channels with the window in registers (16-byte loads and stores):
// u = SiLU(conv_b + Σ_k conv_w[k] · x̃[t - K + 1 + k]), x̃ the x branch of
// the input projection, positions before the prompt taken from the stored
// window (read only here).
constexpr int kConvRun = 8;
template <int K>
__global__ __launch_bounds__(kConvThreads) void mamba_conv_seq_kernel(const bf16_t *__restrict__ xz, int ldxz,
                                                                      const float *__restrict__ conv_state,
                                                                      const float *__restrict__ conv_w,
                                                                      const float *__restrict__ conv_b,
                                                                      bf16_t *__restrict__ u, int T, int d_inner) {
    const int c = 8 * (blockIdx.x * kConvThreads + threadIdx.x), t0 = blockIdx.y * kConvRun, b = blockIdx.z;
    if (c >= d_inner) return;
    constexpr int NW = K - 1 + kConvRun;
    u32x4 raw[NW];  // raw[j]: the 8 channels of x̃ at position t0 - (K - 1) + j (bf16)
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const int i = min(max(t0 - (K - 1) + j, 0), T - 1);
        raw[j] = ld16(xz + ((size_t)b * T + i) * ldxz + c);
    }
    float w[K][8], bias[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        bias[e] = conv_b[c + e];
#pragma unroll
        for (int k = 0; k < K; ++k) w[k][e] = conv_w[(size_t)(c + e) * K + k];
    }
    float win[NW][8];
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const int i = t0 - (K - 1) + j;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = (e & 1) ? hi_bf16(raw[j][e / 2]) : lo_bf16(raw[j][e / 2]);
            if (i < 0) x = conv_state[((size_t)b * d_inner + c + e) * (K - 1) + (K - 1 + i)];
            win[j][e] = x;
        }
    }
#pragma unroll
    for (int r = 0; r < kConvRun; ++r) {
        if (t0 + r >= T) break;
        u32x4 o;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            float y[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int e = 2 * e2 + h;
                float acc = bias[e];
#pragma unroll
                for (int k = 0; k < K; ++k) acc += w[k][e] * win[r + k][e];
                y[h] = acc / (1.f + __expf(-acc));
            }
            o[e2] = pack_bf16x2(y[0], y[1]);
        }
        *reinterpret_cast<u32x4 *>(u + ((size_t)b * T + t0 + r) * d_inner + c) = o;
    }
}

// Sum of the step/B/C projection's K-slices (fp32 [ks, rows, P]): δ to its own
// rows [rows, R] (the step projection's operand), B | C to [rows, 2·NS], bf16.
__global__ __launch_bounds__(256) void xproj_reduce_kernel(const float *__restrict__ part, int ks, int rows, int P,
                                                           int R, bf16_t *__restrict__ delta, bf16_t *__restrict__ bc) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x, per = (size_t)P / 8;
    if (idx >= (size_t)rows * per) return;
    const size_t r = idx / per;
    const int c = 8 * (int)(idx % per);
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < ks; ++s) {
        const float *p = part + ((size_t)s * rows + r) * P + c;
        const f32x4 lo = *reinterpret_cast<const f32x4 *>(p), hi = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] += lo[e], a[4 + e] += hi[e];
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(a[2 * e], a[2 * e + 1]);
    bf16_t *dst = c < R ? delta + r * R + c : bc + r * (P - R) + (c - R);
    *reinterpret_cast<u32x4 *>(dst) = o;
}

// One thread per (b, channel): the stored window after the prompt (its last
// K - 1 inputs, or older stored ones when T < K - 1), updated in place.
__global__ __launch_bounds__(kConvThreads) void mamba_conv_state_kernel(const bf16_t *__restrict__ xz, int ldxz,
                                                                        float *__restrict__ conv_state, int B, int T,
                                                                        int d_inner, int K) {
    const size_t idx = (size_t)blockIdx.x * kConvThreads + threadIdx.x;
    if (idx >= (size_t)B * d_inner || K < 2) return;
    const int b = (int)(idx / d_inner), c = (int)(idx % d_inner);
    float *st = conv_state + idx * (K - 1);
    float old[kMaxConv], nw[kMaxConv];
#pragma unroll
    for (int k = 0; k < kMaxConv - 1; ++k)
        if (k < K - 1) old[k] = st[k];
#pragma unroll
    for (int k = 0; k < kMaxConv - 1; ++k)
        if (k < K - 1) {
            const int i = T - (K - 1) + k;  // position of the k-th kept input
            nw[k] = i >= 0 ? bf16_to_f32(xz[((size_t)b * T + i) * ldxz + c]) : old[K - 1 + i];
        }
#pragma unroll
    for (int k = 0; k < kMaxConv - 1; ++k)
        if (k < K - 1) st[k] = nw[k];
}

// The selective scan over the prompt, in chunks of Lc tokens so that every
// chunk of every channel runs in parallel:
//   A: each chunk from a zero state: its end state S and its total decay
//      P = exp(A · ΣΔ) per (channel, state);
//   B: per (channel, state), in chunk order: the state entering each chunk
//      (init_k = s; s = P_k·s + S_k) and the state after the prompt;
//   C: each chunk again from its entering state, with the readout
//      M_t = Σ_n C_n s_n + D·u_t and the gate g_t = M_t·SiLU(z_t).
// A lane holds NPL states of one channel in registers (G = NS / NPL lanes per
// channel, adjacent, their readouts summed by shuffles); a one-wave
// workgroup covers 64 / G channels of one chunk.  Δ, u, z are read per lane
// (consecutive channels: coalesced); B and C of a token are the same for the
// whole wave when G == 1 (scalar loads).  Steps past the prompt's end run
// with Δ = 0, which leaves the state as it is, so the loop has no tail.
constexpr int kScanUnroll = 8;

__host__ __device__ constexpr int scan_lanes_per_channel(int NS) { return NS > 16 ? NS / 16 : 1; }

template <int NPL, int G, bool OUT>
__global__ __launch_bounds__(64) void mamba_chunk_scan_kernel(
    const bf16_t *__restrict__ xz, int ldxz, const bf16_t *__restrict__ u, const bf16_t *__restrict__ xdbl, int P,
    int R, const float *__restrict__ delta, const float *__restrict__ A_log, const float *__restrict__ Dp,
    float *__restrict__ SP,  // [B, nchunks, d_inner, NS] x2: S (A) / entering state (C), then P (A)
    bf16_t *__restrict__ M_out, bf16_t *__restrict__ g_out, int T, int Lc, int d_inner) {
    constexpr int NS = NPL * G, U = kScanUnroll;
    const int k = blockIdx.x, b = blockIdx.z, nchunks = gridDim.x;
    const int gi = threadIdx.x % G, c = blockIdx.y * (64 / G) + threadIdx.x / G;
    const int t0 = k * Lc, len = min(Lc, T - t0);
    const size_t row0 = (size_t)b * T + t0;
    const size_t spi = (((size_t)b * nchunks + k) * d_inner + c) * NS + NPL * gi;
    const size_t half = (size_t)gridDim.z * nchunks * d_inner * NS;  // offset of the P array
    float a2[NPL], st[NPL];
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
        a2[q] = -expf(A_log[(size_t)c * NS + NPL * gi + q]) * kLog2e;
        st[q] = OUT ? SP[spi + q] : 0.f;
    }
    const float dsk = OUT ? Dp[c] : 0.f;
    float dsum = 0.f;
    for (int tb = 0; tb < len; tb += U) {
        float dl[U], uu[U], zz[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int t = min(tb + i, len - 1);
            const size_t row = row0 + t;
            const float d = delta[row * d_inner + c];
            dl[i] = tb + i < len ? d : 0.f;
            uu[i] = bf16_to_f32(u[row * d_inner + c]);
            if (OUT) zz[i] = bf16_to_f32(xz[row * ldxz + d_inner + c]);
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int t = min(tb + i, len - 1);
            const bf16_t *bc = xdbl + (row0 + t) * P + R + NPL * gi;
            const float du = dl[i] * uu[i];
            float m = 0.f;
#pragma unroll
            for (int q2 = 0; q2 < NPL; q2 += 8) {
                const u32x4 bw = ld16(bc + q2);
                const float bq[8] = {lo_bf16(bw[0]), hi_bf16(bw[0]), lo_bf16(bw[1]), hi_bf16(bw[1]),
                                     lo_bf16(bw[2]), hi_bf16(bw[2]), lo_bf16(bw[3]), hi_bf16(bw[3])};
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    st[q2 + q] = exp2_fast(dl[i] * a2[q2 + q]) * st[q2 + q] + du * bq[q];
                if (OUT) {
                    const u32x4 cw = ld16(bc + NS + q2);
                    const float cq[8] = {lo_bf16(cw[0]), hi_bf16(cw[0]), lo_bf16(cw[1]), hi_bf16(cw[1]),
                                         lo_bf16(cw[2]), hi_bf16(cw[2]), lo_bf16(cw[3]), hi_bf16(cw[3])};
#pragma unroll
                    for (int q = 0; q < 8; ++q) m += cq[q] * st[q2 + q];
                }
            }
            if (OUT) {
#pragma unroll
                for (int x = 1; x < G; x <<= 1) m += __shfl_xor(m, x);
                if (gi == 0 && tb + i < len) {
                    const size_t o = (row0 + tb + i) * d_inner + c;
                    const float mm = m + dsk * uu[i];
                    M_out[o] = f32_to_bf16(mm);
                    g_out[o] = f32_to_bf16(mm * (zz[i] / (1.f + __expf(-zz[i]))));
                }
            } else {
                dsum += dl[i];
            }
        }
    }
    if (!OUT) {
#pragma unroll
        for (int q = 0; q < NPL; ++q) {
            SP[spi + q] = st[q];
            SP[half + spi + q] = exp2_fast(a2[q] * dsum);
        }
    }
}

// One thread per (b, channel, state): the state entering each chunk, in
// order, written over that chunk's S; the state after the prompt.
__global__ __launch_bounds__(256) void mamba_chunk_combine_kernel(float *__restrict__ SP,
                                                                  float *__restrict__ ssm_state, int B, int nchunks,
                                                                  int d_inner, int NS) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x, per = (size_t)d_inner * NS;
    if (idx >= (size_t)B * per) return;
    const size_t b = idx / per, cn = idx % per, half = (size_t)B * nchunks * per;
    float s = ssm_state[idx];
    for (int k = 0; k < nchunks; ++k) {
        const size_t i = (b * nchunks + k) * per + cn;
        const float S = SP[i], Pk = SP[half + i];
        SP[i] = s;
        s = Pk * s + S;
    }
    ssm_state[idx] = s;
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
    // Eight (from 8 tokens) or four (from 4) tokens per workgroup share its
    // staged W_dt rows; below four tokens one wave per workgroup reads its
    // rows directly.
    const int TW = T >= kScanWavesWide ? kScanWavesWide : T >= kScanWaves ? kScanWaves : 1;
    const dim3 grid((unsigned)((d_inner + kScanChannels - 1) / kScanChannels), (unsigned)((T + TW - 1) / TW));
#define SB_SCAN(N_, TW_)                                                                                             \
    hipLaunchKernelGGL((mamba_scan_kernel<N_, TW_>), grid, dim3(64 * TW_), 0, stream, xz, ldxz, u, xdbl, P, R, W_dt, \
                       dt_bias, A_log, Dp, ssm_state, M_out, g_hi, g_lo, T, d_inner)
#define SB_SCAN_TW(N_)                         \
    if (TW == kScanWavesWide) SB_SCAN(N_, 8);  \
    else if (TW == kScanWaves) SB_SCAN(N_, 4); \
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

// Tokens per scan chunk: 64, halved (to 16 at least) while the scan would
// have fewer than 8192 waves (32 per CU).
static int mamba_scan_chunk(int64_t B, int64_t T, int64_t d_inner, int64_t NS) {
    // SAMBAY_SCAN_CHUNK (a multiple of 8, 8..512) overrides the rule (measurement).
    const char *env = getenv("SAMBAY_SCAN_CHUNK");
    if (env && *env) {
        const int v = atoi(env);
        if (v >= 8 && v <= 512 && v % 8 == 0) return v;
    }
    int Lc = 64;
    const int64_t waves = B * d_inner * scan_lanes_per_channel((int)NS) / 64;
    while (Lc > 16 && waves * ((T + Lc - 1) / Lc) < 8192) Lc /= 2;
    return Lc;
}

// K-slices of the step/B/C projection (rows × (R + 2·NS) × d_inner: few
// output tiles, a long K): up to 512 workgroups, slices of >= 512.
static int xproj_splits(int64_t rows, int64_t P, int64_t d_inner) {
    const int64_t tiles = ((rows + 127) / 128) * ((P + 127) / 128);
    int ks = 1;
    while (ks < 8 && tiles * ks * 2 <= 512 && d_inner % (64 * ks * 2) == 0 && d_inner / (ks * 2) >= 512) ks *= 2;
    return ks;
}

namespace {
struct PrefillLayout {
    bf16_t *xz, *u, *bc, *delta, *g;
    float *part, *dpre, *sp;
    size_t bytes;
};
PrefillLayout prefill_layout(void *base, int64_t B, int64_t T, int64_t d_inner, int64_t NS, int64_t R) {
    const int64_t rows = B * T, P = R + 2 * NS;
    const int64_t Lc = mamba_scan_chunk(B, T, d_inner, NS), nch = (T + Lc - 1) / Lc;
    auto r = [](size_t v) { return (v + 255) & ~(size_t)255; };
    char *b = reinterpret_cast<char *>(base);
    size_t off = 0;
    auto take = [&](size_t n) { char *q = b ? b + off : nullptr; off += r(n); return q; };
    PrefillLayout L;
    L.xz = reinterpret_cast<bf16_t *>(take((size_t)rows * 2 * d_inner * 2));
    L.u = reinterpret_cast<bf16_t *>(take((size_t)rows * d_inner * 2));
    L.part = reinterpret_cast<float *>(take((size_t)xproj_splits(rows, P, d_inner) * rows * P * 4));
    L.bc = reinterpret_cast<bf16_t *>(take((size_t)rows * 2 * NS * 2));
    L.delta = reinterpret_cast<bf16_t *>(take((size_t)rows * R * 2));
    L.dpre = reinterpret_cast<float *>(take((size_t)rows * d_inner * 4));
    L.g = reinterpret_cast<bf16_t *>(take((size_t)rows * d_inner * 2));
    L.sp = reinterpret_cast<float *>(take((size_t)2 * B * nch * d_inner * NS * 4));
    L.bytes = off;
    return L;
}
}  // namespace

size_t mamba_prefill_workspace_need(int64_t B, int64_t T, int64_t d_inner, int64_t d_state, int64_t dt_rank) {
    return prefill_layout(nullptr, B, T, d_inner, d_state, dt_rank).bytes;
}

hipError_t launch_mamba_prefill(const bf16_t *x, const bf16_t *W_in, const float *conv_w, const float *conv_b,
                                const bf16_t *W_x, const bf16_t *W_dt, const float *dt_bias, const float *A_log,
                                const float *Dp, const bf16_t *W_out, float *conv_state, float *ssm_state,
                                bf16_t *M_out, bf16_t *y_out, int B, int T, int d_model, int d_inner, int NS, int R,
                                int K, void *workspace, hipStream_t stream, bool resid) {
    const int rows = B * T, P = R + 2 * NS, di2 = 2 * d_inner;
    const PrefillLayout L = prefill_layout(workspace, B, T, d_inner, NS, R);
    bf16_t *xz = L.xz, *u = L.u, *bc = L.bc, *delta = L.delta, *g = L.g;
    float *dpre = L.dpre, *sp = L.sp;

    auto blocks = [](size_t n, int per) { return dim3((unsigned)((n + per - 1) / per)); };
    hipError_t e = launch_gemm(x, W_in, rows, di2, d_model, EPI_BF16, xz, nullptr, stream);
    if (e != hipSuccess) return e;
    const dim3 conv_grid((unsigned)((d_inner / 8 + kConvThreads - 1) / kConvThreads),
                         (unsigned)((T + kConvRun - 1) / kConvRun), (unsigned)B);
#define SB_CONV(K_)                                                                                                  \
    case K_:                                                                                                         \
        hipLaunchKernelGGL(mamba_conv_seq_kernel<K_>, conv_grid, dim3(kConvThreads), 0, stream, xz, di2, conv_state, \
                           conv_w, conv_b, u, T, d_inner);                                                           \
        break
    switch (K) {
        SB_CONV(1); SB_CONV(2); SB_CONV(3); SB_CONV(4); SB_CONV(5); SB_CONV(6); SB_CONV(7); SB_CONV(8);
        default: return hipErrorInvalidValue;
    }
#undef SB_CONV
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(mamba_conv_state_kernel, blocks((size_t)B * d_inner, kConvThreads), dim3(kConvThreads), 0,
                       stream, xz, di2, conv_state, B, T, d_inner, K);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // [δ | B | C] = u W_x^T in K-slices (fp32 partials), then summed into δ
    // rows and B | C rows (bf16).
    const int ks = xproj_splits(rows, P, d_inner);
    e = launch_gemm(u, W_x, rows, P, d_inner, EPI_F32, reinterpret_cast<bf16_t *>(L.part), nullptr, stream, ks);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(xproj_reduce_kernel, blocks((size_t)rows * P / 8, 256), dim3(256), 0, stream, L.part, ks, rows,
                       P, R, delta, bc);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // Δ = softplus(δ W_dt^T + dt_bias) in the GEMM's epilogue (fp32).
    e = launch_gemm(delta, W_dt, rows, d_inner, R, EPI_SOFTPLUS, reinterpret_cast<bf16_t *>(dpre),
                    reinterpret_cast<const bf16_t *>(dt_bias), stream);
    if (e != hipSuccess) return e;
    // The chunked scan (dpre now holds Δ; SP after g in the workspace).
    const int Lc = mamba_scan_chunk(B, T, d_inner, NS), nch = (T + Lc - 1) / Lc;
    const dim3 cgrid((unsigned)nch, (unsigned)(d_inner * scan_lanes_per_channel(NS) / 64), (unsigned)B);
#define SB_CHUNK(N_, OUT_)                                                                                          \
    hipLaunchKernelGGL((mamba_chunk_scan_kernel<N_ / scan_lanes_per_channel(N_), scan_lanes_per_channel(N_), OUT_>), \
                       cgrid, dim3(64), 0, stream, xz, di2, u, bc, 2 * NS, 0, dpre, A_log, Dp, sp, M_out, g, T, Lc,  \
                       d_inner)
#define SB_CHUNK_NS(OUT_)                  \
    switch (NS) {                          \
        case 8: SB_CHUNK(8, OUT_); break;  \
        case 16: SB_CHUNK(16, OUT_); break; \
        case 32: SB_CHUNK(32, OUT_); break; \
        case 64: SB_CHUNK(64, OUT_); break; \
        default: return hipErrorInvalidValue; \
    }
    SB_CHUNK_NS(false);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(mamba_chunk_combine_kernel, blocks((size_t)B * d_inner * NS, 256), dim3(256), 0, stream, sp,
                       ssm_state, B, nch, d_inner, NS);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    SB_CHUNK_NS(true);
#undef SB_CHUNK_NS
#undef SB_CHUNK
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_gemm(g, W_out, rows, d_model, d_inner, resid ? EPI_RESID : EPI_BF16, y_out, nullptr, stream);
}

}  // namespace sambay
