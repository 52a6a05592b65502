// The self-decoder over the prompt in a YOCO-style prefill (gfx950): only
// the self-decoder runs over all prompt tokens, its final full-attention
// layer writes the shared KV cache once, and the cross-decoder then runs on
// the last prompt token alone (Paper-Notes reading notes on
// "Decoder-Hybrid-Decoder Architecture for Efficient Reasoning with Long
// Generation", section 整体框架; the Samba self-decoder alternates Mamba and
// sliding-window attention, section 消融实验).
//
// Every product is the MFMA GEMM over the B·T prompt rows (residual adds
// fused into its epilogues, the MLP's gate and up products paired in one),
// the SSM layers are the chunked prefill of mamba.hip, the attention layers
// the prefill kernel of prefill.hip.  This file adds the cache stores and the last-row gathers.
// Nothing after the final full-attention layer looks at earlier positions,
// so when that layer is the last one only its keys and values are computed
// for every token here; its attention, output projection and MLP run on the
// last token as the first layer of the cross-decoder step (a cross-attention
// layer over the cache it has just written).
#include "device.hpp"
#include "launch.hpp"

namespace sambay {

namespace {

constexpr int kThreads = 256;

// Positions p in [first, T) of k, v [B, T, Hkv, 128] go to slot p % slots of
// the caches [B, Hkv, slots, 128]: the shared cache (slots = L >= T,
// first = 0) or a sliding-window ring (slots = window, first = T - window).
// One thread per 16-byte piece.  lens (nullable) receives T per sequence.
__global__ __launch_bounds__(kThreads) void kv_store_kernel(const bf16_t *__restrict__ k, const bf16_t *__restrict__ v,
                                                            bf16_t *__restrict__ kc, bf16_t *__restrict__ vc, int B,
                                                            int T, int Hkv, int slots, int first,
                                                            int32_t *__restrict__ lens) {
    const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
    const int npos = T - first;
    const size_t total = (size_t)B * npos * Hkv * 16;
    if (lens && idx < (size_t)B) lens[idx] = T;
    if (idx >= total) return;
    const int piece = (int)(idx % 16);
    size_t r = idx / 16;
    const int g = (int)(r % Hkv);
    r /= Hkv;
    const int p = first + (int)(r % npos), b = (int)(r / npos);
    const size_t src = (((size_t)b * T + p) * Hkv + g) * kHeadDim + 8 * piece;
    const size_t dst = (((size_t)b * Hkv + g) * slots + p % slots) * kHeadDim + 8 * piece;
    *reinterpret_cast<u32x4 *>(kc + dst) = ld16(k + src);
    *reinterpret_cast<u32x4 *>(vc + dst) = ld16(v + src);
}

// dst[b, :] = src[b·T + T - 1, :] (rows of `cols` bf16, cols % 8 == 0).
__global__ __launch_bounds__(kThreads) void last_rows_kernel(const bf16_t *__restrict__ src, int T, int cols,
                                                             bf16_t *__restrict__ dst, int B) {
    const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x, per = (size_t)cols / 8;
    if (idx >= (size_t)B * per) return;
    const size_t b = idx / per, c = 8 * (idx % per);
    *reinterpret_cast<u32x4 *>(dst + b * cols + c) = ld16(src + (b * T + T - 1) * cols + c);
}

__global__ __launch_bounds__(kThreads) void copy16_kernel(const bf16_t *__restrict__ src, bf16_t *__restrict__ dst,
                                                          size_t n8) {
    const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx < n8) *reinterpret_cast<u32x4 *>(dst + 8 * idx) = ld16(src + 8 * idx);
}

dim3 blocks_for(size_t n) { return dim3((unsigned)((n + kThreads - 1) / kThreads)); }

size_t r256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

SelfDecoderLayout self_decoder_layout(void *base, int64_t B, int64_t T, int64_t d_model, int64_t d_inner,
                                      int64_t d_state, int64_t dt_rank, int64_t d_ff, int64_t Hq, int64_t Hkv) {
    const int64_t rows = B * T, D = kHeadDim;
    char *b = static_cast<char *>(base);
    size_t off = 0;
    auto take = [&](size_t n) { char *q = b ? b + off : nullptr; off += r256(n); return q; };
    SelfDecoderLayout L;
    L.h = reinterpret_cast<bf16_t *>(take((size_t)rows * d_model * 2));
    L.xn = reinterpret_cast<bf16_t *>(take((size_t)rows * d_model * 2));
    L.M = reinterpret_cast<bf16_t *>(take((size_t)rows * d_inner * 2));
    L.lens = reinterpret_cast<int32_t *>(take((size_t)B * 4));
    L.m_last = reinterpret_cast<bf16_t *>(take((size_t)B * d_inner * 2));
    // One region, used in turn by the attention layers, the MLPs and the SSM
    // layers' own workspace.
    const size_t attn = r256((size_t)rows * Hq * D * 2) * 2 + r256((size_t)rows * Hkv * D * 2) * 2 +
                        r256(attn_prefill_workspace_need(B, T, Hkv));
    const size_t mlp = d_ff > 0 ? r256((size_t)rows * d_ff * 2) : 0;
    const size_t ssm = r256(mamba_prefill_workspace_need(B, T, d_inner, d_state, dt_rank));
    size_t shared = attn > mlp ? attn : mlp;
    if (ssm > shared) shared = ssm;
    char *s = take(shared);
    L.scratch = s;
    L.q = reinterpret_cast<bf16_t *>(s);
    L.k = reinterpret_cast<bf16_t *>(s ? s + r256((size_t)rows * Hq * D * 2) : nullptr);
    L.v = reinterpret_cast<bf16_t *>(s ? (char *)L.k + r256((size_t)rows * Hkv * D * 2) : nullptr);
    L.o = reinterpret_cast<bf16_t *>(s ? (char *)L.v + r256((size_t)rows * Hkv * D * 2) : nullptr);
    L.attn_ws = s ? (char *)L.o + r256((size_t)rows * Hq * D * 2) : nullptr;
    L.hid = reinterpret_cast<bf16_t *>(s);
    L.bytes = off;
    return L;
}

hipError_t launch_self_decoder(const SelfDecoderArgs &a, const SelfDecoderLayout &L, hipStream_t stream) {
    const int B = a.B, T = a.T, dm = a.d_model, rows = B * T;
    const int qd = a.Hq * kHeadDim, kvd = a.Hkv * kHeadDim;
    hipError_t e = hipSuccess;
    auto chk = [&]() { return e == hipSuccess ? (e = hipGetLastError()) : e; };
    hipLaunchKernelGGL(copy16_kernel, blocks_for((size_t)rows * dm / 8), dim3(kThreads), 0, stream, a.x, L.h,
                       (size_t)rows * dm / 8);
    if (chk() != hipSuccess) return e;
    for (int li = 0; li < a.n && e == hipSuccess; ++li) {
        const sb_self_layer &ly = a.layers[li];
        const bf16_t *xin = L.h;
        if (ly.norm1) {
            if ((e = launch_rmsnorm(L.h, (const bf16_t *)ly.norm1, rows, dm, a.eps, L.xn, nullptr, stream)) !=
                hipSuccess)
                return e;
            xin = L.xn;
        }
        if (ly.kind == SB_SELF_MAMBA) {
            const sb_mamba_weights &w = ly.mamba;
            e = launch_mamba_prefill(xin, (const bf16_t *)w.w_in, w.conv_w, w.conv_b, (const bf16_t *)w.w_x,
                                     (const bf16_t *)w.w_dt, w.dt_bias, w.a_log, w.d_skip, (const bf16_t *)w.w_out,
                                     ly.conv_state, ly.ssm_state, L.M, L.h, B, T, dm, a.d_inner, a.d_state,
                                     a.dt_rank, a.d_conv, L.scratch, stream, /*resid=*/true);
        } else {
            const bool swa = ly.kind == SB_SELF_SWA;
            // The last layer, full attention, when the caller finishes it on
            // the last token (kv_only): its keys and values for the cache only.
            const bool kv_only = a.last_kv_only && li == a.n - 1 && !swa;
            e = launch_gemm(xin, (const bf16_t *)ly.wk, rows, kvd, dm, EPI_BF16, L.k, nullptr, stream);
            if (e == hipSuccess) e = launch_gemm(xin, (const bf16_t *)ly.wv, rows, kvd, dm, EPI_BF16, L.v, nullptr, stream);
            if (e == hipSuccess && !kv_only)
                e = launch_gemm(xin, (const bf16_t *)ly.wq, rows, qd, dm, EPI_BF16, L.q, nullptr, stream);
            if (e == hipSuccess && !kv_only)
                e = launch_attn_prefill(L.q, L.k, L.v, L.o, B, T, a.Hq, a.Hkv, swa ? a.window : 0, a.scale,
                                        L.attn_ws, stream);
            if (e == hipSuccess) {
                const int slots = swa ? a.window : a.L, first = swa && T > a.window ? T - a.window : 0;
                bf16_t *kc = static_cast<bf16_t *>(swa ? ly.kring : a.kcache);
                bf16_t *vc = static_cast<bf16_t *>(swa ? ly.vring : a.vcache);
                hipLaunchKernelGGL(kv_store_kernel, blocks_for((size_t)B * (T - first) * a.Hkv * 16), dim3(kThreads),
                                   0, stream, L.k, L.v, kc, vc, B, T, a.Hkv, slots, first, nullptr);
                e = hipGetLastError();
            }
            if (kv_only) continue;
            if (e == hipSuccess) e = launch_gemm(L.o, (const bf16_t *)ly.wo, rows, dm, qd, EPI_RESID, L.h, nullptr, stream);
        }
        if (e != hipSuccess || !ly.w_gate) continue;
        const bf16_t *xm = L.h;
        if (ly.norm2) {
            if ((e = launch_rmsnorm(L.h, (const bf16_t *)ly.norm2, rows, dm, a.eps, L.xn, nullptr, stream)) !=
                hipSuccess)
                return e;
            xm = L.xn;
        }
        // hid = SiLU(x W_gate^T) ⊙ (x W_up^T) in one paired product, then h += hid W_down^T.
        e = launch_gemm(xm, (const bf16_t *)ly.w_gate, rows, a.d_ff, dm, EPI_SWIGLU, L.hid,
                        (const bf16_t *)ly.w_up, stream);
        if (e == hipSuccess)
            e = launch_gemm(L.hid, (const bf16_t *)ly.w_down, rows, dm, a.d_ff, EPI_RESID, L.h, nullptr, stream);
    }
    if (e != hipSuccess) return e;
    // The last prompt token's hidden state and memory, and the cache length.
    hipLaunchKernelGGL(last_rows_kernel, blocks_for((size_t)B * dm / 8), dim3(kThreads), 0, stream, L.h, T, dm,
                       a.h_out, B);
    if (chk() != hipSuccess) return e;
    hipLaunchKernelGGL(last_rows_kernel, blocks_for((size_t)B * a.d_inner / 8), dim3(kThreads), 0, stream, L.M, T,
                       a.d_inner, a.M_out ? a.M_out : L.m_last, B);
    if (chk() != hipSuccess) return e;
    hipLaunchKernelGGL(kv_store_kernel, blocks_for((size_t)B), dim3(kThreads), 0, stream, L.k, L.v, (bf16_t *)nullptr,
                       (bf16_t *)nullptr, B, T, 1, 1, T, L.lens);
    return chk();
}

}  // namespace sambay
