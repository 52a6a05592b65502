// Host-side launchers for the gfx950 kernels.  The C ABI (api.hip) validates
// every argument first; these functions assume valid shapes and only enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sambay.h"

namespace sambay {

typedef uint16_t bf16_t;

// Optional HIP-event bracket around one kernel launch (sb_timing_enable).
class TimingScope {
  public:
    TimingScope(uint32_t kind, hipStream_t stream);
    ~TimingScope();
    TimingScope(const TimingScope &) = delete;
    TimingScope &operator=(const TimingScope &) = delete;

  private:
    uint32_t kind_;
    hipStream_t stream_;
    hipEvent_t start_ = nullptr, stop_ = nullptr;
    bool active_ = false;
};
constexpr uint32_t kTimeXattnSplit = 1, kTimeXattnMerge = 2, kTimeSkinny = 4, kTimeGemm = 8, kTimeGmuF32 = 16,
                   kTimeProbe = 32, kTimeDiffSplit = 64, kTimeDiffMerge = 128,
                   kTimePrefill = 256;

// ------------------------------------------------------- cross-attention
constexpr int kHeadDim = 128;     // supported head dimension
constexpr int kMaxGroup = 16;     // query heads per KV head handled by one tile
constexpr int kKeyBlock = 32;     // cache positions per wave iteration
constexpr int kMaxSplits = 64;

struct XattnPlan {
    int splits;  // number of key chunks per (sequence, KV head)
    int chunk;   // keys per chunk, a multiple of kKeyBlock; every chunk is non-empty
    // Lengths batches: keys per chunk when every length is within one chunk
    // of L (decided on the device, where the lengths are): the full plan's
    // chunk, twice `chunk` when the plan halved it for ragged lengths.
    int chunk_full;
};

// ragged: a lengths array limits each sequence to a prefix of the L positions.
XattnPlan xattn_plan(int64_t B, int64_t Hkv, int64_t L, bool ragged = false);
// Bytes of fp32 partials for `splits` chunks: (max, sum) pairs then D-wide sums.
size_t xattn_partial_bytes(int64_t B, int64_t Hq, int splits);
// Partial bytes for either plan (what a workspace must hold).
size_t xattn_workspace_need(int64_t B, int64_t Hq, int64_t Hkv, int64_t L);
// q is fp32 ([B, Hq, D]) when q_f32, else bf16.  out: bf16 [B, Hq, D]; out_lo
// (nullable) receives bf16(o - out), the low part of a bf16 hi + lo pair.
hipError_t launch_xattn(const void *q, bool q_f32, const bf16_t *K, const bf16_t *V, const int32_t *lens,
                        bf16_t *out, bf16_t *out_lo, int B, int Hq, int Hkv, int L, float scale, const XattnPlan &plan,
                        void *partials, hipStream_t stream);

// Differential attention decode: q, K, V bf16 with 128-wide rows split into
// two 64-wide halves (one per map); partials hold 2·Hq score columns per
// sequence (xattn_partial_bytes(B, 2·Hq, splits)); gamma [128] bf16 or null.
hipError_t launch_diffattn(const bf16_t *q, const bf16_t *K, const bf16_t *V, const int32_t *lens, const bf16_t *gamma,
                           bf16_t *out, int B, int Hq, int Hkv, int L, float scale, float lam, float lam_init,
                           float eps, const XattnPlan &plan, void *partials, hipStream_t stream);

// Self-decoder cache append: sequence b's new K/V rows ([B, Hkv, 128] each)
// go to position pos[b] (window 0, cache of L positions; not stored when
// pos[b] >= L) or ring slot pos[b] % window (cache of window == L slots);
// nothing for pos[b] < 0.  lens_out (nullable, B int32) receives the visible
// count: 0 for pos[b] < 0, else min(pos[b] + 1, L).
hipError_t launch_kv_append(const bf16_t *k_new, const bf16_t *v_new, bf16_t *K, bf16_t *V, const int32_t *pos,
                            int32_t *lens_out, int B, int Hkv, int L, int window, hipStream_t stream);

// Prefill attention: q [B, T, Hq, 128], k, v [B, T, Hkv, 128] bf16 ->
// out [B, T, Hq, 128] bf16; query i sees keys j <= i (and j > i - window when
// window > 0).  Grid (ceil(T / 64), Hq, B).
// workspace: attn_prefill_workspace_need(B, T, Hkv) bytes (V transposed).
size_t attn_prefill_workspace_need(int64_t B, int64_t T, int64_t Hkv);
// Query heads that one prefill-attention workgroup takes (1 to 4, a divisor of Hq / Hkv).
int attn_prefill_heads(int64_t B, int64_t T, int64_t Hq, int64_t Hkv);
hipError_t launch_attn_prefill(const bf16_t *q, const bf16_t *k, const bf16_t *v, bf16_t *out, int B, int T, int Hq,
                               int Hkv, int window, float scale, void *workspace, hipStream_t stream);

// ------------------------------------------------------ SSM decode step
constexpr int kMaxConv = 8;      // convolution taps supported
constexpr int kMaxDtRank = 256;  // step-projection rank supported (a multiple of 8)
// u = SiLU(conv(window, xi)) per (token, channel); conv_state [T, d_inner, K-1]
// fp32 shifted in place; u fp32 and as a bf16 hi + lo pair.
hipError_t launch_mamba_conv(const float *xz, int ldxz, float *conv_state, const float *conv_w, const float *conv_b,
                             float *u, bf16_t *u_hi, bf16_t *u_lo, int T, int d_inner, int K, hipStream_t stream);
// Δ = softplus(W_dt δ + dt_bias), the NS-state update of ssm_state [T, d_inner,
// NS] fp32 in place, M (bf16) and g = M·SiLU(z) (bf16 hi + lo).  xdbl [T, P]
// holds δ [R] | B [NS] | C [NS]; z is xz[:, d_inner:].  NS in {8, 16, 32, 64}.
hipError_t launch_mamba_scan(const float *xz, int ldxz, const float *u, const float *xdbl, int P, int R,
                             const bf16_t *W_dt, const float *dt_bias, const float *A_log, const float *Dp,
                             float *ssm_state, bf16_t *M_out, bf16_t *g_hi, bf16_t *g_lo, int T, int d_inner, int NS,
                             hipStream_t stream);

// The SSM layer over T prompt tokens (x [B·T, d_model] rows): GEMM
// projections, the convolution and the selective scan over the sequence;
// conv_state / ssm_state in and out; M [B·T, d_inner], y [B·T, d_model]
// (resid: y_out holds h and receives bf16(h + y) instead).
// Requires d_model, d_inner, R multiples of 64, NS in {8, 16, 32, 64}.
size_t mamba_prefill_workspace_need(int64_t B, int64_t T, int64_t d_inner, int64_t d_state, int64_t dt_rank);
hipError_t launch_mamba_prefill(const bf16_t *x, const bf16_t *W_in, const float *conv_w, const float *conv_b,
                                const bf16_t *W_x, const bf16_t *W_dt, const float *dt_bias, const float *A_log,
                                const float *Dp, const bf16_t *W_out, float *conv_state, float *ssm_state,
                                bf16_t *M_out, bf16_t *y_out, int B, int T, int d_model, int d_inner, int NS, int R,
                                int K, void *workspace, hipStream_t stream, bool resid = false);

// ------------------------------------------------ skinny (decode) products
// out[t, n] = epi( Σ_k X[t, k] · W[n, k] ) for t < T <= 64 tokens.
enum Epilogue {
    EPI_F32 = 0,    // out fp32
    EPI_BF16 = 1,   // out bf16
    EPI_GATE = 2,   // out bf16 = aux[t, n] · SiLU(acc)   (aux = M, bf16)
    EPI_RESID = 3,  // out bf16 = out[t, n] + acc         (in-place residual add)
    EPI_SWIGLU = 4,  // out bf16 = SiLU(X W^T) · (X W_b^T): gate and up in one pass (W_b required)
    EPI_SOFTPLUS = 5 // prefill GEMM only: out fp32 = softplus(acc + bias[n]), bias = aux as fp32 [N]
};
constexpr int kSkinnyMaxTokens = 64;

struct SkinnyPlan {
    int rows_per_wg;   // weight rows per workgroup
    int k_splits;      // workgroups along K (1 = epilogue fused)
    int k_slice;       // K elements per split (multiple of 64)
    int slab_rtw = 0;  // > 0: the slab product, 128 x slab_rtw weight rows per workgroup (k_splits > 1 always)
};
// xlo: the token operand is a bf16 hi + lo pair (twice the bytes per workgroup).
SkinnyPlan skinny_plan(int T, int N, int K, bool xlo);
size_t skinny_partial_bytes(int T, int N, const SkinnyPlan &p);
size_t skinny_partial_bytes_max(int T, int N, int K);  // over both operand kinds (workspace sizing)

struct SkinnyArgs {
    const bf16_t *X = nullptr;     // [T, ldx] bf16
    const bf16_t *X_lo = nullptr;  // optional low part: the product uses X + X_lo (a bf16 hi + lo pair)
    int ldx = 0;
    const bf16_t *W = nullptr;     // [N, K] bf16
    const bf16_t *W_b = nullptr;   // EPI_SWIGLU: the up weights [N, K]; W is then the gate (one pass, plan
                                   // with skinny_plan_dual).  Stacked products: below
    int T = 0, N = 0, K = 0;
    Epilogue epi = EPI_F32;
    void *out = nullptr;           // [T, ldo]
    int ldo = 0;
    bf16_t *out_lo = nullptr;      // EPI_GATE / EPI_SWIGLU, optional: bf16(value - out)
    const bf16_t *aux = nullptr;   // EPI_GATE: M [T, ldaux]
    int ldaux = 0;
    // EPI_RESID only: also produce the next sublayer's input RMSNorm(h_new;
    // next_norm) as a bf16 hi + lo pair [T, ldo] — fused into the finishing
    // pass when the plan splits K (skinny_fuses_norm), else left to the caller.
    const bf16_t *next_norm = nullptr;
    bf16_t *next_x = nullptr, *next_x_lo = nullptr;
    float eps = 0.f;
    // The 16-token tiled layout of a token operand [T, K] (element (t, k) at
    // tiled_index(t, k, ceil(T / 16)); tiled_elems(T, K) elements, tokens past
    // T undefined): one load instruction of the MFMA token operand reads 1 KB
    // contiguous instead of 64 bytes of 16 rows.  For operands the library
    // produces and consumes itself (the GMU's gated hidden H); only the
    // LDS-streaming product takes it (skinny_tiles).
    bool x_tiled = false;    // X (and X_lo) in the tiled layout (ldx unused)
    bool out_tiled = false;  // EPI_GATE: out (and out_lo) written in the tiled layout, K = N (ldo unused)
    // The deferred RMSNorm (slab product only, slab_norm_ok): X is the
    // residual stream h (X_lo null) and the operand is RMSNorm(h; norm_g),
    // from the chunk sums of squares norm_stats [T][norm_stats_stride(K)]
    // that the residual product which last wrote h left (stats_out).
    const bf16_t *norm_g = nullptr;
    const float *norm_stats = nullptr;
    float norm_eps = 0.f;
    // EPI_RESID, slab product only: also write those chunk sums of h_new
    // ([T][norm_stats_stride(N)]) for the next sublayer's deferred norm.
    float *stats_out = nullptr;
    // Stacked products (EPI_BF16, slab product only; na > 0): several
    // products of one operand in one pass.  Output rows [0, na) come from W
    // into out [T, ldo], rows [na, nb) from W_b (row n - na) into out_b
    // [T, ldo_b], rows [nb, N) from W_c (row n - nb) into out_c [T, ldo_c];
    // na, nb, the leading dimensions multiples of 4.
    const bf16_t *W_c = nullptr;
    int na = 0, nb = 0;
    bf16_t *out_b = nullptr, *out_c = nullptr;
    int ldo_b = 0, ldo_c = 0;
};
__host__ __device__ inline size_t tiled_index(int t, int k, int ntiles) {
    return ((size_t)(k >> 5) * ntiles + (t >> 4)) * 512 + ((k >> 3) & 3) * 128 + (t & 15) * 8 + (k & 7);
}
inline size_t tiled_elems(int T, int K) { return (size_t)((T + 15) / 16) * 16 * K; }
// Whether launch_skinny runs this product on the LDS-streaming kernel (the
// only one that reads or writes the tiled layout).
// Whether a product of T tokens, Nrows weight rows (the SwiGLU pair: both
// matrices' rows) and K columns runs as the slab product with a hi + lo
// operand: then its operand may be a deferred RMSNorm, and a residual
// product of that shape may leave the statistics for one.
bool slab_norm_ok(int T, int Nrows, int K);
// SAMBAY_NO_NORM_FUSION=1: every RMSNorm by its own launch (same bits).
bool norm_fusion_off();
// Whether the plan's kernel takes the 16-token tiled layout for this
// product's token operand (x_tiled) and, for the gate epilogue, its output
// (out_tiled).
bool skinny_tiles(const SkinnyArgs &a, const SkinnyPlan &plan);
hipError_t launch_skinny(const SkinnyArgs &a, const SkinnyPlan &plan, float *partials, hipStream_t stream);
bool skinny_fuses_norm(const SkinnyArgs &a, const SkinnyPlan &plan);
SkinnyPlan skinny_plan_dual(int T, int N, int K);
size_t skinny_partial_bytes_dual(int T, int N, const SkinnyPlan &p);

// ------------------------------------------------------- prefill product
// out[r, n] = epi( Σ_k X[r, k] · W[n, k] ), any row count, N % 8 == 0, K % 64 == 0.
// epi: EPI_BF16, EPI_GATE (aux = M), EPI_RESID (out = bf16(out + acc), in
// place), EPI_F32 or EPI_SOFTPLUS (out is then a float array; EPI_SOFTPLUS
// reads its fp32 bias [N] through aux), EPI_SWIGLU (out = bf16(SiLU(X W^T) ·
// (X aux^T)): W the gate and aux the up weights, both [N, K]; the hidden
// activation of a SwiGLU MLP in one pass).  ksplit > 1
// (EPI_F32 only, K % (64·ksplit) == 0): slice s of K writes its partial sums
// to out + s·rows·N.
hipError_t launch_gemm(const bf16_t *X, const bf16_t *W, int rows, int N, int K, Epilogue epi, bf16_t *out,
                       const bf16_t *aux, hipStream_t stream, int ksplit = 1);

// ------------------------------------------------------------- RMSNorm
// out_hi + out_lo = h[r, :] / sqrt(mean(h[r, :]^2) + eps) * g, d % 8 == 0
// (out_lo may be null: plain bf16 output).
hipError_t launch_rmsnorm(const bf16_t *h, const bf16_t *g, int rows, int d, float eps, bf16_t *out_hi,
                          bf16_t *out_lo, hipStream_t stream);

// ------------------------------------------------- YOCO-style prefill
// The self-decoder over B·T prompt rows (sambay_prefill's first part): the
// caches and states written, h and M of position T-1 gathered into h_out
// ([B, d_model]) and M_out ([B, d_inner]; the layout's m_last when null),
// and lens ([B] int32 in the workspace) set to T for the cross-decoder step
// that follows.
struct SelfDecoderArgs {
    const bf16_t *x = nullptr;          // [B, T, d_model]
    const sb_self_layer *layers = nullptr;
    int n = 0;
    int B = 0, T = 0, d_model = 0, d_inner = 0, d_state = 0, dt_rank = 0, d_conv = 0, d_ff = 0;
    int Hq = 0, Hkv = 0, L = 0, window = 0;
    float scale = 0.f, eps = 0.f;
    void *kcache = nullptr, *vcache = nullptr;
    bf16_t *h_out = nullptr, *M_out = nullptr;
    bool last_kv_only = false;          // a last SB_SELF_ATTN layer computes only its cache rows
};
struct SelfDecoderLayout {
    bf16_t *h, *xn, *M;
    int32_t *lens;
    bf16_t *m_last;                      // [B, d_inner]: M at position T-1 when the caller keeps none
    void *scratch;                       // shared by the attention, MLP and SSM layers in turn
    bf16_t *q, *k, *v, *o, *hid;         // views into scratch
    void *attn_ws;
    size_t bytes;
};
// base == nullptr: sizes only (bytes).
SelfDecoderLayout self_decoder_layout(void *base, int64_t B, int64_t T, int64_t d_model, int64_t d_inner,
                                      int64_t d_state, int64_t dt_rank, int64_t d_ff, int64_t Hq, int64_t Hkv);
hipError_t launch_self_decoder(const SelfDecoderArgs &a, const SelfDecoderLayout &L, hipStream_t stream);

// ------------------------------------------------------------- fp32 GMU
hipError_t launch_gmu_f32(const float *M, const float *X, const float *W1, const float *W2, float *Y, float *H,
                          int64_t rows, int64_t d_model, int64_t d_inner, hipStream_t stream);

}  // namespace sambay
