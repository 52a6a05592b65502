/*
 * sambay.h — C ABI of the SambaY cross-decoder decode-path library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (web pages about "Decoder-Hybrid-Decoder Architecture for
 * Efficient Reasoning with Long Generation"; the Paper-Notes reading-notes
 * page is cited as [Notes], the authors' abstract as [Abstract]):
 *   - the cross-decoder, the second half of the layers, alternates
 *     cross-attention layers over the single KV cache written once by the
 *     self-decoder's final full-attention layer, and Gated Memory Units that
 *     reuse the memory readout M of the self-decoder's last SSM layer
 *     ([Notes] section 整体框架);
 *   - GMU: Y = (M ⊙ SiLU(X W1^T)) W2, SiLU(z) = z·sigmoid(z)
 *     ([Notes] section 关键设计);
 *   - at decode time a cross-attention layer reads the whole cache, O(d_kv·N)
 *     bytes, while a GMU reads state whose size does not depend on N
 *     ([Notes] sections 现有痛点 and 关键设计);
 *   - no positional encoding is applied ([Notes] section 关键发现, [Abstract]).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller, dense and
 *     row-major, with a base address aligned to 16 bytes.  The library never
 *     retains a pointer after the call returns.
 *   - `workspace` is caller-owned device memory of at least the size the
 *     matching *_workspace_bytes() query returns, aligned to 256 bytes; its
 *     contents on entry are irrelevant and are clobbered.
 *   - Calls only enqueue kernels on `stream` (0 = the null stream).  They never
 *     allocate, free or synchronise.  Results are ready when `stream` is.
 *   - All arguments are validated before anything is enqueued: on any
 *     non-SB_OK status nothing was launched and sb_last_error() describes the
 *     problem.  A zero batch (rows == 0, B == 0) is a successful no-op.
 *   - Device faults inside a kernel are asynchronous: they surface at the
 *     caller's next synchronisation on the stream, not as a status here.
 *   - bf16 values are IEEE binary32 values truncated to their top 16 bits
 *     (bfloat16); every conversion to bf16 rounds to nearest, ties to even.
 *   - Entry points may be called from several host threads; sb_last_error()
 *     is per thread.  Calls that overlap on one device share nothing.
 */
#ifndef SAMBAY_H
#define SAMBAY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SB_OK = 0,
    SB_EINVAL = 1,        /* null pointer, negative or inconsistent size, misaligned or aliased buffer */
    SB_EUNSUPPORTED = 2,  /* a valid request outside what the kernels implement (see each call) */
    SB_EWORKSPACE = 3,    /* workspace null or smaller than the matching query returns */
    SB_EHIP = 4           /* the HIP runtime reported an error while enqueuing */
} sb_status;

typedef enum { SB_F32 = 0, SB_BF16 = 1 } sb_dtype;

typedef enum { SB_LAYER_XATTN = 0, SB_LAYER_GMU = 1 } sb_layer_kind;

/* One cross-decoder layer.  kind SB_LAYER_XATTN: w_a = Wq, w_b = Wo, both
 * [d_model, d_model] bf16 (q = h Wq^T, branch = o Wo^T).  kind SB_LAYER_GMU:
 * w_a = W1 [d_inner, d_model], w_b = W2 [d_model, d_inner], bf16. */
typedef struct {
    int32_t kind;       /* an sb_layer_kind value */
    const void *w_a;
    const void *w_b;
} sb_layer;

/* Text describing the last non-SB_OK status returned on this thread ("" if none). */
const char *sb_last_error(void);

/* Library version string: "sambay-mi355x <version> (gfx950) sources <hash>", where <hash> is the
 * first 16 hex digits of the SHA-256 over the kernel and header sources the library was built from
 * (attention_decoding_amd/build.py, source_hash()).  Static storage; never null. */
const char *sb_version(void);

/* ------------------------------------------------------------------ GMU --
 * Gated Memory Unit, [Notes] section 关键设计:
 *   Y[rows, d_model] = (M[rows, d_inner] ⊙ SiLU(X[rows, d_model] · W1^T)) · W2^T
 * with W1 [d_inner, d_model] and W2 [d_model, d_inner] (linear-layer layout:
 * the page's "· W2" with W2 stored transposed).  rows = batch·tokens for
 * prefill, or batch for one decode step (one new token per sequence).  M is
 * the memory readout of the earlier token-mixing layer, one row per token.
 * All five tensors share `dt`:
 *   SB_BF16: products accumulate in fp32; the gated hidden H = M ⊙ SiLU(·)
 *            is rounded to bf16 before the second product; Y is stored as
 *            bf16.
 *   SB_F32 : everything in fp32.
 * Y must not overlap any input.  Errors: SB_EINVAL (null pointer, negative
 * size, d_model or d_inner == 0 with rows > 0, overlap, misalignment),
 * SB_EUNSUPPORTED (bf16 with d_model or d_inner not a multiple of 64),
 * SB_EWORKSPACE, SB_EHIP. */
size_t gmu_workspace_bytes(int64_t rows, int64_t d_model, int64_t d_inner, sb_dtype dt);
sb_status gmu_forward(const void *M, const void *X, const void *W1, const void *W2, void *Y, int64_t rows,
                      int64_t d_model, int64_t d_inner, sb_dtype dt, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* ------------------------------------------------------ cross-attention --
 * Decode-time attention of one new token per sequence over the single shared
 * KV cache ([Notes] sections 整体框架 and 现有痛点), no positional encoding:
 *   out[b, h, :] = Σ_j softmax_j(scale · q[b, h, :] · K[b, g, j, :]) · V[b, g, j, :]
 * over all L cached positions j, with g = h / (Hq / Hkv) (grouped-query
 * heads, contiguous groups).  q, out: [B, Hq, D]; kcache, vcache: [B, Hkv, L, D];
 * all bf16; logits, softmax and the weighted sum run in fp32 (q is scaled and
 * split into two bf16 parts so that q·k keeps ~16 significant bits).
 * Computed as split-K flash decoding: the L positions are cut into chunks whose
 * (max, sum, weighted sum) partials are merged by log-sum-exp, an exact
 * rewriting of the softmax.
 * Errors: SB_EINVAL (null pointer, negative size, L == 0 with B > 0,
 * Hq % Hkv != 0, out overlapping an input, misalignment), SB_EUNSUPPORTED
 * (D != 128, Hq / Hkv > 16, L >= 2^31), SB_EWORKSPACE, SB_EHIP. */
size_t xattn_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L);
sb_status xattn_decode(const void *q, const void *kcache, const void *vcache, void *out, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t D, int64_t L, float scale, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* xattn_decode without a workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same computation, kernels
 * and results as xattn_decode, with the split partials kept in a file-scope device array of the
 * library (16 MiB per GPU, allocated when the library is loaded, held until the process ends).  The
 * partials take xattn_workspace_bytes(B, Hq, Hkv, D, L) bytes; a larger request returns
 * SB_EWORKSPACE before anything is enqueued (e.g. B = 32, 24q/8kv heads, any L: 3.2 MB).  Every call
 * on one GPU uses that GPU's one array, which keeps the last call's contents: calls that overlap on
 * one GPU (other streams, other host threads) race and must be ordered by the caller.  Allocates
 * and frees nothing; errors as xattn_decode. */
sb_status xattn_decode_noalloc(const void *q, const void *kcache, const void *vcache, void *out, int64_t B,
                               int64_t Hq, int64_t Hkv, int64_t D, int64_t L, float scale, hipStream_t stream);

/* ---------------------------------------------------- cross-decoder step --
 * One decode step of the cross-decoder ([Notes] section 整体框架): for each
 * layer in array order, a residual branch on the bf16 stream h [B, d_model]:
 *   SB_LAYER_XATTN: q = h Wq^T (fp32, not rounded), o = attention of q over
 *                   the shared kcache/vcache [B, Hkv, L, D] (as xattn_decode;
 *                   o feeds Wo as a bf16 hi + lo pair), h = bf16(h + o Wo^T);
 *   SB_LAYER_GMU:   h = bf16(h + GMU(M, h, W1, W2)) with the one memory
 *                   readout M [B, d_inner] shared by every GMU layer; H
 *                   feeds W2 as a bf16 hi + lo pair (~16 significant bits).
 * h is updated in place.  Requires Hq·D == d_model.  All tensors bf16.
 * Errors: as gmu_forward and xattn_decode, plus SB_EINVAL for a null layer
 * array with n_layers > 0, a null layer weight, an unknown kind, or
 * Hq·D != d_model. */
size_t crossdecoder_workspace_bytes(int64_t B, int64_t d_model, int64_t d_inner, int64_t Hq, int64_t Hkv, int64_t D,
                                    int64_t L);
sb_status crossdecoder_step(void *h, const void *M, const void *kcache, const void *vcache, const sb_layer *layers,
                            int32_t n_layers, int64_t B, int64_t d_model, int64_t d_inner, int64_t Hq, int64_t Hkv,
                            int64_t D, int64_t L, float scale, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* ------------------------------------------------------ ragged batches --
 * xattn_decode for a serving batch whose sequences are at different lengths.
 * kcache/vcache [B, Hkv, L, D] have room for L positions per (sequence, KV
 * head); sequence b attends to its first lens[b] positions only (lens: B
 * int32 in device memory, 4-byte aligned, read by the kernels; values are
 * clamped to [0, L], and a sequence with lens[b] == 0 gets a zero output: its
 * softmax has no terms).  Positions at or past lens[b] are never read, so
 * they may hold anything.  Same workspace as xattn_decode.  The pages define
 * only the full-cache case; this is its plain per-sequence reading.
 * Errors: as xattn_decode, plus SB_EINVAL for a null or misaligned lens with
 * B > 0. */
sb_status xattn_decode_varlen(const void *q, const void *kcache, const void *vcache, const int32_t *lens, void *out,
                              int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L, float scale,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------ differential attention --
 * Decode-time Differential Attention over the shared cache.  The pages name
 * the method for their largest model and note that its serving
 * implementation makes four plain attention passes ([Notes] section
 * 局限性 / 可改进方向) but do not define it; this is the published definition
 * (Differential Transformer, section 2.1) read for one query per sequence:
 * every D-wide query row q [B, Hq, D] and cached key row [B, Hkv, L, D] is two
 * halves of width D/2, (q1 | q2) and (k1 | k2); value rows keep all D; for
 * query head h (KV head h / (Hq / Hkv)):
 *   a1 = softmax_j(scale · q1·k1_j),  a2 = softmax_j(scale · q2·k2_j)
 *   o  = Σ_j a1_j v_j − lambda · Σ_j a2_j v_j
 *   out[b, h] = (1 − lambda_init) · o / sqrt(mean(o²) + eps) · gamma
 * gamma [D] bf16 (one gain for every head) or NULL for all ones.  lens as in
 * xattn_decode_varlen (NULL: all L positions); a sequence with no position
 * gets a zero output.  Callers usually pass scale = 1/sqrt(D/2).  Both maps
 * are computed in one pass over the cache (it is read once).  All tensors
 * bf16; out [B, Hq, D] must not overlap any input.
 * Errors: as xattn_decode_varlen (lens may be NULL here), plus SB_EINVAL for
 * a non-finite lambda or lambda_init, eps < 0 or non-finite, or a misaligned
 * gamma, and SB_EUNSUPPORTED for 2·(Hq/Hkv) > 16. */
size_t diffattn_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L);
sb_status diffattn_decode(const void *q, const void *kcache, const void *vcache, const int32_t *lens,
                          const void *gamma, void *out, int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L,
                          float scale, float lambda, float lambda_init, float eps, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------- self-decoder attention step --
 * One decode step of a self-decoder attention layer, the producer side of
 * the caches ([Notes] section 整体框架: the final full-attention layer writes
 * the one KV cache that every cross-attention layer reads; section 消融实验:
 * the other attention layers attend over a 256-position sliding window).
 * Sequence b's new token is at position p = pos[b] (pos: B int32 in device
 * memory, 4-byte aligned).  First its key and value rows k_new, v_new
 * [B, Hkv, D] are stored into kcache/vcache [B, Hkv, L, D]:
 *   window == 0: at position p (the cache has room for L positions);
 *   window  > 0: in ring slot p mod window (the cache has L == window slots,
 *                token t living in slot t mod window);
 * then q [B, Hq, D] attends, as xattn_decode, over the visible positions:
 * 0 .. p (window 0) or the min(p + 1, window) slots holding the window most
 * recent tokens.  No positional encoding, so the ring order is irrelevant.
 * p < 0 marks an inactive sequence: nothing stored, zero output.  With
 * window 0 a position p >= L has no slot: nothing is stored and all L
 * positions are visible (the device clamps; the host cannot check device
 * values).  kcache/vcache are updated in place; out [B, Hq, D]; all bf16.
 * Errors: as xattn_decode_varlen, plus SB_EINVAL for window < 0, window > 0
 * with L != window, a null or misaligned pos, and overlaps between the cache,
 * out and the other arguments. */
size_t selfattn_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L);
sb_status selfattn_decode(const void *q, const void *k_new, const void *v_new, void *kcache, void *vcache,
                          const int32_t *pos, void *out, int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L,
                          int64_t window, float scale, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------- prefill attention --
 * Attention of the self-decoder's layers over the prompt during a YOCO-style
 * prefill, which keeps pre-filling linear ([Notes] sections 领域现状 and
 * 现有痛点; the sliding window of section 消融实验): q [B, T, Hq, D], k, v
 * [B, T, Hkv, D] (token-major, as the projections write them), out
 * [B, T, Hq, D]; query i of head h attends to keys j of KV head
 * h / (Hq / Hkv) with j <= i and, when window > 0, j > i - window:
 *   out[b, i, h] = Σ_j softmax_j(scale · q[b, i, h]·k[b, j, g]) v[b, j, g].
 * window == 0 (or >= T) is plain causal attention.  No positional encoding.
 * All bf16; fp32 accumulation.  The workspace holds V transposed.
 * Errors: SB_EINVAL for null or misaligned pointers, Hq % Hkv != 0, a
 * non-finite scale, out or the workspace overlapping an input;
 * SB_EUNSUPPORTED for D != 128 or B, Hq > 65535; SB_EWORKSPACE.  B == 0 or
 * T == 0 is a no-op. */
size_t attn_prefill_workspace_bytes(int64_t B, int64_t T, int64_t Hkv, int64_t D);
sb_status attn_prefill(const void *q, const void *k, const void *v, void *out, int64_t B, int64_t T, int64_t Hq,
                       int64_t Hkv, int64_t D, int64_t window, float scale, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* ------------------------------------------------- SSM decode step (M) --
 * One decode step of the self-decoder's SSM layer, whose token-mixing output
 * M is the memory that every GMU layer reuses ([Notes] sections 关键设计 and
 * 整体框架: the GMU gates M of the last SSM layer, which keeps a state of
 * constant size at decode time; the SSM is Mamba with per-channel decay,
 * section 消融实验).  The pages do not spell the layer out; this is the
 * published Mamba layer, for B sequences with input x [B, d_model]:
 *   [xi | z] = x W_in^T                  W_in  [2·d_inner, d_model], bf16
 *   u  = SiLU(conv_b + Σ_k conv_w[:, k] · window[k]),   window = the d_conv-1
 *        stored inputs (oldest first) then xi; the stored window shifts by one
 *   [δ | Bv | Cv] = u W_x^T              W_x   [dt_rank + 2·d_state, d_inner], bf16
 *   Δ  = softplus(δ W_dt^T + dt_bias)    W_dt  [d_inner, dt_rank], bf16
 *   s  = exp(Δ·A) ⊙ s + Δ·Bv·u,  A = -exp(a_log)   (per channel c and state n)
 *   M  = Σ_n Cv[n] · s[:, n] + d_skip ⊙ u           -> M_out [B, d_inner], bf16
 *   y  = (M ⊙ SiLU(z)) W_out^T           W_out [d_model, d_inner], bf16
 *                                                   -> y_out [B, d_model], bf16
 * conv_w [d_inner, d_conv], conv_b, dt_bias, d_skip [d_inner] and a_log
 * [d_inner, d_state] are fp32.  conv_state [B, d_inner, d_conv-1] and
 * ssm_state [B, d_inner, d_state] are fp32 and updated in place (conv_state
 * may be NULL when d_conv == 1: there is no stored input).  u and the
 * gated readout feed their products as bf16 hi + lo pairs; everything else
 * accumulates in fp32.  Supported: d_model, d_inner multiples of 64; d_state
 * in {8, 16, 32, 64}; dt_rank a multiple of 8, at most 256; d_conv <= 8.
 * Errors: SB_EINVAL for null pointers or weights, misaligned pointers, a
 * zero dimension, overlaps between an output (states, M, y) and anything
 * else; SB_EUNSUPPORTED for other shapes; SB_EWORKSPACE. */
typedef struct {
    const void *w_in;     /* [2·d_inner, d_model] bf16: rows 0 .. d_inner-1 the x branch, then z */
    const float *conv_w;  /* [d_inner, d_conv] fp32, tap d_conv-1 multiplies the newest input */
    const float *conv_b;  /* [d_inner] fp32 */
    const void *w_x;      /* [dt_rank + 2·d_state, d_inner] bf16: rows δ | B | C */
    const void *w_dt;     /* [d_inner, dt_rank] bf16 */
    const float *dt_bias; /* [d_inner] fp32 */
    const float *a_log;   /* [d_inner, d_state] fp32 */
    const float *d_skip;  /* [d_inner] fp32 */
    const void *w_out;    /* [d_model, d_inner] bf16 */
} sb_mamba_weights;
size_t mamba_workspace_bytes(int64_t B, int64_t d_model, int64_t d_inner, int64_t d_state, int64_t dt_rank,
                             int64_t d_conv);
sb_status mamba_decode_step(const void *x, const sb_mamba_weights *w, float *conv_state, float *ssm_state,
                            void *M_out, void *y_out, int64_t B, int64_t d_model, int64_t d_inner, int64_t d_state,
                            int64_t dt_rank, int64_t d_conv, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* --------------------------------------------- SSM layer over the prompt --
 * The same layer as mamba_decode_step over T prompt tokens in one call (the
 * self-decoder's SSM layers in a YOCO-style prefill, which stays linear in T,
 * [Notes] sections 领域现状 and 现有痛点): equal, up to rounding, to T
 * successive mamba_decode_step calls on x[:, 0], ..., x[:, T-1] starting from
 * the given states.  x [B, T, d_model]; M_out [B, T, d_inner] and y_out
 * [B, T, d_model] for every token; conv_state and ssm_state in and out.  The
 * projections are MFMA GEMMs over the B·T rows with bf16 operands (xz, u,
 * [δ | B | C] and the gated readout are stored bf16; the step projection
 * and the scan are fp32); the convolution and the selective scan run over
 * the sequence.  Additionally requires dt_rank % 64 == 0.
 * Errors: as mamba_decode_step, plus SB_EUNSUPPORTED for T > 65535 or
 * B·T >= 2^31.  B == 0 or T == 0 is a no-op. */
size_t mamba_prefill_workspace_bytes(int64_t B, int64_t T, int64_t d_model, int64_t d_inner, int64_t d_state,
                                     int64_t dt_rank, int64_t d_conv);
sb_status mamba_prefill(const void *x, const sb_mamba_weights *w, float *conv_state, float *ssm_state, void *M_out,
                        void *y_out, int64_t B, int64_t T, int64_t d_model, int64_t d_inner, int64_t d_state,
                        int64_t dt_rank, int64_t d_conv, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------- complete cross-decoder layer --
 * The pages define the GMU and the shared-cache cross-attention but not the
 * rest of a layer; this step takes the plain pre-norm Transformer reading.
 * For each layer, with RMSNorm(x; g) = x / sqrt(mean(x^2) + eps) * g:
 *   x = RMSNorm(h; norm1)            (x = h when norm1 is NULL)
 *   SB_LAYER_XATTN: q = x Wq^T, o = attention over the first lens[b] cached
 *                   positions (all L when lens is NULL), h = bf16(h + o Wo^T)
 *   SB_LAYER_GMU:   h = bf16(h + GMU(M, x, W1, W2))
 *   when w_gate is not NULL (a SwiGLU MLP):
 *     x = RMSNorm(h; norm2)          (x = h when norm2 is NULL)
 *     h = bf16(h + (SiLU(x Wg^T) ⊙ (x Wu^T)) Wd^T)
 * The normalised x, the attention output, the GMU hidden and the SwiGLU
 * product feed their next product as bf16 hi + lo pairs; everything else
 * accumulates in fp32.  With every norm1, norm2, w_gate NULL and lens NULL
 * this is crossdecoder_step.  Gains norm1, norm2 [d_model]; w_gate, w_up
 * [d_ff, d_model]; w_down [d_model, d_ff]; all bf16, 16-byte aligned.
 * d_ff may be 0 when no layer has an MLP.  h is updated in place.
 * Errors: as crossdecoder_step and xattn_decode_varlen, plus SB_EINVAL for
 * an MLP with a missing weight or d_ff == 0, a negative or non-finite eps,
 * and SB_EUNSUPPORTED for d_ff not a multiple of 64. */
typedef struct {
    int32_t kind;          /* an sb_layer_kind value */
    const void *w_a;       /* as sb_layer */
    const void *w_b;
    const void *norm1;     /* RMSNorm gain before the mixer, or NULL */
    const void *norm2;     /* RMSNorm gain before the MLP, or NULL */
    const void *w_gate;    /* SwiGLU MLP weights, or all NULL: no MLP */
    const void *w_up;
    const void *w_down;
} sb_layer_ex;

size_t crossdecoder_ex_workspace_bytes(int64_t B, int64_t d_model, int64_t d_inner, int64_t d_ff, int64_t Hq,
                                       int64_t Hkv, int64_t D, int64_t L);
sb_status crossdecoder_step_ex(void *h, const void *M, const void *kcache, const void *vcache, const int32_t *lens,
                               const sb_layer_ex *layers, int32_t n_layers, int64_t B, int64_t d_model,
                               int64_t d_inner, int64_t d_ff, int64_t Hq, int64_t Hkv, int64_t D, int64_t L,
                               float scale, float eps, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------ YOCO-style prefill --
 * The SambaY prefill ([Notes] section 整体框架: only the self-decoder runs
 * over the prompt, so pre-filling stays linear; [Summary] key claims): the
 * self-decoder over the T prompt tokens of B sequences, its final
 * full-attention layer writing the shared KV cache once, then the
 * cross-decoder on the last prompt token only.  The self-decoder is Samba
 * (SSM layers alternating with sliding-window attention layers) followed by
 * one full-attention layer; no positional encoding ([Summary] abstract).
 * Each self-decoder layer takes the same plain pre-norm reading as the
 * complete cross-decoder layer:
 *   x = RMSNorm(h; norm1)                      (x = h when norm1 is NULL)
 *   SB_SELF_MAMBA: h = bf16(h + y), (M, y) = mamba_prefill(x) with the
 *                  layer's states (in and out); M is kept for the GMUs
 *   SB_SELF_SWA:   q, k, v = x Wq^T, x Wk^T, x Wv^T; o = attn_prefill(q, k, v,
 *                  window); h = bf16(h + o Wo^T); the last min(T, window)
 *                  positions p of k, v go to ring slot p % window of
 *                  kring / vring [B, Hkv, window, D]
 *   SB_SELF_ATTN:  the same with plain causal attention; k, v of positions
 *                  0 .. T-1 go to the shared cache kcache / vcache
 *                  [B, Hkv, L, D] (the cache the cross-decoder reads)
 *   when w_gate is not NULL: x = RMSNorm(h; norm2);
 *                  h = bf16(h + (SiLU(x Wg^T) ⊙ (x Wu^T)) Wd^T)
 * Then h_last = h at position T-1 and M_last = M (of the last SSM layer) at
 * position T-1 run through crossdecoder_step_ex(cross_layers) with every
 * sequence's cache length T; h_out [B, d_model] receives the result and
 * M_out [B, d_inner] (nullable) receives M_last, the memory the GMUs used.
 * Prefill activations (x, q, k, v, o, M, the MLP hidden) are bf16 with fp32
 * accumulation; the residual stream h is bf16.  The prompt starts at
 * position 0 (the caches are written from there); the SSM states start from
 * the values given (zero for a fresh prompt).
 * Shapes: x [B, T, d_model] bf16; Wq, Wo [d_model, d_model] (Hq·D ==
 * d_model), Wk, Wv [Hkv·D, d_model]; MLP and norms as in sb_layer_ex; the
 * SSM layer as mamba_prefill.  Requires D == 128, Hq % Hkv == 0, d_model,
 * d_inner, d_ff, dt_rank multiples of 64, 1 <= T <= L, B, T <= 65535,
 * window >= 1 when an SB_SELF_SWA layer is present, at least one
 * SB_SELF_ATTN layer when a cross layer is SB_LAYER_XATTN and at least one
 * SB_SELF_MAMBA layer when a cross layer is SB_LAYER_GMU.
 * Errors: SB_EINVAL for null or misaligned pointers, unknown kinds, missing
 * weights or states, a non-finite scale or eps, h_out / M_out / the caches /
 * the workspace overlapping another argument; SB_EUNSUPPORTED for other
 * shapes; SB_EWORKSPACE.  B == 0 is a no-op. */
typedef enum { SB_SELF_MAMBA = 0, SB_SELF_SWA = 1, SB_SELF_ATTN = 2 } sb_self_kind;
typedef struct {
    int32_t kind;             /* an sb_self_kind value */
    sb_mamba_weights mamba;   /* SB_SELF_MAMBA */
    float *conv_state;        /* SB_SELF_MAMBA: [B, d_inner, d_conv-1] fp32, in and out (NULL when d_conv == 1) */
    float *ssm_state;         /* SB_SELF_MAMBA: [B, d_inner, d_state] fp32, in and out */
    const void *wq, *wk, *wv, *wo;  /* SB_SELF_SWA, SB_SELF_ATTN */
    void *kring, *vring;      /* SB_SELF_SWA: [B, Hkv, window, D] bf16, written */
    const void *norm1;        /* RMSNorm gain before the mixer, or NULL */
    const void *norm2;        /* RMSNorm gain before the MLP, or NULL */
    const void *w_gate;       /* SwiGLU MLP weights, or all NULL: no MLP */
    const void *w_up;
    const void *w_down;
} sb_self_layer;

size_t sambay_prefill_workspace_bytes(int64_t B, int64_t T, int64_t d_model, int64_t d_inner, int64_t d_state,
                                      int64_t dt_rank, int64_t d_conv, int64_t d_ff, int64_t Hq, int64_t Hkv,
                                      int64_t D, int64_t L);
sb_status sambay_prefill(const void *x, void *h_out, void *M_out, const sb_self_layer *self_layers, int32_t n_self,
                         const sb_layer_ex *cross_layers, int32_t n_cross, void *kcache, void *vcache, int64_t B,
                         int64_t T, int64_t d_model, int64_t d_inner, int64_t d_state, int64_t dt_rank,
                         int64_t d_conv, int64_t d_ff, int64_t Hq, int64_t Hkv, int64_t D, int64_t L, int64_t window,
                         float scale, float eps, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------ whole-model decode --
 * One decode step of the whole model after a prefill: the new token of each
 * sequence (at position pos[b], the number of tokens before it) through the
 * self-decoder's layers, each one step of the layer sambay_prefill runs over
 * the prompt (same norms and MLPs):
 *   SB_SELF_MAMBA: mamba_decode_step on the normalised x (states in place),
 *                  h = bf16(h + y); M of the last SSM layer kept for the GMUs
 *   SB_SELF_SWA:   q, k, v projections of x; k, v stored in ring slot
 *                  pos % window; attention over the min(pos + 1, window)
 *                  ring entries; h = bf16(h + o Wo^T)
 *   SB_SELF_ATTN:  the same on the shared cache [B, Hkv, L, D] at position
 *                  pos (nothing stored when pos >= L, attention over L then),
 *                  attention over positions 0 .. pos
 * then crossdecoder_step_ex(cross_layers) with cache lengths min(pos + 1, L),
 * in place on h [B, d_model] (bf16: the new token's input row in, its last
 * hidden state out).  M_out [B, d_inner] (nullable) receives the last SSM
 * layer's M.  pos [B] int32 on the device; pos[b] < 0 marks an inactive
 * sequence for the attention layers (nothing stored, zero attention output)
 * — the other layers still run on its row.  The normalised x, the attention
 * output, the MLP hidden and the SSM step's inner rows feed their products
 * as bf16 hi + lo pairs.  At most one SB_SELF_ATTN layer (it writes the
 * shared cache).  Requirements and errors as sambay_prefill, without T; B
 * == 0 is a no-op. */
size_t sambay_decode_workspace_bytes(int64_t B, int64_t d_model, int64_t d_inner, int64_t d_state, int64_t dt_rank,
                                     int64_t d_conv, int64_t d_ff, int64_t Hq, int64_t Hkv, int64_t D, int64_t L,
                                     int64_t window);
sb_status sambay_decode_step(void *h, void *M_out, const sb_self_layer *self_layers, int32_t n_self,
                             const sb_layer_ex *cross_layers, int32_t n_cross, void *kcache, void *vcache,
                             const int32_t *pos, int64_t B, int64_t d_model, int64_t d_inner, int64_t d_state,
                             int64_t dt_rank, int64_t d_conv, int64_t d_ff, int64_t Hq, int64_t Hkv, int64_t D,
                             int64_t L, int64_t window, float scale, float eps, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------ benchmark instrumentation --
 * For measuring kernels inside the calls above (benchmarks and profiling
 * only; not meant for production loops).  While a kind's bit is enabled,
 * every launch of that kernel kind is bracketed by a pair of HIP events
 * recorded on the stream the kernel is launched on.  sb_timing_collect waits
 * for the recorded events of the kinds in `mask`, returns the number of
 * launches and their summed duration in milliseconds, and forgets them.
 * These two calls may synchronise on the recorded events.  Errors: SB_EHIP. */
typedef enum {
    SB_TIME_XATTN_SPLIT = 1,   /* split-K attention partial kernel */
    SB_TIME_XATTN_MERGE = 2,   /* log-sum-exp merge kernel */
    SB_TIME_SKINNY = 4,        /* decode weight-streaming products (GMU, Wq, Wo) */
    SB_TIME_GEMM = 8,          /* prefill MFMA GEMM */
    SB_TIME_GMU_F32 = 16,      /* fp32 GMU kernels */
    SB_TIME_PROBE = 32,        /* the two probes below */
    SB_TIME_DIFF_SPLIT = 64,   /* differential-attention partial kernel */
    SB_TIME_DIFF_MERGE = 128,  /* differential-attention merge + normalisation */
    SB_TIME_PREFILL = 256      /* prefill attention kernel */
} sb_timing_kind;

sb_status sb_timing_enable(uint32_t mask);
sb_status sb_timing_collect(uint32_t mask, int64_t *launches, double *total_ms);

/* Measured-ceiling probes (benchmarks only; not part of the method).
 * sb_probe_stream_read reads `bytes` bytes of device memory `data` (16-byte
 * aligned, bytes a multiple of 16) once with a plain grid-stride streaming
 * read that does nothing else: its rate is a practical HBM read ceiling for
 * this machine at that size.  sb_probe_mfma runs `iters` dependent steps of the
 * 32x32x16 bf16 MFMA on four independent accumulators per wave in 4096 waves
 * (sb_probe_mfma_flops(iters) floating-point operations): a practical dense
 * bf16 MFMA ceiling.  `sink` is 4 bytes of device memory the kernels may
 * write.  Errors: SB_EINVAL, SB_EHIP. */
sb_status sb_probe_stream_read(const void *data, size_t bytes, void *sink, hipStream_t stream);
sb_status sb_probe_mfma(int64_t iters, void *sink, hipStream_t stream);
double sb_probe_mfma_flops(int64_t iters);

#ifdef __cplusplus
}
#endif

#endif /* SAMBAY_H */
