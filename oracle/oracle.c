/*
 * Plain fp64 CPU oracle for the SambaY cross-decoder step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the tests, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no source, header, table or helper with the HIP library under
 * attention_decoding_amd/csrc, and it never touches a GPU.
 *
 * Every function below is the plain definition of what the method computes,
 * written out as loops in double precision, in the order the pages state it.
 * OpenMP splits only independent rows / (batch, head) pairs; no blocking,
 * fusion or reordering of any single result's arithmetic.
 *
 * Sources (all are web pages about the paper "Decoder-Hybrid-Decoder
 * Architecture for Efficient Reasoning with Long Generation"):
 *   [Notes]    Paper-Notes reading notes page with that title; sections
 *              "关键设计" (key designs: the GMU equation and the 3-D mixing
 *              lift), "整体框架" (overall framework: self-/cross-decoder,
 *              single KV cache, GMU/cross-attention alternation),
 *              "现有痛点" (pain point: O(d_kv·N) decode I/O of cross-attention),
 *              "关键发现" (findings: NoPE).
 *   [Abstract] the authors' abstract (chatpaper.ai and fugumt.com pages).
 *
 * Inputs may be fp64, fp32 or bf16 (raw 16-bit patterns); bf16 and fp32 are
 * widened exactly to fp64 before use.  Outputs are fp64.
 *
 * Byte-count mode: when a `bytes` array is passed, the call runs on one
 * thread and records every distinct element it reads from each input tensor
 * and writes to each output tensor; the sums (element count x nominal element
 * size) are returned per category.  This makes the I/O claim of [Notes]
 * "现有痛点"/"关键设计" (cross-attention decode reads O(d_kv·N); a GMU decode
 * step reads state whose size does not depend on N) checkable by counting.
 *
 * Parity pins (the tests under tests/test_oracle_*.py): GMU against the
 * brute-force 3-D mixing identity, closed forms and special cases; attention
 * against torch's fp64 scaled_dot_product_attention, a brute-force two-pass
 * softmax, closed forms and invariances; byte counts against the analytic
 * formulas.  See the test files for which mistake each pin catches.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F64 = 0, OR_F32 = 1, OR_BF16 = 2 };
enum { OR_CAT_KV = 0, OR_CAT_STATE_IN = 1, OR_CAT_STATE_OUT = 2, OR_CAT_WEIGHT = 3, OR_NCAT = 4 };

/* ------------------------------------------------------------------ loads */

static double widen(const void *p, int dt, int64_t i) {
    if (dt == OR_F64) return ((const double *)p)[i];
    if (dt == OR_F32) return (double)((const float *)p)[i];
    /* bf16: the 16 stored bits are the top half of an IEEE binary32. */
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int dt_bytes(int dt) { return dt == OR_F64 ? 8 : dt == OR_F32 ? 4 : 2; }

/* --------------------------------------------------------------- tracking */

typedef struct {
    unsigned char *seen;
    int64_t n;
    int elem_bytes;
    int cat;
} trk_tensor;

typedef struct {
    trk_tensor t[8];
} tracker;

static int trk_add(tracker *tr, int slot, int64_t n, int elem_bytes, int cat) {
    if (!tr) return 0;
    tr->t[slot].seen = (unsigned char *)calloc((size_t)(n > 0 ? n : 1), 1);
    tr->t[slot].n = n;
    tr->t[slot].elem_bytes = elem_bytes;
    tr->t[slot].cat = cat;
    return tr->t[slot].seen ? 0 : -2;
}

static inline void trk_mark(tracker *tr, int slot, int64_t i) {
    if (tr && tr->t[slot].seen) tr->t[slot].seen[i] = 1;
}

/* Adds the distinct-element byte sums into bytes[cat] and frees the maps. */
static void trk_finish(tracker *tr, int64_t *bytes) {
    if (!tr) return;
    for (int s = 0; s < 8; ++s) {
        if (!tr->t[s].seen) continue;
        int64_t c = 0;
        for (int64_t i = 0; i < tr->t[s].n; ++i) c += tr->t[s].seen[i];
        if (bytes) bytes[tr->t[s].cat] += c * tr->t[s].elem_bytes;
        free(tr->t[s].seen);
        tr->t[s].seen = NULL;
    }
}

/* ------------------------------------------------------------ bf16 round */

/* Round a double to the nearest bfloat16 value, ties to even, directly (no
 * detour through binary32, which could round twice).  bfloat16 keeps 8
 * significant bits and binary32's exponent range. */
double oracle_round_bf16(double x) {
    if (!isfinite(x) || x == 0.0) return x;
    int e;
    (void)frexp(x, &e);          /* |x| = m * 2^e with 0.5 <= m < 1 */
    int q = e - 8;               /* weight of the last kept bit */
    if (q < -133) q = -133;      /* below the normal range: fixed quantum 2^-133 */
    double r = nearbyint(ldexp(x, -q));  /* default mode: nearest, ties to even */
    double y = ldexp(r, q);
    if (fabs(y) > 3.3895313892515355e38) return copysign(INFINITY, x);
    return y;
}

/* ------------------------------------------------------------------ GMU */

/* One row of the Gated Memory Unit, [Notes] "关键设计":
 *   Y = (M ⊙ SiLU(X W1^T)) W2, where SiLU(z) = z·sigmoid(z) = z / (1 + e^{-z}).
 * Weights are stored as linear-layer matrices, W1 [d_inner, d_model] and
 * W2 [d_model, d_inner], so the output projection is H · W2^T (the same
 * linear map as the page's "H W2" with W2 stored transposed).  No bias. */
static void gmu_row(const void *M, int dt_m, const void *X, int dt_x, const void *W1, const void *W2,
                    int dt_w, double *y, int64_t r, int64_t d_model, int64_t d_inner, double *H,
                    tracker *tr, int sM, int sX, int sW1, int sW2) {
    for (int64_t k = 0; k < d_inner; ++k) {
        double z = 0.0;                                  /* z = X[r,:] · W1[k,:] */
        for (int64_t c = 0; c < d_model; ++c) {
            trk_mark(tr, sX, r * d_model + c);
            trk_mark(tr, sW1, k * d_model + c);
            z += widen(X, dt_x, r * d_model + c) * widen(W1, dt_w, k * d_model + c);
        }
        double g = z / (1.0 + exp(-z));                  /* SiLU(z) */
        trk_mark(tr, sM, r * d_inner + k);
        H[k] = widen(M, dt_m, r * d_inner + k) * g;      /* memory gated channel-wise */
    }
    for (int64_t o = 0; o < d_model; ++o) {
        double acc = 0.0;                                /* Y[r,o] = H · W2[o,:] */
        for (int64_t k = 0; k < d_inner; ++k) {
            trk_mark(tr, sW2, o * d_inner + k);
            acc += H[k] * widen(W2, dt_w, o * d_inner + k);
        }
        y[o] = acc;
    }
}

/* Y[rows, d_model] = (M[rows, d_inner] ⊙ SiLU(X[rows, d_model] W1^T)) W2^T.
 * dt_act is the dtype of M and X, dt_w of W1 and W2.
 * bytes (nullable, 4 entries, accumulated): distinct bytes per category. */
int oracle_gmu(const void *M, const void *X, int dt_act, const void *W1, const void *W2, int dt_w,
               double *Y, int64_t rows, int64_t d_model, int64_t d_inner, int64_t *bytes) {
    if (!M || !X || !W1 || !W2 || !Y || rows < 0 || d_model <= 0 || d_inner <= 0) return -1;
    tracker trs, *tr = NULL;
    if (bytes) {
        memset(&trs, 0, sizeof trs);
        tr = &trs;
        int ab = dt_bytes(dt_act), wb = dt_bytes(dt_w);
        if (trk_add(tr, 0, rows * d_inner, ab, OR_CAT_STATE_IN) || trk_add(tr, 1, rows * d_model, ab, OR_CAT_STATE_IN) ||
            trk_add(tr, 2, d_inner * d_model, wb, OR_CAT_WEIGHT) || trk_add(tr, 3, d_model * d_inner, wb, OR_CAT_WEIGHT) ||
            trk_add(tr, 4, rows * d_model, ab, OR_CAT_STATE_OUT)) {
            trk_finish(tr, NULL);
            return -2;
        }
    }
    int fail = 0;
#pragma omp parallel if (!tr)
    {
        double *H = (double *)malloc((size_t)d_inner * sizeof(double));
        if (!H) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            if (!H) continue;
            gmu_row(M, dt_act, X, dt_act, W1, W2, dt_w, Y + r * d_model, r, d_model, d_inner, H, tr, 0, 1, 2, 3);
            for (int64_t o = 0; o < d_model; ++o) trk_mark(tr, 4, r * d_model + o);
        }
        free(H);
    }
    trk_finish(tr, bytes);
    return fail ? -2 : 0;
}

/* ------------------------------------------------------ cross-attention */

/* Decode-time softmax attention of one query head over all L cached
 * positions of the single shared KV cache ([Notes] "整体框架": the
 * self-decoder's final full-attention layer writes one KV cache that every
 * cross-attention layer reuses).  No positional encoding is applied ([Notes]
 * "关键发现", [Abstract]: no explicit positional encoding).  Grouped-query
 * layout: query head h reads KV head h / (Hq / Hkv).
 *   s_j = scale · q·k_j,  m = max_j s_j,  w_j = e^{s_j - m},
 *   out = Σ_j w_j v_j / Σ_j w_j.                                        */
static void xattn_head(const void *q, int dt_q, int64_t q_off, const void *K, const void *V, int dt_kv,
                       int64_t kv_off, double *out, int64_t D, int64_t L, double scale, double *s,
                       tracker *tr, int sQ, int sK, int sV) {
    double m = -INFINITY;
    for (int64_t j = 0; j < L; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) {
            trk_mark(tr, sQ, q_off + d);
            trk_mark(tr, sK, kv_off + j * D + d);
            dot += widen(q, dt_q, q_off + d) * widen(K, dt_kv, kv_off + j * D + d);
        }
        s[j] = dot * scale;
        if (s[j] > m) m = s[j];
    }
    double den = 0.0;
    for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
    for (int64_t j = 0; j < L; ++j) {
        double w = exp(s[j] - m);
        den += w;
        for (int64_t d = 0; d < D; ++d) {
            trk_mark(tr, sV, kv_off + j * D + d);
            out[d] += w * widen(V, dt_kv, kv_off + j * D + d);
        }
    }
    for (int64_t d = 0; d < D; ++d) out[d] /= den;
}

static int xattn_args_ok(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L) {
    return B >= 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0 && D > 0 && L > 0;
}

/* out[B, Hq, D] = softmax(scale · q K^T) V with q [B, Hq, D], K, V [B, Hkv, L, D].
 * bytes (nullable, 4 entries, accumulated). */
int oracle_xattn(const void *q, int dt_q, const void *K, const void *V, int dt_kv, double *out, int64_t B,
                 int64_t Hq, int64_t Hkv, int64_t D, int64_t L, double scale, int64_t *bytes) {
    if (!q || !K || !V || !out || !xattn_args_ok(B, Hq, Hkv, D, L)) return -1;
    const int64_t G = Hq / Hkv;
    tracker trs, *tr = NULL;
    if (bytes) {
        memset(&trs, 0, sizeof trs);
        tr = &trs;
        int qb = dt_bytes(dt_q), kb = dt_bytes(dt_kv);
        if (trk_add(tr, 0, B * Hq * D, qb, OR_CAT_STATE_IN) || trk_add(tr, 1, B * Hkv * L * D, kb, OR_CAT_KV) ||
            trk_add(tr, 2, B * Hkv * L * D, kb, OR_CAT_KV) || trk_add(tr, 3, B * Hq * D, qb, OR_CAT_STATE_OUT)) {
            trk_finish(tr, NULL);
            return -2;
        }
    }
    int fail = 0;
#pragma omp parallel if (!tr)
    {
        double *s = (double *)malloc((size_t)L * sizeof(double));
        if (!s) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * Hq; ++bh) {
            if (!s) continue;
            int64_t b = bh / Hq, h = bh % Hq, g = h / G;
            xattn_head(q, dt_q, bh * D, K, V, dt_kv, (b * Hkv + g) * L * D, out + bh * D, D, L, scale, s, tr, 0, 1, 2);
            for (int64_t d = 0; d < D; ++d) trk_mark(tr, 3, bh * D + d);
        }
        free(s);
    }
    trk_finish(tr, bytes);
    return fail ? -2 : 0;
}

/* The same attention computed as S independent chunks of keys, each reduced
 * to (m_c, l_c, o_c) = (max s, Σ e^{s-m_c}, Σ e^{s-m_c} v), then merged:
 *   m = max_c m_c,  l = Σ_c l_c e^{m_c - m},  out = Σ_c o_c e^{m_c - m} / l.
 * This is an exact rewriting of the softmax (split-K flash decoding); the
 * pins check it against oracle_xattn.  Chunk c covers keys
 * [c·ceil(L/S), min(L, (c+1)·ceil(L/S))); empty chunks are skipped. */
int oracle_xattn_chunked(const void *q, int dt_q, const void *K, const void *V, int dt_kv, double *out,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L, double scale, int64_t S) {
    if (!q || !K || !V || !out || !xattn_args_ok(B, Hq, Hkv, D, L) || S <= 0) return -1;
    const int64_t G = Hq / Hkv, chunk = (L + S - 1) / S;
    int fail = 0;
#pragma omp parallel
    {
        double *mc = (double *)malloc((size_t)S * sizeof(double));
        double *lc = (double *)malloc((size_t)S * sizeof(double));
        double *oc = (double *)malloc((size_t)(S * D) * sizeof(double));
        double *sv = (double *)malloc((size_t)(chunk > 0 ? chunk : 1) * sizeof(double));
        int ok = mc && lc && oc && sv;
        if (!ok) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * Hq; ++bh) {
            if (!ok) continue;
            int64_t b = bh / Hq, h = bh % Hq, g = h / G;
            int64_t kv = (b * Hkv + g) * L * D;
            int64_t nc = 0;
            for (int64_t c = 0; c < S; ++c) {
                int64_t j0 = c * chunk, j1 = j0 + chunk < L ? j0 + chunk : L;
                if (j0 >= j1) continue;
                double m = -INFINITY;
                for (int64_t j = j0; j < j1; ++j) {
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d) dot += widen(q, dt_q, bh * D + d) * widen(K, dt_kv, kv + j * D + d);
                    sv[j - j0] = dot * scale;
                    if (sv[j - j0] > m) m = sv[j - j0];
                }
                double l = 0.0;
                for (int64_t d = 0; d < D; ++d) oc[nc * D + d] = 0.0;
                for (int64_t j = j0; j < j1; ++j) {
                    double w = exp(sv[j - j0] - m);
                    l += w;
                    for (int64_t d = 0; d < D; ++d) oc[nc * D + d] += w * widen(V, dt_kv, kv + j * D + d);
                }
                mc[nc] = m;
                lc[nc] = l;
                ++nc;
            }
            double M = -INFINITY;
            for (int64_t c = 0; c < nc; ++c) M = mc[c] > M ? mc[c] : M;
            double l = 0.0;
            for (int64_t c = 0; c < nc; ++c) l += lc[c] * exp(mc[c] - M);
            for (int64_t d = 0; d < D; ++d) {
                double acc = 0.0;
                for (int64_t c = 0; c < nc; ++c) acc += oc[c * D + d] * exp(mc[c] - M);
                out[bh * D + d] = acc / l;
            }
        }
        free(mc);
        free(lc);
        free(oc);
        free(sv);
    }
    return fail ? -2 : 0;
}

/* --------------------------------------------------------- cross-decoder */

/* One decode step of the cross-decoder ([Notes] "整体框架": the second half
 * of the layers alternates cross-attention over the single shared KV cache
 * and GMUs that reuse the memory readout M of the self-decoder's last SSM
 * layer).  Every layer is a residual branch:
 *   cross-attention layer (weights Wq, Wo, each [d_model, d_model]):
 *       q = h Wq^T (kept exact, viewed as [B, Hq, D]);  o = attention(q, K, V);
 *       h = h + o Wo^T
 *   GMU layer (weights W1 [d_inner, d_model], W2 [d_model, d_inner]):
 *       h = h + GMU(M, h, W1, W2)
 * When round_bf16 is set, h is rounded to bfloat16 after every residual add
 * (the bf16 residual stream); nothing else is rounded.
 * kinds[l]: 0 = cross-attention, 1 = GMU.  wa[l]/wb[l]: (Wq, Wo) or (W1, W2),
 * all of dtype dt_w.  h0, M of dtype dt_act; K, V of dtype dt_kv.
 * h_out [B, d_model] receives the final residual stream.
 * bytes (nullable, n_layers x 4 entries, accumulated) counts each layer's
 * distinct bytes with h and M counted at dt_act's size. */
int oracle_crossdecoder(const void *h0, const void *M, int dt_act, const void *K, const void *V, int dt_kv,
                        const int32_t *kinds, const void *const *wa, const void *const *wb, int dt_w, int32_t n_layers,
                        int64_t B, int64_t d_model, int64_t d_inner, int64_t Hq, int64_t Hkv, int64_t D, int64_t L,
                        double scale, int round_bf16, double *h_out, int64_t *bytes) {
    if (!h0 || !M || !K || !V || !kinds || !wa || !wb || !h_out || n_layers < 0 || B < 0 || d_model <= 0 ||
        d_inner <= 0 || !xattn_args_ok(B, Hq, Hkv, D, L) || Hq * D != d_model)
        return -1;
    const int64_t G = Hq / Hkv;
    const int ab = dt_bytes(dt_act), wbyt = dt_bytes(dt_w), kb = dt_bytes(dt_kv);
    double *h = (double *)malloc((size_t)(B * d_model) * sizeof(double));
    double *y = (double *)malloc((size_t)(B * d_model) * sizeof(double));
    double *qv = (double *)malloc((size_t)(B * d_model) * sizeof(double));
    double *o = (double *)malloc((size_t)(B * d_model) * sizeof(double));
    if (!h || !y || !qv || !o) {
        free(h); free(y); free(qv); free(o);
        return -2;
    }
    for (int64_t i = 0; i < B * d_model; ++i) h[i] = widen(h0, dt_act, i);
    int fail = 0;
    for (int32_t li = 0; li < n_layers && !fail; ++li) {
        if (!wa[li] || !wb[li] || (kinds[li] != 0 && kinds[li] != 1)) {
            fail = -1;
            break;
        }
        tracker trs, *tr = NULL;
        if (bytes) {
            memset(&trs, 0, sizeof trs);
            tr = &trs;
            int e = trk_add(tr, 0, B * d_model, ab, OR_CAT_STATE_IN) | trk_add(tr, 1, B * d_model, ab, OR_CAT_STATE_OUT);
            if (kinds[li] == 0)
                e |= trk_add(tr, 2, d_model * d_model, wbyt, OR_CAT_WEIGHT) |
                     trk_add(tr, 3, d_model * d_model, wbyt, OR_CAT_WEIGHT) |
                     trk_add(tr, 4, B * Hkv * L * D, kb, OR_CAT_KV) | trk_add(tr, 5, B * Hkv * L * D, kb, OR_CAT_KV);
            else
                e |= trk_add(tr, 2, d_inner * d_model, wbyt, OR_CAT_WEIGHT) |
                     trk_add(tr, 3, d_model * d_inner, wbyt, OR_CAT_WEIGHT) |
                     trk_add(tr, 4, B * d_inner, ab, OR_CAT_STATE_IN);
            if (e) {
                trk_finish(tr, NULL);
                fail = -2;
                break;
            }
        }
        if (kinds[li] == 0) {
            /* q = h Wq^T, exact */
#pragma omp parallel for schedule(static) if (!tr)
            for (int64_t i = 0; i < B * d_model; ++i) {
                int64_t b = i / d_model, n = i % d_model;
                double acc = 0.0;
                for (int64_t c = 0; c < d_model; ++c) {
                    trk_mark(tr, 0, b * d_model + c);
                    trk_mark(tr, 2, n * d_model + c);
                    acc += h[b * d_model + c] * widen(wa[li], dt_w, n * d_model + c);
                }
                qv[i] = acc;
            }
            /* o = attention(q) over the shared cache */
#pragma omp parallel if (!tr)
            {
                double *s = (double *)malloc((size_t)L * sizeof(double));
                if (!s) {
#pragma omp atomic write
                    fail = -2;
                }
#pragma omp for schedule(dynamic, 1)
                for (int64_t bh = 0; bh < B * Hq; ++bh) {
                    if (!s) continue;
                    int64_t b = bh / Hq, hh = bh % Hq, g = hh / G;
                    xattn_head(qv, OR_F64, bh * D, K, V, dt_kv, (b * Hkv + g) * L * D, o + bh * D, D, L, scale, s,
                               tr, 7, 4, 5);
                }
                free(s);
            }
            /* y = o Wo^T */
#pragma omp parallel for schedule(static) if (!tr)
            for (int64_t i = 0; i < B * d_model; ++i) {
                int64_t b = i / d_model, n = i % d_model;
                double acc = 0.0;
                for (int64_t c = 0; c < d_model; ++c) {
                    trk_mark(tr, 3, n * d_model + c);
                    acc += o[b * d_model + c] * widen(wb[li], dt_w, n * d_model + c);
                }
                y[i] = acc;
            }
        } else {
#pragma omp parallel if (!tr)
            {
                double *H = (double *)malloc((size_t)d_inner * sizeof(double));
                if (!H) {
#pragma omp atomic write
                    fail = -2;
                }
#pragma omp for schedule(static)
                for (int64_t r = 0; r < B; ++r) {
                    if (!H) continue;
                    gmu_row(M, dt_act, h, OR_F64, wa[li], wb[li], dt_w, y + r * d_model, r, d_model, d_inner, H, tr,
                            4, 0, 2, 3);
                }
                free(H);
            }
        }
        for (int64_t i = 0; i < B * d_model; ++i) {
            trk_mark(tr, 0, i);
            trk_mark(tr, 1, i);
            double v = h[i] + y[i];
            h[i] = round_bf16 ? oracle_round_bf16(v) : v;
        }
        trk_finish(tr, bytes ? bytes + (int64_t)li * OR_NCAT : NULL);
    }
    if (!fail) memcpy(h_out, h, (size_t)(B * d_model) * sizeof(double));
    free(h); free(y); free(qv); free(o);
    return fail;
}

/* ------------------------------------- ragged batch and the complete layer
 *
 * The pages define the GMU and the shared-cache cross-attention but not the
 * rest of a layer.  The complete cross-decoder layer below takes the plain
 * Transformer reading: a pre-normalised residual mixer (cross-attention or
 * GMU) followed by a pre-normalised residual SwiGLU MLP, RMSNorm as the norm.
 * A serving batch holds sequences at different lengths: the cache has room
 * for L positions per (sequence, KV head) and sequence b uses its first
 * lens[b] of them. */

/* Attention of a ragged batch.  K, V [B, Hkv, L, D] hold room for L
 * positions; sequence b attends to positions 0 .. lens[b]-1 (0 <= lens[b] <=
 * L).  lens[b] == 0 leaves the softmax without terms and is defined to give a
 * zero output. */
int oracle_xattn_varlen(const void *q, int dt_q, const void *K, const void *V, int dt_kv, const int32_t *lens,
                        double *out, int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L, double scale) {
    if (!q || !K || !V || !lens || !out || !xattn_args_ok(B, Hq, Hkv, D, L)) return -1;
    for (int64_t b = 0; b < B; ++b)
        if (lens[b] < 0 || lens[b] > L) return -1;
    const int64_t G = Hq / Hkv;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)L * sizeof(double));
        if (!s) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * Hq; ++bh) {
            if (!s) continue;
            int64_t b = bh / Hq, h = bh % Hq, g = h / G;
            if (lens[b] == 0) {
                for (int64_t d = 0; d < D; ++d) out[bh * D + d] = 0.0;
                continue;
            }
            xattn_head(q, dt_q, bh * D, K, V, dt_kv, (b * Hkv + g) * L * D, out + bh * D, D, lens[b], scale, s, NULL,
                       0, 0, 0);
        }
        free(s);
    }
    return fail ? -2 : 0;
}

/* RMSNorm of one row: y_i = x_i / sqrt(mean_j x_j^2 + eps) * g_i. */
static void rmsnorm_row(const double *x, const void *g, int dt_g, int64_t n, double eps, double *y) {
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
    const double r = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t i = 0; i < n; ++i) y[i] = x[i] * r * widen(g, dt_g, i);
}

/* SwiGLU MLP of one row: u_k = SiLU(x . Wg[k]) * (x . Wu[k]) for k < d_ff,
 * y_n = u . Wd[n] for n < d_model (Wg, Wu [d_ff, d_model], Wd [d_model, d_ff]). */
static void swiglu_row(const double *x, const void *Wg, const void *Wu, const void *Wd, int dt_w, int64_t d_model,
                       int64_t d_ff, double *u, double *y) {
    for (int64_t k = 0; k < d_ff; ++k) {
        double a = 0.0, b = 0.0;
        for (int64_t c = 0; c < d_model; ++c) {
            a += x[c] * widen(Wg, dt_w, k * d_model + c);
            b += x[c] * widen(Wu, dt_w, k * d_model + c);
        }
        u[k] = a / (1.0 + exp(-a)) * b;
    }
    for (int64_t n = 0; n < d_model; ++n) {
        double acc = 0.0;
        for (int64_t k = 0; k < d_ff; ++k) acc += u[k] * widen(Wd, dt_w, n * d_ff + k);
        y[n] = acc;
    }
}

/* Row-wise RMSNorm of x [rows, n] (any input dtype) with gain g [n]. */
int oracle_rmsnorm(const void *x, int dt_x, const void *g, int dt_g, int64_t rows, int64_t n, double eps,
                   double *out) {
    if (!x || !g || !out || rows < 0 || n <= 0 || !(eps >= 0.0)) return -1;
    double *xr = (double *)malloc((size_t)n * sizeof(double));
    if (!xr) return -2;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t i = 0; i < n; ++i) xr[i] = widen(x, dt_x, r * n + i);
        rmsnorm_row(xr, g, dt_g, n, eps, out + r * n);
    }
    free(xr);
    return 0;
}

/* Row-wise SwiGLU MLP of x [rows, d_model]. */
int oracle_swiglu(const void *x, int dt_x, const void *Wg, const void *Wu, const void *Wd, int dt_w, int64_t rows,
                  int64_t d_model, int64_t d_ff, double *out) {
    if (!x || !Wg || !Wu || !Wd || !out || rows < 0 || d_model <= 0 || d_ff <= 0) return -1;
    int fail = 0;
#pragma omp parallel
    {
        double *xr = (double *)malloc((size_t)d_model * sizeof(double));
        double *u = (double *)malloc((size_t)d_ff * sizeof(double));
        if (!xr || !u) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            if (!xr || !u) continue;
            for (int64_t i = 0; i < d_model; ++i) xr[i] = widen(x, dt_x, r * d_model + i);
            swiglu_row(xr, Wg, Wu, Wd, dt_w, d_model, d_ff, u, out + r * d_model);
        }
        free(xr);
        free(u);
    }
    return fail ? -2 : 0;
}

/* One decode step of the complete cross-decoder.  For each layer l, with
 * x = RMSNorm(h; norm1[l]) (x = h when norm1[l] is NULL):
 *   cross-attention: q = x Wq^T; o = ragged attention(q, K, V, lens); y = o Wo^T
 *   GMU:             y = GMU(M, x, W1, W2)
 *   h = h + y                                  (rounded to bf16 if round_bf16)
 * then, when wg[l] is not NULL, with x = RMSNorm(h; norm2[l]) (or h):
 *   h = h + SwiGLU(x; Wg, Wu, Wd)              (rounded to bf16 if round_bf16)
 * lens may be NULL (every sequence uses all L positions).  Norm gains and
 * weights share dtype dt_w. */
int oracle_crossdecoder_ex(const void *h0, const void *M, int dt_act, const void *K, const void *V, int dt_kv,
                           const int32_t *lens, const int32_t *kinds, const void *const *wa, const void *const *wb,
                           const void *const *norm1, const void *const *norm2, const void *const *wg,
                           const void *const *wu, const void *const *wd, int dt_w, int32_t n_layers, int64_t B,
                           int64_t d_model, int64_t d_inner, int64_t d_ff, int64_t Hq, int64_t Hkv, int64_t D,
                           int64_t L, double scale, double eps, int round_bf16, double *h_out) {
    if (!h0 || !M || !K || !V || !kinds || !wa || !wb || !norm1 || !norm2 || !wg || !wu || !wd || !h_out ||
        n_layers < 0 || B < 0 || d_model <= 0 || d_inner <= 0 || d_ff < 0 || !xattn_args_ok(B, Hq, Hkv, D, L) ||
        Hq * D != d_model || !(eps >= 0.0))
        return -1;
    if (lens)
        for (int64_t b = 0; b < B; ++b)
            if (lens[b] < 0 || lens[b] > L) return -1;
    const int64_t G = Hq / Hkv;
    const size_t nbd = (size_t)(B * d_model) * sizeof(double);
    double *h = (double *)malloc(nbd), *x = (double *)malloc(nbd), *y = (double *)malloc(nbd);
    double *qv = (double *)malloc(nbd), *o = (double *)malloc(nbd);
    if (!h || !x || !y || !qv || !o) {
        free(h); free(x); free(y); free(qv); free(o);
        return -2;
    }
    for (int64_t i = 0; i < B * d_model; ++i) h[i] = widen(h0, dt_act, i);
    int fail = 0;
    for (int32_t li = 0; li < n_layers && !fail; ++li) {
        if (!wa[li] || !wb[li] || (kinds[li] != 0 && kinds[li] != 1) || (wg[li] && (!wu[li] || !wd[li] || d_ff == 0))) {
            fail = -1;
            break;
        }
        for (int64_t r = 0; r < B; ++r) {
            if (norm1[li])
                rmsnorm_row(h + r * d_model, norm1[li], dt_w, d_model, eps, x + r * d_model);
            else
                memcpy(x + r * d_model, h + r * d_model, (size_t)d_model * sizeof(double));
        }
        if (kinds[li] == 0) {
#pragma omp parallel for schedule(static)
            for (int64_t i = 0; i < B * d_model; ++i) {
                int64_t b = i / d_model, n = i % d_model;
                double acc = 0.0;
                for (int64_t c = 0; c < d_model; ++c) acc += x[b * d_model + c] * widen(wa[li], dt_w, n * d_model + c);
                qv[i] = acc;
            }
#pragma omp parallel
            {
                double *s = (double *)malloc((size_t)L * sizeof(double));
                if (!s) {
#pragma omp atomic write
                    fail = -2;
                }
#pragma omp for schedule(dynamic, 1)
                for (int64_t bh = 0; bh < B * Hq; ++bh) {
                    if (!s) continue;
                    int64_t b = bh / Hq, hh = bh % Hq, g = hh / G;
                    int64_t Lb = lens ? lens[b] : L;
                    if (Lb == 0) {
                        for (int64_t d = 0; d < D; ++d) o[bh * D + d] = 0.0;
                        continue;
                    }
                    xattn_head(qv, OR_F64, bh * D, K, V, dt_kv, (b * Hkv + g) * L * D, o + bh * D, D, Lb, scale, s,
                               NULL, 0, 0, 0);
                }
                free(s);
            }
#pragma omp parallel for schedule(static)
            for (int64_t i = 0; i < B * d_model; ++i) {
                int64_t b = i / d_model, n = i % d_model;
                double acc = 0.0;
                for (int64_t c = 0; c < d_model; ++c) acc += o[b * d_model + c] * widen(wb[li], dt_w, n * d_model + c);
                y[i] = acc;
            }
        } else {
#pragma omp parallel
            {
                double *H = (double *)malloc((size_t)d_inner * sizeof(double));
                if (!H) {
#pragma omp atomic write
                    fail = -2;
                }
#pragma omp for schedule(static)
                for (int64_t r = 0; r < B; ++r) {
                    if (!H) continue;
                    gmu_row(M, dt_act, x, OR_F64, wa[li], wb[li], dt_w, y + r * d_model, r, d_model, d_inner, H, NULL,
                            0, 0, 0, 0);
                }
                free(H);
            }
        }
        for (int64_t i = 0; i < B * d_model; ++i) {
            double v = h[i] + y[i];
            h[i] = round_bf16 ? oracle_round_bf16(v) : v;
        }
        if (fail || !wg[li]) continue;
        for (int64_t r = 0; r < B; ++r) {
            if (norm2[li])
                rmsnorm_row(h + r * d_model, norm2[li], dt_w, d_model, eps, x + r * d_model);
            else
                memcpy(x + r * d_model, h + r * d_model, (size_t)d_model * sizeof(double));
        }
#pragma omp parallel
        {
            double *u = (double *)malloc((size_t)d_ff * sizeof(double));
            if (!u) {
#pragma omp atomic write
                fail = -2;
            }
#pragma omp for schedule(static)
            for (int64_t r = 0; r < B; ++r) {
                if (!u) continue;
                swiglu_row(x + r * d_model, wg[li], wu[li], wd[li], dt_w, d_model, d_ff, u, y + r * d_model);
            }
            free(u);
        }
        for (int64_t i = 0; i < B * d_model; ++i) {
            double v = h[i] + y[i];
            h[i] = round_bf16 ? oracle_round_bf16(v) : v;
        }
    }
    if (!fail) memcpy(h_out, h, nbd);
    free(h); free(x); free(y); free(qv); free(o);
    return fail;
}

/* ------------------------------------------------- differential attention
 *
 * The pages name Differential Attention as part of their largest model and
 * note that its serving implementation runs four plain attention passes
 * ([Notes] "局限性 / 可改进方向"), but do not define it.  The definition used
 * here is the published one (Differential Transformer, Ye et al. 2024,
 * section 2.1), read for decoding over the shared cache:
 *   each query head row q [D] and each cached key row k [D] are two halves
 *   of width d = D/2, (q1 | q2) and (k1 | k2); value rows v keep all D;
 *   a1 = softmax_j(scale · q1·k1_j),  a2 = softmax_j(scale · q2·k2_j),
 *   o = Σ_j a1_j v_j − λ Σ_j a2_j v_j                      (width D),
 *   out = (1 − λ_init) · o / sqrt(mean_c o_c² + eps) · γ   (per head).
 * λ and λ_init are inputs (the paper derives λ from learned vectors; that
 * reparametrisation lives with the weights).  γ is one D-wide gain shared by
 * all heads, or all ones when NULL.  A ragged batch (lens non-NULL) uses the
 * first lens[b] positions; a sequence with none gives a zero output. */

/* One attention map: softmax over positions j < n of scale · Σ_{c0<=c<c1}
 * q[c]·k_j[c], applied to the full D-wide value rows. */
static void diff_map(const void *q, int dt_q, int64_t q_off, const void *K, const void *V, int dt_kv,
                     int64_t kv_off, int64_t D, int64_t c0, int64_t c1, int64_t n, double scale, double *s,
                     double *o) {
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int64_t c = c0; c < c1; ++c)
            dot += widen(q, dt_q, q_off + c) * widen(K, dt_kv, kv_off + j * D + c);
        s[j] = dot * scale;
        if (s[j] > m) m = s[j];
    }
    double den = 0.0;
    for (int64_t c = 0; c < D; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double w = exp(s[j] - m);
        den += w;
        for (int64_t c = 0; c < D; ++c) o[c] += w * widen(V, dt_kv, kv_off + j * D + c);
    }
    for (int64_t c = 0; c < D; ++c) o[c] /= den;
}

/* out[B, Hq, D] from q [B, Hq, D], K, V [B, Hkv, L, D] (GQA: head h reads KV
 * head h / (Hq / Hkv)), lens [B] or NULL, gamma [D] or NULL. */
int oracle_diffattn(const void *q, int dt_q, const void *K, const void *V, int dt_kv, const int32_t *lens,
                    const void *gamma, int dt_g, double *out, int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                    int64_t L, double scale, double lambda, double lambda_init, double eps) {
    if (!q || !K || !V || !out || !xattn_args_ok(B, Hq, Hkv, D, L) || D % 2 != 0 || !(eps >= 0.0)) return -1;
    if (lens)
        for (int64_t b = 0; b < B; ++b)
            if (lens[b] < 0 || lens[b] > L) return -1;
    const int64_t G = Hq / Hkv, d = D / 2;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)L * sizeof(double));
        double *o1 = (double *)malloc((size_t)D * sizeof(double));
        double *o2 = (double *)malloc((size_t)D * sizeof(double));
        int ok = s && o1 && o2;
        if (!ok) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * Hq; ++bh) {
            if (!ok) continue;
            int64_t b = bh / Hq, h = bh % Hq, g = h / G;
            int64_t n = lens ? lens[b] : L, kv = (b * Hkv + g) * L * D;
            double *y = out + bh * D;
            if (n == 0) {
                for (int64_t c = 0; c < D; ++c) y[c] = 0.0;
                continue;
            }
            diff_map(q, dt_q, bh * D, K, V, dt_kv, kv, D, 0, d, n, scale, s, o1);
            diff_map(q, dt_q, bh * D, K, V, dt_kv, kv, D, d, D, n, scale, s, o2);
            double ss = 0.0;
            for (int64_t c = 0; c < D; ++c) {
                y[c] = o1[c] - lambda * o2[c];
                ss += y[c] * y[c];
            }
            const double r = (1.0 - lambda_init) / sqrt(ss / (double)D + eps);
            for (int64_t c = 0; c < D; ++c) y[c] *= r * (gamma ? widen(gamma, dt_g, c) : 1.0);
        }
        free(s);
        free(o1);
        free(o2);
    }
    return fail ? -2 : 0;
}

/* ----------------------------------------- self-decoder attention decode
 *
 * The producer side of the cache ([Notes] "整体框架": the self-decoder's
 * final full-attention layer writes the one KV cache that every
 * cross-attention layer reads; its other attention layers use a sliding
 * window, 256 positions in the model the pages favour, [Notes] "消融实验").
 * One decode step of such a layer for a batch: sequence b's new token sits
 * at position p = pos[b] (0-based; p < 0 marks an inactive sequence, which
 * writes nothing and gets a zero output).  Its key and value rows (k_new,
 * v_new [B, Hkv, D]) are stored, then its query attends:
 *   window == 0: the cache [B, Hkv, L, D] holds positions 0 .. L-1; the new
 *                row goes to position p (p < L) and positions 0 .. p are
 *                visible;
 *   window == W: the cache holds W slots (L == W) used as a ring, token t in
 *                slot t mod W; the new row goes to slot p mod W and the W
 *                most recent tokens (all of p + 1 when p < W) are visible.
 * No positional encoding, so the order of the slots does not matter to the
 * softmax.  K_out, V_out receive the whole updated cache (fp64). */
int oracle_selfattn(const void *q, int dt_q, const void *k_new, const void *v_new, int dt_new, const void *K,
                    const void *V, int dt_kv, const int32_t *pos, double *out, double *K_out, double *V_out,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L, int64_t window, double scale) {
    if (!q || !k_new || !v_new || !K || !V || !pos || !out || !K_out || !V_out || !xattn_args_ok(B, Hq, Hkv, D, L) ||
        window < 0 || (window > 0 && L != window))
        return -1;
    for (int64_t b = 0; b < B; ++b)
        if (window == 0 && pos[b] >= L) return -1;
    const int64_t G = Hq / Hkv, n_cache = B * Hkv * L * D;
    for (int64_t i = 0; i < n_cache; ++i) {
        K_out[i] = widen(K, dt_kv, i);
        V_out[i] = widen(V, dt_kv, i);
    }
    for (int64_t b = 0; b < B; ++b) {
        if (pos[b] < 0) continue;
        const int64_t slot = window ? pos[b] % window : pos[b];
        for (int64_t g = 0; g < Hkv; ++g)
            for (int64_t d = 0; d < D; ++d) {
                K_out[((b * Hkv + g) * L + slot) * D + d] = widen(k_new, dt_new, (b * Hkv + g) * D + d);
                V_out[((b * Hkv + g) * L + slot) * D + d] = widen(v_new, dt_new, (b * Hkv + g) * D + d);
            }
    }
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)L * sizeof(double));
        if (!s) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * Hq; ++bh) {
            if (!s) continue;
            const int64_t b = bh / Hq, h = bh % Hq, g = h / G, p = pos[b];
            const int64_t n = p < 0 ? 0 : (window && p + 1 > window ? window : p + 1);
            if (n == 0) {
                for (int64_t d = 0; d < D; ++d) out[bh * D + d] = 0.0;
                continue;
            }
            xattn_head(q, dt_q, bh * D, K_out, V_out, OR_F64, (b * Hkv + g) * L * D, out + bh * D, D, n, scale, s,
                       NULL, 0, 0, 0);
        }
        free(s);
    }
    return fail ? -2 : 0;
}

/* ------------------------------------------- SSM decode step (memory M)
 *
 * The GMU layers reuse M, the token-mixing output of the self-decoder's last
 * SSM layer ([Notes] "关键设计", "整体框架"; at decode time that layer keeps a
 * state of constant size, [Notes] "关键设计").  The pages do not spell out
 * the SSM; the self-decoder is Samba's, whose SSM layers are Mamba layers
 * with per-channel state decay ([Notes] "消融实验": the scalar-decay Mamba-2
 * variant loses).  This is one decode step of a Mamba layer (selective SSM
 * with zero-order-hold decay and Euler input term, as published) for B
 * sequences, in the order the layer computes it:
 *   [xi | z] = W_in x                           (W_in [2·d_inner, d_model])
 *   u_c  = SiLU(Σ_k conv_w[c,k] · win_c[k] + conv_b[c]),
 *          win_c = (conv_state[c, 0 .. K-2], xi_c)   oldest first, K = d_conv
 *   [δ | Bv | Cv] = W_x u                       (W_x [R + 2N, d_inner])
 *   Δ_c  = softplus(W_dt[c] · δ + dt_bias[c]),  softplus(a) = log(1 + e^a)
 *   s[c,n] <- exp(Δ_c · A[c,n]) · s[c,n] + Δ_c · Bv[n] · u_c,  A = -exp(A_log)
 *   M_c  = Σ_n Cv[n] · s[c,n] + D[c] · u_c      (the memory readout)
 *   y    = W_out (M ⊙ SiLU(z))                  (W_out [d_model, d_inner])
 * conv_state shifts by one (the new xi enters last).  Matrices share dt_w,
 * per-channel parameters (conv_w [d_inner, K], conv_b, dt_bias, D [d_inner],
 * A_log [d_inner, N]) share dt_p; states arrive in any dtype and leave as
 * fp64 (conv_state [B, d_inner, K-1], ssm_state [B, d_inner, N]). */
static double softplus_def(double a) {
    /* log(1 + e^a), written without overflowing e^a for large a */
    return a > 30.0 ? a + log1p(exp(-a)) : log1p(exp(a));
}

int oracle_mamba_step(const void *x, int dt_x, const void *W_in, const void *W_x, const void *W_dt,
                      const void *W_out, int dt_w, const void *conv_w, const void *conv_b, const void *dt_bias,
                      const void *A_log, const void *Dp, int dt_p, const void *conv_state, const void *ssm_state,
                      int dt_s, double *conv_state_out, double *ssm_state_out, double *M_out, double *y_out,
                      int64_t B, int64_t d_model, int64_t d_inner, int64_t N, int64_t R, int64_t K) {
    if (!x || !W_in || !W_x || !W_dt || !W_out || !conv_w || !conv_b || !dt_bias || !A_log || !Dp ||
        !conv_state || !ssm_state || !conv_state_out || !ssm_state_out || !M_out || !y_out || B < 0 ||
        d_model <= 0 || d_inner <= 0 || N <= 0 || R <= 0 || K < 1)
        return -1;
    const int64_t P = R + 2 * N, KS = K - 1;
    /* Per-sequence intermediates; every stage below is a loop over independent
       (sequence, channel) pairs, so it runs in parallel also for one sequence. */
    double *XI = (double *)malloc((size_t)B * d_inner * sizeof(double));
    double *Z = (double *)malloc((size_t)B * d_inner * sizeof(double));
    double *U = (double *)malloc((size_t)B * d_inner * sizeof(double));
    double *XD = (double *)malloc((size_t)B * P * sizeof(double));
    double *GM = (double *)malloc((size_t)B * d_inner * sizeof(double));
    if (B > 0 && !(XI && Z && U && XD && GM)) {
        free(XI); free(Z); free(U); free(XD); free(GM);
        return -2;
    }
    /* input projection: the x branch and the gate branch */
#pragma omp parallel for schedule(static)
    for (int64_t bc = 0; bc < B * 2 * d_inner; ++bc) {
        const int64_t b = bc / (2 * d_inner), c = bc % (2 * d_inner);
        double acc = 0.0;
        for (int64_t k = 0; k < d_model; ++k) acc += widen(W_in, dt_w, c * d_model + k) * widen(x, dt_x, b * d_model + k);
        if (c < d_inner) XI[b * d_inner + c] = acc; else Z[b * d_inner + c - d_inner] = acc;
    }
    /* causal depthwise convolution over the last K inputs, SiLU; shift the window */
#pragma omp parallel for schedule(static)
    for (int64_t bc = 0; bc < B * d_inner; ++bc) {
        const int64_t b = bc / d_inner, c = bc % d_inner;
        const double *xi = XI + b * d_inner;
        const int64_t so = (b * d_inner + c) * KS;
        double acc = widen(conv_b, dt_p, c);
        for (int64_t k = 0; k < KS; ++k) acc += widen(conv_w, dt_p, c * K + k) * widen(conv_state, dt_s, so + k);
        acc += widen(conv_w, dt_p, c * K + KS) * xi[c];
        U[b * d_inner + c] = acc / (1.0 + exp(-acc));
        for (int64_t k = 0; k + 1 < KS; ++k) conv_state_out[so + k] = widen(conv_state, dt_s, so + k + 1);
        if (KS > 0) conv_state_out[so + KS - 1] = xi[c];
    }
    /* the data-dependent step, input and output vectors */
#pragma omp parallel for schedule(static)
    for (int64_t bp = 0; bp < B * P; ++bp) {
        const int64_t b = bp / P, p = bp % P;
        const double *u = U + b * d_inner;
        double acc = 0.0;
        for (int64_t c = 0; c < d_inner; ++c) acc += widen(W_x, dt_w, p * d_inner + c) * u[c];
        XD[b * P + p] = acc;
    }
    /* the state update, the readout M = C·s + D·u and the gate */
#pragma omp parallel for schedule(static)
    for (int64_t bc = 0; bc < B * d_inner; ++bc) {
        const int64_t b = bc / d_inner, c = bc % d_inner;
        const double *u = U + b * d_inner, *z = Z + b * d_inner, *xd = XD + b * P;
        const double *delta = xd, *Bv = xd + R, *Cv = xd + R + N;
        double a = widen(dt_bias, dt_p, c);
        for (int64_t r = 0; r < R; ++r) a += widen(W_dt, dt_w, c * R + r) * delta[r];
        const double dlt = softplus_def(a);
        double m = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const int64_t si = (b * d_inner + c) * N + n;
            const double A = -exp(widen(A_log, dt_p, c * N + n));
            const double st = exp(dlt * A) * widen(ssm_state, dt_s, si) + dlt * Bv[n] * u[c];
            ssm_state_out[si] = st;
            m += Cv[n] * st;
        }
        m += widen(Dp, dt_p, c) * u[c];
        M_out[b * d_inner + c] = m;
        GM[b * d_inner + c] = m * (z[c] / (1.0 + exp(-z[c])));
    }
    /* output projection of the gated readout */
#pragma omp parallel for schedule(static)
    for (int64_t bo = 0; bo < B * d_model; ++bo) {
        const int64_t b = bo / d_model, o = bo % d_model;
        const double *gm = GM + b * d_inner;
        double acc = 0.0;
        for (int64_t c = 0; c < d_inner; ++c) acc += widen(W_out, dt_w, o * d_inner + c) * gm[c];
        y_out[b * d_model + o] = acc;
    }
    free(XI); free(Z); free(U); free(XD); free(GM);
    return 0;
}

/* ------------------------------------------------ self-decoder prefill
 *
 * Prefill in the YOCO manner keeps the pages' linear pre-filling cost
 * ([Notes] "现有痛点" and "领域现状": the decoder-decoder structure caches KV
 * once and pre-fills in linear time; [Summary] "Key results": 4.9x faster
 * long-context processing): the self-decoder runs over every prompt token,
 * its sliding-window attention layers attending causally over the last
 * `window` tokens (256 in the model the pages favour, [Notes] "消融实验").
 * Causal attention of T prompt tokens, grouped heads, no positional
 * encoding: q [B, T, Hq, D], k, v [B, T, Hkv, D] (token-major, as
 * projections produce them), out [B, T, Hq, D]; query i of head h attends
 * to keys j of KV head h / (Hq / Hkv) with j <= i and, for window > 0,
 * j > i - window:  out_i = Σ_j softmax_j(scale · q_i·k_j) v_j. */
int oracle_attn_prefill(const void *q, int dt_q, const void *k, const void *v, int dt_kv, double *out, int64_t B,
                        int64_t T, int64_t Hq, int64_t Hkv, int64_t D, int64_t window, double scale) {
    if (!q || !k || !v || !out || B < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || window < 0)
        return -1;
    const int64_t G = Hq / Hkv;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)(T > 0 ? T : 1) * sizeof(double));
        if (!s) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < B * T * Hq; ++r) {
            if (!s) continue;
            const int64_t b = r / (T * Hq), i = (r / Hq) % T, h = r % Hq, g = h / G;
            const int64_t j0 = window > 0 && i + 1 > window ? i + 1 - window : 0, j1 = i;  /* keys j0 .. j1 */
            double m = -INFINITY;
            for (int64_t j = j0; j <= j1; ++j) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += widen(q, dt_q, r * D + d) * widen(k, dt_kv, ((b * T + j) * Hkv + g) * D + d);
                s[j] = dot * scale;
                if (s[j] > m) m = s[j];
            }
            double den = 0.0;
            double *o = out + r * D;
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            for (int64_t j = j0; j <= j1; ++j) {
                const double w = exp(s[j] - m);
                den += w;
                for (int64_t d = 0; d < D; ++d) o[d] += w * widen(v, dt_kv, ((b * T + j) * Hkv + g) * D + d);
            }
            for (int64_t d = 0; d < D; ++d) o[d] /= den;
        }
        free(s);
    }
    return fail ? -2 : 0;
}

/* --------------------------------------------------------------- threads */

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
