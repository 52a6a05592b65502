// C ABI of the library: argument validation, workspace layout, dispatch by
// shape regime and cross-decoder sequencing.  Kernels live in the other
// translation units; nothing here allocates, frees or synchronises.
#include "sambay.h"

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>

#include "launch.hpp"
#include "norm_order.hpp"

#include <vector>

using namespace sambay;

namespace {

thread_local std::string g_last_error;

sb_status fail(sb_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

sb_status ok() {
    g_last_error.clear();
    return SB_OK;
}

sb_status hip_fail(const char *where, hipError_t e) {
    return fail(SB_EHIP, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
}

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi)
};

Range rng(const char *name, const void *p, size_t bytes) {
    return Range{name, (uintptr_t)p, (uintptr_t)p + bytes};
}

bool overlaps(const Range &a, const Range &b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

// Workspace carving: sequential 256-byte-aligned sub-buffers.
struct Carver {
    char *base;
    size_t used = 0;
    void *take(size_t bytes) {
        void *p = base ? base + used : nullptr;
        used += round_up(bytes);
        return p;
    }
};

constexpr int64_t kMaxDim = (int64_t)1 << 30;

// SAMBAY_LOG=1 prints each call's dispatch decisions (kernel path, plans) to stderr.
bool log_enabled() {
    static const bool on = [] {
        const char *e = getenv("SAMBAY_LOG");
        return e && *e && *e != '0';
    }();
    return on;
}

// ----------------------------------------------------------------- GMU

// Elements of the GMU's gated hidden H for a group of T decode tokens: above
// 16 tokens it travels in the 16-token tiled layout (whole tiles), below it
// row-major.
size_t gmu_hidden_elems(int T, int d_inner) {
    return T > 16 ? tiled_elems(T, d_inner) : (size_t)T * d_inner;
}

size_t gmu_ws(int64_t rows, int64_t d_model, int64_t d_inner, sb_dtype dt) {
    if (rows <= 0 || d_model <= 0 || d_inner <= 0) return 0;
    if (dt == SB_F32) return round_up((size_t)rows * d_inner * sizeof(float));
    // bf16 H [rows, d_inner] (decode: a hi + lo pair in whole 16-token tiles,
    // plus room for k-split partials).
    size_t bytes = round_up((size_t)rows * d_inner * sizeof(bf16_t));
    if (rows <= kSkinnyMaxTokens) {
        bytes = 2 * round_up(gmu_hidden_elems((int)rows, (int)d_inner) * sizeof(bf16_t));
        size_t part = skinny_partial_bytes_max((int)rows, (int)d_inner, (int)d_model);
        const size_t part2 = skinny_partial_bytes_max((int)rows, (int)d_model, (int)d_inner);
        if (part2 > part) part = part2;
        bytes += round_up(part);
    }
    return bytes;
}

// bf16 GMU on rows <= 64 tokens (decode): two weight-streaming launches.  With
// h_lo the gated hidden H travels as a bf16 hi + lo pair between them (used in
// the layer stack, where rounding errors compound; a single call's error is
// dominated by its bf16 output, and the pair costs up to ~20% at 64 rows).
hipError_t gmu_decode_bf16(const bf16_t *M, const bf16_t *X, const bf16_t *X_lo, int ldx, const bf16_t *W1,
                           const bf16_t *W2, void *Y, Epilogue out_epi, int T, int d_model, int d_inner, bool h_lo,
                           Carver &ws, hipStream_t stream) {
    bf16_t *H = static_cast<bf16_t *>(ws.take(gmu_hidden_elems(T, d_inner) * sizeof(bf16_t)));
    bf16_t *H_lo = static_cast<bf16_t *>(ws.take(gmu_hidden_elems(T, d_inner) * sizeof(bf16_t)));
    if (!h_lo) H_lo = nullptr;
    const SkinnyPlan p1 = skinny_plan(T, d_inner, d_model, X_lo != nullptr);
    const SkinnyPlan p2 = skinny_plan(T, d_model, d_inner, H_lo != nullptr);
    size_t part = skinny_partial_bytes(T, d_inner, p1);
    if (skinny_partial_bytes(T, d_model, p2) > part) part = skinny_partial_bytes(T, d_model, p2);
    float *partials = static_cast<float *>(ws.take(part));
    SkinnyArgs a1;
    a1.X = X; a1.X_lo = X_lo; a1.ldx = ldx; a1.W = W1; a1.T = T; a1.N = d_inner; a1.K = d_model; a1.epi = EPI_GATE;
    a1.out = H; a1.ldo = d_inner; a1.out_lo = H_lo; a1.aux = M; a1.ldaux = d_inner;
    SkinnyArgs a2;
    a2.X = H; a2.X_lo = H_lo; a2.ldx = d_inner; a2.W = W2; a2.T = T; a2.N = d_model; a2.K = d_inner;
    a2.epi = out_epi; a2.out = Y; a2.ldo = d_model;
    // Above 16 tokens H travels in the 16-token tiled layout when both
    // products' kernels take it: each token-operand load then reads 1 KB
    // contiguous (a 32-token product of 37.7 MB: 11.4 -> 10.0 us; at 8
    // tokens no gain).
    if (T > 16 && p1.k_splits == 1 && skinny_tiles(a1, p1) && skinny_tiles(a2, p2)) {
        a1.out_tiled = true;
        a2.x_tiled = true;
    }
    hipError_t e = launch_skinny(a1, p1, partials, stream);
    if (e != hipSuccess) return e;
    return launch_skinny(a2, p2, partials, stream);
}

// ------------------------------------------------------- cross-attention

sb_status check_xattn_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L) {
    if (B < 0 || Hq < 0 || Hkv < 0 || D < 0 || L < 0) return fail(SB_EINVAL, "negative size");
    if (Hq == 0 || Hkv == 0) return fail(SB_EINVAL, "Hq and Hkv must be positive");
    if (L == 0) return fail(SB_EINVAL, "L == 0: the cache holds no position");
    if (Hq % Hkv != 0) return fail(SB_EINVAL, "Hq (%lld) is not a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
    if (D != kHeadDim) return fail(SB_EUNSUPPORTED, "head dim %lld unsupported (only %d)", (long long)D, kHeadDim);
    if (Hq / Hkv > kMaxGroup)
        return fail(SB_EUNSUPPORTED, "group size Hq/Hkv = %lld exceeds %d", (long long)(Hq / Hkv), kMaxGroup);
    if (L >= ((int64_t)1 << 31)) return fail(SB_EUNSUPPORTED, "L >= 2^31");
    if (B > 65535 || Hkv > 65535) return fail(SB_EUNSUPPORTED, "B and Hkv must be <= 65535");
    if (B * Hq > ((int64_t)1 << 31) - 1) return fail(SB_EUNSUPPORTED, "B*Hq too large");
    return SB_OK;
}

size_t xattn_ws(int64_t B, int64_t Hq, int64_t Hkv, int64_t L) {
    return round_up(xattn_workspace_need(B, Hq, Hkv, L));
}

}  // namespace

// =================================================================== ABI

extern "C" const char *sb_last_error(void) { return g_last_error.c_str(); }

#ifndef SAMBAY_SOURCE_HASH
#define SAMBAY_SOURCE_HASH "unknown"
#endif
extern "C" const char *sb_version(void) { return "sambay-mi355x 0.2 (gfx950) sources " SAMBAY_SOURCE_HASH; }

extern "C" size_t gmu_workspace_bytes(int64_t rows, int64_t d_model, int64_t d_inner, sb_dtype dt) {
    return gmu_ws(rows, d_model, d_inner, dt);
}

extern "C" sb_status gmu_forward(const void *M, const void *X, const void *W1, const void *W2, void *Y, int64_t rows,
                                 int64_t d_model, int64_t d_inner, sb_dtype dt, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    if (rows < 0 || d_model < 0 || d_inner < 0) return fail(SB_EINVAL, "negative size");
    if (dt != SB_F32 && dt != SB_BF16) return fail(SB_EINVAL, "unknown dtype %d", (int)dt);
    if (rows == 0) return ok();
    if (d_model == 0 || d_inner == 0) return fail(SB_EINVAL, "d_model and d_inner must be positive");
    if (!M || !X || !W1 || !W2 || !Y) return fail(SB_EINVAL, "null tensor pointer");
    if (!aligned16(M) || !aligned16(X) || !aligned16(W1) || !aligned16(W2) || !aligned16(Y))
        return fail(SB_EINVAL, "tensor base pointers must be 16-byte aligned");
    if (rows > kMaxDim || d_model > kMaxDim || d_inner > kMaxDim) return fail(SB_EUNSUPPORTED, "dimension >= 2^30");
    if (rows * d_inner > ((int64_t)1 << 40) || rows * d_model > ((int64_t)1 << 40))
        return fail(SB_EUNSUPPORTED, "tensor too large");
    const size_t es = dt == SB_F32 ? 4 : 2;
    const Range ry = rng("Y", Y, (size_t)rows * d_model * es);
    const Range ins[] = {rng("M", M, (size_t)rows * d_inner * es), rng("X", X, (size_t)rows * d_model * es),
                         rng("W1", W1, (size_t)d_inner * d_model * es), rng("W2", W2, (size_t)d_model * d_inner * es)};
    for (const Range &r : ins)
        if (overlaps(ry, r)) return fail(SB_EINVAL, "Y overlaps %s", r.name);
    if (dt == SB_BF16 && (d_model % 64 != 0 || d_inner % 64 != 0))
        return fail(SB_EUNSUPPORTED, "bf16 GMU needs d_model and d_inner multiples of 64");
    const size_t need = gmu_ws(rows, d_model, d_inner, dt);
    if (!workspace || workspace_bytes < need)
        return fail(SB_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    if (!aligned16(workspace)) return fail(SB_EINVAL, "workspace must be 16-byte aligned");
    const Range rw = rng("workspace", workspace, need);
    if (overlaps(rw, ry)) return fail(SB_EINVAL, "workspace overlaps Y");
    for (const Range &r : ins)
        if (overlaps(rw, r)) return fail(SB_EINVAL, "workspace overlaps %s", r.name);

    Carver ws{static_cast<char *>(workspace)};
    if (log_enabled()) {
        if (dt == SB_F32) {
            fprintf(stderr, "[sambay] gmu_forward rows=%lld %lldx%lld fp32 -> gmu_f32 kernels\n", (long long)rows,
                    (long long)d_model, (long long)d_inner);
        } else if (rows == 1 && (d_model == 3072 || d_model == 6144 || d_model == 8192) &&
                   (d_inner == 3072 || d_inner == 6144 || d_inner == 8192)) {
            fprintf(stderr, "[sambay] gmu_forward rows=1 %lldx%lld bf16 -> one-token dot-product products\n",
                    (long long)d_model, (long long)d_inner);
        } else if (rows <= kSkinnyMaxTokens) {
            const SkinnyPlan p1 = skinny_plan((int)rows, (int)d_inner, (int)d_model, false);
            const SkinnyPlan p2 = skinny_plan((int)rows, (int)d_model, (int)d_inner, false);
            fprintf(stderr,
                    "[sambay] gmu_forward rows=%lld %lldx%lld bf16 -> decode products: gate rows/wg=%d ksplit=%d, "
                    "out rows/wg=%d ksplit=%d\n",
                    (long long)rows, (long long)d_model, (long long)d_inner, p1.rows_per_wg, p1.k_splits,
                    p2.rows_per_wg, p2.k_splits);
        } else {
            fprintf(stderr, "[sambay] gmu_forward rows=%lld %lldx%lld bf16 -> prefill GEMMs (MFMA tiles)\n",
                    (long long)rows, (long long)d_model, (long long)d_inner);
        }
    }
    hipError_t e;
    if (dt == SB_F32) {
        float *H = static_cast<float *>(ws.take((size_t)rows * d_inner * sizeof(float)));
        e = launch_gmu_f32((const float *)M, (const float *)X, (const float *)W1, (const float *)W2, (float *)Y, H,
                           rows, d_model, d_inner, stream);
    } else if (rows <= kSkinnyMaxTokens) {
        e = gmu_decode_bf16((const bf16_t *)M, (const bf16_t *)X, nullptr, (int)d_model, (const bf16_t *)W1,
                            (const bf16_t *)W2, Y, EPI_BF16, (int)rows, (int)d_model, (int)d_inner, false, ws, stream);
    } else {
        bf16_t *H = static_cast<bf16_t *>(ws.take((size_t)rows * d_inner * sizeof(bf16_t)));
        e = launch_gemm((const bf16_t *)X, (const bf16_t *)W1, (int)rows, (int)d_inner, (int)d_model, EPI_GATE, H,
                        (const bf16_t *)M, stream);
        if (e == hipSuccess)
            e = launch_gemm(H, (const bf16_t *)W2, (int)rows, (int)d_model, (int)d_inner, EPI_BF16, (bf16_t *)Y,
                            nullptr, stream);
    }
    if (e != hipSuccess) return hip_fail("gmu_forward launch", e);
    return ok();
}

extern "C" size_t xattn_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || L <= 0 || D != kHeadDim || Hq % Hkv != 0) return 0;
    return xattn_ws(B, Hq, Hkv, L);
}

namespace {

sb_status xattn_decode_impl(const char *fn, const void *q, const void *kcache, const void *vcache, const int32_t *lens,
                            void *out, int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L, float scale,
                            void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (B < 0 || Hq < 0 || Hkv < 0 || D < 0 || L < 0) return fail(SB_EINVAL, "negative size");
    if (B == 0) return ok();
    sb_status st = check_xattn_shape(B, Hq, Hkv, D, L);
    if (st != SB_OK) return st;
    if (!q || !kcache || !vcache || !out) return fail(SB_EINVAL, "null tensor pointer");
    if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(out))
        return fail(SB_EINVAL, "tensor base pointers must be 16-byte aligned");
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
        return fail(SB_EINVAL, "scale must be finite");
    const size_t qbytes = (size_t)B * Hq * D * 2, kvbytes = (size_t)B * Hkv * L * D * 2;
    const Range ro = rng("out", out, qbytes);
    const Range ins[] = {rng("q", q, qbytes), rng("kcache", kcache, kvbytes), rng("vcache", vcache, kvbytes),
                         rng("lens", lens, lens ? (size_t)B * sizeof(int32_t) : 0)};
    for (const Range &r : ins)
        if (overlaps(ro, r)) return fail(SB_EINVAL, "out overlaps %s", r.name);
    const size_t need = xattn_ws(B, Hq, Hkv, L);
    if (!workspace || workspace_bytes < need)
        return fail(SB_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    if (!aligned16(workspace)) return fail(SB_EINVAL, "workspace must be 16-byte aligned");
    const Range rw = rng("workspace", workspace, need);
    if (overlaps(rw, ro)) return fail(SB_EINVAL, "workspace overlaps out");
    for (const Range &r : ins)
        if (overlaps(rw, r)) return fail(SB_EINVAL, "workspace overlaps %s", r.name);

    const XattnPlan plan = xattn_plan(B, Hkv, L, lens != nullptr);
    if (log_enabled())
        fprintf(stderr, "[sambay] %s B=%lld Hq=%lld Hkv=%lld L=%lld%s -> %d chunks of %d positions, grid %dx%lldx%lld\n",
                fn, (long long)B, (long long)Hq, (long long)Hkv, (long long)L, lens ? " (ragged)" : "", plan.splits,
                plan.chunk, plan.splits, (long long)Hkv, (long long)B);
    hipError_t e = launch_xattn(q, false, (const bf16_t *)kcache, (const bf16_t *)vcache, lens, (bf16_t *)out, nullptr,
                                (int)B, (int)Hq, (int)Hkv, (int)L, scale, plan, workspace, stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

}  // namespace

extern "C" sb_status xattn_decode(const void *q, const void *kcache, const void *vcache, void *out, int64_t B,
                                  int64_t Hq, int64_t Hkv, int64_t D, int64_t L, float scale, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    return xattn_decode_impl("xattn_decode", q, kcache, vcache, nullptr, out, B, Hq, Hkv, D, L, scale, workspace,
                             workspace_bytes, stream);
}

// ---------------------------------------------------- no-allocation entry
// The partials of xattn_decode_noalloc live in this file-scope device array:
// one copy per GPU the library runs on, held until the process ends.  On the
// host its name is only a stand-in: the device address is looked up once per
// device with hipGetSymbolAddress (with that device current), and only that
// address is ever passed on.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

sb_status scratch_for_current_device(const char *fn, void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(fn, e);
    if (dev < 0 || dev >= kMaxDevices) return fail(SB_EUNSUPPORTED, "%s: device %d (at most %d)", fn, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail("hipGetSymbolAddress(scratch)", e);
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return SB_OK;
}

}  // namespace

extern "C" sb_status xattn_decode_noalloc(const void *q, const void *kcache, const void *vcache, void *out, int64_t B,
                                          int64_t Hq, int64_t Hkv, int64_t D, int64_t L, float scale,
                                          hipStream_t stream) {
    const char *fn = "xattn_decode_noalloc";
    if (B < 0 || Hq < 0 || Hkv < 0 || D < 0 || L < 0) return fail(SB_EINVAL, "negative size");
    if (B == 0) return ok();
    const sb_status st = check_xattn_shape(B, Hq, Hkv, D, L);
    if (st != SB_OK) return st;
    const size_t need = xattn_ws(B, Hq, Hkv, L);
    if (need > kNoAllocScratchBytes)
        return fail(SB_EWORKSPACE, "%s: %zu bytes of partials needed, the library's scratch holds %zu", fn, need,
                    kNoAllocScratchBytes);
    void *ws = nullptr;
    const sb_status sst = scratch_for_current_device(fn, &ws);
    if (sst != SB_OK) return sst;
    return xattn_decode_impl(fn, q, kcache, vcache, nullptr, out, B, Hq, Hkv, D, L, scale, ws, kNoAllocScratchBytes,
                             stream);
}

extern "C" sb_status xattn_decode_varlen(const void *q, const void *kcache, const void *vcache, const int32_t *lens,
                                         void *out, int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L,
                                         float scale, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (B > 0 && !lens) return fail(SB_EINVAL, "null lens");
    if (((uintptr_t)lens & 3u) != 0) return fail(SB_EINVAL, "lens must be 4-byte aligned");
    return xattn_decode_impl("xattn_decode_varlen", q, kcache, vcache, lens, out, B, Hq, Hkv, D, L, scale, workspace,
                             workspace_bytes, stream);
}

extern "C" size_t diffattn_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || L <= 0 || D != kHeadDim || Hq % Hkv != 0) return 0;
    return round_up(xattn_workspace_need(B, 2 * Hq, Hkv, L));
}

extern "C" sb_status diffattn_decode(const void *q, const void *kcache, const void *vcache, const int32_t *lens,
                                     const void *gamma, void *out, int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                                     int64_t L, float scale, float lambda, float lambda_init, float eps,
                                     void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const char *fn = "diffattn_decode";
    if (B < 0 || Hq < 0 || Hkv < 0 || D < 0 || L < 0) return fail(SB_EINVAL, "negative size");
    if (B == 0) return ok();
    sb_status st = check_xattn_shape(B, Hq, Hkv, D, L);
    if (st != SB_OK) return st;
    if (2 * (Hq / Hkv) > kMaxGroup)
        return fail(SB_EUNSUPPORTED, "group size Hq/Hkv = %lld exceeds %d for two maps", (long long)(Hq / Hkv),
                    kMaxGroup / 2);
    if (B * 2 * Hq > ((int64_t)1 << 31) - 1) return fail(SB_EUNSUPPORTED, "B*Hq too large");
    if (!q || !kcache || !vcache || !out) return fail(SB_EINVAL, "null tensor pointer");
    if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(out) || !aligned16(gamma))
        return fail(SB_EINVAL, "tensor base pointers must be 16-byte aligned");
    if (((uintptr_t)lens & 3u) != 0) return fail(SB_EINVAL, "lens must be 4-byte aligned");
    const float inf = __builtin_inff();
    if (!(scale == scale) || scale == inf || scale == -inf) return fail(SB_EINVAL, "scale must be finite");
    if (!(lambda == lambda) || lambda == inf || lambda == -inf || !(lambda_init == lambda_init) ||
        lambda_init == inf || lambda_init == -inf)
        return fail(SB_EINVAL, "lambda and lambda_init must be finite");
    if (!(eps >= 0.f) || eps == inf) return fail(SB_EINVAL, "eps must be finite and >= 0");
    const size_t qbytes = (size_t)B * Hq * D * 2, kvbytes = (size_t)B * Hkv * L * D * 2;
    const Range ro = rng("out", out, qbytes);
    const Range ins[] = {rng("q", q, qbytes), rng("kcache", kcache, kvbytes), rng("vcache", vcache, kvbytes),
                         rng("lens", lens, lens ? (size_t)B * sizeof(int32_t) : 0),
                         rng("gamma", gamma, gamma ? (size_t)D * 2 : 0)};
    for (const Range &r : ins)
        if (overlaps(ro, r)) return fail(SB_EINVAL, "out overlaps %s", r.name);
    const size_t need = diffattn_workspace_bytes(B, Hq, Hkv, D, L);
    if (!workspace || workspace_bytes < need)
        return fail(SB_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    if (!aligned16(workspace)) return fail(SB_EINVAL, "workspace must be 16-byte aligned");
    const Range rw = rng("workspace", workspace, need);
    if (overlaps(rw, ro)) return fail(SB_EINVAL, "workspace overlaps out");
    for (const Range &r : ins)
        if (overlaps(rw, r)) return fail(SB_EINVAL, "workspace overlaps %s", r.name);

    const XattnPlan plan = xattn_plan(B, Hkv, L, lens != nullptr);
    if (log_enabled())
        fprintf(stderr, "[sambay] %s B=%lld Hq=%lld Hkv=%lld L=%lld%s -> %d chunks of %d positions, %lld score "
                "columns per group\n", fn, (long long)B, (long long)Hq, (long long)Hkv, (long long)L,
                lens ? " (ragged)" : "", plan.splits, plan.chunk, (long long)(2 * (Hq / Hkv)));
    hipError_t e = launch_diffattn((const bf16_t *)q, (const bf16_t *)kcache, (const bf16_t *)vcache, lens,
                                   (const bf16_t *)gamma, (bf16_t *)out, (int)B, (int)Hq, (int)Hkv, (int)L, scale,
                                   lambda, lambda_init, eps, plan, workspace, stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

extern "C" size_t selfattn_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t L) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || L <= 0 || D != kHeadDim || Hq % Hkv != 0) return 0;
    // The visible counts, then the attention partials of a ragged batch.
    return round_up((size_t)B * sizeof(int32_t)) + round_up(xattn_partial_bytes(B, Hq, xattn_plan(B, Hkv, L, true).splits));
}

extern "C" sb_status selfattn_decode(const void *q, const void *k_new, const void *v_new, void *kcache, void *vcache,
                                     const int32_t *pos, void *out, int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                                     int64_t L, int64_t window, float scale, void *workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
    const char *fn = "selfattn_decode";
    if (B < 0 || Hq < 0 || Hkv < 0 || D < 0 || L < 0) return fail(SB_EINVAL, "negative size");
    if (window < 0) return fail(SB_EINVAL, "window must be >= 0");
    if (B == 0) return ok();
    sb_status st = check_xattn_shape(B, Hq, Hkv, D, L);
    if (st != SB_OK) return st;
    if (window > 0 && L != window)
        return fail(SB_EINVAL, "a sliding-window cache has exactly window slots (L %lld, window %lld)", (long long)L,
                    (long long)window);
    if (!q || !k_new || !v_new || !kcache || !vcache || !pos || !out) return fail(SB_EINVAL, "null pointer");
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(kcache) || !aligned16(vcache) ||
        !aligned16(out))
        return fail(SB_EINVAL, "tensor base pointers must be 16-byte aligned");
    if (((uintptr_t)pos & 3u) != 0) return fail(SB_EINVAL, "pos must be 4-byte aligned");
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
        return fail(SB_EINVAL, "scale must be finite");
    const size_t qbytes = (size_t)B * Hq * D * 2, rowbytes = (size_t)B * Hkv * D * 2,
                 kvbytes = (size_t)B * Hkv * L * D * 2;
    const Range rk = rng("kcache", kcache, kvbytes), rv = rng("vcache", vcache, kvbytes), ro = rng("out", out, qbytes);
    const Range ins[] = {rng("q", q, qbytes), rng("k_new", k_new, rowbytes), rng("v_new", v_new, rowbytes),
                         rng("pos", pos, (size_t)B * sizeof(int32_t))};
    if (overlaps(rk, rv)) return fail(SB_EINVAL, "kcache overlaps vcache");
    for (const Range *w : {&rk, &rv, &ro})
        for (const Range &r : ins)
            if (overlaps(*w, r)) return fail(SB_EINVAL, "%s overlaps %s", w->name, r.name);
    if (overlaps(ro, rk) || overlaps(ro, rv)) return fail(SB_EINVAL, "out overlaps the cache");
    const size_t need = selfattn_workspace_bytes(B, Hq, Hkv, D, L);
    if (!workspace || workspace_bytes < need)
        return fail(SB_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    if (!aligned16(workspace)) return fail(SB_EINVAL, "workspace must be 16-byte aligned");
    const Range rw = rng("workspace", workspace, need);
    for (const Range *w : {&rk, &rv, &ro})
        if (overlaps(rw, *w)) return fail(SB_EINVAL, "workspace overlaps %s", w->name);
    for (const Range &r : ins)
        if (overlaps(rw, r)) return fail(SB_EINVAL, "workspace overlaps %s", r.name);

    int32_t *lens = reinterpret_cast<int32_t *>(workspace);
    void *partials = reinterpret_cast<char *>(workspace) + round_up((size_t)B * sizeof(int32_t));
    const XattnPlan plan = xattn_plan(B, Hkv, L, true);
    if (log_enabled())
        fprintf(stderr, "[sambay] %s B=%lld Hq=%lld Hkv=%lld L=%lld window=%lld -> append, %d chunks of %d positions\n",
                fn, (long long)B, (long long)Hq, (long long)Hkv, (long long)L, (long long)window, plan.splits,
                plan.chunk);
    hipError_t e = launch_kv_append((const bf16_t *)k_new, (const bf16_t *)v_new, (bf16_t *)kcache, (bf16_t *)vcache,
                                    pos, lens, (int)B, (int)Hkv, (int)L, (int)window, stream);
    if (e == hipSuccess)
        e = launch_xattn(q, false, (const bf16_t *)kcache, (const bf16_t *)vcache, lens, (bf16_t *)out, nullptr,
                         (int)B, (int)Hq, (int)Hkv, (int)L, scale, plan, partials, stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

extern "C" size_t attn_prefill_workspace_bytes(int64_t B, int64_t T, int64_t Hkv, int64_t D) {
    if (B <= 0 || T <= 0 || Hkv <= 0 || D != kHeadDim) return 0;
    return round_up(attn_prefill_workspace_need(B, T, Hkv));
}

extern "C" sb_status attn_prefill(const void *q, const void *k, const void *v, void *out, int64_t B, int64_t T,
                                  int64_t Hq, int64_t Hkv, int64_t D, int64_t window, float scale, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    const char *fn = "attn_prefill";
    if (B < 0 || T < 0 || Hq < 0 || Hkv < 0 || D < 0 || window < 0) return fail(SB_EINVAL, "negative size");
    if (B == 0 || T == 0) return ok();
    if (Hq == 0 || Hkv == 0) return fail(SB_EINVAL, "Hq and Hkv must be positive");
    if (Hq % Hkv != 0) return fail(SB_EINVAL, "Hq (%lld) is not a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
    if (D != kHeadDim) return fail(SB_EUNSUPPORTED, "head dim %lld unsupported (only %d)", (long long)D, kHeadDim);
    if (B > 65535 || Hq > 65535 || T >= ((int64_t)1 << 31) || B * T * Hq * D >= ((int64_t)1 << 62))
        return fail(SB_EUNSUPPORTED, "size out of range");
    if (!q || !k || !v || !out) return fail(SB_EINVAL, "null tensor pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(SB_EINVAL, "tensor base pointers must be 16-byte aligned");
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
        return fail(SB_EINVAL, "scale must be finite");
    const size_t qbytes = (size_t)B * T * Hq * D * 2, kvbytes = (size_t)B * T * Hkv * D * 2;
    const Range ro = rng("out", out, qbytes);
    const Range ins[] = {rng("q", q, qbytes), rng("k", k, kvbytes), rng("v", v, kvbytes)};
    for (const Range &r : ins)
        if (overlaps(ro, r)) return fail(SB_EINVAL, "out overlaps %s", r.name);
    const size_t need = attn_prefill_workspace_bytes(B, T, Hkv, D);
    if (!workspace || workspace_bytes < need)
        return fail(SB_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    if (!aligned16(workspace)) return fail(SB_EINVAL, "workspace must be 16-byte aligned");
    const Range rw = rng("workspace", workspace, need);
    if (overlaps(rw, ro)) return fail(SB_EINVAL, "workspace overlaps out");
    for (const Range &r : ins)
        if (overlaps(rw, r)) return fail(SB_EINVAL, "workspace overlaps %s", r.name);
    if (log_enabled())
        fprintf(stderr, "[sambay] %s B=%lld T=%lld Hq=%lld Hkv=%lld window=%lld -> %lld workgroups\n", fn,
                (long long)B, (long long)T, (long long)Hq, (long long)Hkv, (long long)window,
                (long long)(B * Hq * ((T + 63) / 64)));
    const int W = window >= T ? 0 : (int)window;  // a window covering the prompt is plain causal attention
    hipError_t e = launch_attn_prefill((const bf16_t *)q, (const bf16_t *)k, (const bf16_t *)v, (bf16_t *)out, (int)B,
                                       (int)T, (int)Hq, (int)Hkv, W, scale, workspace, stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

namespace {

// Workspace of one Mamba decode step, per token group of <= 64 sequences
// (groups run one after another and reuse it).
struct MambaLayout {
    size_t xz, u, u_hi, u_lo, xdbl, g_hi, g_lo, part, total;
};

MambaLayout mamba_layout(int64_t B, int64_t d_model, int64_t d_inner, int64_t N, int64_t R) {
    const int T = (int)(B < kSkinnyMaxTokens ? B : kSkinnyMaxTokens);
    const int64_t P = R + 2 * N;
    MambaLayout l;
    Carver c{nullptr};
    l.xz = c.used; c.take((size_t)T * 2 * d_inner * sizeof(float));
    l.u = c.used; c.take((size_t)T * d_inner * sizeof(float));
    l.u_hi = c.used; c.take((size_t)T * d_inner * 2);
    l.u_lo = c.used; c.take((size_t)T * d_inner * 2);
    l.xdbl = c.used; c.take((size_t)T * P * sizeof(float));
    l.g_hi = c.used; c.take((size_t)T * d_inner * 2);
    l.g_lo = c.used; c.take((size_t)T * d_inner * 2);
    size_t part = skinny_partial_bytes_max(T, (int)(2 * d_inner), (int)d_model);
    const size_t p2 = skinny_partial_bytes_max(T, (int)P, (int)d_inner),
                 p3 = skinny_partial_bytes_max(T, (int)d_model, (int)d_inner);
    if (p2 > part) part = p2;
    if (p3 > part) part = p3;
    l.part = c.used; c.take(part);
    l.total = c.used;
    return l;
}

bool mamba_dims_ok(int64_t B, int64_t d_model, int64_t d_inner, int64_t N, int64_t R, int64_t K) {
    return B > 0 && d_model > 0 && d_inner > 0 && d_model % 64 == 0 && d_inner % 64 == 0 && d_model <= kMaxDim &&
           d_inner <= kMaxDim && (N == 8 || N == 16 || N == 32 || N == 64) && R >= 8 && R <= kMaxDtRank &&
           R % 8 == 0 && K >= 1 && K <= kMaxConv;
}


// Deferred RMSNorms of the whole-model step, per token group of
// kSkinnyMaxTokens rows.  in_deferred[g]: the group's input is RMSNorm(h;
// norm_in) and the input product normalises its own K slab from h and the
// chunk sums of squares in stats (no RMSNorm launch).  out_defer[g]: the
// output product (a residual add into h) leaves the group's chunk sums in
// stats for the next sublayer's norm.  stats: [token][stride] floats.
struct DeferredNorms {
    const bf16_t *h = nullptr;
    const bf16_t *norm_in = nullptr;
    const bool *in_deferred = nullptr;
    const bool *out_defer = nullptr;
    float *stats = nullptr;
    int stride = 0;
    float eps = 0.f;
};

// The decode step's launches for B sequences in token groups of <= 64 (the
// arguments already validated): x may come with a low part x_lo (a bf16
// hi + lo pair); out_epi EPI_BF16 stores y, EPI_RESID adds it into y_out (h);
// dn (optional) defers the input's and the next sublayer's RMSNorm.
hipError_t run_mamba_step(const bf16_t *x, const bf16_t *x_lo, const sb_mamba_weights *w, float *conv_state,
                          float *ssm_state, bf16_t *M_out, bf16_t *y_out, Epilogue out_epi, int64_t B,
                          int64_t d_model, int64_t d_inner, int64_t d_state, int64_t dt_rank, int64_t d_conv,
                          void *workspace, hipStream_t stream, const DeferredNorms *dn = nullptr) {
    const MambaLayout lay = mamba_layout(B, d_model, d_inner, d_state, dt_rank);
    const int64_t P = dt_rank + 2 * d_state;
    char *ws = reinterpret_cast<char *>(workspace);
    float *xz = reinterpret_cast<float *>(ws + lay.xz), *u = reinterpret_cast<float *>(ws + lay.u);
    float *xdbl = reinterpret_cast<float *>(ws + lay.xdbl), *part = reinterpret_cast<float *>(ws + lay.part);
    bf16_t *u_hi = reinterpret_cast<bf16_t *>(ws + lay.u_hi), *u_lo = reinterpret_cast<bf16_t *>(ws + lay.u_lo);
    bf16_t *g_hi = reinterpret_cast<bf16_t *>(ws + lay.g_hi), *g_lo = reinterpret_cast<bf16_t *>(ws + lay.g_lo);
    const int di = (int)d_inner, dm = (int)d_model, Pi = (int)P;
    hipError_t e = hipSuccess;
    for (int64_t t0 = 0; t0 < B && e == hipSuccess; t0 += kSkinnyMaxTokens) {
        const int T = (int)(B - t0 < kSkinnyMaxTokens ? B - t0 : kSkinnyMaxTokens);
        const int grp = (int)(t0 / kSkinnyMaxTokens);
        SkinnyArgs a;
        a.X = x + t0 * d_model;
        a.X_lo = x_lo ? x_lo + t0 * d_model : nullptr;
        if (dn && dn->in_deferred && dn->in_deferred[grp]) {
            a.X = dn->h + t0 * d_model;
            a.X_lo = nullptr;
            a.norm_g = dn->norm_in;
            a.norm_stats = dn->stats + t0 * dn->stride;
            a.norm_eps = dn->eps;
        }
        a.ldx = dm;
        a.W = (const bf16_t *)w->w_in;
        a.T = T;
        a.N = 2 * di;
        a.K = dm;
        a.epi = EPI_F32;
        a.out = xz;
        a.ldo = 2 * di;
        const SkinnyPlan p_in = skinny_plan(T, 2 * di, dm, a.X_lo != nullptr || a.norm_g != nullptr);
        if (log_enabled() && t0 == 0)
            fprintf(stderr, "[sambay] SSM step B=%lld d_model=%d d_inner=%d N=%lld R=%lld K=%lld: in-proj %d k-splits\n",
                    (long long)B, dm, di, (long long)d_state, (long long)dt_rank, (long long)d_conv, p_in.k_splits);
        e = launch_skinny(a, p_in, part, stream);
        if (e != hipSuccess) break;
        e = launch_mamba_conv(xz, 2 * di, conv_state + t0 * d_inner * (d_conv - 1), (const float *)w->conv_w,
                              (const float *)w->conv_b, u, u_hi, u_lo, T, di, (int)d_conv, stream);
        if (e != hipSuccess) break;
        SkinnyArgs b;
        b.X = u_hi;
        b.X_lo = u_lo;
        b.ldx = di;
        b.W = (const bf16_t *)w->w_x;
        b.T = T;
        b.N = Pi;
        b.K = di;
        b.epi = EPI_F32;
        b.out = xdbl;
        b.ldo = Pi;
        e = launch_skinny(b, skinny_plan(T, Pi, di, true), part, stream);
        if (e != hipSuccess) break;
        e = launch_mamba_scan(xz, 2 * di, u, xdbl, Pi, (int)dt_rank, (const bf16_t *)w->w_dt,
                              (const float *)w->dt_bias, (const float *)w->a_log, (const float *)w->d_skip,
                              ssm_state + t0 * d_inner * d_state, M_out + t0 * d_inner, g_hi, g_lo, T, di,
                              (int)d_state, stream);
        if (e != hipSuccess) break;
        SkinnyArgs o;
        o.X = g_hi;
        o.X_lo = g_lo;
        o.ldx = di;
        o.W = (const bf16_t *)w->w_out;
        o.T = T;
        o.N = dm;
        o.K = di;
        o.epi = out_epi;
        o.out = y_out + t0 * d_model;
        o.ldo = dm;
        if (dn && dn->out_defer && dn->out_defer[grp]) o.stats_out = dn->stats + t0 * dn->stride;
        e = launch_skinny(o, skinny_plan(T, dm, di, true), part, stream);
    }
    return e;
}
}  // namespace

extern "C" size_t mamba_workspace_bytes(int64_t B, int64_t d_model, int64_t d_inner, int64_t d_state,
                                        int64_t dt_rank, int64_t d_conv) {
    if (!mamba_dims_ok(B, d_model, d_inner, d_state, dt_rank, d_conv)) return 0;
    return mamba_layout(B, d_model, d_inner, d_state, dt_rank).total;
}

extern "C" sb_status mamba_decode_step(const void *x, const sb_mamba_weights *w, float *conv_state, float *ssm_state,
                                       void *M_out, void *y_out, int64_t B, int64_t d_model, int64_t d_inner,
                                       int64_t d_state, int64_t dt_rank, int64_t d_conv, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    const char *fn = "mamba_decode_step";
    if (B < 0 || d_model < 0 || d_inner < 0 || d_state < 0 || dt_rank < 0 || d_conv < 0)
        return fail(SB_EINVAL, "negative size");
    if (B == 0) return ok();
    if (d_model == 0 || d_inner == 0 || d_state == 0 || dt_rank == 0 || d_conv == 0)
        return fail(SB_EINVAL, "every dimension must be positive");
    if (!mamba_dims_ok(B, d_model, d_inner, d_state, dt_rank, d_conv))
        return fail(SB_EUNSUPPORTED,
                    "unsupported Mamba shape (d_model, d_inner multiples of 64; d_state in {8, 16, 32, 64}; "
                    "dt_rank a multiple of 8, <= %d; d_conv <= %d)", kMaxDtRank, kMaxConv);
    if (!x || !w || (!conv_state && d_conv > 1) || !ssm_state || !M_out || !y_out)
        return fail(SB_EINVAL, "null pointer");
    if (!w->w_in || !w->conv_w || !w->conv_b || !w->w_x || !w->w_dt || !w->dt_bias || !w->a_log || !w->d_skip ||
        !w->w_out)
        return fail(SB_EINVAL, "null weight");
    const void *al[] = {x, conv_state, ssm_state, M_out, y_out, w->w_in, w->conv_w, w->conv_b, w->w_x, w->w_dt,
                        w->dt_bias, w->a_log, w->d_skip, w->w_out};
    for (const void *p : al)
        if (!aligned16(p)) return fail(SB_EINVAL, "tensor base pointers must be 16-byte aligned");
    const int64_t P = dt_rank + 2 * d_state;
    const Range outs[] = {rng("conv_state", conv_state, (size_t)B * d_inner * (d_conv - 1) * 4),
                          rng("ssm_state", ssm_state, (size_t)B * d_inner * d_state * 4),
                          rng("M", M_out, (size_t)B * d_inner * 2), rng("y", y_out, (size_t)B * d_model * 2)};
    const Range ins[] = {rng("x", x, (size_t)B * d_model * 2), rng("w_in", w->w_in, (size_t)2 * d_inner * d_model * 2),
                         rng("conv_w", w->conv_w, (size_t)d_inner * d_conv * 4),
                         rng("conv_b", w->conv_b, (size_t)d_inner * 4), rng("w_x", w->w_x, (size_t)P * d_inner * 2),
                         rng("w_dt", w->w_dt, (size_t)d_inner * dt_rank * 2),
                         rng("dt_bias", w->dt_bias, (size_t)d_inner * 4),
                         rng("a_log", w->a_log, (size_t)d_inner * d_state * 4),
                         rng("d_skip", w->d_skip, (size_t)d_inner * 4),
                         rng("w_out", w->w_out, (size_t)d_model * d_inner * 2)};
    for (size_t i = 0; i < 4; ++i) {
        for (size_t j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], outs[j])) return fail(SB_EINVAL, "%s overlaps %s", outs[i].name, outs[j].name);
        for (const Range &r : ins)
            if (overlaps(outs[i], r)) return fail(SB_EINVAL, "%s overlaps %s", outs[i].name, r.name);
    }
    const MambaLayout lay = mamba_layout(B, d_model, d_inner, d_state, dt_rank);
    if (!workspace || workspace_bytes < lay.total)
        return fail(SB_EWORKSPACE, "workspace of %zu bytes needed, %zu given", lay.total,
                    workspace ? workspace_bytes : 0);
    if (!aligned16(workspace)) return fail(SB_EINVAL, "workspace must be 16-byte aligned");
    const Range rw = rng("workspace", workspace, lay.total);
    for (const Range &r : outs)
        if (overlaps(rw, r)) return fail(SB_EINVAL, "workspace overlaps %s", r.name);
    for (const Range &r : ins)
        if (overlaps(rw, r)) return fail(SB_EINVAL, "workspace overlaps %s", r.name);

    const hipError_t e = run_mamba_step((const bf16_t *)x, nullptr, w, conv_state, ssm_state, (bf16_t *)M_out,
                                        (bf16_t *)y_out, EPI_BF16, B, d_model, d_inner, d_state, dt_rank, d_conv,
                                        workspace, stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

extern "C" size_t mamba_prefill_workspace_bytes(int64_t B, int64_t T, int64_t d_model, int64_t d_inner,
                                                int64_t d_state, int64_t dt_rank, int64_t d_conv) {
    if (T <= 0 || !mamba_dims_ok(B, d_model, d_inner, d_state, dt_rank, d_conv) || dt_rank % 64 != 0) return 0;
    return round_up(mamba_prefill_workspace_need(B, T, d_inner, d_state, dt_rank));
}

extern "C" sb_status mamba_prefill(const void *x, const sb_mamba_weights *w, float *conv_state, float *ssm_state,
                                   void *M_out, void *y_out, int64_t B, int64_t T, int64_t d_model, int64_t d_inner,
                                   int64_t d_state, int64_t dt_rank, int64_t d_conv, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    const char *fn = "mamba_prefill";
    if (B < 0 || T < 0 || d_model < 0 || d_inner < 0 || d_state < 0 || dt_rank < 0 || d_conv < 0)
        return fail(SB_EINVAL, "negative size");
    if (B == 0 || T == 0) return ok();
    if (d_model == 0 || d_inner == 0 || d_state == 0 || dt_rank == 0 || d_conv == 0)
        return fail(SB_EINVAL, "every dimension must be positive");
    if (!mamba_dims_ok(B, d_model, d_inner, d_state, dt_rank, d_conv) || dt_rank % 64 != 0)
        return fail(SB_EUNSUPPORTED,
                    "unsupported Mamba prefill shape (d_model, d_inner, dt_rank multiples of 64, dt_rank <= %d; "
                    "d_state in {8, 16, 32, 64}; d_conv <= %d)", kMaxDtRank, kMaxConv);
    if (B * T > ((int64_t)1 << 31) - 1 || B > 65535 || T > 65535)
        return fail(SB_EUNSUPPORTED, "B, T <= 65535 and B*T < 2^31 required");
    if (!x || !w || (!conv_state && d_conv > 1) || !ssm_state || !M_out || !y_out)
        return fail(SB_EINVAL, "null pointer");
    if (!w->w_in || !w->conv_w || !w->conv_b || !w->w_x || !w->w_dt || !w->dt_bias || !w->a_log || !w->d_skip ||
        !w->w_out)
        return fail(SB_EINVAL, "null weight");
    const void *al[] = {x, conv_state, ssm_state, M_out, y_out, w->w_in, w->conv_w, w->conv_b, w->w_x, w->w_dt,
                        w->dt_bias, w->a_log, w->d_skip, w->w_out};
    for (const void *p : al)
        if (!aligned16(p)) return fail(SB_EINVAL, "tensor base pointers must be 16-byte aligned");
    const int64_t P = dt_rank + 2 * d_state, rows = B * T;
    const Range outs[] = {rng("conv_state", conv_state, (size_t)B * d_inner * (d_conv - 1) * 4),
                          rng("ssm_state", ssm_state, (size_t)B * d_inner * d_state * 4),
                          rng("M", M_out, (size_t)rows * d_inner * 2), rng("y", y_out, (size_t)rows * d_model * 2)};
    const Range ins[] = {rng("x", x, (size_t)rows * d_model * 2),
                         rng("w_in", w->w_in, (size_t)2 * d_inner * d_model * 2),
                         rng("conv_w", w->conv_w, (size_t)d_inner * d_conv * 4),
                         rng("conv_b", w->conv_b, (size_t)d_inner * 4), rng("w_x", w->w_x, (size_t)P * d_inner * 2),
                         rng("w_dt", w->w_dt, (size_t)d_inner * dt_rank * 2),
                         rng("dt_bias", w->dt_bias, (size_t)d_inner * 4),
                         rng("a_log", w->a_log, (size_t)d_inner * d_state * 4),
                         rng("d_skip", w->d_skip, (size_t)d_inner * 4),
                         rng("w_out", w->w_out, (size_t)d_model * d_inner * 2)};
    for (size_t i = 0; i < 4; ++i) {
        for (size_t j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], outs[j])) return fail(SB_EINVAL, "%s overlaps %s", outs[i].name, outs[j].name);
        for (const Range &r : ins)
            if (overlaps(outs[i], r)) return fail(SB_EINVAL, "%s overlaps %s", outs[i].name, r.name);
    }
    const size_t need = mamba_prefill_workspace_bytes(B, T, d_model, d_inner, d_state, dt_rank, d_conv);
    if (!workspace || workspace_bytes < need)
        return fail(SB_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    if (!aligned16(workspace)) return fail(SB_EINVAL, "workspace must be 16-byte aligned");
    const Range rw = rng("workspace", workspace, need);
    for (const Range &r : outs)
        if (overlaps(rw, r)) return fail(SB_EINVAL, "workspace overlaps %s", r.name);
    for (const Range &r : ins)
        if (overlaps(rw, r)) return fail(SB_EINVAL, "workspace overlaps %s", r.name);
    if (log_enabled())
        fprintf(stderr, "[sambay] %s B=%lld T=%lld d_model=%lld d_inner=%lld N=%lld R=%lld K=%lld\n", fn,
                (long long)B, (long long)T, (long long)d_model, (long long)d_inner, (long long)d_state,
                (long long)dt_rank, (long long)d_conv);
    hipError_t e = launch_mamba_prefill(
        (const bf16_t *)x, (const bf16_t *)w->w_in, w->conv_w, w->conv_b, (const bf16_t *)w->w_x,
        (const bf16_t *)w->w_dt, w->dt_bias, w->a_log, w->d_skip, (const bf16_t *)w->w_out, conv_state, ssm_state,
        (bf16_t *)M_out, (bf16_t *)y_out, (int)B, (int)T, (int)d_model, (int)d_inner, (int)d_state, (int)dt_rank,
        (int)d_conv, workspace, stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

namespace {

// Workspace layout of one cross-decoder step (all reused layer to layer).
struct StepLayout {
    size_t q, o, gmu, partials, total;  // o holds the bf16 hi + lo pair of the attention output
};

StepLayout step_layout(int64_t B, int64_t d_model, int64_t d_inner, int64_t Hq, int64_t Hkv, int64_t L) {
    StepLayout s;
    const int64_t T = B < kSkinnyMaxTokens ? B : kSkinnyMaxTokens;  // token group processed per product
    s.q = round_up((size_t)B * d_model * sizeof(float));
    s.o = 2 * round_up((size_t)B * d_model * sizeof(bf16_t));
    // GMU: H for one token group plus k-split partials; projections share the partial space.
    size_t part = 0;
    const size_t cands[] = {skinny_partial_bytes_max((int)T, (int)d_inner, (int)d_model),
                            skinny_partial_bytes_max((int)T, (int)d_model, (int)d_inner),
                            skinny_partial_bytes_max((int)T, (int)d_model, (int)d_model)};
    for (size_t c : cands)
        if (c > part) part = c;
    s.gmu = 2 * round_up(gmu_hidden_elems((int)T, (int)d_inner) * sizeof(bf16_t)) + round_up(part);
    s.partials = round_up(xattn_partial_bytes(B, Hq, xattn_plan(B, Hkv, L).splits));
    s.total = s.q + s.o + s.gmu + s.partials;
    return s;
}

}  // namespace

extern "C" size_t crossdecoder_workspace_bytes(int64_t B, int64_t d_model, int64_t d_inner, int64_t Hq, int64_t Hkv,
                                               int64_t D, int64_t L) {
    if (B <= 0 || d_model <= 0 || d_inner <= 0 || Hq <= 0 || Hkv <= 0 || L <= 0 || D != kHeadDim || Hq % Hkv != 0)
        return 0;
    return step_layout(B, d_model, d_inner, Hq, Hkv, L).total;
}

extern "C" sb_status crossdecoder_step(void *h, const void *M, const void *kcache, const void *vcache,
                                       const sb_layer *layers, int32_t n_layers, int64_t B, int64_t d_model,
                                       int64_t d_inner, int64_t Hq, int64_t Hkv, int64_t D, int64_t L, float scale,
                                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (B < 0 || d_model < 0 || d_inner < 0 || Hq < 0 || Hkv < 0 || D < 0 || L < 0 || n_layers < 0)
        return fail(SB_EINVAL, "negative size");
    if (B == 0 || n_layers == 0) return ok();
    sb_status st = check_xattn_shape(B, Hq, Hkv, D, L);
    if (st != SB_OK) return st;
    if (d_model == 0 || d_inner == 0) return fail(SB_EINVAL, "d_model and d_inner must be positive");
    if (Hq * D != d_model)
        return fail(SB_EINVAL, "Hq*D (%lld) != d_model (%lld)", (long long)(Hq * D), (long long)d_model);
    if (d_model % 64 != 0 || d_inner % 64 != 0)
        return fail(SB_EUNSUPPORTED, "d_model and d_inner must be multiples of 64");
    if (d_model > kMaxDim || d_inner > kMaxDim) return fail(SB_EUNSUPPORTED, "dimension >= 2^30");
    if (!h || !M || !kcache || !vcache) return fail(SB_EINVAL, "null tensor pointer");
    if (!layers) return fail(SB_EINVAL, "null layer array");
    if (!aligned16(h) || !aligned16(M) || !aligned16(kcache) || !aligned16(vcache))
        return fail(SB_EINVAL, "tensor base pointers must be 16-byte aligned");
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
        return fail(SB_EINVAL, "scale must be finite");
    const size_t kvbytes = (size_t)B * Hkv * L * D * 2;
    const Range rh = rng("h", h, (size_t)B * d_model * 2);
    const Range fixed[] = {rng("M", M, (size_t)B * d_inner * 2), rng("kcache", kcache, kvbytes),
                           rng("vcache", vcache, kvbytes)};
    for (const Range &r : fixed)
        if (overlaps(rh, r)) return fail(SB_EINVAL, "h overlaps %s", r.name);
    for (int32_t i = 0; i < n_layers; ++i) {
        const sb_layer &ly = layers[i];
        if (ly.kind != SB_LAYER_XATTN && ly.kind != SB_LAYER_GMU)
            return fail(SB_EINVAL, "layer %d: unknown kind %d", (int)i, (int)ly.kind);
        if (!ly.w_a || !ly.w_b) return fail(SB_EINVAL, "layer %d: null weight", (int)i);
        if (!aligned16(ly.w_a) || !aligned16(ly.w_b)) return fail(SB_EINVAL, "layer %d: misaligned weight", (int)i);
        const size_t ba = (size_t)(ly.kind == SB_LAYER_GMU ? d_inner : d_model) * d_model * 2;
        const size_t bb = (size_t)d_model * (ly.kind == SB_LAYER_GMU ? d_inner : d_model) * 2;
        if (overlaps(rh, rng("w_a", ly.w_a, ba)) || overlaps(rh, rng("w_b", ly.w_b, bb)))
            return fail(SB_EINVAL, "layer %d: weight overlaps h", (int)i);
    }
    const StepLayout lay = step_layout(B, d_model, d_inner, Hq, Hkv, L);
    if (!workspace || workspace_bytes < lay.total)
        return fail(SB_EWORKSPACE, "workspace of %zu bytes needed, %zu given", lay.total,
                    workspace ? workspace_bytes : 0);
    if (!aligned16(workspace)) return fail(SB_EINVAL, "workspace must be 16-byte aligned");
    const Range rw = rng("workspace", workspace, lay.total);
    if (overlaps(rw, rh)) return fail(SB_EINVAL, "workspace overlaps h");
    for (const Range &r : fixed)
        if (overlaps(rw, r)) return fail(SB_EINVAL, "workspace overlaps %s", r.name);

    char *base = static_cast<char *>(workspace);
    float *q = reinterpret_cast<float *>(base);
    bf16_t *o = reinterpret_cast<bf16_t *>(base + lay.q);
    bf16_t *o_lo = reinterpret_cast<bf16_t *>(base + lay.q + lay.o / 2);
    char *gmu_ws_base = base + lay.q + lay.o;
    void *partials = base + lay.q + lay.o + lay.gmu;
    const XattnPlan plan = xattn_plan(B, Hkv, L);
    if (log_enabled())
        fprintf(stderr, "[sambay] crossdecoder_step B=%lld layers=%d d_model=%lld d_inner=%lld L=%lld -> attention "
                        "%d chunks of %d positions; workspace %zu bytes\n",
                (long long)B, (int)n_layers, (long long)d_model, (long long)d_inner, (long long)L, plan.splits,
                plan.chunk, lay.total);
    bf16_t *hb = static_cast<bf16_t *>(h);
    const int dm = (int)d_model, di = (int)d_inner;

    for (int32_t li = 0; li < n_layers; ++li) {
        const sb_layer &ly = layers[li];
        hipError_t e = hipSuccess;
        if (ly.kind == SB_LAYER_XATTN) {
            // Projection partials share the GMU region's partial space (after the H pair).
            const int64_t Tm = B < kSkinnyMaxTokens ? B : kSkinnyMaxTokens;
            float *proj_partials =
                reinterpret_cast<float *>(gmu_ws_base + 2 * round_up(gmu_hidden_elems((int)Tm, di) * sizeof(bf16_t)));
            for (int64_t t0 = 0; t0 < B && e == hipSuccess; t0 += kSkinnyMaxTokens) {
                const int T = (int)(B - t0 < kSkinnyMaxTokens ? B - t0 : kSkinnyMaxTokens);
                SkinnyArgs aq;
                aq.X = hb + t0 * dm; aq.ldx = dm; aq.W = (const bf16_t *)ly.w_a; aq.T = T; aq.N = dm; aq.K = dm;
                aq.epi = EPI_F32; aq.out = q + t0 * dm; aq.ldo = dm;
                e = launch_skinny(aq, skinny_plan(T, dm, dm, false), proj_partials, stream);
            }
            if (e == hipSuccess)
                e = launch_xattn(q, true, (const bf16_t *)kcache, (const bf16_t *)vcache, nullptr, o, o_lo, (int)B, (int)Hq,
                                 (int)Hkv, (int)L, scale, plan, partials, stream);
            for (int64_t t0 = 0; t0 < B && e == hipSuccess; t0 += kSkinnyMaxTokens) {
                const int T = (int)(B - t0 < kSkinnyMaxTokens ? B - t0 : kSkinnyMaxTokens);
                SkinnyArgs ao;
                ao.X = o + t0 * dm; ao.X_lo = o_lo + t0 * dm; ao.ldx = dm; ao.W = (const bf16_t *)ly.w_b; ao.T = T;
                ao.N = dm; ao.K = dm; ao.epi = EPI_RESID; ao.out = hb + t0 * dm; ao.ldo = dm;
                e = launch_skinny(ao, skinny_plan(T, dm, dm, true), proj_partials, stream);
            }
        } else {
            for (int64_t t0 = 0; t0 < B && e == hipSuccess; t0 += kSkinnyMaxTokens) {
                const int T = (int)(B - t0 < kSkinnyMaxTokens ? B - t0 : kSkinnyMaxTokens);
                Carver ws{gmu_ws_base};
                e = gmu_decode_bf16((const bf16_t *)M + t0 * di, hb + t0 * dm, nullptr, dm, (const bf16_t *)ly.w_a,
                                    (const bf16_t *)ly.w_b, hb + t0 * dm, EPI_RESID, T, dm, di, true, ws, stream);
            }
        }
        if (e != hipSuccess) return hip_fail("crossdecoder_step launch", e);
    }
    return ok();
}

// ===================================================== complete cross-decoder

namespace {

// Workspace of one complete-layer step (all reused layer to layer).
struct ExLayout {
    size_t q, o, xn, gmu, mlp_u, part, attn, stats, total;
};

ExLayout ex_layout(int64_t B, int64_t d_model, int64_t d_inner, int64_t d_ff, int64_t Hq, int64_t Hkv, int64_t L) {
    ExLayout s;
    const int64_t T = B < kSkinnyMaxTokens ? B : kSkinnyMaxTokens;
    const int t = (int)T, dm = (int)d_model, di = (int)d_inner, df = (int)d_ff;
    s.q = round_up((size_t)B * d_model * sizeof(float));
    s.o = 2 * round_up((size_t)B * d_model * sizeof(bf16_t));
    s.xn = 2 * round_up((size_t)B * d_model * sizeof(bf16_t));
    s.gmu = 2 * round_up((size_t)T * d_inner * sizeof(bf16_t));
    s.mlp_u = d_ff > 0 ? 2 * round_up((size_t)T * d_ff * sizeof(bf16_t)) : 0;
    size_t part = 0;
    const int shapes[][2] = {{di, dm}, {dm, di}, {dm, dm}, {dm, df}};
    for (const auto &nk : shapes) {
        if (nk[0] <= 0 || nk[1] <= 0) continue;
        const size_t c = skinny_partial_bytes_max(t, nk[0], nk[1]);
        if (c > part) part = c;
    }
    if (df > 0) {
        const size_t c = skinny_partial_bytes_dual(t, df, skinny_plan_dual(t, df, dm));
        if (c > part) part = c;
    }
    s.part = round_up(part);
    s.attn = round_up(xattn_workspace_need(B, Hq, Hkv, L));
    s.stats = round_up((size_t)B * norm_stats_stride(dm) * sizeof(float));
    s.total = s.q + s.o + s.xn + s.gmu + s.mlp_u + s.part + s.attn + s.stats;
    return s;
}

}  // namespace

extern "C" size_t crossdecoder_ex_workspace_bytes(int64_t B, int64_t d_model, int64_t d_inner, int64_t d_ff,
                                                  int64_t Hq, int64_t Hkv, int64_t D, int64_t L) {
    if (B <= 0 || d_model <= 0 || d_inner <= 0 || d_ff < 0 || Hq <= 0 || Hkv <= 0 || L <= 0 || D != kHeadDim ||
        Hq % Hkv != 0)
        return 0;
    return ex_layout(B, d_model, d_inner, d_ff, Hq, Hkv, L).total;
}

extern "C" sb_status crossdecoder_step_ex(void *h, const void *M, const void *kcache, const void *vcache,
                                          const int32_t *lens, const sb_layer_ex *layers, int32_t n_layers, int64_t B,
                                          int64_t d_model, int64_t d_inner, int64_t d_ff, int64_t Hq, int64_t Hkv,
                                          int64_t D, int64_t L, float scale, float eps, void *workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
    if (B < 0 || d_model < 0 || d_inner < 0 || d_ff < 0 || Hq < 0 || Hkv < 0 || D < 0 || L < 0 || n_layers < 0)
        return fail(SB_EINVAL, "negative size");
    if (B == 0 || n_layers == 0) return ok();
    sb_status st = check_xattn_shape(B, Hq, Hkv, D, L);
    if (st != SB_OK) return st;
    if (d_model == 0 || d_inner == 0) return fail(SB_EINVAL, "d_model and d_inner must be positive");
    if (Hq * D != d_model)
        return fail(SB_EINVAL, "Hq*D (%lld) != d_model (%lld)", (long long)(Hq * D), (long long)d_model);
    if (d_model % 64 != 0 || d_inner % 64 != 0 || d_ff % 64 != 0)
        return fail(SB_EUNSUPPORTED, "d_model, d_inner and d_ff must be multiples of 64");
    if (d_model > kMaxDim || d_inner > kMaxDim || d_ff > kMaxDim) return fail(SB_EUNSUPPORTED, "dimension >= 2^30");
    if (!h || !M || !kcache || !vcache) return fail(SB_EINVAL, "null tensor pointer");
    if (!layers) return fail(SB_EINVAL, "null layer array");
    if (!aligned16(h) || !aligned16(M) || !aligned16(kcache) || !aligned16(vcache))
        return fail(SB_EINVAL, "tensor base pointers must be 16-byte aligned");
    if (((uintptr_t)lens & 3u) != 0) return fail(SB_EINVAL, "lens must be 4-byte aligned");
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
        return fail(SB_EINVAL, "scale must be finite");
    if (!(eps >= 0.f) || eps == __builtin_inff()) return fail(SB_EINVAL, "eps must be finite and >= 0");
    const size_t kvbytes = (size_t)B * Hkv * L * D * 2;
    const Range rh = rng("h", h, (size_t)B * d_model * 2);
    const Range fixed[] = {rng("M", M, (size_t)B * d_inner * 2), rng("kcache", kcache, kvbytes),
                           rng("vcache", vcache, kvbytes), rng("lens", lens, lens ? (size_t)B * 4 : 0)};
    for (const Range &r : fixed)
        if (overlaps(rh, r)) return fail(SB_EINVAL, "h overlaps %s", r.name);
    for (int32_t i = 0; i < n_layers; ++i) {
        const sb_layer_ex &ly = layers[i];
        if (ly.kind != SB_LAYER_XATTN && ly.kind != SB_LAYER_GMU)
            return fail(SB_EINVAL, "layer %d: unknown kind %d", (int)i, (int)ly.kind);
        if (!ly.w_a || !ly.w_b) return fail(SB_EINVAL, "layer %d: null weight", (int)i);
        const bool mlp = ly.w_gate != nullptr;
        if (mlp && (!ly.w_up || !ly.w_down)) return fail(SB_EINVAL, "layer %d: incomplete MLP", (int)i);
        if (mlp && d_ff == 0) return fail(SB_EINVAL, "layer %d has an MLP but d_ff == 0", (int)i);
        const void *ptrs[] = {ly.w_a, ly.w_b, ly.norm1, ly.norm2, ly.w_gate, ly.w_up, ly.w_down};
        for (const void *p : ptrs)
            if (!aligned16(p)) return fail(SB_EINVAL, "layer %d: misaligned weight or gain", (int)i);
        const size_t ba = (size_t)(ly.kind == SB_LAYER_GMU ? d_inner : d_model) * d_model * 2;
        const size_t bb = (size_t)d_model * (ly.kind == SB_LAYER_GMU ? d_inner : d_model) * 2;
        const Range wr[] = {rng("w_a", ly.w_a, ba), rng("w_b", ly.w_b, bb),
                            rng("norm1", ly.norm1, ly.norm1 ? (size_t)d_model * 2 : 0),
                            rng("norm2", ly.norm2, ly.norm2 ? (size_t)d_model * 2 : 0),
                            rng("w_gate", ly.w_gate, mlp ? (size_t)d_ff * d_model * 2 : 0),
                            rng("w_up", ly.w_up, mlp ? (size_t)d_ff * d_model * 2 : 0),
                            rng("w_down", ly.w_down, mlp ? (size_t)d_model * d_ff * 2 : 0)};
        for (const Range &r : wr)
            if (overlaps(rh, r)) return fail(SB_EINVAL, "layer %d: %s overlaps h", (int)i, r.name);
    }
    const ExLayout lay = ex_layout(B, d_model, d_inner, d_ff, Hq, Hkv, L);
    if (!workspace || workspace_bytes < lay.total)
        return fail(SB_EWORKSPACE, "workspace of %zu bytes needed, %zu given", lay.total,
                    workspace ? workspace_bytes : 0);
    if (!aligned16(workspace)) return fail(SB_EINVAL, "workspace must be 16-byte aligned");
    const Range rw = rng("workspace", workspace, lay.total);
    if (overlaps(rw, rh)) return fail(SB_EINVAL, "workspace overlaps h");
    for (const Range &r : fixed)
        if (overlaps(rw, r)) return fail(SB_EINVAL, "workspace overlaps %s", r.name);

    char *p = static_cast<char *>(workspace);
    float *q = reinterpret_cast<float *>(p);
    p += lay.q;
    bf16_t *o = reinterpret_cast<bf16_t *>(p), *o_lo = reinterpret_cast<bf16_t *>(p + lay.o / 2);
    p += lay.o;
    bf16_t *xn = reinterpret_cast<bf16_t *>(p), *xn_lo = reinterpret_cast<bf16_t *>(p + lay.xn / 2);
    p += lay.xn;
    bf16_t *H = reinterpret_cast<bf16_t *>(p), *H_lo = reinterpret_cast<bf16_t *>(p + lay.gmu / 2);
    p += lay.gmu;
    bf16_t *U = reinterpret_cast<bf16_t *>(p), *U_lo = reinterpret_cast<bf16_t *>(p + lay.mlp_u / 2);
    p += lay.mlp_u;
    float *part = reinterpret_cast<float *>(p);
    p += lay.part;
    void *attn_part = p;
    p += lay.attn;
    float *stats = reinterpret_cast<float *>(p);
    const XattnPlan plan = xattn_plan(B, Hkv, L, lens != nullptr);
    if (log_enabled())
        fprintf(stderr, "[sambay] crossdecoder_step_ex B=%lld layers=%d d_model=%lld d_inner=%lld d_ff=%lld L=%lld%s "
                        "-> attention %d chunks of %d positions; workspace %zu bytes\n",
                (long long)B, (int)n_layers, (long long)d_model, (long long)d_inner, (long long)d_ff, (long long)L,
                lens ? " (ragged)" : "", plan.splits, plan.chunk, lay.total);
    bf16_t *hb = static_cast<bf16_t *>(h);
    const int dm = (int)d_model, di = (int)d_inner, df = (int)d_ff;

    // A sublayer's input RMSNorm(h; g) is either materialised in xn (hi + lo)
    // or deferred: the residual product that last wrote h left each token's
    // chunk sums of squares in `stats`, and the products that read the input
    // normalise their own K slab while staging it (the slab product; same
    // bits as the RMSNorm kernel).  Deferred per token group of <= 64 rows
    // when the residual product and every consumer of the input run as slab
    // products; never for the first layer's input.
    const int sstride = norm_stats_stride(dm);
    constexpr int kMaxGroups = 64;
    bool deferred[kMaxGroups] = {};
    const bool may_defer = (B + kSkinnyMaxTokens - 1) / kSkinnyMaxTokens <= kMaxGroups;
    auto group = [](int64_t t0) { return (int)(t0 / kSkinnyMaxTokens); };
    // The operand of a product of group t0 whose input is RMSNorm(h; g) (g
    // null: h itself).
    auto operand = [&](SkinnyArgs &a, int64_t t0, const void *g) {
        a.ldx = dm;
        if (g && deferred[group(t0)]) {
            a.X = hb + t0 * dm; a.X_lo = nullptr;
            a.norm_g = (const bf16_t *)g; a.norm_stats = stats + t0 * sstride; a.norm_eps = eps;
        } else if (g) {
            a.X = xn + t0 * dm; a.X_lo = xn_lo + t0 * dm;
        } else {
            a.X = hb + t0 * dm; a.X_lo = nullptr;
        }
    };
    auto plan_of = [](const SkinnyArgs &a) { return skinny_plan(a.T, a.N, a.K, a.X_lo != nullptr || a.norm_g != nullptr); };
    // Whether the mixer of layer i (if any) reads its normalised input through the slab product at T tokens.
    auto mixer_takes = [&](int32_t i, int T) {
        if (i >= n_layers || !layers[i].norm1) return false;
        return layers[i].kind == SB_LAYER_XATTN ? slab_norm_ok(T, dm, dm) : slab_norm_ok(T, di, dm);
    };
    // The residual product of a group; when `next_norm` is set the group's
    // rows of the next sublayer's input RMSNorm(h; next_norm) are prepared
    // too: deferred (statistics from this product's finishing pass) when
    // `defer` allows and this product runs as the slab product, else
    // materialised in xn inside the K-split finishing pass or by a separate
    // launch.
    auto residual = [&](const bf16_t *X, const bf16_t *X_lo, int ldx, const void *W, int K, int64_t t0, int T,
                        const void *next_norm, bool defer) -> hipError_t {
        SkinnyArgs a;
        a.X = X; a.X_lo = X_lo; a.ldx = ldx; a.W = (const bf16_t *)W; a.T = T; a.N = dm; a.K = K;
        a.epi = EPI_RESID; a.out = hb + t0 * dm; a.ldo = dm;
        const SkinnyPlan plan_r = plan_of(a);
        const bool d = next_norm && defer && may_defer && plan_r.slab_rtw > 0;
        deferred[group(t0)] = d;
        if (d) {
            a.stats_out = stats + t0 * sstride;
            return launch_skinny(a, plan_r, part, stream);
        }
        a.next_norm = (const bf16_t *)next_norm; a.next_x = xn + t0 * dm; a.next_x_lo = xn_lo + t0 * dm;
        a.eps = eps;
        hipError_t e = launch_skinny(a, plan_r, part, stream);
        if (e == hipSuccess && next_norm && !skinny_fuses_norm(a, plan_r))
            e = launch_rmsnorm(hb + t0 * dm, (const bf16_t *)next_norm, T, dm, eps, xn + t0 * dm, xn_lo + t0 * dm,
                               stream);
        return e;
    };

    // xn holds RMSNorm(h) for the first sublayer when its gain is set.
    hipError_t e0 = layers[0].norm1
                        ? launch_rmsnorm(hb, (const bf16_t *)layers[0].norm1, (int)B, dm, eps, xn, xn_lo, stream)
                        : hipSuccess;
    if (e0 != hipSuccess) return hip_fail("crossdecoder_step_ex launch", e0);
    for (int32_t li = 0; li < n_layers; ++li) {
        const sb_layer_ex &ly = layers[li];
        const bool mlp = ly.w_gate != nullptr;
        const void *after_mixer = mlp ? ly.norm2 : (li + 1 < n_layers ? layers[li + 1].norm1 : nullptr);
        const void *after_mlp = li + 1 < n_layers ? layers[li + 1].norm1 : nullptr;
        hipError_t e = hipSuccess;
        for (int64_t t0 = 0; t0 < B && e == hipSuccess; t0 += kSkinnyMaxTokens) {
            const int T = (int)(B - t0 < kSkinnyMaxTokens ? B - t0 : kSkinnyMaxTokens);
            const bool defer_mixer = mlp ? slab_norm_ok(T, 2 * df, dm) : mixer_takes(li + 1, T);
            if (ly.kind == SB_LAYER_XATTN) {
                SkinnyArgs a;
                operand(a, t0, ly.norm1);
                a.W = (const bf16_t *)ly.w_a; a.T = T; a.N = dm; a.K = dm; a.epi = EPI_F32; a.out = q + t0 * dm;
                a.ldo = dm;
                e = launch_skinny(a, plan_of(a), part, stream);
            } else {
                SkinnyArgs a1;
                operand(a1, t0, ly.norm1);
                a1.W = (const bf16_t *)ly.w_a; a1.T = T; a1.N = di; a1.K = dm; a1.epi = EPI_GATE;
                a1.out = H; a1.ldo = di; a1.out_lo = H_lo; a1.aux = (const bf16_t *)M + t0 * di; a1.ldaux = di;
                e = launch_skinny(a1, plan_of(a1), part, stream);
                if (e == hipSuccess) e = residual(H, H_lo, di, ly.w_b, di, t0, T, after_mixer, defer_mixer);
            }
        }
        if (e == hipSuccess && ly.kind == SB_LAYER_XATTN) {
            e = launch_xattn(q, true, (const bf16_t *)kcache, (const bf16_t *)vcache, lens, o, o_lo, (int)B, (int)Hq,
                             (int)Hkv, (int)L, scale, plan, attn_part, stream);
            for (int64_t t0 = 0; t0 < B && e == hipSuccess; t0 += kSkinnyMaxTokens) {
                const int T = (int)(B - t0 < kSkinnyMaxTokens ? B - t0 : kSkinnyMaxTokens);
                const bool defer_mixer = mlp ? slab_norm_ok(T, 2 * df, dm) : mixer_takes(li + 1, T);
                e = residual(o + t0 * dm, o_lo + t0 * dm, dm, ly.w_b, dm, t0, T, after_mixer, defer_mixer);
            }
        }
        if (e == hipSuccess && mlp) {
            for (int64_t t0 = 0; t0 < B && e == hipSuccess; t0 += kSkinnyMaxTokens) {
                const int T = (int)(B - t0 < kSkinnyMaxTokens ? B - t0 : kSkinnyMaxTokens);
                SkinnyArgs a;  // gate and up weights streamed in one pass
                operand(a, t0, ly.norm2);
                a.W = (const bf16_t *)ly.w_gate; a.W_b = (const bf16_t *)ly.w_up; a.T = T; a.N = df; a.K = dm;
                a.epi = EPI_SWIGLU; a.out = U; a.ldo = df; a.out_lo = U_lo;
                e = launch_skinny(a, skinny_plan_dual(T, df, dm), part, stream);
                if (e == hipSuccess) e = residual(U, U_lo, df, ly.w_down, df, t0, T, after_mlp, mixer_takes(li + 1, T));
            }
        }
        if (e != hipSuccess) return hip_fail("crossdecoder_step_ex launch", e);
    }
    return ok();
}

// ===================================================== YOCO-style prefill

namespace {

size_t sambay_prefill_ws(int64_t B, int64_t T, int64_t d_model, int64_t d_inner, int64_t d_state, int64_t dt_rank,
                         int64_t d_ff, int64_t Hq, int64_t Hkv, int64_t L, bool cross) {
    const size_t self = round_up(self_decoder_layout(nullptr, B, T, d_model, d_inner, d_state, dt_rank, d_ff, Hq,
                                                     Hkv).bytes);
    return self + (cross ? round_up(ex_layout(B, d_model, d_inner, d_ff, Hq, Hkv, L).total) : 0);
}

bool prefill_dims_ok(int64_t B, int64_t T, int64_t d_model, int64_t d_inner, int64_t d_state, int64_t dt_rank,
                     int64_t d_conv, int64_t d_ff, int64_t Hq, int64_t Hkv, int64_t D, int64_t L) {
    return B > 0 && T > 0 && T <= L && B <= 65535 && T <= 65535 && B * T < ((int64_t)1 << 31) && D == kHeadDim &&
           Hq > 0 && Hkv > 0 && Hq % Hkv == 0 && Hq * D == d_model && d_ff >= 0 && d_ff % 64 == 0 &&
           d_ff <= kMaxDim && L <= kMaxDim && mamba_dims_ok(B, d_model, d_inner, d_state, dt_rank, d_conv) &&
           dt_rank % 64 == 0;
}

}  // namespace

extern "C" size_t sambay_prefill_workspace_bytes(int64_t B, int64_t T, int64_t d_model, int64_t d_inner,
                                                 int64_t d_state, int64_t dt_rank, int64_t d_conv, int64_t d_ff,
                                                 int64_t Hq, int64_t Hkv, int64_t D, int64_t L) {
    if (!prefill_dims_ok(B, T, d_model, d_inner, d_state, dt_rank, d_conv, d_ff, Hq, Hkv, D, L)) return 0;
    return sambay_prefill_ws(B, T, d_model, d_inner, d_state, dt_rank, d_ff, Hq, Hkv, L, true);
}

extern "C" sb_status sambay_prefill(const void *x, void *h_out, void *M_out, const sb_self_layer *self_layers,
                                    int32_t n_self, const sb_layer_ex *cross_layers, int32_t n_cross, void *kcache,
                                    void *vcache, int64_t B, int64_t T, int64_t d_model, int64_t d_inner,
                                    int64_t d_state, int64_t dt_rank, int64_t d_conv, int64_t d_ff, int64_t Hq,
                                    int64_t Hkv, int64_t D, int64_t L, int64_t window, float scale, float eps,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const char *fn = "sambay_prefill";
    if (B < 0 || T < 0 || d_model < 0 || d_inner < 0 || d_state < 0 || dt_rank < 0 || d_conv < 0 || d_ff < 0 ||
        Hq < 0 || Hkv < 0 || D < 0 || L < 0 || window < 0 || n_self < 0 || n_cross < 0)
        return fail(SB_EINVAL, "negative size");
    if (B == 0) return ok();
    if (T == 0) return fail(SB_EINVAL, "an empty prompt has no last token");
    if (!prefill_dims_ok(B, T, d_model, d_inner, d_state, dt_rank, d_conv, d_ff, Hq, Hkv, D, L))
        return fail(SB_EUNSUPPORTED,
                    "unsupported prefill shape (D == 128, Hq %% Hkv == 0, Hq*D == d_model; d_model, d_inner, d_ff, "
                    "dt_rank multiples of 64, dt_rank <= %d; d_state in {8, 16, 32, 64}; d_conv <= %d; "
                    "1 <= T <= L; B, T <= 65535)", kMaxDtRank, kMaxConv);
    if (!x || !h_out || !kcache || !vcache) return fail(SB_EINVAL, "null tensor pointer");
    if (n_self > 0 && !self_layers) return fail(SB_EINVAL, "null self-decoder layer array");
    if (n_cross > 0 && !cross_layers) return fail(SB_EINVAL, "null cross-decoder layer array");
    if (!aligned16(x) || !aligned16(h_out) || !aligned16(M_out) || !aligned16(kcache) || !aligned16(vcache))
        return fail(SB_EINVAL, "tensor base pointers must be 16-byte aligned");
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
        return fail(SB_EINVAL, "scale must be finite");
    if (!(eps >= 0.f) || eps == __builtin_inff()) return fail(SB_EINVAL, "eps must be finite and >= 0");
    const int64_t rows = B * T, kvd = Hkv * D;
    const size_t kvbytes = (size_t)B * Hkv * L * D * 2;
    // Everything the call writes, against each other and everything it reads.
    std::vector<Range> outs = {rng("h_out", h_out, (size_t)B * d_model * 2),
                               rng("M_out", M_out, M_out ? (size_t)B * d_inner * 2 : 0),
                               rng("kcache", kcache, kvbytes), rng("vcache", vcache, kvbytes)};
    std::vector<Range> ins = {rng("x", x, (size_t)rows * d_model * 2)};
    bool has_attn = false, has_mamba = false, has_swa = false;
    for (int32_t i = 0; i < n_self; ++i) {
        const sb_self_layer &ly = self_layers[i];
        const bool mlp = ly.w_gate != nullptr;
        if (mlp && (!ly.w_up || !ly.w_down)) return fail(SB_EINVAL, "self layer %d: incomplete MLP", (int)i);
        if (mlp && d_ff == 0) return fail(SB_EINVAL, "self layer %d has an MLP but d_ff == 0", (int)i);
        const void *common[] = {ly.norm1, ly.norm2, ly.w_gate, ly.w_up, ly.w_down};
        for (const void *p : common)
            if (!aligned16(p)) return fail(SB_EINVAL, "self layer %d: misaligned weight or gain", (int)i);
        ins.push_back(rng("norm1", ly.norm1, ly.norm1 ? (size_t)d_model * 2 : 0));
        ins.push_back(rng("norm2", ly.norm2, ly.norm2 ? (size_t)d_model * 2 : 0));
        ins.push_back(rng("w_gate", ly.w_gate, mlp ? (size_t)d_ff * d_model * 2 : 0));
        ins.push_back(rng("w_up", ly.w_up, mlp ? (size_t)d_ff * d_model * 2 : 0));
        ins.push_back(rng("w_down", ly.w_down, mlp ? (size_t)d_model * d_ff * 2 : 0));
        if (ly.kind == SB_SELF_MAMBA) {
            has_mamba = true;
            const sb_mamba_weights &w = ly.mamba;
            if (!w.w_in || !w.conv_w || !w.conv_b || !w.w_x || !w.w_dt || !w.dt_bias || !w.a_log || !w.d_skip ||
                !w.w_out)
                return fail(SB_EINVAL, "self layer %d: null SSM weight", (int)i);
            if (!ly.ssm_state || (!ly.conv_state && d_conv > 1))
                return fail(SB_EINVAL, "self layer %d: null SSM state", (int)i);
            const void *al[] = {w.w_in, w.conv_w, w.conv_b, w.w_x, w.w_dt, w.dt_bias, w.a_log, w.d_skip, w.w_out,
                                ly.conv_state, ly.ssm_state};
            for (const void *p : al)
                if (!aligned16(p)) return fail(SB_EINVAL, "self layer %d: misaligned SSM tensor", (int)i);
            const int64_t P = dt_rank + 2 * d_state;
            outs.push_back(rng("conv_state", ly.conv_state, (size_t)B * d_inner * (d_conv - 1) * 4));
            outs.push_back(rng("ssm_state", ly.ssm_state, (size_t)B * d_inner * d_state * 4));
            ins.push_back(rng("w_in", w.w_in, (size_t)2 * d_inner * d_model * 2));
            ins.push_back(rng("conv_w", w.conv_w, (size_t)d_inner * d_conv * 4));
            ins.push_back(rng("conv_b", w.conv_b, (size_t)d_inner * 4));
            ins.push_back(rng("w_x", w.w_x, (size_t)P * d_inner * 2));
            ins.push_back(rng("w_dt", w.w_dt, (size_t)d_inner * dt_rank * 2));
            ins.push_back(rng("dt_bias", w.dt_bias, (size_t)d_inner * 4));
            ins.push_back(rng("a_log", w.a_log, (size_t)d_inner * d_state * 4));
            ins.push_back(rng("d_skip", w.d_skip, (size_t)d_inner * 4));
            ins.push_back(rng("w_out", w.w_out, (size_t)d_model * d_inner * 2));
        } else if (ly.kind == SB_SELF_SWA || ly.kind == SB_SELF_ATTN) {
            if (!ly.wq || !ly.wk || !ly.wv || !ly.wo)
                return fail(SB_EINVAL, "self layer %d: null attention weight", (int)i);
            const void *al[] = {ly.wq, ly.wk, ly.wv, ly.wo, ly.kring, ly.vring};
            for (const void *p : al)
                if (!aligned16(p)) return fail(SB_EINVAL, "self layer %d: misaligned attention tensor", (int)i);
            ins.push_back(rng("wq", ly.wq, (size_t)d_model * d_model * 2));
            ins.push_back(rng("wk", ly.wk, (size_t)kvd * d_model * 2));
            ins.push_back(rng("wv", ly.wv, (size_t)kvd * d_model * 2));
            ins.push_back(rng("wo", ly.wo, (size_t)d_model * d_model * 2));
            if (ly.kind == SB_SELF_SWA) {
                has_swa = true;
                if (!ly.kring || !ly.vring) return fail(SB_EINVAL, "self layer %d: null ring cache", (int)i);
                const size_t rb = (size_t)B * Hkv * (window > 0 ? window : 0) * D * 2;
                outs.push_back(rng("kring", ly.kring, rb));
                outs.push_back(rng("vring", ly.vring, rb));
            } else {
                has_attn = true;
            }
        } else {
            return fail(SB_EINVAL, "self layer %d: unknown kind %d", (int)i, (int)ly.kind);
        }
    }
    if (has_swa && (window < 1 || window > 65535))
        return fail(SB_EUNSUPPORTED, "a sliding-window layer needs 1 <= window <= 65535");
    for (int32_t i = 0; i < n_cross; ++i) {
        if (cross_layers[i].kind == SB_LAYER_XATTN && !has_attn)
            return fail(SB_EINVAL, "cross layer %d attends to a cache no self-decoder layer writes", (int)i);
        if (cross_layers[i].kind == SB_LAYER_GMU && !has_mamba)
            return fail(SB_EINVAL, "cross layer %d gates a memory no SSM layer produces", (int)i);
    }
    for (size_t i = 0; i < outs.size(); ++i) {
        for (size_t j = i + 1; j < outs.size(); ++j)
            if (overlaps(outs[i], outs[j])) return fail(SB_EINVAL, "%s overlaps %s", outs[i].name, outs[j].name);
        for (const Range &r : ins)
            if (overlaps(outs[i], r)) return fail(SB_EINVAL, "%s overlaps %s", outs[i].name, r.name);
    }
    // A final full-attention layer finishes on the last token only, as the
    // first layer of the cross-decoder step.
    const bool last_kv_only = n_self > 0 && self_layers[n_self - 1].kind == SB_SELF_ATTN;
    const size_t need =
        sambay_prefill_ws(B, T, d_model, d_inner, d_state, dt_rank, d_ff, Hq, Hkv, L, n_cross > 0 || last_kv_only);
    if (!workspace || workspace_bytes < need)
        return fail(SB_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    if (!aligned16(workspace)) return fail(SB_EINVAL, "workspace must be 16-byte aligned");
    const Range rw = rng("workspace", workspace, need);
    for (const Range &r : outs)
        if (overlaps(rw, r)) return fail(SB_EINVAL, "workspace overlaps %s", r.name);
    for (const Range &r : ins)
        if (overlaps(rw, r)) return fail(SB_EINVAL, "workspace overlaps %s", r.name);
    if (log_enabled())
        fprintf(stderr, "[sambay] %s B=%lld T=%lld self=%d cross=%d d_model=%lld window=%lld workspace %zu bytes\n",
                fn, (long long)B, (long long)T, (int)n_self, (int)n_cross, (long long)d_model, (long long)window,
                need);

    const SelfDecoderLayout lay = self_decoder_layout(workspace, B, T, d_model, d_inner, d_state, dt_rank, d_ff, Hq,
                                                      Hkv);
    // M_last for the cross-decoder: the caller's M_out, else workspace rows.
    bf16_t *m_last = M_out ? static_cast<bf16_t *>(M_out) : lay.m_last;
    SelfDecoderArgs a;
    a.x = (const bf16_t *)x; a.layers = self_layers; a.n = n_self;
    a.B = (int)B; a.T = (int)T; a.d_model = (int)d_model; a.d_inner = (int)d_inner; a.d_state = (int)d_state;
    a.dt_rank = (int)dt_rank; a.d_conv = (int)d_conv; a.d_ff = (int)d_ff; a.Hq = (int)Hq; a.Hkv = (int)Hkv;
    a.L = (int)L; a.window = (int)window; a.scale = scale; a.eps = eps; a.kcache = kcache; a.vcache = vcache;
    a.h_out = static_cast<bf16_t *>(h_out); a.M_out = m_last; a.last_kv_only = last_kv_only;
    hipError_t e = launch_self_decoder(a, lay, stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    std::vector<sb_layer_ex> cross;
    if (last_kv_only) {
        const sb_self_layer &ly = self_layers[n_self - 1];
        cross.push_back(sb_layer_ex{SB_LAYER_XATTN, ly.wq, ly.wo, ly.norm1, ly.norm2, ly.w_gate, ly.w_up, ly.w_down});
    }
    for (int32_t i = 0; i < n_cross; ++i) cross.push_back(cross_layers[i]);
    if (cross.empty()) return ok();
    char *cws = static_cast<char *>(workspace) + round_up(lay.bytes);
    const size_t cbytes = need - round_up(lay.bytes);
    return crossdecoder_step_ex(h_out, m_last, kcache, vcache, lay.lens, cross.data(), (int32_t)cross.size(), B,
                                d_model, d_inner, d_ff, Hq, Hkv, D, L, scale, eps, cws, cbytes, stream);
}

// ====================================================== whole-model decode

namespace {

// Workspace of one whole-model decode step: per-layer activations (reused
// layer to layer), the cache lengths, then the SSM step's, the attention's
// and the cross-decoder step's own regions.
struct DecodeLayout {
    size_t xn, xn_lo, q, kn, vn, o, o_lo, m, lens, lens_ring, hid, hid_lo, stats, part, attn, ssm, cross, total;
};

DecodeLayout decode_layout(int64_t B, int64_t d_model, int64_t d_inner, int64_t d_state, int64_t dt_rank,
                           int64_t d_ff, int64_t Hq, int64_t Hkv, int64_t L, int64_t window) {
    const int64_t T = B < kSkinnyMaxTokens ? B : kSkinnyMaxTokens;
    const int t = (int)T, dm = (int)d_model, kvd = (int)(Hkv * kHeadDim), df = (int)d_ff;
    DecodeLayout l;
    Carver c{nullptr};
    l.xn = c.used; c.take((size_t)B * d_model * 2);
    l.xn_lo = c.used; c.take((size_t)B * d_model * 2);
    l.q = c.used; c.take((size_t)B * d_model * 2);
    l.kn = c.used; c.take((size_t)B * kvd * 2);
    l.vn = c.used; c.take((size_t)B * kvd * 2);
    l.o = c.used; c.take((size_t)B * d_model * 2);
    l.o_lo = c.used; c.take((size_t)B * d_model * 2);
    l.m = c.used; c.take((size_t)B * d_inner * 2);
    l.lens = c.used; c.take((size_t)B * 4);
    l.lens_ring = c.used; c.take((size_t)B * 4);
    l.hid = c.used; c.take((size_t)T * (d_ff > 0 ? d_ff : 1) * 2);
    l.hid_lo = c.used; c.take((size_t)T * (d_ff > 0 ? d_ff : 1) * 2);
    l.stats = c.used; c.take((size_t)B * norm_stats_stride(dm) * 4);
    size_t part = 0;
    const int shapes[][2] = {{dm, dm}, {kvd, dm}, {dm + 2 * kvd, dm}, {dm, df}};
    for (const auto &nk : shapes) {
        if (nk[0] <= 0 || nk[1] <= 0) continue;
        const size_t v = skinny_partial_bytes_max(t, nk[0], nk[1]);
        if (v > part) part = v;
    }
    if (df > 0) {
        const size_t v = skinny_partial_bytes_dual(t, df, skinny_plan_dual(t, df, dm));
        if (v > part) part = v;
    }
    l.part = c.used; c.take(part);
    const int64_t Lmax = L > window ? L : window;
    l.attn = c.used; c.take(xattn_workspace_need(B, Hq, Hkv, Lmax));
    l.ssm = c.used; c.take(mamba_layout(B, d_model, d_inner, d_state, dt_rank).total);
    l.cross = c.used; c.take(ex_layout(B, d_model, d_inner, d_ff, Hq, Hkv, L).total);
    l.total = c.used;
    return l;
}

bool decode_dims_ok(int64_t B, int64_t d_model, int64_t d_inner, int64_t d_state, int64_t dt_rank, int64_t d_conv,
                    int64_t d_ff, int64_t Hq, int64_t Hkv, int64_t D, int64_t L) {
    return B > 0 && D == kHeadDim && Hq > 0 && Hkv > 0 && Hq % Hkv == 0 && Hq * D == d_model && Hq <= 65535 &&
           L > 0 && L <= kMaxDim && d_ff >= 0 && d_ff % 64 == 0 && d_ff <= kMaxDim &&
           mamba_dims_ok(B, d_model, d_inner, d_state, dt_rank, d_conv);
}

}  // namespace

extern "C" size_t sambay_decode_workspace_bytes(int64_t B, int64_t d_model, int64_t d_inner, int64_t d_state,
                                                int64_t dt_rank, int64_t d_conv, int64_t d_ff, int64_t Hq,
                                                int64_t Hkv, int64_t D, int64_t L, int64_t window) {
    if (!decode_dims_ok(B, d_model, d_inner, d_state, dt_rank, d_conv, d_ff, Hq, Hkv, D, L) || window < 0)
        return 0;
    return decode_layout(B, d_model, d_inner, d_state, dt_rank, d_ff, Hq, Hkv, L, window).total;
}

extern "C" sb_status sambay_decode_step(void *h, void *M_out, const sb_self_layer *self_layers, int32_t n_self,
                                        const sb_layer_ex *cross_layers, int32_t n_cross, void *kcache, void *vcache,
                                        const int32_t *pos, int64_t B, int64_t d_model, int64_t d_inner,
                                        int64_t d_state, int64_t dt_rank, int64_t d_conv, int64_t d_ff, int64_t Hq,
                                        int64_t Hkv, int64_t D, int64_t L, int64_t window, float scale, float eps,
                                        void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const char *fn = "sambay_decode_step";
    if (B < 0 || d_model < 0 || d_inner < 0 || d_state < 0 || dt_rank < 0 || d_conv < 0 || d_ff < 0 || Hq < 0 ||
        Hkv < 0 || D < 0 || L < 0 || window < 0 || n_self < 0 || n_cross < 0)
        return fail(SB_EINVAL, "negative size");
    if (B == 0) return ok();
    if (!decode_dims_ok(B, d_model, d_inner, d_state, dt_rank, d_conv, d_ff, Hq, Hkv, D, L))
        return fail(SB_EUNSUPPORTED,
                    "unsupported decode shape (D == 128, Hq %% Hkv == 0, Hq*D == d_model; d_model, d_inner, d_ff "
                    "multiples of 64; d_state in {8, 16, 32, 64}; dt_rank a multiple of 8, <= %d; d_conv <= %d)",
                    kMaxDtRank, kMaxConv);
    if (!h || !kcache || !vcache || !pos) return fail(SB_EINVAL, "null tensor pointer");
    if (n_self > 0 && !self_layers) return fail(SB_EINVAL, "null self-decoder layer array");
    if (n_cross > 0 && !cross_layers) return fail(SB_EINVAL, "null cross-decoder layer array");
    if (!aligned16(h) || !aligned16(M_out) || !aligned16(kcache) || !aligned16(vcache))
        return fail(SB_EINVAL, "tensor base pointers must be 16-byte aligned");
    if (((uintptr_t)pos & 3u) != 0) return fail(SB_EINVAL, "pos must be 4-byte aligned");
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
        return fail(SB_EINVAL, "scale must be finite");
    if (!(eps >= 0.f) || eps == __builtin_inff()) return fail(SB_EINVAL, "eps must be finite and >= 0");
    const int64_t kvd = Hkv * D;
    const size_t kvbytes = (size_t)B * Hkv * L * D * 2;
    std::vector<Range> outs = {rng("h", h, (size_t)B * d_model * 2),
                               rng("M_out", M_out, M_out ? (size_t)B * d_inner * 2 : 0),
                               rng("kcache", kcache, kvbytes), rng("vcache", vcache, kvbytes)};
    std::vector<Range> ins = {rng("pos", pos, (size_t)B * 4)};
    bool has_attn = false, has_mamba = false, has_swa = false;
    for (int32_t i = 0; i < n_self; ++i) {
        const sb_self_layer &ly = self_layers[i];
        const bool mlp = ly.w_gate != nullptr;
        if (mlp && (!ly.w_up || !ly.w_down)) return fail(SB_EINVAL, "self layer %d: incomplete MLP", (int)i);
        if (mlp && d_ff == 0) return fail(SB_EINVAL, "self layer %d has an MLP but d_ff == 0", (int)i);
        const void *common[] = {ly.norm1, ly.norm2, ly.w_gate, ly.w_up, ly.w_down};
        for (const void *p : common)
            if (!aligned16(p)) return fail(SB_EINVAL, "self layer %d: misaligned weight or gain", (int)i);
        ins.push_back(rng("w_gate", ly.w_gate, mlp ? (size_t)d_ff * d_model * 2 : 0));
        ins.push_back(rng("w_up", ly.w_up, mlp ? (size_t)d_ff * d_model * 2 : 0));
        ins.push_back(rng("w_down", ly.w_down, mlp ? (size_t)d_model * d_ff * 2 : 0));
        if (ly.kind == SB_SELF_MAMBA) {
            has_mamba = true;
            const sb_mamba_weights &w = ly.mamba;
            if (!w.w_in || !w.conv_w || !w.conv_b || !w.w_x || !w.w_dt || !w.dt_bias || !w.a_log || !w.d_skip ||
                !w.w_out)
                return fail(SB_EINVAL, "self layer %d: null SSM weight", (int)i);
            if (!ly.ssm_state || (!ly.conv_state && d_conv > 1))
                return fail(SB_EINVAL, "self layer %d: null SSM state", (int)i);
            const void *al[] = {w.w_in, w.conv_w, w.conv_b, w.w_x, w.w_dt, w.dt_bias, w.a_log, w.d_skip, w.w_out,
                                ly.conv_state, ly.ssm_state};
            for (const void *p : al)
                if (!aligned16(p)) return fail(SB_EINVAL, "self layer %d: misaligned SSM tensor", (int)i);
            outs.push_back(rng("conv_state", ly.conv_state, (size_t)B * d_inner * (d_conv - 1) * 4));
            outs.push_back(rng("ssm_state", ly.ssm_state, (size_t)B * d_inner * d_state * 4));
            ins.push_back(rng("w_in", w.w_in, (size_t)2 * d_inner * d_model * 2));
            ins.push_back(rng("w_out", w.w_out, (size_t)d_model * d_inner * 2));
        } else if (ly.kind == SB_SELF_SWA || ly.kind == SB_SELF_ATTN) {
            if (!ly.wq || !ly.wk || !ly.wv || !ly.wo)
                return fail(SB_EINVAL, "self layer %d: null attention weight", (int)i);
            const void *al[] = {ly.wq, ly.wk, ly.wv, ly.wo, ly.kring, ly.vring};
            for (const void *p : al)
                if (!aligned16(p)) return fail(SB_EINVAL, "self layer %d: misaligned attention tensor", (int)i);
            ins.push_back(rng("wq", ly.wq, (size_t)d_model * d_model * 2));
            ins.push_back(rng("wk", ly.wk, (size_t)kvd * d_model * 2));
            ins.push_back(rng("wv", ly.wv, (size_t)kvd * d_model * 2));
            ins.push_back(rng("wo", ly.wo, (size_t)d_model * d_model * 2));
            if (ly.kind == SB_SELF_SWA) {
                has_swa = true;
                if (!ly.kring || !ly.vring) return fail(SB_EINVAL, "self layer %d: null ring cache", (int)i);
                const size_t rb = (size_t)B * Hkv * (window > 0 ? window : 0) * D * 2;
                outs.push_back(rng("kring", ly.kring, rb));
                outs.push_back(rng("vring", ly.vring, rb));
            } else {
                if (has_attn) return fail(SB_EINVAL, "self layer %d: a second full-attention layer", (int)i);
                has_attn = true;
            }
        } else {
            return fail(SB_EINVAL, "self layer %d: unknown kind %d", (int)i, (int)ly.kind);
        }
    }
    if (has_swa && (window < 1 || window > kMaxDim))
        return fail(SB_EUNSUPPORTED, "a sliding-window layer needs 1 <= window < 2^30");
    for (int32_t i = 0; i < n_cross; ++i) {
        if (cross_layers[i].kind == SB_LAYER_XATTN && !has_attn)
            return fail(SB_EINVAL, "cross layer %d attends to a cache no self-decoder layer writes", (int)i);
        if (cross_layers[i].kind == SB_LAYER_GMU && !has_mamba)
            return fail(SB_EINVAL, "cross layer %d gates a memory no SSM layer produces", (int)i);
    }
    for (size_t i = 0; i < outs.size(); ++i) {
        for (size_t j = i + 1; j < outs.size(); ++j)
            if (overlaps(outs[i], outs[j])) return fail(SB_EINVAL, "%s overlaps %s", outs[i].name, outs[j].name);
        for (const Range &r : ins)
            if (overlaps(outs[i], r)) return fail(SB_EINVAL, "%s overlaps %s", outs[i].name, r.name);
    }
    const DecodeLayout lay = decode_layout(B, d_model, d_inner, d_state, dt_rank, d_ff, Hq, Hkv, L, window);
    if (!workspace || workspace_bytes < lay.total)
        return fail(SB_EWORKSPACE, "workspace of %zu bytes needed, %zu given", lay.total,
                    workspace ? workspace_bytes : 0);
    if (!aligned16(workspace)) return fail(SB_EINVAL, "workspace must be 16-byte aligned");
    const Range rw = rng("workspace", workspace, lay.total);
    for (const Range &r : outs)
        if (overlaps(rw, r)) return fail(SB_EINVAL, "workspace overlaps %s", r.name);
    for (const Range &r : ins)
        if (overlaps(rw, r)) return fail(SB_EINVAL, "workspace overlaps %s", r.name);
    if (log_enabled())
        fprintf(stderr, "[sambay] %s B=%lld self=%d cross=%d d_model=%lld L=%lld window=%lld workspace %zu bytes\n",
                fn, (long long)B, (int)n_self, (int)n_cross, (long long)d_model, (long long)L, (long long)window,
                lay.total);

    char *w8 = static_cast<char *>(workspace);
    bf16_t *xn = reinterpret_cast<bf16_t *>(w8 + lay.xn), *xn_lo = reinterpret_cast<bf16_t *>(w8 + lay.xn_lo);
    bf16_t *q = reinterpret_cast<bf16_t *>(w8 + lay.q), *kn = reinterpret_cast<bf16_t *>(w8 + lay.kn);
    bf16_t *vn = reinterpret_cast<bf16_t *>(w8 + lay.vn), *o = reinterpret_cast<bf16_t *>(w8 + lay.o);
    bf16_t *o_lo = reinterpret_cast<bf16_t *>(w8 + lay.o_lo);
    bf16_t *mbuf = M_out ? static_cast<bf16_t *>(M_out) : reinterpret_cast<bf16_t *>(w8 + lay.m);
    int32_t *lens = reinterpret_cast<int32_t *>(w8 + lay.lens);
    int32_t *lens_ring = reinterpret_cast<int32_t *>(w8 + lay.lens_ring);
    bf16_t *hid = reinterpret_cast<bf16_t *>(w8 + lay.hid), *hid_lo = reinterpret_cast<bf16_t *>(w8 + lay.hid_lo);
    float *part = reinterpret_cast<float *>(w8 + lay.part);
    void *attn_part = w8 + lay.attn, *ssm_ws = w8 + lay.ssm;
    bf16_t *hb = static_cast<bf16_t *>(h);
    const int dm = (int)d_model, kvi = (int)kvd, df = (int)d_ff;

    // A sublayer's input RMSNorm(h; g) is materialised in xn (hi + lo) by an
    // RMSNorm launch, or deferred: the residual product that last wrote the
    // group's rows of h left their chunk sums of squares in `stats`, and each
    // product that reads the input normalises its own K slab while staging
    // it (the slab product; the same bits as the RMSNorm kernel).  Deferred
    // per token group of <= 64 rows when the residual product and every
    // consumer of the input run as slab products; never for the first
    // layer's input or the cross-decoder's.
    float *stats = reinterpret_cast<float *>(w8 + lay.stats);
    const int sstride = norm_stats_stride(dm), di = (int)d_inner;
    constexpr int kMaxGroups = 64;
    const int ngroups = (int)((B + kSkinnyMaxTokens - 1) / kSkinnyMaxTokens);
    const bool may_defer = ngroups <= kMaxGroups;
    bool deferred[kMaxGroups] = {};  // the pending norm's sums are in stats for the group
    bool out_defer[kMaxGroups] = {};
    auto group_T = [&](int gi) {
        const int64_t t0 = (int64_t)gi * kSkinnyMaxTokens;
        return (int)(B - t0 < kSkinnyMaxTokens ? B - t0 : kSkinnyMaxTokens);
    };
    // Whether every consumer of layer i's first (second) norm takes it deferred at T tokens.
    auto takes_norm1 = [&](int32_t i, int T) {
        if (i >= n_self || !self_layers[i].norm1) return false;
        if (self_layers[i].kind == SB_SELF_MAMBA) return slab_norm_ok(T, 2 * di, dm);
        return slab_norm_ok(T, dm + 2 * kvi, dm);  // q, k and v as one stacked product
    };
    auto takes_norm2 = [&](int32_t i, int T) {
        return self_layers[i].w_gate && self_layers[i].norm2 && slab_norm_ok(T, 2 * df, dm);
    };
    // out_defer for a residual product of K columns whose next norm is taken when `takes` says so.
    auto plan_defer = [&](int K, auto takes) {
        for (int gi = 0; gi < ngroups; ++gi) {
            const int T = group_T(gi);
            out_defer[gi] = may_defer && takes(T) && skinny_plan(T, dm, K, true).slab_rtw > 0;
        }
    };
    // RMSNorm(h; g) into xn for the groups whose norm is not deferred (one
    // launch when none is).
    auto materialise = [&](const void *g) -> hipError_t {
        bool any = false;
        for (int gi = 0; gi < ngroups; ++gi) any = any || deferred[gi];
        if (!any) return launch_rmsnorm(hb, (const bf16_t *)g, (int)B, dm, eps, xn, xn_lo, stream);
        hipError_t e = hipSuccess;
        for (int gi = 0; gi < ngroups && e == hipSuccess; ++gi) {
            const int64_t t0 = (int64_t)gi * kSkinnyMaxTokens;
            if (!deferred[gi])
                e = launch_rmsnorm(hb + t0 * dm, (const bf16_t *)g, group_T(gi), dm, eps, xn + t0 * dm,
                                   xn_lo + t0 * dm, stream);
        }
        return e;
    };
    // The operand of a product of group t0 whose input is RMSNorm(h; g) (g null: h itself).
    auto operand = [&](SkinnyArgs &a, int64_t t0, const void *g) {
        a.ldx = dm;
        if (g && deferred[t0 / kSkinnyMaxTokens]) {
            a.X = hb + t0 * dm; a.X_lo = nullptr;
            a.norm_g = (const bf16_t *)g; a.norm_stats = stats + t0 * sstride; a.norm_eps = eps;
        } else if (g) {
            a.X = xn + t0 * dm; a.X_lo = xn_lo + t0 * dm;
        } else {
            a.X = hb + t0 * dm; a.X_lo = nullptr;
        }
    };
    auto plan_of = [](const SkinnyArgs &a) { return skinny_plan(a.T, a.N, a.K, a.X_lo != nullptr || a.norm_g != nullptr); };

    hipError_t e = hipSuccess;
    for (int32_t li = 0; li < n_self && e == hipSuccess; ++li) {
        const sb_self_layer &ly = self_layers[li];
        const bool mlp = ly.w_gate != nullptr;
        if (ly.norm1 && (e = materialise(ly.norm1)) != hipSuccess) break;
        // The sublayer after the mixer: the MLP's norm2, else the next layer's norm1.
        auto takes_after_mixer = [&](int T) { return mlp ? takes_norm2(li, T) : takes_norm1(li + 1, T); };
        if (ly.kind == SB_SELF_MAMBA) {
            plan_defer(di, takes_after_mixer);
            DeferredNorms dn;
            dn.h = hb; dn.norm_in = (const bf16_t *)ly.norm1; dn.in_deferred = ly.norm1 ? deferred : nullptr;
            dn.out_defer = out_defer; dn.stats = stats; dn.stride = sstride; dn.eps = eps;
            e = run_mamba_step(ly.norm1 ? xn : hb, ly.norm1 ? xn_lo : nullptr, &ly.mamba, ly.conv_state,
                               ly.ssm_state, mbuf, hb, EPI_RESID, B, d_model, d_inner, d_state, dt_rank, d_conv,
                               ssm_ws, stream, &dn);
        } else {
            const bool swa = ly.kind == SB_SELF_SWA;
            const int slots = swa ? (int)window : (int)L;
            bf16_t *kc = static_cast<bf16_t *>(swa ? ly.kring : kcache);
            bf16_t *vc = static_cast<bf16_t *>(swa ? ly.vring : vcache);
            int32_t *ln = swa ? lens_ring : lens;
            // q, k and v of every token group: one stacked pass over the three
            // weight matrices when the slab product takes it (the deferred
            // norm only then), else three products.
            for (int64_t t0 = 0; t0 < B && e == hipSuccess; t0 += kSkinnyMaxTokens) {
                const int T = (int)(B - t0 < kSkinnyMaxTokens ? B - t0 : kSkinnyMaxTokens);
                SkinnyArgs s3;
                operand(s3, t0, ly.norm1);
                s3.W = (const bf16_t *)ly.wq; s3.W_b = (const bf16_t *)ly.wk; s3.W_c = (const bf16_t *)ly.wv;
                s3.T = T; s3.N = dm + 2 * kvi; s3.K = dm; s3.epi = EPI_BF16;
                s3.na = dm; s3.nb = dm + kvi;
                s3.out = q + t0 * dm; s3.ldo = dm; s3.out_b = kn + t0 * kvi; s3.ldo_b = kvi;
                s3.out_c = vn + t0 * kvi; s3.ldo_c = kvi;
                const SkinnyPlan p3 = plan_of(s3);
                if (p3.slab_rtw > 0 && kvi % 4 == 0) {
                    e = launch_skinny(s3, p3, part, stream);
                    continue;
                }
                const void *ws[3] = {ly.wq, ly.wk, ly.wv};
                bf16_t *outs[3] = {q, kn, vn};
                const int ns[3] = {dm, kvi, kvi};
                for (int j = 0; j < 3 && e == hipSuccess; ++j) {
                    SkinnyArgs a;
                    operand(a, t0, ly.norm1);
                    a.W = (const bf16_t *)ws[j]; a.T = T; a.N = ns[j]; a.K = dm; a.epi = EPI_BF16;
                    a.out = outs[j] + t0 * ns[j]; a.ldo = ns[j];
                    e = launch_skinny(a, plan_of(a), part, stream);
                }
            }
            if (e == hipSuccess)
                e = launch_kv_append(kn, vn, kc, vc, pos, ln, (int)B, (int)Hkv, slots, swa ? (int)window : 0,
                                     stream);
            if (e == hipSuccess)
                e = launch_xattn(q, false, kc, vc, ln, o, o_lo, (int)B, (int)Hq, (int)Hkv, slots, scale,
                                 xattn_plan(B, Hkv, slots, true), attn_part, stream);
            plan_defer(dm, takes_after_mixer);
            for (int64_t t0 = 0; t0 < B && e == hipSuccess; t0 += kSkinnyMaxTokens) {
                const int T = (int)(B - t0 < kSkinnyMaxTokens ? B - t0 : kSkinnyMaxTokens);
                SkinnyArgs a;
                a.X = o + t0 * dm; a.X_lo = o_lo + t0 * dm; a.ldx = dm; a.W = (const bf16_t *)ly.wo; a.T = T;
                a.N = dm; a.K = dm; a.epi = EPI_RESID; a.out = hb + t0 * dm; a.ldo = dm;
                if (out_defer[t0 / kSkinnyMaxTokens]) a.stats_out = stats + t0 * sstride;
                e = launch_skinny(a, skinny_plan(T, dm, dm, true), part, stream);
            }
        }
        for (int gi = 0; gi < ngroups; ++gi) deferred[gi] = out_defer[gi];
        if (e != hipSuccess || !mlp) continue;
        if (ly.norm2 && (e = materialise(ly.norm2)) != hipSuccess) break;
        plan_defer(df, [&](int T) { return takes_norm1(li + 1, T); });
        // Token group by token group: hid = SiLU(x Wg^T) ⊙ (x Wu^T), h += hid Wd^T.
        for (int64_t t0 = 0; t0 < B && e == hipSuccess; t0 += kSkinnyMaxTokens) {
            const int T = (int)(B - t0 < kSkinnyMaxTokens ? B - t0 : kSkinnyMaxTokens);
            SkinnyArgs a;
            operand(a, t0, ly.norm2);
            a.W = (const bf16_t *)ly.w_gate; a.W_b = (const bf16_t *)ly.w_up; a.T = T; a.N = df; a.K = dm;
            a.epi = EPI_SWIGLU; a.out = hid; a.ldo = df; a.out_lo = hid_lo;
            e = launch_skinny(a, skinny_plan_dual(T, df, dm), part, stream);
            if (e != hipSuccess) break;
            SkinnyArgs d;
            d.X = hid; d.X_lo = hid_lo; d.ldx = df; d.W = (const bf16_t *)ly.w_down; d.T = T; d.N = dm; d.K = df;
            d.epi = EPI_RESID; d.out = hb + t0 * dm; d.ldo = dm;
            if (out_defer[t0 / kSkinnyMaxTokens]) d.stats_out = stats + t0 * sstride;
            e = launch_skinny(d, skinny_plan(T, dm, df, true), part, stream);
        }
        for (int gi = 0; gi < ngroups; ++gi) deferred[gi] = out_defer[gi];
    }
    if (e != hipSuccess) return hip_fail(fn, e);
    if (n_cross == 0) return ok();
    return crossdecoder_step_ex(h, mbuf, kcache, vcache, lens, cross_layers, n_cross, B, d_model, d_inner, d_ff, Hq,
                                Hkv, D, L, scale, eps, w8 + lay.cross, lay.total - lay.cross, stream);
}
