// Split-K flash decoding over the single shared GQA KV cache (gfx950).
//
// What is computed: for each sequence b and query head h, the softmax
// attention of the new token's query over all L cached positions of KV head
// g = h / G (G = Hq / Hkv), with no positional encoding — the decode-time
// cross-attention of the cross-decoder (Paper-Notes reading notes on
// "Decoder-Hybrid-Decoder Architecture for Efficient Reasoning with Long
// Generation", sections 整体框架 and 现有痛点; NoPE: section 关键发现).
//
// Design (HBM-bound: the cache is read once, ~3 FLOP per byte):
//  * One workgroup per (chunk s, KV head g, sequence b); its four waves take
//    32-position blocks of the chunk round-robin.  All G query heads of the
//    group share every K/V byte loaded, so the cache is read exactly once.
//  * K and V stream into per-wave LDS buffers by direct global -> LDS copies
//    of whole rows with the non-temporal policy (the next block's copies in
//    flight while the wave computes on the current one).
//  * Scores: one 16x16x32 MFMA tile per 16 positions and 32 dims, K rows as
//    the A operand read from LDS, the group's queries as the B operand
//    (padded to 16 heads).
//    The query is pre-scaled by scale·log2(e) and split into bf16 hi + lo
//    parts, so q·k keeps ~16 significant bits with exact bf16 keys.
//  * Online softmax in the log2 domain per lane (each lane owns one head of
//    8 positions); the block max is shared across the 4 lane groups.
//  * P·V: the score tile's accumulator layout is already the B operand of
//    the second product (each lane holds 8 probabilities of one head), so P
//    never moves.  V is read back from its LDS buffer transposed
//    (position-major per lane) as the A operand.
//  * Partials (m, l, o) per (b, head, chunk) in fp32; a merge kernel combines
//    the chunks by log-sum-exp in a fixed order (deterministic, no atomics)
//    and stores bf16 (plus, on request, the bf16 low part of the fp32 value).
//    With a single chunk per head (short caches) the split kernel stores the
//    normalised output itself, with the same arithmetic, and no merge runs.
//  * Ragged batches: with a lengths array, sequence b reads only its first
//    lens[b] positions of a cache laid out with room for L.  The workgroups
//    enumerate only the chunks that hold positions (same order as the full
//    case; a sequence without positions keeps one empty item so that its
//    output is written), so every workgroup streams a full chunk except each
//    sequence's last; the merge reads only the chunks that hold positions and
//    a sequence with no position gets a zero output.
//
// Differential attention (the same kernel, DIFF = true): each query and key
// row is two 64-wide halves, one per attention map, and both maps weight the
// full 128-wide value rows (Differential Transformer, section 2.1; the pages
// name the method in the Paper-Notes page's section 局限性 / 可改进方向, where
// its serving implementation makes four plain attention passes).  The score
// tile's 16 columns hold the group's G heads twice: column i < G is map 1 of
// head i (query half 2 zeroed), column G + i is map 2 (half 1 zeroed), so one
// 128-deep contraction yields both maps' logits and each column keeps its own
// online softmax and P·V accumulator.  The cache is still read once, with
// the same MFMA count as the plain decode (2G <= 16 columns either way).  The
// merge combines each head's two columns as o1 − λ·o2 and applies the
// per-head RMS normalisation, its gain and the (1 − λ_init) factor.
#include "device.hpp"
#include "launch.hpp"

#include <math.h>
#include <stdlib.h>

namespace sambay {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlockElems = kKeyBlock * kHeadDim;  // bf16 per 32-position K or V block (8 KB)
constexpr int kWaitLds = 0xc07f;  // lgkmcnt(0): this wave's LDS reads have returned
constexpr int kWaitVm = 0x3f70;   // vmcnt(0): this wave's loads and direct-to-LDS copies have landed

// Copy policy of the cache streams: non-temporal (each byte is read once).
constexpr int kStreamPolicy = 2;

template <bool QF32, bool DIFF>
// Two workgroups per CU (64 KB of K and V buffers each); every wave keeps the
// next block's copies in flight while it computes on the current one.
__global__ __launch_bounds__(kThreads, 2) void xattn_split_kernel(const void *__restrict__ qv,
                                                               const bf16_t *__restrict__ K,
                                                               const bf16_t *__restrict__ V,
                                                               float2 *__restrict__ part_ml,
                                                               float *__restrict__ part_o,
                                                               bf16_t *__restrict__ out, bf16_t *__restrict__ out_lo,
                                                               int B, int Hq, int Hkv, int L,
                                                               const int32_t *__restrict__ lens, int chunk,
                                                               int chunk_full, int S, float qscale) {
    __shared__ __attribute__((aligned(16))) bf16_t kbuf[kWaves][kBlockElems];
    __shared__ __attribute__((aligned(16))) bf16_t vbuf[kWaves][kBlockElems];
    __shared__ float red_m[kWaves][kMaxGroup];
    __shared__ float red_l[kWaves][kMaxGroup];

    __shared__ int item[3];  // ragged batches: sequence, item index in it, its length
    int s, g, b, Lb, ck;      // ck: positions per chunk
    if (!lens) {
        // Full caches: grid (S, Hkv, B), a head's chunks in consecutive workgroups.
        s = blockIdx.x;
        g = blockIdx.y;
        b = blockIdx.z;
        Lb = L;
        ck = chunk;
    } else {
        // Ragged batches: a 1-D grid over the (sequence, KV head, chunk) items
        // that hold positions, in that order (the same order as above, without
        // the empty chunks); workgroups past the last item exit.  Each thread
        // counts the items of a contiguous run of sequences (reading each
        // length once), a prefix sum over the threads (a scan inside each
        // wave, the wave totals through LDS) gives each run's first item, and
        // the thread whose run holds this workgroup's item publishes it.
        // Chunks hold chunk_full positions when every length is within one
        // chunk of L (a uniform batch: fewer, longer workgroups, as the full
        // plan), else chunk; both counts are formed in the same pass, and the
        // batch's shortest length picks one.
        int *wsum = reinterpret_cast<int *>(&kbuf[0][0]);  // [0, 4) / [4, 8) wave totals, [8, 12) wave minima
        // Sequence i's length (clamped to [0, L]) and chunks: those holding
        // positions, at least one (an empty item still writes its zero result).
        auto len_of = [&](int i) { return min(max(lens[i], 0), L); };
        auto chunks = [&](int len, int c) { return max(1, (len + c - 1) / c); };
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int per = (B + kThreads - 1) / kThreads;
        const int lo = min(B, (int)threadIdx.x * per), hi = min(B, lo + per);
        const int len_lo = lo < hi ? len_of(lo) : 0;
        int cnt_s = 0, cnt_f = 0, mn = L;
        for (int i = lo; i < hi; ++i) {
            const int len = i == lo ? len_lo : len_of(i);
            cnt_s += Hkv * chunks(len, chunk);
            cnt_f += Hkv * chunks(len, chunk_full);
            mn = min(mn, len);
        }
        int incl_s = cnt_s, incl_f = cnt_f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int vs = __shfl_up(incl_s, off), vf = __shfl_up(incl_f, off);
            if (lane >= off) {
                incl_s += vs;
                incl_f += vf;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mn = min(mn, __shfl_xor(mn, off));
        if (lane == 63) {
            wsum[wave] = incl_s;
            wsum[kWaves + wave] = incl_f;
            wsum[2 * kWaves + wave] = mn;
        }
        if (threadIdx.x == 0) item[0] = -1;
        __syncthreads();
        int bmin = L;
        for (int w2 = 0; w2 < kWaves; ++w2) bmin = min(bmin, wsum[2 * kWaves + w2]);
        const bool uniform = bmin >= L - chunk;
        ck = uniform ? chunk_full : chunk;
        const int cnt = uniform ? cnt_f : cnt_s;
        int start = (uniform ? incl_f : incl_s) - cnt;
        for (int w2 = 0; w2 < wave; ++w2) start += wsum[(uniform ? kWaves : 0) + w2];
        const int w = (int)blockIdx.x;
        if (w >= start && w < start + cnt) {  // at most one thread
            int acc = start;
            for (int i = lo; i < hi; ++i) {
                const int len = i == lo ? len_lo : len_of(i), n = Hkv * chunks(len, ck);
                if (w < acc + n) {
                    item[0] = i;
                    item[1] = w - acc;
                    item[2] = len;
                    break;
                }
                acc += n;
            }
        }
        __syncthreads();
        if (item[0] < 0) return;  // uniform across the workgroup
        b = item[0];
        Lb = item[2];
        const int nch = chunks(Lb, ck);
        g = item[1] / nch;
        s = item[1] % nch;  // (wsum's region is read only before the second barrier)
    }
    const int G = Hq / Hkv;
    const int NC = DIFF ? 2 * G : G;  // score columns of this group
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
    // Ragged batch: sequence b uses its first Lb = lens[b] positions (clamped
    // to [0, L]); chunks past that end are empty and write an empty partial.
    const int j0 = s * ck;
    const int j1 = max(j0, min(Lb, j0 + ck));
    const size_t kv0 = ((size_t)b * Hkv + g) * (size_t)L * kHeadDim;
    const bf16_t *Kb = K + kv0;
    const bf16_t *Vb = V + kv0;

    bf16_t *kw = kbuf[wave], *vw = vbuf[wave];

    // One 32-position block of K or V into this wave's LDS buffer by direct
    // global -> LDS copies: 8 instructions of 1 KB, each 4 whole 256-byte
    // rows, so every request reads whole cache lines (register loads in the
    // MFMA operand layout read 64 bytes of each of 16 rows per instruction,
    // and the non-temporal policy then fetches lines twice).  Lane i copies
    // 16-byte chunk (i % 16) ^ swz(row) of row 4j + i / 16 into slot i % 16:
    // K rows swizzle by row % 16 (16 rows read at one chunk), V rows by
    // 2 · ((row / 4) % 4) (4 rows read at one dimension), so the reads below
    // hit distinct LDS banks.  Rows past the chunk end are clamped to its
    // last row (in bounds) and masked later.
    auto issue_block = [&](const bf16_t *src, bf16_t *dst, int blk, bool is_v) {
        const int base = j0 + blk * kKeyBlock;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 4 * j + (lane >> 4), slot = lane & 15;
            const int c = slot ^ (is_v ? 2 * ((r >> 2) & 3) : (r & 15));
            const int row = min(base + r, j1 - 1);
            __builtin_amdgcn_global_load_lds(src + (size_t)row * kHeadDim + 8 * c,
                                             (__attribute__((address_space(3))) void *)(dst + 512 * j), 16, 0,
                                             kStreamPolicy);
        }
    };

    // B operand of the score product: head `col` of this group (differential:
    // map col / G of head col % G, the other map's half zeroed); MFMA k-step t
    // covers dims 32·t .. 32·t+31, lane group grp holding dims 32·t + 8·grp + e.
    // The query rows are loaded first (16-byte loads; dead columns read a
    // clamped row and are zeroed), then the first block's copies go out, and
    // only then is the query converted: its latency and the first block's
    // overlap instead of adding up.
    const int q_map = DIFF && col >= G ? 1 : 0;
    const int q_head = min(g * G + col - q_map * G, Hq - 1);
    constexpr int QV = QF32 ? 2 : 1;  // 16-byte loads per 8 dims
    u32x4 qraw[4][QV];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const size_t off = ((size_t)b * Hq + q_head) * kHeadDim + 32 * t + 8 * grp;
#pragma unroll
        for (int v = 0; v < QV; ++v)
            qraw[t][v] = QF32 ? ld16((const float *)qv + off + 4 * v) : ld16((const bf16_t *)qv + off);
    }
    __builtin_amdgcn_sched_barrier(0);
    const int nblk = (j1 - j0 + kKeyBlock - 1) / kKeyBlock;
    if (wave < nblk) {
        issue_block(Kb, kw, wave, false);
        issue_block(Vb, vw, wave, true);
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4 qhi[4], qlo[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float f[8];
        const bool live = col < NC && (!DIFF || (t >> 1) == q_map);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = QF32 ? __uint_as_float(qraw[t][QF32 ? e / 4 : 0][e % 4])
                                 : ((e & 1) ? hi_bf16(qraw[t][0][e / 2]) : lo_bf16(qraw[t][0][e / 2]));
            f[e] = (live ? x : 0.f) * qscale;
        }
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bf16_t h0 = f32_to_bf16(f[2 * e]), h1 = f32_to_bf16(f[2 * e + 1]);
            hi[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lo[e] = (uint32_t)split_lo(f[2 * e], h0) | ((uint32_t)split_lo(f[2 * e + 1], h1) << 16);
        }
        qhi[t] = (u32x4){hi[0], hi[1], hi[2], hi[3]};
        qlo[t] = (u32x4){lo[0], lo[1], lo[2], lo[3]};
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // A block is read from LDS into registers whole (K fragments and the
    // transposed V operand) before the next block's copies are issued, so the
    // copies of block blk + 4 fly while the wave computes on block blk.  The
    // wave has one block of copies in flight at a time: an explicit vmcnt(0)
    // before the LDS reads waits for exactly that block (the compiler's own
    // tracking of direct-to-LDS copies does not insert this wait on every
    // path through the loop).
    auto process_block = [&](int blk, bool next) {
        const int base = j0 + blk * kKeyBlock;
        __builtin_amdgcn_s_waitcnt(kWaitVm);  // this wave's copies of block blk have landed
        // K fragments: rows col (k0) and 16 + col (k1), dims 32·t + 8·grp .. +7 (chunk 4t + grp).
        u32x4 k0[4], k1[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int sl = (4 * t + grp) ^ col;
            k0[t] = *reinterpret_cast<const u32x4 *>(&kw[col * kHeadDim + 8 * sl]);
            k1[t] = *reinterpret_cast<const u32x4 *>(&kw[(16 + col) * kHeadDim + 8 * sl]);
        }
        // V^T operand: dim 16·db + col at positions 4·grp + i and 16 + 4·grp + i, whose
        // rows all carry swizzle 2·grp.
        u32x4 va[8];
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const int e = 8 * (2 * (db ^ grp) + (col >> 3)) + (col & 7);
            const bf16_t *v0 = vw + (4 * grp) * kHeadDim + e, *v1 = vw + (16 + 4 * grp) * kHeadDim + e;
            va[db][0] = (uint32_t)v0[0] | ((uint32_t)v0[kHeadDim] << 16);
            va[db][1] = (uint32_t)v0[2 * kHeadDim] | ((uint32_t)v0[3 * kHeadDim] << 16);
            va[db][2] = (uint32_t)v1[0] | ((uint32_t)v1[kHeadDim] << 16);
            va[db][3] = (uint32_t)v1[2 * kHeadDim] | ((uint32_t)v1[3 * kHeadDim] << 16);
        }
        __builtin_amdgcn_s_waitcnt(kWaitLds);  // the buffers are free
        if (next) {
            issue_block(Kb, kw, blk + kWaves, false);
            issue_block(Vb, vw, blk + kWaves, true);
        }
        // Scores of positions base + 4·grp + i (s0) and base + 16 + 4·grp + i (s1) for head col.
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            s0 = mfma16x16x32(k0[t], qhi[t], s0);
            s1 = mfma16x16x32(k1[t], qhi[t], s1);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            s0 = mfma16x16x32(k0[t], qlo[t], s0);
            s1 = mfma16x16x32(k1[t], qlo[t], s1);
        }

#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (base + 4 * grp + i >= j1) s0[i] = -INFINITY;
            if (base + 16 + 4 * grp + i >= j1) s1[i] = -INFINITY;
        }
        float bm = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                         fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
        bm = fmaxf(bm, __shfl_xor(bm, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float m_new = fmaxf(m_run, bm);  // finite: every processed block has a live position
        const float alpha = exp2_fast(m_run - m_new);
        m_run = m_new;
        float p[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = exp2_fast(s0[i] - m_new);
            p[4 + i] = exp2_fast(s1[i] - m_new);
        }
        l_run = l_run * alpha + (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] *= alpha;
        const u32x4 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                          pack_bf16x2(p[6], p[7])};
        // O^T[dim][head] += V^T[dim][pos] · P^T[pos][head].
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[db] = mfma16x16x32(va[db], pb, acc[db]);
    };

    for (int blk = wave; blk < nblk; blk += kWaves) process_block(blk, blk + kWaves < nblk);

    // Row sums: each lane group summed different positions of the same head.
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);

    // Combine the four waves' (m, l, o) in LDS, then write this chunk's partial.
    __syncthreads();
    float *ow = reinterpret_cast<float *>(&kbuf[0][0]);  // [kWaves][16 heads][128 dims] fp32 = 32 KB
    if (grp == 0) {
        red_m[wave][col] = m_run;
        red_l[wave][col] = l_run;
    }
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) ow[(wave * kMaxGroup + col) * kHeadDim + 16 * db + 4 * grp + r] = acc[db][r];
    __syncthreads();
    for (int idx = threadIdx.x; idx < NC * kHeadDim; idx += kThreads) {
        const int hh = idx / kHeadDim, d = idx % kHeadDim;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w][hh]);
        float lsum = 0.f, o = 0.f;
        if (M != -INFINITY) {  // else an empty chunk: (m, l, o) = (-inf, 0, 0)
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float e = exp2_fast(red_m[w][hh] - M);  // waves without positions carry m = -inf: weight 0
                lsum += e * red_l[w][hh];
                o += e * ow[(w * kMaxGroup + hh) * kHeadDim + d];
            }
        }
        if (!DIFF && S == 1) {  // the only chunk: normalise and store here (what the merge would do)
            const float v = lsum > 0.f ? o / lsum : 0.f;
            const size_t oi = ((size_t)b * Hq + (size_t)g * G + hh) * kHeadDim + d;
            const bf16_t hi = f32_to_bf16(v);
            out[oi] = hi;
            if (out_lo) out_lo[oi] = split_lo(v, hi);
        } else {
            const size_t pi = ((size_t)b * (DIFF ? 2 * Hq : Hq) + (size_t)g * NC + hh) * S + s;
            part_o[pi * kHeadDim + d] = o;
            if (d == 0) part_ml[pi] = make_float2(M, lsum);
        }
    }
}

// Log-sum-exp merge of one score column's first Sb chunk partials, in order,
// and the softmax normalisation: dimension d of that column's output.
__device__ __forceinline__ float merge_column(const float2 *__restrict__ ml, const float *__restrict__ po, int Sb,
                                              int d) {
    float M = -INFINITY;
    for (int s = 0; s < Sb; ++s) M = fmaxf(M, ml[s].x);
    float lsum = 0.f, o = 0.f;
    if (M != -INFINITY) {  // else a sequence without visible positions: zero output
        for (int s = 0; s < Sb; ++s) {
            const float e = exp2_fast(ml[s].x - M);  // empty chunks carry m = -inf: weight 0
            lsum += e * ml[s].y;
            o += e * po[(size_t)s * kHeadDim + d];
        }
    }
    return lsum > 0.f ? o / lsum : 0.f;
}

// One workgroup per (sequence, query head): the merge, then the bf16 store.
// Ragged batches: the chunk length the split kernel used (chunk_full when
// every length of the batch is within one chunk of L, else chunk), from the
// batch's shortest length; every thread of the workgroup gets it.
__device__ __forceinline__ int lens_chunk(const int32_t *__restrict__ lens, int B, int L, int chunk, int chunk_full,
                                          int *red) {
    int mn = L;
    for (int i = threadIdx.x; i < B; i += blockDim.x) mn = min(mn, min(max(lens[i], 0), L));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mn = min(mn, __shfl_xor(mn, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mn;
    __syncthreads();
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) mn = min(mn, red[w]);
    return mn >= L - chunk ? chunk_full : chunk;
}

__global__ __launch_bounds__(kHeadDim) void xattn_merge_kernel(const float2 *__restrict__ part_ml,
                                                               const float *__restrict__ part_o,
                                                               bf16_t *__restrict__ out, bf16_t *__restrict__ out_lo,
                                                               int S, int Hq, int L, const int32_t *__restrict__ lens,
                                                               int chunk, int chunk_full) {
    __shared__ int red[kHeadDim / 64];
    const size_t bh = blockIdx.x;
    const int d = threadIdx.x;
    // Ragged batches: only the chunks that hold positions were written.
    const int ck = lens ? lens_chunk(lens, (int)(gridDim.x / Hq), L, chunk, chunk_full, red) : chunk;
    const int Sb = lens ? (min(max(lens[bh / Hq], 0), L) + ck - 1) / ck : S;
    const float v = merge_column(part_ml + bh * S, part_o + bh * S * kHeadDim, Sb, d);
    const bf16_t hi = f32_to_bf16(v);
    out[bh * kHeadDim + d] = hi;
    if (out_lo) out_lo[bh * kHeadDim + d] = split_lo(v, hi);
}

// Differential attention, one workgroup per (sequence, query head): merge the
// head's two map columns, y = o1 − λ·o2, then out = (1 − λ_init)·y / RMS(y)·γ
// over the head's 128 dimensions (RMS with eps; γ all ones when null).  The
// sum of squares is reduced in a fixed order (wave tree, then wave 0 + wave 1).
__global__ __launch_bounds__(kHeadDim) void diffattn_merge_kernel(const float2 *__restrict__ part_ml,
                                                                  const float *__restrict__ part_o,
                                                                  const bf16_t *__restrict__ gamma,
                                                                  bf16_t *__restrict__ out, int S, int Hq, int G,
                                                                  int L, const int32_t *__restrict__ lens, int chunk,
                                                                  int chunk_full, float lam, float lam_init,
                                                                  float eps) {
    __shared__ float red[kHeadDim / 64];
    __shared__ int ired[kHeadDim / 64];
    const size_t bh = blockIdx.x;
    const int d = threadIdx.x;
    const size_t b = bh / Hq;
    const int h = (int)(bh % Hq), g = h / G;
    const size_t c1 = b * 2 * Hq + (size_t)g * 2 * G + (h - g * G), c2 = c1 + G;  // map 1 and map 2 columns
    const int ck = lens ? lens_chunk(lens, (int)(gridDim.x / Hq), L, chunk, chunk_full, ired) : chunk;
    const int Sb = lens ? (min(max(lens[b], 0), L) + ck - 1) / ck : S;
    const float y = merge_column(part_ml + c1 * S, part_o + c1 * S * kHeadDim, Sb, d) -
                    lam * merge_column(part_ml + c2 * S, part_o + c2 * S * kHeadDim, Sb, d);
    float ss = y * y;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    if ((d & 63) == 0) red[d >> 6] = ss;
    __syncthreads();
    const float r = (1.f - lam_init) / sqrtf((red[0] + red[1]) / (float)kHeadDim + eps);
    const float gm = gamma ? bf16_to_f32(gamma[d]) : 1.f;
    out[bh * kHeadDim + d] = f32_to_bf16(Sb > 0 ? y * r * gm : 0.f);
}

int env_splits() {
    const char *e = getenv("SAMBAY_XATTN_SPLITS");
    if (!e || !*e) return 0;
    const int v = atoi(e);
    return v > 0 ? v : 0;
}

}  // namespace

XattnPlan xattn_plan(int64_t B, int64_t Hkv, int64_t L, bool ragged) {
    const int64_t nblk = (L + kKeyBlock - 1) / kKeyBlock;
    const int64_t pairs = B * Hkv > 0 ? B * Hkv : 1;
    // Chunks of >= 4096 positions amortise each workgroup's setup and merge,
    // unless that leaves fewer than ~2 workgroups per CU (256 CUs); never more
    // than ~8 per CU.
    int64_t S = env_splits();
    bool halved = false;  // ragged: chunks half as long as the full plan's
    if (S == 0) {
        const int64_t fill = (512 + pairs - 1) / pairs, cap = (2048 + pairs - 1) / pairs;
        const int64_t by_len = L / 4096 > 1 ? L / 4096 : 1;
        // Splitting to fill the GPU only while every chunk keeps >= 16 blocks
        // (512 positions): below that a workgroup's fixed cost (item lookup,
        // query split, cross-wave combine) outweighs its streaming, and one
        // chunk per head lets the split kernel store the output itself
        // (measured on a 256-position window, 32 x 8 KV heads: 4 chunks
        // 32.4 us, 2 chunks 21.4 us, 1 chunk 20.7 us per call).
        const int64_t fill_cap = nblk / 16;
        S = cap < by_len ? cap : by_len;
        if (S < fill && S < fill_cap) S = fill < fill_cap ? fill : fill_cap;
        // Ragged batches hold fewer positions than L per sequence: chunks half
        // as long keep the workgroup count up and the tail short (measured on
        // lengths uniform in [2048, 34816]: 8 -> 16 chunks, 5.1 -> 5.4 TB/s).
        if (ragged && nblk / (2 * S) >= 16) {
            halved = true;
            S *= 2;
        }
    }
    if (S > kMaxSplits) S = kMaxSplits;
    if (S > nblk) S = nblk;
    if (S < 1) S = 1;
    const int64_t per = (nblk + S - 1) / S;
    XattnPlan p;
    p.chunk = (int)(per * kKeyBlock);
    p.splits = (int)((L + p.chunk - 1) / p.chunk);  // every chunk non-empty
    const int64_t S_full = halved ? S / 2 : S, per_full = (nblk + S_full - 1) / S_full;
    p.chunk_full = halved ? (int)(per_full * kKeyBlock) : p.chunk;
    return p;
}

size_t xattn_workspace_need(int64_t B, int64_t Hq, int64_t Hkv, int64_t L) {
    const int a = xattn_plan(B, Hkv, L, false).splits, b = xattn_plan(B, Hkv, L, true).splits;
    return xattn_partial_bytes(B, Hq, a > b ? a : b);
}

size_t xattn_partial_bytes(int64_t B, int64_t Hq, int splits) {
    const size_t n = (size_t)B * Hq * splits;
    return n * sizeof(float2) + n * kHeadDim * sizeof(float);
}

hipError_t launch_xattn(const void *q, bool q_f32, const bf16_t *K, const bf16_t *V, const int32_t *lens,
                        bf16_t *out, bf16_t *out_lo, int B, int Hq, int Hkv, int L, float scale, const XattnPlan &plan,
                        void *partials, hipStream_t stream) {
    const size_t n = (size_t)B * Hq * plan.splits;
    float2 *ml = reinterpret_cast<float2 *>(partials);
    float *po = reinterpret_cast<float *>(reinterpret_cast<char *>(partials) + n * sizeof(float2));
    // Ragged: an upper bound on the items; those past the last one exit.
    if (lens && (size_t)B * Hkv * plan.splits > 0x7fffffffu) return hipErrorInvalidConfiguration;
    const dim3 grid = lens ? dim3((unsigned)((size_t)B * Hkv * plan.splits)) : dim3(plan.splits, Hkv, B);
    const float qscale = scale * kLog2e;
    {
    TimingScope ts(kTimeXattnSplit, stream);
    if (q_f32)
        hipLaunchKernelGGL((xattn_split_kernel<true, false>), grid, dim3(kThreads), 0, stream, q, K, V, ml, po, out,
                           out_lo, B, Hq, Hkv, L, lens, plan.chunk, plan.chunk_full, plan.splits, qscale);
    else
        hipLaunchKernelGGL((xattn_split_kernel<false, false>), grid, dim3(kThreads), 0, stream, q, K, V, ml, po, out,
                           out_lo, B, Hq, Hkv, L, lens, plan.chunk, plan.chunk_full, plan.splits, qscale);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1) return e;  // one chunk: the split kernel stored the output
    TimingScope ts(kTimeXattnMerge, stream);
    hipLaunchKernelGGL(xattn_merge_kernel, dim3((unsigned)(B * Hq)), dim3(kHeadDim), 0, stream, ml, po, out, out_lo,
                       plan.splits, Hq, L, lens, plan.chunk, plan.chunk_full);
    return hipGetLastError();
}

hipError_t launch_diffattn(const bf16_t *q, const bf16_t *K, const bf16_t *V, const int32_t *lens, const bf16_t *gamma,
                           bf16_t *out, int B, int Hq, int Hkv, int L, float scale, float lam, float lam_init,
                           float eps, const XattnPlan &plan, void *partials, hipStream_t stream) {
    const size_t n = (size_t)B * 2 * Hq * plan.splits;  // two score columns per head
    float2 *ml = reinterpret_cast<float2 *>(partials);
    float *po = reinterpret_cast<float *>(reinterpret_cast<char *>(partials) + n * sizeof(float2));
    if (lens && (size_t)B * Hkv * plan.splits > 0x7fffffffu) return hipErrorInvalidConfiguration;
    const dim3 grid = lens ? dim3((unsigned)((size_t)B * Hkv * plan.splits)) : dim3(plan.splits, Hkv, B);
    {
        TimingScope ts(kTimeDiffSplit, stream);
        hipLaunchKernelGGL((xattn_split_kernel<false, true>), grid, dim3(kThreads), 0, stream, q, K, V, ml, po,
                           nullptr, nullptr, B, Hq, Hkv, L, lens, plan.chunk, plan.chunk_full, plan.splits,
                           scale * kLog2e);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    TimingScope ts(kTimeDiffMerge, stream);
    hipLaunchKernelGGL(diffattn_merge_kernel, dim3((unsigned)(B * Hq)), dim3(kHeadDim), 0, stream, ml, po, gamma, out,
                       plan.splits, Hq, Hq / Hkv, L, lens, plan.chunk, plan.chunk_full, lam, lam_init, eps);
    return hipGetLastError();
}

}  // namespace sambay
