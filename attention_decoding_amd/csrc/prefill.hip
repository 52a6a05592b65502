// Prefill attention of the self-decoder's layers (gfx950): causal attention
// of T prompt tokens over their own keys, optionally limited to a sliding
// window (the Paper-Notes page on "Decoder-Hybrid-Decoder Architecture for
// Efficient Reasoning with Long Generation", sections 领域现状 and 现有痛点:
// the decoder-decoder structure pre-fills in linear time; section 消融实验:
// the self-decoder's attention uses a 256-token window).  Query i of head h
// attends to keys j of KV head h / (Hq / Hkv) with j <= i and, for a window
// W > 0, j > i - W; no positional encoding.
//
// Design (flash attention with the score tile transposed, as in the decode
// kernel): one workgroup per (sequence, NH query heads of one KV head, 64
// queries); its four waves take 16 queries each as the 16 columns of a
// 16x16x32 MFMA tile, one tile per head: every K and V^T operand read from
// LDS serves the NH heads (their visible keys are the same), and a block's
// loads, stores and barrier serve NH times the work.  NH is 3 or 2 of the
// group when that leaves the grid at least two workgroups per CU, else 1 (a
// causal batch-1 prompt, whose longest tiles would then bound the call).
//  * Keys come in 32-position blocks (16 KB of K and V^T, pieces of each
//    row XOR-swizzled against bank conflicts) through a register-to-LDS
//    pipeline: while block n is processed from one LDS stage, blocks n + 1
//    and n + 2 are loading into two register sets; block n + 1 is then
//    stored into the other stage and block n + 3 starts loading, one
//    barrier per block.  A workgroup's work per block is small (16
//    MFMAs per wave), so hiding the memory latency needs that depth; the
//    barrier carries no memory fence, which would wait for the loads in
//    flight.  Workgroups with the longest key ranges (the last tiles of a
//    causal prompt) are dispatched first.
//  * S^T = K·Q^T: K rows from LDS as the A operand, the wave's 16 queries as
//    the B operand (held in registers for the whole key range); the scale
//    (with log2 e) is applied to the fp32 scores.
//  * Online softmax in the log2 domain per query column; keys outside the
//    causal window are masked to -inf (a column can see no key of a block:
//    its running max then stays -inf and the block adds nothing).
//  * O^T += V^T·P^T: the score accumulators are already the B operand (each
//    lane holds 8 probabilities of its query).  V is transposed once per
//    call into the workspace ([dim][key], a small pass over V), and the K
//    rows of the score tiles are permuted so that each lane's 8 keys are
//    consecutive: the A operand is then one 16-byte LDS read per tile.
//  * The output is normalised in registers and stored as bf16.
#include "device.hpp"
#include "launch.hpp"

#include <math.h>
#include <stdlib.h>

namespace sambay {

namespace {

constexpr int kPWaves = 4;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kPQueries = 16 * kPWaves;  // queries per workgroup
constexpr int kPKeys = 32;               // keys per block
constexpr int kPSlots = kPKeys * kHeadDim / 8;  // 16-byte slots of one K (or V^T) block: 512

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Two fp32 to a packed bf16 pair, round to nearest even (one gfx950 instruction).
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// K block slots: piece c (dims 8c .. 8c+7) of key row r, XOR-swizzled so the
// 16 rows an MFMA operand reads at one piece index fall on distinct banks.
// A score tile reads rows 8(l/4) + l%4 (+ 4 for the second tile) for l < 16:
// (r & 3) | ((r >> 3) << 2) is l itself on both sets.  (r & 15 repeats on
// them: rows 0 and 16 shared banks, ~2x the LDS cycles of the key reads.)
__device__ __forceinline__ int kswz(int r) { return (r & 3) | ((r >> 3) << 2); }
__device__ __forceinline__ int kslot(int r, int c) { return 16 * r + (c ^ kswz(r)); }
// V^T block slots: keys 8s .. 8s+7 of dim row d (64-byte rows), swizzled so
// that 16 consecutive dims at one s fall on distinct banks.
__device__ __forceinline__ int vslot(int d, int s) { return 4 * d + (s ^ ((d >> 2) & 3)); }

// Workgroup barrier for the LDS stages without a memory fence: a fence
// would also wait for the global loads of the blocks still in flight
// (vmcnt 0), which is exactly the latency the pipeline is there to hide.
// Only LDS is shared here: this wave's LDS stores and reads are complete
// (lgkmcnt 0) before the barrier, and the asm's memory clobber keeps the
// compiler from moving LDS accesses across it; the compiler itself waits
// for each register load before the store that uses it.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// V [B, T, Hkv, 128] -> V^T [B, Hkv, 128, Tp] (Tp = T rounded up to 32, zeros
// past T): one workgroup per (32 tokens, KV head, sequence) through LDS.
__global__ __launch_bounds__(256) void v_transpose_kernel(const bf16_t *__restrict__ V, bf16_t *__restrict__ VT,
                                                         int T, int Tp, int Hkv) {
    __shared__ bf16_t tile[kPKeys][kHeadDim + 2];
    const int t0 = blockIdx.x * kPKeys, g = blockIdx.y, b = blockIdx.z;
    for (int i = threadIdx.x; i < kPKeys * kHeadDim / 2; i += 256) {  // 2 dims per thread-step
        const int r = i / (kHeadDim / 2), d2 = 2 * (i % (kHeadDim / 2));
        uint32_t w = 0u;
        if (t0 + r < T) w = *reinterpret_cast<const uint32_t *>(V + (((size_t)b * T + t0 + r) * Hkv + g) * kHeadDim + d2);
        tile[r][d2] = (bf16_t)(w & 0xffffu);
        tile[r][d2 + 1] = (bf16_t)(w >> 16);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kHeadDim * kPKeys / 2; i += 256) {  // 2 keys per thread-step
        const int d = i / (kPKeys / 2), r2 = 2 * (i % (kPKeys / 2));
        const uint32_t w = (uint32_t)tile[r2][d] | ((uint32_t)tile[r2 + 1][d] << 16);
        *reinterpret_cast<uint32_t *>(VT + (((size_t)b * Hkv + g) * kHeadDim + d) * Tp + t0 + r2) = w;
    }
}

template <int NH>
__global__ __launch_bounds__(kPThreads, 2) void attn_prefill_kernel(const bf16_t *__restrict__ Q,
                                                                    const bf16_t *__restrict__ K,
                                                                    const bf16_t *__restrict__ VT,
                                                                    bf16_t *__restrict__ out, int T, int Tp, int Hq,
                                                                    int Hkv, int window, float qscale) {
    // Two LDS stages: [stage][K slots | V^T slots], each slot 16 bytes.
    __shared__ __attribute__((aligned(16))) u32x4 stage[2][2 * kPSlots];

    const int ntiles = (T + kPQueries - 1) / kPQueries;
    const int tile = ntiles - 1 - (int)blockIdx.x;  // longest key ranges first (causal: late tiles)
    const int h0 = blockIdx.y * NH, b = blockIdx.z;   // heads h0 .. h0 + NH - 1, one KV head
    const int g = h0 / (Hq / Hkv);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, grp = lane >> 4, col = lane & 15;
    const int i0 = tile * kPQueries;
    const int qi = i0 + 16 * wave + col;  // this lane's query (column)
    const int qlast = min(T, i0 + kPQueries) - 1;
    const int jlo = window > 0 ? max(0, i0 - window + 1) : 0;
    const int kb0 = jlo / kPKeys, kb1 = qlast / kPKeys;

    u32x4 qb[NH][4];
#pragma unroll
    for (int j = 0; j < NH; ++j) {
        const size_t qrow = (((size_t)b * T + min(qi, T - 1)) * Hq + h0 + j) * kHeadDim + 8 * grp;
#pragma unroll
        for (int t = 0; t < 4; ++t) qb[j][t] = ld16(Q + qrow + 32 * t);
    }
    // The queries are complete before the block pipeline starts, so that no
    // wait inside the loop has to count them among the loads in flight.
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)

    const bf16_t *kbase = K + ((size_t)b * T * Hkv + g) * kHeadDim;
    const bf16_t *vbase = VT + ((size_t)b * Hkv + g) * kHeadDim * Tp;
    // Thread t moves slots t, t + 256, t + 512, t + 768 of a block (K then V^T):
    // 4 loads of 16 bytes into registers, later 4 stores into a stage.
    auto load = [&](int kb, u32x4 (&r)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int slot = threadIdx.x + kPThreads * e, sl = slot & (kPSlots - 1);
            if (e < 2) {
                const int row = sl >> 4, c = (sl & 15) ^ kswz(row);
                const int j = min(kb * kPKeys + row, T - 1);  // rows past T: any valid row, masked later
                r[e] = ld16(kbase + (size_t)j * Hkv * kHeadDim + 8 * c);
            } else {
                const int d = sl >> 2, sc = (sl & 3) ^ ((d >> 2) & 3);
                r[e] = ld16(vbase + (size_t)d * Tp + kb * kPKeys + 8 * sc);  // zeros past T
            }
        }
    };
    auto store = [&](int buf, const u32x4 (&r)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) stage[buf][threadIdx.x + kPThreads * e] = r[e];
    };

    float m_run[NH], l_run[NH];
    f32x4 acc[NH][8];
#pragma unroll
    for (int j = 0; j < NH; ++j) {
        m_run[j] = -INFINITY;
        l_run[j] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }

    // Score tile rows: tile 0 row r holds key 8(r/4) + r%4, tile 1 row r key
    // 8(r/4) + 4 + r%4, so that lane group grp ends up with keys 8grp .. 8grp+7
    // in order: exactly the V^T slot it reads for the second product.
    const int r0 = 8 * (col >> 2) + (col & 3), r1 = r0 + 4;
    auto compute = [&](int buf, int kb) {
        const u32x4 *kr = stage[buf];
        const u32x4 *vr = kr + kPSlots;
        const int j0 = kb * kPKeys;
        f32x4 s0[NH], s1[NH];
#pragma unroll
        for (int j = 0; j < NH; ++j) s0[j] = s1[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const u32x4 k0 = kr[kslot(r0, 4 * t + grp)], k1 = kr[kslot(r1, 4 * t + grp)];
#pragma unroll
            for (int j = 0; j < NH; ++j) {
                s0[j] = mfma16x16x32(k0, qb[j][t], s0[j]);
                s1[j] = mfma16x16x32(k1, qb[j][t], s1[j]);
            }
        }
        // s0[j][i]: key j0 + 8grp + i, s1[j][i]: key j0 + 8grp + 4 + i, for query qi of head h0 + j.
        const int jmin = window > 0 ? qi - window + 1 : 0;  // visible keys: jmin <= key <= qi
        u32x4 pb[NH];
#pragma unroll
        for (int j = 0; j < NH; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ja = j0 + 8 * grp + i, jb = ja + 4;
                s0[j][i] = ja <= qi && ja >= jmin ? s0[j][i] * qscale : -INFINITY;
                s1[j][i] = jb <= qi && jb >= jmin ? s1[j][i] * qscale : -INFINITY;
            }
            float bm = fmaxf(fmaxf(fmaxf(s0[j][0], s0[j][1]), fmaxf(s0[j][2], s0[j][3])),
                             fmaxf(fmaxf(s1[j][0], s1[j][1]), fmaxf(s1[j][2], s1[j][3])));
            bm = fmaxf(bm, __shfl_xor(bm, 16));
            bm = fmaxf(bm, __shfl_xor(bm, 32));
            const float m_new = fmaxf(m_run[j], bm);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;  // no visible key yet: nothing to rescale
            const float alpha = exp2_fast(m_run[j] - m_use);
            m_run[j] = m_new;
            float p[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = exp2_fast(s0[j][i] - m_use);
                p[4 + i] = exp2_fast(s1[j][i] - m_use);
            }
            l_run[j] = l_run[j] * alpha + (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[j][i] *= alpha;
            pb[j] = (u32x4){pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7])};
        }
        // O^T[dim][query] += V^T[dim][key] · P^T[key][query]: lane reads keys 8grp .. 8grp+7 of dim 16·db + col.
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const u32x4 v = vr[vslot(16 * db + col, grp)];
#pragma unroll
            for (int j = 0; j < NH; ++j) acc[j][db] = mfma16x16x32(v, pb[j], acc[j][db]);
        }
    };

    // Pipeline: block kb is processed from one stage while block kb + 1 waits
    // in registers for the other and blocks kb + 2, kb + 3 are in flight.
    // Unrolled by two so that each register set is named at compile time.
    // Loads are issued unconditionally (past the last block they repeat it):
    // the compiler then counts the loads in flight exactly and waits only for
    // the register set being stored.
    u32x4 ra[4], rb[4];
    load(kb0, ra);
    store(0, ra);
    load(min(kb0 + 1, kb1), ra);
    load(min(kb0 + 2, kb1), rb);
    ring_barrier();
    for (int kb = kb0; kb <= kb1; kb += 2) {
        compute(0, kb);
        if (kb + 1 <= kb1) store(1, ra);             // block kb + 1; stage 1 was last read before the previous barrier
        load(min(kb + 3, kb1), ra);
        ring_barrier();
        if (kb + 1 > kb1) break;
        compute(1, kb + 1);
        if (kb + 2 <= kb1) store(0, rb);             // block kb + 2
        load(min(kb + 4, kb1), rb);
        ring_barrier();
    }

    // Row sums: the four lane groups summed different keys of the same query.
#pragma unroll
    for (int j = 0; j < NH; ++j) {
        l_run[j] += __shfl_xor(l_run[j], 16);
        l_run[j] += __shfl_xor(l_run[j], 32);
    }
    if (qi >= T) return;
#pragma unroll
    for (int j = 0; j < NH; ++j) {
        const float inv = 1.f / l_run[j];  // every query sees at least itself
        bf16_t *o = out + (((size_t)b * T + qi) * Hq + h0 + j) * kHeadDim;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const int d = 16 * db + 4 * grp;
            const uint32_t w0 = pack_bf16x2(acc[j][db][0] * inv, acc[j][db][1] * inv);
            const uint32_t w1 = pack_bf16x2(acc[j][db][2] * inv, acc[j][db][3] * inv);
            *reinterpret_cast<u32x2 *>(o + d) = (u32x2){w0, w1};
        }
    }
}

}  // namespace

// Query heads per workgroup: 3 or 2 heads of a KV head's group (G = Hq /
// Hkv divisible by them; 4 would not fit the registers) when that still
// gives >= 512 workgroups (two per CU), else 1.  SAMBAY_PREFILL_HEADS (1-3,
// a divisor of G) overrides the rule.
int attn_prefill_heads(int64_t B, int64_t T, int64_t Hq, int64_t Hkv) {
    const int64_t G = Hq / Hkv;
    if (const char *env = getenv("SAMBAY_PREFILL_HEADS")) {
        const int v = atoi(env);
        if (v >= 1 && v <= 3 && G % v == 0) return v;
    }
    const int nh = G % 3 == 0 ? 3 : G % 2 == 0 ? 2 : 1;
    const int64_t tiles = (T + kPQueries - 1) / kPQueries;
    return tiles * B * (Hq / nh) < 512 ? 1 : nh;
}

size_t attn_prefill_workspace_need(int64_t B, int64_t T, int64_t Hkv) {
    const int64_t Tp = (T + kPKeys - 1) / kPKeys * kPKeys;
    return (size_t)B * Hkv * kHeadDim * Tp * sizeof(bf16_t);
}

hipError_t launch_attn_prefill(const bf16_t *q, const bf16_t *k, const bf16_t *v, bf16_t *out, int B, int T, int Hq,
                               int Hkv, int window, float scale, void *workspace, hipStream_t stream) {
    const int Tp = (T + kPKeys - 1) / kPKeys * kPKeys;
    bf16_t *vt = reinterpret_cast<bf16_t *>(workspace);
    hipLaunchKernelGGL(v_transpose_kernel, dim3((unsigned)(Tp / kPKeys), (unsigned)Hkv, (unsigned)B), dim3(256), 0,
                       stream, v, vt, T, Tp, Hkv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int tiles = (T + kPQueries - 1) / kPQueries, G = Hq / Hkv;
    int nh = attn_prefill_heads(B, T, Hq, Hkv);
    if (nh < 1 || nh > 3 || G % nh != 0) nh = 1;
    const dim3 grid((unsigned)tiles, (unsigned)(Hq / nh), (unsigned)B);
    TimingScope ts(kTimePrefill, stream);
#define SB_PREFILL(NH_)                                                                                              \
    hipLaunchKernelGGL(attn_prefill_kernel<NH_>, grid, dim3(kPThreads), 0, stream, q, k, vt, out, T, Tp, Hq, Hkv,   \
                       window, scale * kLog2e)
    switch (nh) {
        case 2: SB_PREFILL(2); break;
        case 3: SB_PREFILL(3); break;
        default: SB_PREFILL(1); break;
    }
#undef SB_PREFILL
    return hipGetLastError();
}

}  // namespace sambay
