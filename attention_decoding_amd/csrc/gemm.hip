// MFMA bf16 GEMM for GMU prefill (gfx950):
//   out[r, n] = epilogue( Σ_k X[r, k] · W[n, k] )   (both operands K-contiguous)
// The GMU (Paper-Notes reading notes on "Decoder-Hybrid-Decoder Architecture
// for Efficient Reasoning with Long Generation", section 关键设计) needs two:
//   H = M ⊙ SiLU(X W1^T)   — the SiLU·M Hadamard product fused in the epilogue,
//   Y = H W2^T.
//
// Design (compute-bound at prefill sizes):
//  * Workgroup tiles of 32x32x16 MFMA blocks (on gfx950 the 32x32x16 bf16
//    form measured ~2.4 PFLOP/s in a register-only loop, the 16x16x32 form
//    ~1.4): 256x320, 256x256 and 256x192 tiles of 8 waves (64x160, 128x64,
//    64x96 per wave; one workgroup per CU) and 128x128 tiles of 4 waves
//    (64x64 each; two per CU), chosen per call by how whole rounds of the
//    256 CUs fill (launch_gemm's rule).
//  * K advances BK = 64 at a time through a two-stage LDS ring filled by direct
//    global -> LDS loads (global_load_lds_dwordx4): no register staging, and
//    the next stage's loads run under this stage's MFMAs.  A bare s_barrier
//    plus an explicit vmcnt wait orders the stages (a __syncthreads fence
//    would also wait for the stage still in flight).  16-byte chunks of each
//    128-byte LDS row are XOR-swizzled by (row / 2): the 16 lanes of an
//    operand read hit 16 distinct bank groups (no bank conflicts counted).
//  * Workgroup ids are remapped so each XCD (ids round-robin over 8) works
//    on a contiguous band of tiles, grouped 8 row-tiles at a time.
//  * The epilogue parks each wave's accumulators in LDS (the ring is free by
//    then) so that M (or, for the residual add, h itself) is read and the
//    output written as 16-byte vectors.  The paired form (EPI_SWIGLU) loads
//    gate and up weight rows into one W tile and forms SiLU(g)·u there.
//  * Inside a stage, the fragments of 16-deep k-step ks + 1 are read into a
//    second register set while k-step ks multiplies, one LDS read placed
//    between two MFMAs (scheduling group barriers); only the first k-step
//    of a stage waits for its reads.  The GMU pair at 8192 x 2560 x 5120:
//    0.409-0.412 against 0.425-0.428 ms with the reads of each k-step ahead
//    of its own MFMAs (same box, alternating runs).
//  * Measured at 8192 x 2560 x 5120 before that change (both GMU products
//    on 256x320 tiles, random data): ~243 us for the gate product and ~193
//    us for the output product (885 and 1112 TFLOP/s).  A 3-5 deep ring (BK
//    64 or 32), 16-wave tiles, 128x160 tiles, 4 waves of 128x128 per 256x256
//    tile, 4 waves of 128x160 per 256x320 tile, reading a whole slice's
//    fragments before its MFMAs (forced with scheduling barriers) and a
//    raised wave priority around the MFMA clusters all measured equal or
//    slower; MFMA busy stays under 70%, LDS bank conflicts are zero.
#include "device.hpp"
#include "launch.hpp"

#include <math.h>

namespace sambay {

namespace {

constexpr int kGroupM = 8;
constexpr int kXcds = 8;

// LDS rows hold BK bf16 (CPR 16-byte chunks); chunk c of row r is stored at
// c ^ ((r / RP) % CPR), RP = rows per 256 bytes, so the 32 rows of an operand
// read are spread over all bank groups.
template <int BK>
__device__ __forceinline__ int swz(int row, int chunk) {
    constexpr int CPR = BK / 8, RP = 256 / (2 * BK);
    return chunk ^ ((row / RP) % CPR);
}

// BM x BN output tile per workgroup of WGM x WGN waves; NS-stage LDS ring of
// BK-deep operand slices.
template <int BM, int BN, int WGM, int WGN, int NS, int BK, int EPI>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm32_kernel(const bf16_t *__restrict__ X,
                                                                const bf16_t *__restrict__ W, int rows, int N,
                                                                int K, bf16_t *__restrict__ out,
                                                                const bf16_t *__restrict__ aux, int ksplit) {
    constexpr int NWAVES = WGM * WGN;
    constexpr int TM = BM / WGM, TN = BN / WGN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int ROWS = BM + BN;
    constexpr int CPR = BK / 8;              // 16-byte chunks per LDS row
    constexpr int IROWS = 64 / CPR;          // rows filled by one wave-wide 16-byte copy
    constexpr int INSTS = ROWS / IROWS;
    constexpr int IPW = INSTS / NWAVES;
    static_assert(IPW * NWAVES == INSTS && FM * 32 == TM && FN * 32 == TN, "tile shape");
    // EPI_SWIGLU: the W tile interleaves, per 64 rows, 32 gate rows (W) and
    // the 32 up rows (aux) of the same output columns, so a wave's fragment
    // pair (2p, 2p + 1) holds g and u of one 32-column block and the tile
    // covers BN / 2 output columns.
    constexpr bool PAIR = EPI == EPI_SWIGLU;
    static_assert(!PAIR || FN % 2 == 0, "paired gate/up fragments");
    constexpr int OBN = PAIR ? BN / 2 : BN, OTN = PAIR ? TN / 2 : TN;  // output columns per tile / wave
    // Epilogue staging: blocks of 32 rows x SC columns per wave, SC = the
    // wave's whole width when that fits in LDS and tiles a wave's lanes, else 32.
    constexpr int SC_FULL = NWAVES * 32 * (OTN + 4) * 4 <= 160 * 1024 && OTN / 8 <= 64 && 64 % (OTN / 8) == 0;
    constexpr int SC = SC_FULL ? OTN : 32;
    constexpr int NJB = OTN / SC;                 // column blocks per 32 rows
    constexpr int SROW = SC + 4;                  // fp32 per staged epilogue row
    constexpr int RING_BYTES = NS * ROWS * BK * 2, STAGE_BYTES = NWAVES * 32 * SROW * 4;
    constexpr int LDS_BYTES = RING_BYTES > STAGE_BYTES ? RING_BYTES : STAGE_BYTES;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(1024))) char lds_raw[LDS_BYTES];
    bf16_t(*lds)[ROWS * BK] = reinterpret_cast<bf16_t(*)[ROWS * BK]>(lds_raw);

    const int tiles_m = (rows + BM - 1) / BM, tiles_n = (N + OBN - 1) / OBN;
    const int ntiles = tiles_m * tiles_n;
    // Split K (EPI_F32 only): slice blockIdx.x / ntiles of K / ksplit, its
    // partial sums to the slice's own [rows, N] block of out.
    const int kslice = blockIdx.x / ntiles, Ks = K / ksplit;
    int pid = blockIdx.x % ntiles;
    if (ntiles % kXcds == 0) pid = (pid % kXcds) * (ntiles / kXcds) + pid / kXcds;
    const int group = pid / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int tm = first_m + (pid % (kGroupM * tiles_n)) % gsize;
    const int tn = (pid % (kGroupM * tiles_n)) / gsize;
    const int bm = tm * BM, bn = tn * OBN;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
    const int wm = wave / WGN, wn = wave % WGN;

    const bf16_t *src[IPW];
#pragma unroll
    for (int q = 0; q < IPW; ++q) {
        const int r = (wave * IPW + q) * IROWS + lane / CPR;
        const int logical = swz<BK>(r, lane % CPR);
        const bf16_t *base;
        if (r < BM) {
            base = X + (size_t)min(bm + r, rows - 1) * K;
        } else if (PAIR) {
            const int rw = r - BM, n = bn + 32 * (rw / 64) + (rw & 31);
            base = ((rw & 32) ? aux : W) + (size_t)min(n, N - 1) * K;
        } else {
            base = W + (size_t)min(bn + r - BM, N - 1) * K;
        }
        src[q] = base + (size_t)kslice * Ks + 8 * logical;
    }
    auto issue = [&](int kt, int slot) {
#pragma unroll
        for (int q = 0; q < IPW; ++q) lds_dma16(src[q] + (size_t)kt * BK, &lds[slot][(wave * IPW + q) * IROWS * BK]);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // The lane's 8 output columns in each column block of the epilogue (the
    // same for every vector it stores there): their softplus biases are
    // loaded before the main loop.
    constexpr int VPR = SC / 8;                   // 8-column vectors per staged row
    static_assert(64 % VPR == 0, "epilogue columns");
    float bias[NJB][8];
    if (EPI == EPI_SOFTPLUS) {
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
            const int n_lane = bn + wn * OTN + jb * SC + 8 * (lane % VPR);
            f32x4 b0 = {0.f, 0.f, 0.f, 0.f}, b1 = b0;
            if (n_lane < N) {
                b0 = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(aux) + n_lane);
                b1 = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(aux) + n_lane + 4);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) bias[jb][e] = b0[e], bias[jb][4 + e] = b1[e];
        }
    }

    const int KT = Ks / BK;
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < KT) issue(s, s);
    for (int kt = 0; kt < KT; ++kt) {
        const int slot = kt % NS;
        if (kt + NS - 2 < KT) __builtin_amdgcn_s_waitcnt(0x3f70 | ((IPW * (NS - 2)) & 0xf) | (((IPW * (NS - 2)) >> 4) << 14));
        else __builtin_amdgcn_s_waitcnt(0x3f70);
        __builtin_amdgcn_s_barrier();
        if (kt + NS - 1 < KT) issue(kt + NS - 1, (kt + NS - 1) % NS);
        const bf16_t *sA = lds[slot];
        const bf16_t *sB = lds[slot] + BM * BK;
        // Fragments of k-step ks + 1 are read while k-step ks multiplies (two
        // register sets), one read between two MFMAs.
        u32x4 fa[2][FM], fb[2][FN];
        auto read_frags = [&](int ks, int b) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = wm * TM + 32 * i + l32;
                fa[b][i] = *reinterpret_cast<const u32x4 *>(&sA[r * BK + 8 * swz<BK>(r, 2 * ks + half)]);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int r = wn * TN + 32 * j + l32;
                fb[b][j] = *reinterpret_cast<const u32x4 *>(&sB[r * BK + 8 * swz<BK>(BM + r, 2 * ks + half)]);
            }
        };
        read_frags(0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int b = ks & 1;
            if (ks + 1 < BK / 16) read_frags(ks + 1, b ^ 1);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(fa[b][i], fb[b][j], acc[i][j]);
            if (ks + 1 < BK / 16) {
                constexpr int NR = FM + FN, NM = FM * FN;
#pragma unroll
                for (int q = 0; q < (NR < NM ? NR : NM); ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                }
                if (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM > NR ? NM - NR : 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Epilogue through LDS: acc[i][j][v] holds row TM·wm + 32·i + 8·(v/4) +
    // 4·half + v%4, col TN·wn + 32·j + l32 of the tile, so each lane owns one
    // column.  Each wave parks a 32 x SC block of its accumulators in its own
    // LDS area, then every lane handles 8 consecutive columns: one 16-byte
    // load of M (gate) or h (residual) and one 16-byte store per vector
    // instead of 2-byte accesses.  Those loads run PD - 1 blocks ahead (all
    // blocks when they fit in 64 registers).
    constexpr int VPL = 32 * VPR / 64;            // vectors per lane per block
    static_assert(VPL * 64 == 32 * VPR, "epilogue shape");
    constexpr int NB = FM * NJB;                  // blocks per wave
    constexpr int PD = NB * VPL <= 16 ? NB : 2;
    constexpr bool AUX = EPI == EPI_GATE || EPI == EPI_RESID;
    float *stage = reinterpret_cast<float *>(lds_raw) + wave * 32 * SROW;
    u32x4 mv[PD][VPL];
    auto load_aux = [&](int blk) {  // M (gate) or the residual h itself (out)
        const bf16_t *src = EPI == EPI_GATE ? aux : out;
        const int i = blk / NJB, jb = blk % NJB;
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
            const int idx = u * 64 + lane, r = idx / VPR, c8 = idx % VPR;
            const int m = bm + wm * TM + 32 * i + r, n = bn + wn * OTN + jb * SC + 8 * c8;
            mv[blk % PD][u] = (m < rows && n < N) ? ld16(src + (size_t)m * N + n) : (u32x4){0u, 0u, 0u, 0u};
        }
    };
    if (AUX) {
#pragma unroll
        for (int blk = 0; blk < PD - 1; ++blk) load_aux(blk);
    }
    __syncthreads();  // every wave is done with the operand ring
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
        const int i = blk / NJB, jb = blk % NJB;
        if (AUX && blk + PD - 1 < NB) load_aux(blk + PD - 1);
#pragma unroll
        for (int jj = 0; jj < SC / 32; ++jj) {
            const int q = jb * (SC / 32) + jj;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                float val;
                if constexpr (PAIR) {  // SiLU(g) · u
                    const float g = acc[i][2 * q][v];
                    val = (g / (1.f + expf(-g))) * acc[i][2 * q + 1][v];
                } else {
                    val = acc[i][q][v];
                }
                stage[(8 * (v / 4) + 4 * half + (v % 4)) * SROW + 32 * jj + l32] = val;
            }
        }
        wave_lds_fence();
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
            const int idx = u * 64 + lane, r = idx / VPR, c8 = idx % VPR;
            const int m = bm + wm * TM + 32 * i + r, n = bn + wn * OTN + jb * SC + 8 * c8;
            const f32x4 lo = *reinterpret_cast<const f32x4 *>(&stage[r * SROW + 8 * c8]);
            const f32x4 hi = *reinterpret_cast<const f32x4 *>(&stage[r * SROW + 8 * c8 + 4]);
            float x[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            if (EPI == EPI_GATE) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t w = mv[blk % PD][u][e / 2];
                    const float mm = (e & 1) ? hi_bf16(w) : lo_bf16(w);
                    x[e] = mm * (x[e] / (1.f + expf(-x[e])));
                }
            }
            if (EPI == EPI_RESID) {  // h = bf16(h + acc)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t w = mv[blk % PD][u][e / 2];
                    x[e] += (e & 1) ? hi_bf16(w) : lo_bf16(w);
                }
            }
            if (EPI == EPI_SOFTPLUS) {  // softplus(acc + bias[n]), the SSM layer's step sizes
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float a = x[e] + bias[jb][e];
                    // log(1 + e^a) with the hardware exp/log: exact enough where it matters (|a| <= 20);
                    // a itself above, e^a below -15 (1 + e^a would round to 1).
                    x[e] = a > 20.f ? a : (a < -15.f ? __expf(a) : __logf(1.f + __expf(a)));
                }
            }
            if (EPI == EPI_F32 || EPI == EPI_SOFTPLUS) {  // fp32 output: out is a float array
                if (m < rows && n < N) {
                    float *of = reinterpret_cast<float *>(out) + ((size_t)kslice * rows + m) * N + n;
                    *reinterpret_cast<f32x4 *>(of) = (f32x4){x[0], x[1], x[2], x[3]};
                    *reinterpret_cast<f32x4 *>(of + 4) = (f32x4){x[4], x[5], x[6], x[7]};
                }
            } else {
                u32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
                if (m < rows && n < N) *reinterpret_cast<u32x4 *>(out + (size_t)m * N + n) = o;
            }
        }
        wave_lds_fence();
    }
}

template <int BM, int BN, int WGM, int WGN, int NS, int BK>
hipError_t launch_tile(const bf16_t *X, const bf16_t *W, int rows, int N, int K, Epilogue epi, bf16_t *out,
                     const bf16_t *aux, int ksplit, hipStream_t stream) {
    const int obn = epi == EPI_SWIGLU ? BN / 2 : BN;
    const int tiles = ((rows + BM - 1) / BM) * ((N + obn - 1) / obn) * ksplit;
    TimingScope ts(kTimeGemm, stream);
    if (epi == EPI_GATE)
        hipLaunchKernelGGL((gemm32_kernel<BM, BN, WGM, WGN, NS, BK, EPI_GATE>), dim3(tiles), dim3(64 * WGM * WGN), 0,
                           stream, X, W, rows, N, K, out, aux, ksplit);
    else if (epi == EPI_F32)
        hipLaunchKernelGGL((gemm32_kernel<BM, BN, WGM, WGN, NS, BK, EPI_F32>), dim3(tiles), dim3(64 * WGM * WGN), 0,
                           stream, X, W, rows, N, K, out, aux, ksplit);
    else if (epi == EPI_RESID)
        hipLaunchKernelGGL((gemm32_kernel<BM, BN, WGM, WGN, NS, BK, EPI_RESID>), dim3(tiles), dim3(64 * WGM * WGN), 0,
                           stream, X, W, rows, N, K, out, aux, ksplit);
    else if (epi == EPI_SWIGLU) {
        if constexpr ((BN / WGN / 32) % 2 == 0)
            hipLaunchKernelGGL((gemm32_kernel<BM, BN, WGM, WGN, NS, BK, EPI_SWIGLU>), dim3(tiles), dim3(64 * WGM * WGN),
                               0, stream, X, W, rows, N, K, out, aux, ksplit);
        else
            return hipErrorInvalidValue;  // the paired form needs fragment pairs per wave
    }
    else if (epi == EPI_SOFTPLUS)
        hipLaunchKernelGGL((gemm32_kernel<BM, BN, WGM, WGN, NS, BK, EPI_SOFTPLUS>), dim3(tiles),
                           dim3(64 * WGM * WGN), 0, stream, X, W, rows, N, K, out, aux, ksplit);
    else
        hipLaunchKernelGGL((gemm32_kernel<BM, BN, WGM, WGN, NS, BK, EPI_BF16>), dim3(tiles), dim3(64 * WGM * WGN), 0,
                           stream, X, W, rows, N, K, out, aux, ksplit);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const bf16_t *X, const bf16_t *W, int rows, int N, int K, Epilogue epi, bf16_t *out,
                       const bf16_t *aux, hipStream_t stream, int ksplit) {
    if (ksplit < 1 || K % (64 * ksplit) != 0 || (ksplit > 1 && epi != EPI_F32)) return hipErrorInvalidValue;
    // Tile shape by how the grid fills the 256 CUs.  The large tiles (8
    // waves, one workgroup per CU) read less LDS per MFMA; two 128x128
    // workgroups per CU fill 512 slots per round.  Each shape is priced as
    // its rounds of tiles times a round's area over the shape's rate, a last
    // partial round at 0.4 + 0.6 x its fill (a part-filled chip runs each
    // tile faster).  Rates per unit of tile area, measured on MI355X over
    // 2048-32768 rows and the prefill products (random operands): 256x320
    // and 256x256 1.0, 256x192 0.9, 128x128 0.8; the rule's choice was
    // within 0.7% of the fastest shape in all 24 measured cases (e.g. the
    // GMU products at 8192 rows on 256x320 tiles, 5120 x 2560: 253 vs 284
    // us with 128x128; 2560 x 5120: 203 vs 255 us; 3072-wide outputs at
    // 8192 rows on 256x192, 3072 x 6144: 325 vs 340 us).  All shapes add
    // the same products in the same order (identical bits).  The softplus
    // epilogue keeps 320-wide tiles out (its 5 bias vectors spill).
    if (ksplit > 1) return launch_tile<128, 128, 2, 2, 2, 64>(X, W, rows, N, K, epi, out, aux, ksplit, stream);
    struct Shape { int bm, bn, per_cu; double rate; };
    const Shape shapes[] = {{256, 320, 1, 1.0}, {256, 256, 1, 1.0}, {256, 192, 1, 0.9}, {128, 128, 2, 0.8}};
    int best = -1;
    double best_t = 0.0;
    for (int i = 0; i < 4; ++i) {
        const Shape &c = shapes[i];
        if (c.bn == 320 && epi == EPI_SOFTPLUS) continue;
        // The paired SwiGLU form needs an even number of 32-column fragments
        // per wave (256x256 and 128x128); its tiles cover bn / 2 outputs.
        if (epi == EPI_SWIGLU && (c.bn == 320 || c.bn == 192)) continue;
        const int obn = epi == EPI_SWIGLU ? c.bn / 2 : c.bn;
        const int64_t tiles = (int64_t)((rows + c.bm - 1) / c.bm) * ((N + obn - 1) / obn);
        const int64_t slots = 256LL * c.per_cu, full = tiles / slots, rem = tiles % slots;
        const double rounds = (double)full + (rem ? 0.4 + 0.6 * (double)rem / (double)slots : 0.0);
        const double t = rounds * c.bm * c.bn * c.per_cu / c.rate;
        if (best < 0 || t < best_t) best = i, best_t = t;
    }
    switch (best) {
        case 0: return launch_tile<256, 320, 4, 2, 2, 64>(X, W, rows, N, K, epi, out, aux, ksplit, stream);
        case 1: return launch_tile<256, 256, 2, 4, 2, 64>(X, W, rows, N, K, epi, out, aux, ksplit, stream);
        case 2: return launch_tile<256, 192, 4, 2, 2, 64>(X, W, rows, N, K, epi, out, aux, ksplit, stream);
        default: return launch_tile<128, 128, 2, 2, 2, 64>(X, W, rows, N, K, epi, out, aux, ksplit, stream);
    }
}

}  // namespace sambay
