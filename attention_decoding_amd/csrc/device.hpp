// Device-side building blocks shared by the gfx950 kernels: bf16 bit
// conversions, 16-byte vector types, and the wave64 MFMA tile used by every
// matrix product in the library.
//
// MFMA tile (v_mfma_f32_16x16x32_bf16, CDNA4): D[16x16] += A[16x32] · B[32x16].
// Operand layout per lane l of the wave (row/col = l % 16, grp = l / 16):
//   A: row (l % 16), k elements 8·grp .. 8·grp+7   (eight bf16, 16 bytes)
//   B: col (l % 16), k elements 8·grp .. 8·grp+7
//   D: col (l % 16), rows 4·grp .. 4·grp+3         (four fp32)
// The kernels only rely on A and B pairing the same (grp, element) slots, so
// any fixed assignment of the 32 contraction indices to those slots is valid;
// they pick the one that lets every lane load 16 contiguous bytes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sambay {

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

typedef __attribute__((ext_vector_type(2))) float f32x2v;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;

// Round to nearest, ties to even (NaN stays a NaN), by gfx950's packed
// conversion (v_cvt_pk_bf16_f32): for every finite fp32 value it gives the
// bits of the integer rounding u + 0x7fff + ((u >> 16) & 1) >> 16 (checked
// over all 2^32 patterns), in one instruction per pair.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){lo, hi}, bf16x2v));
}

// The low part of y's bf16 hi + lo pair: bf16(y - hi), hi = bf16(y), y as
// rounded to fp32.  No multiply-add contraction here: fusing the subtraction
// with the multiply that produced y would form lo from the unrounded product
// in some kernels and not in others.
__device__ __forceinline__ bf16_t split_lo(float y, bf16_t hi) {
#pragma clang fp contract(off)
    return f32_to_bf16(y - bf16_to_f32(hi));
}

// Low / high bf16 of a packed pair, widened to fp32.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16: D[32x32] += A[32x16] · B[16x32].  Lane l supplies
// A row (l % 32) and B col (l % 32), k elements 8·(l/32) .. 8·(l/32)+7; D
// register v of lane l is row 8·(v/4) + 4·(l/32) + (v%4), col l % 32.  On
// gfx950 it delivers twice the bf16 rate of the 16x16x32 form (measured).
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Non-temporal 16-byte load (streamed weights: read once per step).
__device__ __forceinline__ u32x4 ld16_nt(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Register loads in MFMA operand layouts (64 bytes of each of 16 rows per
// instruction) stay plain: the non-temporal hint measured ~8% slower there.
// Whole-row streams copied into LDS (the attention kernel's K and V) take
// it: 6.9-7.0 against 6.0-6.3 TB/s in a read probe of the same block walk.

// 16-byte global -> LDS copy (gfx950 global_load_lds_dwordx4): lane i's 16
// bytes land at lds_base + 16·i; lds_base must be wave-uniform.  Completion
// is tracked by vmcnt, not lgkmcnt.
__device__ __forceinline__ void lds_dma16(const void *gsrc, void *lds_base) {
    __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void *)(lds_base), 16, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Orders this wave's LDS accesses across lanes without a workgroup barrier.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace sambay
