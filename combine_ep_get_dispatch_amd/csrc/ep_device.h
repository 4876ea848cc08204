// Device-side helpers for the gfx950 kernels: bf16 unpacking, the fp32 ->
// OCP E4M3 and fp32 -> bf16 conversions, and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 16-byte loads and stores with the non-temporal hint, for data that is
// streamed exactly once (rows read once, outputs written once): they do not
// displace reused data from the caches.
__device__ __forceinline__ uint4 load_nt(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(void* p, const uint4& v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, static_cast<u32x4*>(p));
}

// 16-byte store with the device-scope cache policy (sc1): the line is
// written through the XCD's L2 instead of staying dirty there.  Used for the
// receive rows, which the next kernel reads from other XCDs: it leaves less
// L2 write-back for the end of the kernel (measured faster than ordinary and
// than non-temporal stores for dispatch's scattered rows).  A store of more
// than 8 bytes needs two wait states on gfx950 before a VALU instruction may
// overwrite its data registers; the compiler inserts them after the stores it
// generates but cannot see into inline asm, so the asm carries its own.
__device__ __forceinline__ void store_wt(void* p, const uint4& v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" : : "v"(p), "v"(w) : "memory");
}

// The same for 8 bytes (no wait states needed after a store of 8 bytes or less).
__device__ __forceinline__ void store_wt8(void* p, const uint2& v) {
    const u32x2 w = {v.x, v.y};
    asm volatile("global_store_dwordx2 %0, %1, off sc1" : : "v"(p), "v"(w) : "memory");
}

// bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> two bf16 (round to nearest even) packed low/high, with gfx950's
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

// Four fp32 -> four OCP E4M3 codes packed into a dword (byte i = value i),
// with gfx950's v_cvt_pk_fp8_f32: round to nearest even.  Inputs of the
// quantiser never exceed 448 * (1 + 2^-23) in magnitude, which rounds to 448,
// so the instruction's out-of-range behaviour is never reached there.
__device__ __forceinline__ uint32_t e4m3x4_hw(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Bit-level fp32 -> OCP E4M3, round to nearest even, saturating to +-448,
// sign kept, NaN -> S.1111.111.  Normal results keep the top 3 fp32 mantissa
// bits after rounding the 20 dropped bits to nearest even (a carry moves into
// the exponent); results below 2^-6 are multiples of 2^-9, found by scaling
// by 2^9 (exact) and rounding to an integer.
__device__ __forceinline__ uint32_t e4m3_sw(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7fu;           // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;          // |v| >= 448
    if (a < 0x3c800000u) {                              // |v| < 2^-6
        const float q = __builtin_rintf(__uint_as_float(a) * 512.0f);
        return sign | (uint32_t)q;                      // 0..8 (8 = 2^-6)
    }
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
    uint32_t code = r - ((127u - 7u) << 3);
    if (code > 0x7eu) code = 0x7eu;
    return sign | code;
}

__device__ __forceinline__ uint32_t e4m3x4_sw(float a, float b, float c, float d) {
    return e4m3_sw(a) | (e4m3_sw(b) << 8) | (e4m3_sw(c) << 16) | (e4m3_sw(d) << 24);
}

// Unsigned maximum over the 8 lanes of an aligned group of 8, with three DPP
// moves (no LDS round trip): swap neighbours (quad_perm 1,0,3,2), swap pairs
// (quad_perm 2,3,0,1), then mirror each half row of 8 lanes, which pairs the
// two quads.  A source lane that is inactive reads as 0, which leaves an
// unsigned maximum unchanged.
__device__ __forceinline__ uint32_t group8_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));
    return v;
}

// Unsigned maximum over the 16 lanes of a DPP row: the maximum over each
// half row, then a row mirror (lane i reads lane 15 - i) pairs the halves.
__device__ __forceinline__ uint32_t group16_max_u32(uint32_t v) {
    v = group8_max_u32(v);
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));
    return v;
}

// Sum over aligned segments of S lanes (S a power of two, 1..64), every lane
// of a segment receiving its segment's total.  Segments of up to 16 lanes lie
// inside a DPP row and take DPP moves: neighbour and pair swaps, then the
// half-row and row mirrors, which pair the halves; wider segments finish with
// cross-row shuffles.  All 64 lanes must be active.
__device__ __forceinline__ int segment_sum(int v, int S) {
    if (S >= 2) v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xf, 0xf, false);
    if (S >= 4) v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xf, 0xf, false);
    if (S >= 8) v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, false);
    if (S >= 16) v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, false);
    if (S >= 32) v += __shfl_xor(v, 16);
    if (S >= 64) v += __shfl_xor(v, 32);
    return v;
}

}  // namespace ep
