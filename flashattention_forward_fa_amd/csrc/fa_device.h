// fa_device.h -- device helpers shared by the forward and backward kernels.
#pragma once

#include "fa_ns.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

FA_NS_BEGIN

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;


// Swizzled tile layout in LDS (rows of D bf16 values, e.g. keys of a V block):
// row r holds its 16-byte chunks with chunk c stored at position c ^ vswz<D>(r).
// Two read patterns must be free of bank conflicts:
//  * transpose reads (ds_read_b64_tr_b16), served 32 lanes at a time: lanes
//    0-31 read rows 4g+0..3 (+8, +16 k) at the four chunks 4t..4t+3;
//  * 16-byte row reads, served 16 lanes at a time: rows 0..15 at one chunk.
// At D = 128 a row is 256 B (all 64 banks), so f must be a permutation of
// 0..15 over 16 consecutive rows and give rows 4g+0..3 disjoint quarters.  At
// D = 64 a row is 128 B: odd rows sit on the upper 32 banks, rows r and r+2
// must take opposite 64-byte halves, and the 8 even (odd) rows of a 16-row
// read must land on distinct chunks.  16-byte writes are conflict-free in any
// layout.
template <int D>
__device__ __forceinline__ int vswz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) ^ ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// The lane index, computed afresh: the mask passes through an empty asm, so
// the compiler cannot reuse (and keep live) a lane index computed earlier.
// Used where a lane-dependent value is needed only after or rarely inside a
// long loop whose register budget is full.
__device__ __forceinline__ int fresh_lane() {
    unsigned m = ~0u;
    asm volatile("" : "+s"(m));
    return (int)__builtin_amdgcn_mbcnt_hi(m, __builtin_amdgcn_mbcnt_lo(m, 0u));
}

__device__ __forceinline__ float lane_pair_max(float x) {
    // Combine lanes l and l^32 (both halves see the maximum of the pair).
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
    const f32x2 f = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

// Sum of the two bf16 halves of a word, accumulated in fp32 (v_dot2 with (1, 1)).
__device__ __forceinline__ float add_bf16x2(unsigned word, float acc) {
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, word), ones, acc, false);
}

// Two floats -> two fp16 (round to nearest even) in one v_cvt_pk_f16_f32.
__device__ __forceinline__ unsigned pack_f16x2(float a, float b) {
    const f32x2 f = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f, f16x2));
}

// Sum of the two fp16 halves of a word, accumulated in fp32 (v_dot2 with (1, 1)).
__device__ __forceinline__ float add_f16x2(unsigned word, float acc) {
    const f16x2 ones = __builtin_bit_cast(f16x2, 0x3C003C00u);
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, word), ones, acc, false);
}

// Two bf16 (one word) -> two fp16, exactly for magnitudes below 65536 (bf16
// has 8 significant bits and fp16 11, with the wider exponent range above
// 2^-14; bf16 values from 2^16 up become infinite).
__device__ __forceinline__ unsigned bf16x2_to_f16x2(unsigned word) {
    return pack_f16x2(__uint_as_float(word << 16), __uint_as_float(word & 0xFFFF0000u));
}

// As bf16x2_to_f16x2 for values scaled by `sc` (a power of two) first.
__device__ __forceinline__ unsigned bf16x2_to_f16x2_scaled(unsigned word, float sc) {
    return pack_f16x2(__uint_as_float(word << 16) * sc, __uint_as_float(word & 0xFFFF0000u) * sc);
}

// 2^x without the transcendental unit: 2^j * p(f), j = floor(x), f = x - j in
// [0, 1), with p the degree-3 polynomial of least relative error on [0, 1]
// (Remez exchange; csrc/fit_exp2_poly.py prints these coefficients and the
// bound, 7.48e-5) and 2^j applied to the exponent field (v_ldexp_f32).  For
// the forward's split exp2 ("Flash Attention 4", section "algorithm
// structure": part of a block's exponentials on the FMA pipes).  x is clamped
// at -200 so -inf (masked scores) gives exactly 0; a NaN x also gives 0.
constexpr float kExp2C0 = 0.99992521856271555f;
constexpr float kExp2C1 = 0.69583354049475288f;
constexpr float kExp2C2 = 0.22606715542748335f;
constexpr float kExp2C3 = 0.078024522640479307f;

__device__ __forceinline__ float exp2_poly(float x) {
    x = fmaxf(x, -200.f);
    const float f = __builtin_amdgcn_fractf(x);   // x - floor(x), v_fract_f32
    const float p = fmaf(fmaf(fmaf(kExp2C3, f, kExp2C2), f, kExp2C1), f, kExp2C0);
    return ldexpf(p, (int)floorf(x));
}

// Global loads go through buffer resources: a descriptor per K/V block whose
// range ends at the block's last valid key, so keys past the end read as 0
// with no branch and no address arithmetic per block.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, unsigned voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

FA_NS_END  // namespace fa
