// Internal helpers shared by the gfx950 kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// ---- number formats ---------------------------------------------------------

__device__ __forceinline__ float bf16_to_float(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// fp16 -> f32 through the hardware conversion (exact, subnormals included).
__device__ __forceinline__ float half_to_float(uint32_t h16) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)h16);
    return (float)h;
}

// f32 -> fp16 with the hardware conversion in the default round-to-nearest-even
// mode (fp16 denormals are kept). The empty asm keeps the value in a register
// so that a producing multiply is not folded into a mixed-precision FMA with a
// +0 addend, which would turn a -0 product into +0.
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
    __asm__ volatile("" : "+v"(f));
    _Float16 h = (_Float16)f;
    return __builtin_bit_cast(uint16_t, h);
}

// f32 -> bf16, round half to even on the 16 discarded bits (finite inputs
// and infinities; a NaN keeps a quiet NaN pattern).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
    uint32_t round_bit = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + round_bit) >> 16);
}

// ---- wavefront reductions ---------------------------------------------------

// Sum over the 64 lanes of a wavefront; every lane receives the total.
// Within each row of 16 lanes: DPP quad permutes and row mirrors; across the
// four rows: lane reads of the row totals.
__device__ __forceinline__ float wave_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)); // row_half_mirror
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)); // row_mirror
    float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
}

// ---- nibble unpacking ---------------------------------------------------------

// Low and high nibbles of each byte of a packed dword, as bytes 0..15.
__device__ __forceinline__ uint32_t lo_nibbles(uint32_t w) { return w & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t hi_nibbles(uint32_t w) { return (w >> 4) & 0x0F0F0F0Fu; }

// 6-bit codes: bytes b = 0..3 of the result take bits 2j and 2j + 1 of byte b
// of the high-bit plane word w, moved to bits 4 and 5 (the two bits above the
// code's low nibble).
__device__ __forceinline__ uint32_t two_bits_high(uint32_t w, int j) { return ((w >> (2 * j)) & 0x03030303u) << 4; }

// Bytes q in 0..15 -> signed bytes q - 8. Adding 0x78 keeps every byte below
// 0x88 (no carry between bytes); flipping bit 7 then subtracts 128.
__device__ __forceinline__ uint32_t minus8_bytes(uint32_t q) { return (q + 0x78787878u) ^ 0x80808080u; }

// ---- activation codes -----------------------------------------------------------

// Inverse of a block scale for the fast path of act_code, or 0 when the fast
// path must not be used (scale zero or subnormal).
__device__ __forceinline__ float act_inverse(float s) {
    return (s >= 0x1p-125f) ? __builtin_amdgcn_rcpf(s) : 0.0f;
}

// Code of one activation: clamp(round_half_even(v / s), -127, 127) with the
// correctly rounded float32 quotient v / s, for |v| <= 127 s (s = amax / 127).
// Fast path: r = v * rcp(s). v_rcp_f32 is within 1 ulp, so for |v / s| < 128
// r is within 2^-15 of the rounded quotient; when r is at least 2^-12 away from
// the nearest half-integer both sit inside the same rounding cell and round to
// the same integer. Near a half-integer (and when `inv` is 0) the exact
// quotient decides.
__device__ __forceinline__ int act_code(float v, float s, float inv) {
    float r = v * inv;
    const float f = r - floorf(r);
    if (inv == 0.0f || fabsf(f - 0.5f) < 0x1p-12f) r = v / s;
    const int c = (int)rintf(r);
    return min(127, max(-127, c));
}

}  // namespace q4
