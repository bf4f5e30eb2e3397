// Device helpers shared by the gfx950 kernels: number formats, wave64
// primitives and MFMA operand types.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;

// ---- bfloat16 (raw 16-bit patterns) ----------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even to bfloat16 (finite inputs): add 0x7FFF plus the
// lowest kept bit, then truncate.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---- OCP FP8 E4M3FN encode -------------------------------------------------
// Round to nearest even, saturate the magnitude at 448 (code 0x7E), keep the
// sign bit of the input.  Normal results (|v| >= 2^-6) round the fp32
// significand at bit 20 (3 fraction bits kept); smaller magnitudes are
// multiples of 2^-9 (subnormal codes 0..7, 8 meaning 2^-6).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
    // v_cvt_pk_fp8_f32 rounds to nearest even into OCP e4m3 (finite range
    // +-448, subnormals kept); inputs are clamped to that range first.  On
    // gfx950 this equals the bitwise rounding of the value for every fp32
    // input of magnitude <= 448 (checked exhaustively on the device).
    const float c = fmaxf(fminf(v, 448.0f), -448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}

// four values to four e4m3 codes, little-endian in one word
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
    a = fmaxf(fminf(a, 448.0f), -448.0f);
    b = fmaxf(fminf(b, 448.0f), -448.0f);
    c = fmaxf(fminf(c, 448.0f), -448.0f);
    d = fmaxf(fminf(d, 448.0f), -448.0f);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// ---- OCP MX (microscaling) block exponents ----------------------------------
// A block of 32 values shares the scale 2^(E-127) (E8M0).  Per the OCP MX
// conversion rule E - 127 = floor(log2(amax)) - emax_elem, clamped to the
// E8M0 range; emax_elem = 8 for FP8 E4M3 elements (448 = 1.75 * 2^8).  For a
// normal amax, floor(log2(amax)) is its exponent field minus 127, so
// E = exponent field - 8; a zero or subnormal amax gives E = 0.  Finite fp32
// inputs keep E <= 246.
__device__ __forceinline__ uint32_t mx_e8m0_for_e4m3(float amax) {
    const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
    return (uint32_t)max(ef - 8, 0);
}

// 2^(127 - E) as an fp32 number (exact and normal for E <= 253): values times
// this factor are the block's elements before rounding.
__device__ __forceinline__ float mx_inv_scale(uint32_t E) { return __uint_as_float((254u - E) << 23); }

// ---- wave64 helpers ----------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo = __shfl_xor(lo, m, kWave);
    hi = __shfl_xor(hi, m, kWave);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o = shfl_xor_u64(v, m);
        v = o > v ? o : v;
    }
    return v;
}

// Order-preserving map of an fp32 value to uint32 (for -0 == +0 callers must
// canonicalise first).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace moe
