// Shared device helpers for the gfx950 MoE kernels: vector types, bf16 and
// e4m3fn conversions, MFMA wrappers and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (inputs are finite here), by
// gfx950's v_cvt_pk_bf16_f32 (fp32 denormals are kept in these kernels, so
// it rounds every finite value as the bit-level rule u + 0x7FFF + lsb, >> 16,
// does); pack_bf16x2 rounds two values into one word with one instruction.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Unpack 8 bf16 values held in a 16-byte word.
__device__ __forceinline__ void unpack_bf16x8(const u32x4_t v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ u32x4_t pack_bf16x8(const float* f) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return r;
}

// --------------------------------------------------------------- e4m3fn ----
// Round-to-nearest-even encoding of a finite fp32 value with |v| <= 448 into
// an OCP e4m3fn code (bias 7, 3 mantissa bits, subnormals below 2^-6), by
// gfx950's v_cvt_pk_fp8_f32.  Measured identical to the bit-level definition
// (exponent rebias, 3 mantissa bits, ties to even, subnormals as m * 2^-9) on
// 10^6 normal samples scaled by 2^-12 .. 2^11 (clamped to +-448) plus every
// e4m3 value, every midpoint between neighbours and the fp32 values on either
// side of it, both signs.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.f, 0, false) & 0xFFu;
}

// a / s rounded to nearest even, from y = 1 / s (itself rounded to nearest),
// for scales s >= kDivFastMin; callers divide outright below that.  The
// product |a| y is within 2 ulps of |a| / s; each step q += (|a| - q s) y takes
// the exact FMA residual, and the second starts within 1 ulp and so rounds
// correctly (Markstein's theorem for FMA division).  The residuals are exact
// while s >= kDivFastMin and |a| / s >= 2^-10 (half the smallest e4m3 step);
// below that the quotient may be off by an ulp, but every such value maps to
// the e4m3 code 0 either way.  The sign is restored last, so -0 stays -0.
// Four FMA-rate operations per value instead of a full-precision division.
constexpr float kDivFastMin = 0x1p-64f;
__device__ __forceinline__ float div_rn_by(float a, float s, float y) {
  const float m = fabsf(a);
  float q = m * y;
  q = __builtin_fmaf(__builtin_fmaf(-q, s, m), y, q);
  q = __builtin_fmaf(__builtin_fmaf(-q, s, m), y, q);
  return __builtin_copysignf(q, a);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t ef = (c >> 3) & 0xFu, mf = c & 7u;
  float mag = ef == 0 ? (float)mf * 0.001953125f
                      : __uint_as_float(((ef + 120u) << 23) | (mf << 20));
  return (c & 0x80u) ? -mag : mag;
}

// ----------------------------------------------------------------- MXFP8 ----
// E8M0 code of an MX block (32 values) with absolute maximum amax >= 0:
// floor(log2(amax)) - 8 + 127, clamped at 0 (an all-zero block, and blocks
// below 2^-118, take 2^-127).  For a normal amax the biased fp32 exponent E
// is floor(log2(amax)) + 127, so the code is max(E - 8, 0).
__device__ __forceinline__ uint32_t mx_e8m0(float amax) {
  const int E = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return (uint32_t)max(E - 8, 0);
}

// 2^-(code - 127) as fp32 (codes 0 .. 253): the factor that scales a block's
// values into its e4m3 range, exactly.
__device__ __forceinline__ float mx_inv_scale(uint32_t code) {
  return __uint_as_float((254u - code) << 23);
}

// ----------------------------------------------------------------- MFMA ----
// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16).  Lane l supplies row l%16
// of A and column l%16 of B, 8 consecutive k each; lane l receives
// D[4*(l/16) + i][l%16], i = 0..3.
__device__ __forceinline__ f32x4_t mfma_bf16_16x16x32(const u32x4_t a, const u32x4_t b,
                                                     f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D(16x16 fp32) += A(16x128 e4m3) * B(128x16 e4m3), unit scales.  Lane l
// supplies 32 codes of row l%16 of A and of column l%16 of B.
__device__ __forceinline__ f32x4_t mfma_fp8_16x16x128(const i32x8_t a, const i32x8_t b,
                                                     f32x4_t c) {
  // cbsz = blgp = 0 selects e4m3 for both operands; scale 127 = 2^0 (e8m0).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// D += A(16x128 e4m3) * B(128x16 e4m3) with MX block scales: lane l holds
// row / column l%16, bytes 0..15 at K 16*(l/16) and bytes 16..31 at K
// 64 + 16*(l/16); its E8M0 scale (bits 7:0 of sa / sb) applies to K block
// l/16 (K 32*(l/16) .. +32) of its row / column (measured on gfx950).
__device__ __forceinline__ f32x4_t mfma_mx8_16x16x128(const i32x8_t a, const i32x8_t b, f32x4_t c,
                                                      uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, (int)sa, 0, (int)sb);
}

// ------------------------------------------------------- wave reductions ----
__device__ __forceinline__ float wave_max_xor(float v, int lanes) {
  for (int m = 1; m < lanes; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// Maximum over each row of 16 lanes (lanes 16 r .. 16 r + 15), returned in
// every lane of the row, by DPP moves (no LDS crossbar): swap neighbours,
// swap pairs, then mirror within 8 and within 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));    // quad_perm 1,0,3,2
  v = fmaxf(v, dpp_mov<0x4E>(v));    // quad_perm 2,3,0,1
  v = fmaxf(v, dpp_mov<0x141>(v));   // row_half_mirror
  v = fmaxf(v, dpp_mov<0x140>(v));   // row_mirror
  return v;
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace moe
