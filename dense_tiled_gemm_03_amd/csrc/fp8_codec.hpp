// fp32 -> OCP E4M3FN block quantisation, element by element: the scale of
// a block from its absolute maximum and the code of one element.  Shared by
// the block quantiser kernels and the GEMM's fp8-output epilogue, so both
// round the same way ("TileKernels deep dive", section 7.2: scale = block
// maximum over 448, code = x / scale cast to E4M3; section 4.3: E4M3 FN).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

// e4m3fn codes of |y| <= 448, rounded to nearest with ties to the even
// fraction, sign kept (-0 and negatives that round to zero give 0x80): the
// hardware conversion, two values per instruction.  On every fp32 value in
// [-448, 448] it gives the code of the plain definition -- below 2^-6 the
// nearest multiple of 2^-9, above it the fraction rounded to 3 bits with the
// carry moving into the exponent, exponent bias 7 -- which a comparison over
// all 2.28e9 such values on the GPU confirmed.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xFFu;
}

// Four codes packed little-endian (a in the lowest byte).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// The block's scale, and whether it is an all-zero block.
__device__ __forceinline__ float block_scale(float amax, bool& zero) {
  const float s = amax / 448.0f;
  zero = s == 0.0f;
  return zero ? 1.0f : s;
}

// x / s correctly rounded to fp32, clamped to +-448: the value a code rounds.
__device__ __forceinline__ float scaled(float x, float s) {
  return fminf(fmaxf(x / s, -448.0f), 448.0f);
}

// Code of x in a block of scale s: the rounded quotient x / s, clamped to
// +-448, rounded to e4m3fn; 0 in an all-zero block.
__device__ __forceinline__ uint32_t code_of(float x, float s, bool zero) {
  const uint32_t c = e4m3_code(scaled(x, s));
  return zero ? 0u : c;
}

// Scales for which quotient_by() is exact.
__device__ __forceinline__ bool scale_in_fast_range(float s) {
  return s >= 0x1p-60f && s <= 0x1p60f;
}

// The correctly rounded quotient x / s from r = 1 / s correctly rounded:
// q = x r is within one ulp of x / s, the FMA gives the remainder x - s q
// exactly, and q + (x - s q) r rounded to nearest is the correctly rounded
// quotient (Markstein's theorem for division), as long as nothing
// underflows.  For 2^-60 <= s <= 2^60 that holds whenever the quotient is at
// least 2^-10, the least magnitude that does not round to a zero code; below
// it the result stays below 2^-10, which is all the code needs.  The sign is
// x's (s > 0): copying it back keeps -0, which the correction step would turn
// into +0.
__device__ __forceinline__ float quotient_by(float x, float s, float r) {
  const float q = x * r;
  const float e = __builtin_fmaf(-q, s, x);
  return copysignf(__builtin_fmaf(e, r, q), x);
}

// scaled() and code_of() with the quotient from quotient_by(), for scales
// in the fast range.
__device__ __forceinline__ float scaled_fast(float x, float s, float r) {
  return fminf(fmaxf(quotient_by(x, s, r), -448.0f), 448.0f);
}
__device__ __forceinline__ uint32_t code_of_fast(float x, float s, float r, bool zero) {
  const uint32_t c = e4m3_code(scaled_fast(x, s, r));
  return zero ? 0u : c;
}

}  // namespace tg
