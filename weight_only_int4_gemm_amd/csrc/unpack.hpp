// In-register unpack and scale: one permuted 32-bit word -> eight FP16
// weights (q - 8) * s, in the order the 16x16x32 FP16 matrix instruction
// takes its B operand.
//
// The pages: each thread unpacks INT4 codes to FP16 with bitwise operations
// and a small lookup trick, then multiplies by the group scale ("Quant
// Marlin kernel" explainer, "The architecture: every piece explained",
// middle row), a handful of instructions per group of weights ("Why
// architecture matters here").
//
// The trick used here: OR-ing a 4-bit code q into the low mantissa bits of
// the FP16 value 1024 (0x6400, whose mantissa unit is exactly 1) gives the
// FP16 value 1024 + q with no conversion instruction.  One shift and one
// and-or per pair of codes build two such values in the halves of a 32-bit
// register.  Subtracting 1032 in FP16 is exact (the result is an integer in
// -8..7), and the FP16 multiply by the scale rounds the exact product once,
// round-to-nearest-even.  So every weight equals fp16_rne((q - 8) * s)
// exactly.  (Folding the subtraction into one fused multiply-add with
// 1032 * s would round 1032 * s first and cancel catastrophically; it is not
// used.)
//
// This is the one routine both the GEMM and the dequantisation check use.
#pragma once

#include <stdint.h>

namespace w4a16 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

union Half8 {
  half8_t v;
  half2_t h2[4];
  uint32_t u[4];
};

__device__ __forceinline__ half8_t unpack_scale(uint32_t word, half2_t scale2) {
#pragma clang fp contract(off)
  const half2_t bias = {(_Float16)1032.0f, (_Float16)1032.0f};
  Half8 out;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t bits = ((word >> (4 * r)) & 0x000F000Fu) | 0x64006400u;
    half2_t h = __builtin_bit_cast(half2_t, bits);   // (1024 + q_2r, 1024 + q_2r+1)
    h = h - bias;                                    // exact: q - 8
    out.h2[r] = h * scale2;                          // one rounding
  }
  return out.v;
}

}  // namespace w4a16
