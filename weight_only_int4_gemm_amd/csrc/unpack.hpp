// In-register unpack and scale: one permuted 32-bit word -> eight FP16
// weights (q - 8) * s, in the order the 16x16x32 FP16 matrix instruction
// takes its B operand.
//
// The pages have every thread turn its 4-bit codes into FP16 values with a
// few bit operations and then apply the group scale ("Quant Marlin kernel"
// explainer, "The architecture: every piece explained", middle row; "Why
// architecture matters here" on keeping it to a handful of instructions).
//
// The conversion is the published FP16 "magic number" method for 4-bit
// integers (NVIDIA FasterTransformer's mixed-precision GEMM; Kim et al.,
// "Who Says Elephants Can't Run: Bringing Large Scale MoE Models into Cloud
// Scale Production", 2022): OR-ing a small integer into the low mantissa
// bits of a suitable FP16 constant gives "constant + integer" with no
// conversion instruction, and one exact subtraction removes the constant.
// This routine restates it for this library's nibble order:
//  * A code in bits 0..3 of a 16-bit half, OR-ed into 1024.0 (0x6400,
//    mantissa unit 1), gives 1024 + q.
//  * A code in bits 4..7, OR-ed into 64.0 (0x5400, mantissa unit 1/16),
//    gives 64 + 16q/16 = 64 + q: no shift is needed for it.
// Bits 8..15 of a half reach the exponent, so the upper two codes of each
// half are first shifted down by 8.  One mask-and-or per pair of codes, plus
// one shift per word, builds the four FP16 pairs (code k+0 and k+1 in the two
// halves of a register, as the matrix instruction wants them) -- this is why
// the permuted layout stores code i of a fragment at nibble {0,4,1,5,2,6,3,7}
// [i].  Subtracting 1032 (or 72) in FP16 is exact (the result is an integer
// in -8..7), and the FP16 multiply by the scale rounds the exact product
// once, round-to-nearest-even.  So every weight equals fp16_rne((q - 8) * s)
// exactly.  (Folding the subtraction into one fused multiply-add with
// 1032 * s would round 1032 * s first and cancel catastrophically; it is not
// used.)
//
// Cost: 5 bit operations, 4 packed subtractions and 4 packed multiplies per
// eight weights.  The dequantisation check and the GEMM tiles of 64 rows
// or more run all of it; the streaming kernel and the 16- and 32-row tiles
// of the stream-K and LDS kernels run its bit operations and subtractions
// (codes_minus_eight) and scale the FP32 sums instead.
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

// (x & mask) | magic as one instruction.  Left to itself the compiler emits
// an AND and an OR with literal operands (two issue slots); the three-operand
// form needs both constants in registers, which it then keeps across the loop.
// VIS = false writes the instruction out; the compiler's scheduling groups
// do not count it as a vector instruction then.  VIS = true hands the
// compiler the constants as opaque register values and the plain expression,
// from which it forms the same instruction, visible to those groups (the
// LDS kernel's interleaved schedule relies on that; the other kernels were
// measured slower with it).
template <bool VIS = false>
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
  if constexpr (VIS) {
    asm("" : "+v"(mask));
    asm("" : "+v"(magic));
    return (x & mask) | magic;
  } else {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(mask), "v"(magic));
    return r;
  }
}

// The exact integers q - 8 of one word as four FP16 pairs, unscaled: the
// first two steps of unpack_scale.  The streaming GEMM kernel multiplies
// these and applies the scale to the FP32 sums instead.
template <bool VIS = false>
__device__ __forceinline__ Half8 codes_minus_eight(uint32_t word) {
#pragma clang fp contract(off)
  const half2_t bias_lo = {(_Float16)1032.0f, (_Float16)1032.0f};  // 1024 + 8
  const half2_t bias_hi = {(_Float16)72.0f, (_Float16)72.0f};      //   64 + 8
  const uint32_t w8 = word >> 8;
  Half8 raw;
  raw.u[0] = and_or<VIS>(word, 0x000F000Fu, 0x64006400u);  // codes 0, 1: 1024 + q
  raw.u[1] = and_or<VIS>(word, 0x00F000F0u, 0x54005400u);  // codes 2, 3:   64 + q
  raw.u[2] = and_or<VIS>(w8, 0x000F000Fu, 0x64006400u);    // codes 4, 5
  raw.u[3] = and_or<VIS>(w8, 0x00F000F0u, 0x54005400u);    // codes 6, 7
  Half8 d;
  d.h2[0] = raw.h2[0] - bias_lo;  // exact subtraction
  d.h2[1] = raw.h2[1] - bias_hi;
  d.h2[2] = raw.h2[2] - bias_lo;
  d.h2[3] = raw.h2[3] - bias_hi;
  return d;
}

template <bool VIS = false>
__device__ __forceinline__ half8_t unpack_scale(uint32_t word, half2_t scale2) {
#pragma clang fp contract(off)
  Half8 out = codes_minus_eight<VIS>(word);
#pragma unroll
  for (int i = 0; i < 4; ++i) out.h2[i] = out.h2[i] * scale2;  // one rounding
  return out.v;
}

}  // namespace w4a16
