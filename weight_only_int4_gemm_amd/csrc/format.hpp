// Weight and activation formats of the GEMM kernels.
//
// Format 0 is the path the pages describe: FP16 activations, scales and
// output, codes centred on 8, w = fp16_rne((q - 8) * s) ("Quant Marlin
// kernel" explainer, "The architecture: every piece explained").  Serving
// stacks also run AWQ checkpoints through the same kernel ("Low-Precision
// Quantization Kernels in Production", section 1 on production engines, and
// the comparison table of section 5: GPTQ and AWQ formats), whose codes
// carry a zero point per group and column, and models kept in BF16 (same
// page: the introduction's 16-bit FP16/BF16 weights, section 4's FP16 and
// BF16 activation formats).  The other formats add those:
//
//   1  FP16, zero point z per (group, column):   w = fp16_rne((q - z) * s)
//   2  BF16 activations, scales and output:      w = bf16_rne((q - 8) * s)
//   3  BF16 with zero points:                    w = bf16_rne((q - z) * s)
//   4  FP16, 8-bit codes centred on 128:         w = fp16_rne((q - 128) * s)
//      (same page, section 1: the kernel serves 4-bit and 8-bit checkpoints)
//   5  FP16, 2:4-sparse 4-bit codes: at most two kept weights in every four
//      consecutive in-features of a column, w = fp16_rne((q - 8) * s) for
//      the kept ones ("The anthology of the SOTA", the MARLIN note, "Key
//      results": the Sparse-MARLIN variant), multiplied by the sparse matrix
//      instruction with the weights as its compressed operand
//
// In every format (q - z) is an integer in -15..15 and the product with the
// scale is exact before its one rounding to the 16-bit type.
//
// FP16 with a zero point uses the magic-number conversion of unpack.hpp
// (FasterTransformer; Kim et al. 2022) with the
// subtrahends 1024 + z and 64 + z instead of 1032 and 72: both are exact in
// FP16, so the difference is the exact integer q - z.  The BF16 formats take
// that same exact q - z in FP16, widen each half to FP32, multiply by the
// scale in FP32 (exact: at most 9 by 8 significant bits) and convert the
// pair to BF16, which rounds once, to nearest even.  The FP32 product is
// exact for every BF16 scale (BF16 and FP32 share their exponent range), and
// a code equal to its zero point gives 0 * s, signed as the scale.  That is
// 29 vector instructions per eight weights against 13 for FP16: BF16 pays in
// unpacking, not in bytes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "unpack.hpp"

namespace w4a16 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_fmt_t __attribute__((ext_vector_type(4)));

enum : int { kFmtF16 = 0, kFmtF16Zp = 1, kFmtBf16 = 2, kFmtBf16Zp = 3, kFmtW8 = 4, kFmtSp24 = 5 };

template <int FMT>
struct Format {
  static_assert(FMT >= 0 && FMT <= 5, "six formats");
  static constexpr bool kBf16 = FMT == kFmtBf16 || FMT == kFmtBf16Zp;
  static constexpr bool kZp = FMT == kFmtF16Zp || FMT == kFmtBf16Zp;
  static constexpr bool kW8 = FMT == kFmtW8;  // two code words per 32-deep step
  static constexpr bool kSp = FMT == kFmtSp24;  // compressed 2:4 codes + positions
};

// What the unpack of one (group, column) needs, made once per K block and
// column from the raw 16-bit scale (FP16 or BF16 bits, in both halves of s2)
// and the zero point z (8 for the formats without one).
struct ColParams {
  half2_t s2;        // FP16 formats: the scale in both halves
  half2_t zlo, zhi;  // formats 1-3: 1024 + z and 64 + z in both halves
  float s;           // BF16 formats: the scale as FP32
};

template <int FMT>
__device__ __forceinline__ ColParams make_col(half2_t s2, uint32_t z) {
  ColParams p;
  p.s2 = s2;
  if constexpr (FMT != kFmtF16 && FMT != kFmtW8 && FMT != kFmtSp24) {
    const _Float16 lo = (_Float16)(float)(1024u + z);  // exact: integers to 2048
    const _Float16 hi = (_Float16)(float)(64u + z);    // exact: quarter units above 256
    p.zlo = half2_t{lo, lo};
    p.zhi = half2_t{hi, hi};
  }
  if constexpr (Format<FMT>::kBf16) {
    // BF16 bits in the low half of the register; as FP32 they sit in the
    // upper half
    const uint32_t bits = __builtin_bit_cast(uint32_t, s2) << 16;
    p.s = __builtin_bit_cast(float, bits);
  }
  return p;
}

// The exact integers q - z of one word, as four FP16 pairs in B-operand
// order: unpack_scale's steps with the subtrahends 1024 + z (codes at bits
// 0..3) and 64 + z (codes at bits 4..7).
template <bool VIS = false>
__device__ __forceinline__ Half8 codes_minus_zero(uint32_t word, half2_t zlo, half2_t zhi) {
#pragma clang fp contract(off)
  const uint32_t w8 = word >> 8;
  Half8 raw;
  raw.u[0] = and_or<VIS>(word, 0x000F000Fu, 0x64006400u);
  raw.u[1] = and_or<VIS>(word, 0x00F000F0u, 0x54005400u);
  raw.u[2] = and_or<VIS>(w8, 0x000F000Fu, 0x64006400u);
  raw.u[3] = and_or<VIS>(w8, 0x00F000F0u, 0x54005400u);
  Half8 d;
  d.h2[0] = raw.h2[0] - zlo;  // exact
  d.h2[1] = raw.h2[1] - zhi;
  d.h2[2] = raw.h2[2] - zlo;
  d.h2[3] = raw.h2[3] - zhi;
  return d;
}

// FP16 with a zero point: (q - z) * s, one rounding.
template <bool VIS = false>
__device__ __forceinline__ half8_t unpack_scale_zp(uint32_t word, half2_t scale2, half2_t zlo,
                                                   half2_t zhi) {
#pragma clang fp contract(off)
  Half8 out = codes_minus_zero<VIS>(word, zlo, zhi);
#pragma unroll
  for (int i = 0; i < 4; ++i) out.h2[i] = out.h2[i] * scale2;
  return out.v;
}

// BF16: eight weights bf16_rne((q - z) * s) in the B-operand order of the
// 16x16x32 BF16 matrix instruction (the same order as FP16), as raw bits.
template <bool VIS = false>
__device__ __forceinline__ half8_t unpack_scale_bf16(uint32_t word, float s, half2_t zlo,
                                                     half2_t zhi) {
#pragma clang fp contract(off)
  const Half8 d = codes_minus_zero<VIS>(word, zlo, zhi);
  Half8 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2_t pair = {(__bf16)((float)d.h2[i][0] * s), (__bf16)((float)d.h2[i][1] * s)};
    out.u[i] = __builtin_bit_cast(uint32_t, pair);
  }
  return out.v;
}

// The FP16 formats 0 and 1 unscaled: the exact integers q - z of one word
// (z = 8 for format 0), for kernels that apply the scale to FP32 sums.
template <int FMT, bool VIS = false>
__device__ __forceinline__ half8_t unpack_col_codes(uint32_t word, const ColParams& p) {
  static_assert(FMT == kFmtF16 || FMT == kFmtF16Zp, "FP16 formats with 4-bit codes");
  if constexpr (FMT == kFmtF16)
    return codes_minus_eight<VIS>(word).v;
  else
    return codes_minus_zero<VIS>(word, p.zlo, p.zhi).v;
}

// VIS: the AND-OR steps in the form the compiler's scheduling groups see
// (and_or in unpack.hpp).
template <int FMT, bool VIS = false>
__device__ __forceinline__ half8_t unpack_col(uint32_t word, const ColParams& p) {
  if constexpr (FMT == kFmtF16 || FMT == kFmtSp24)
    return unpack_scale<VIS>(word, p.s2);
  else if constexpr (FMT == kFmtF16Zp)
    return unpack_scale_zp<VIS>(word, p.s2, p.zlo, p.zhi);
  else
    return unpack_scale_bf16<VIS>(word, p.s, p.zlo, p.zhi);
}

// 8-bit codes: the eight FP16 weights (q - 128) * s of one 32-deep step
// from its two words.  A byte code OR-ed into 1024.0 (0x6400, mantissa unit
// 1, ten mantissa bits) gives 1024 + q exactly; the mask 0x00FF00FF keeps
// bytes 0 and 2 (codes k, k+1 in the layout), the same mask after a shift
// by 8 bytes 1 and 3 (codes k+2, k+3); subtracting 1152 = 1024 + 128 is
// exact and the multiply by the scale rounds once.  14 instructions per
// eight weights.
__device__ __forceinline__ half8_t unpack8_scale(uint32_t w0, uint32_t w1, half2_t scale2) {
#pragma clang fp contract(off)
  const half2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  Half8 raw;
  raw.u[0] = and_or(w0, 0x00FF00FFu, 0x64006400u);        // codes k, k+1
  raw.u[1] = and_or(w0 >> 8, 0x00FF00FFu, 0x64006400u);   // codes k+2, k+3
  raw.u[2] = and_or(w1, 0x00FF00FFu, 0x64006400u);        // codes k+4, k+5
  raw.u[3] = and_or(w1 >> 8, 0x00FF00FFu, 0x64006400u);   // codes k+6, k+7
  Half8 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out.h2[i] = (raw.h2[i] - bias) * scale2;
  return out.v;
}

// One 16x16x32 matrix instruction on raw 16-bit fragments.
template <int FMT>
__device__ __forceinline__ float4_fmt_t mma16(half8_t a, half8_t b, float4_fmt_t acc) {
  if constexpr (Format<FMT>::kBf16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}

// 2:4 sparsity.  One sparse 16x16x64 FP16 matrix instruction,
// D (16 x 16) += S (16 x 64, 2:4-sparse along its 64) . B (64 x 16).  The
// sparse operand comes compressed: lane L gives row L % 16 of S as eight
// values, slot i of which sits at column 16 (L / 16) + 4 (i / 2) + p_i of S,
// p_i = bits 2i .. 2i+1 of `pos` (the two slots of one group of four must
// name different positions).  The dense operand: lane l gives column l % 16
// of B, element j at row 32 (j / 8) + 8 (l / 16) + j % 8 -- i.e. the
// activation fragments of two consecutive 32-deep steps of the dense
// instruction, side by side.  The result lands as in the dense
// instruction: lane l holds D rows 4 (l / 16) .. +3 of column l % 16.  (The
// lane maps were read off the hardware with one-hot operands.)
// Here S is a block of transposed weights (rows = output columns) and B a
// block of transposed activations (columns = batch rows), so D is a block of
// C transposed.
typedef _Float16 half16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float4_fmt_t smma16(half8_t s, half8_t b_lo, half8_t b_hi,
                                               uint32_t pos, float4_fmt_t acc) {
  const half16_t b = __builtin_shufflevector(b_lo, b_hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11,
                                             12, 13, 14, 15);
  return __builtin_amdgcn_smfmac_f32_16x16x64_f16(s, b, acc, (int)pos, 0, 0);
}

// An FP32 result rounded to the output type (to nearest even), as the raw
// 16 bits in a _Float16 container.
template <int FMT>
__device__ __forceinline__ _Float16 out16(float x) {
  if constexpr (Format<FMT>::kBf16)
    return __builtin_bit_cast(_Float16, (__bf16)x);
  else
    return (_Float16)x;
}

}  // namespace w4a16
