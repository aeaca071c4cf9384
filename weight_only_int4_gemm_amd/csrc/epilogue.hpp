// The output stage's fused operation, y = act(x + bias[col]), computed in
// FP32 on the GEMM's sum before the one rounding to FP16.  The kernels take
// a compile-time switch EPI: without it (plain w4a16_gemm) the output stage
// is the plain rounding and the epilogue's arguments are never read, so the
// plain kernels are not burdened by the option.
#pragma once

#include "internal.hpp"
#include "w4a16.h"

namespace w4a16 {

// act(x + b), b the column's bias as FP32 (ignored without a bias).
// SiLU is x * sigmoid(x) = x * 1 / (1 + e^-x), with the hardware exponential
// and reciprocal (each within a few FP32 ulps, far below the FP16 rounding
// that follows); for x below about -88 e^-x overflows to infinity, its
// reciprocal is 0 and the product the correctly signed zero.
__device__ __forceinline__ float epilogue_apply(const Epilogue& ep, float x, float b) {
  if (ep.bias) x += b;
  if (ep.act == W4A16_ACT_RELU) return x > 0.f ? x : 0.f;
  if (ep.act == W4A16_ACT_SILU) return x * __builtin_amdgcn_rcpf(1.f + __expf(-x));
  return x;
}

// Host side: does this call need the epilogue instantiation?
inline bool epilogue_needed(const Epilogue& ep) {
  return ep.bias != nullptr || ep.act != W4A16_ACT_NONE;
}

}  // namespace w4a16
