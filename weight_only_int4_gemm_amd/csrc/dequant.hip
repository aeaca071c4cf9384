// w4a16_dequant_debug's kernel: permuted words -> W[K][N] (FP16, or BF16
// for the BF16 formats of w4a16_dequant_awq_debug).
//
// It runs the GEMM's own unpack-and-scale routine of the format on every
// word, so W shows bit for bit the weights the GEMM feeds to the matrix
// instruction.  One
// wave handles one fragment block (16 columns x 128 in-features): lane l
// reads its four words (16 bytes) and the scale of its column, exactly as
// the GEMM does, and writes its 32 weights.
#include "format.hpp"
#include "internal.hpp"
#include "layout.hpp"
#include "unpack.hpp"

namespace w4a16 {

template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ Bp,
                                                      const _Float16* __restrict__ S,
                                                      const uint8_t* __restrict__ Z,
                                                      _Float16* __restrict__ W,
                                                      int K, int N, int group) {
  const int KB = K / kBlockK;
  const int64_t blocks = (int64_t)(N / kBlockN) * KB;
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t wstride = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t blk = wave0; blk < blocks; blk += wstride) {
    const int n16 = (int)(blk / KB);
    const int kb = (int)(blk % KB);
    const int n = n16 * kBlockN + (lane & 15);
    const uint4 words =
        *reinterpret_cast<const uint4*>(Bp + block_word_offset(n16, kb, K) + lane * 4);
    const int64_t g = (int64_t)(kb * kBlockK / group) * N + n;
    const _Float16 s = S[g];
    const ColParams cp = make_col<FMT>(half2_t{s, s}, Format<FMT>::kZp ? (uint32_t)Z[g] : 8u);
    const uint32_t w4[4] = {words.x, words.y, words.z, words.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Half8 h;
      h.v = unpack_col<FMT>(w4[j], cp);
      const int k0 = kb * kBlockK + 32 * j + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) W[(int64_t)(k0 + i) * N + n] = h.v[i];
    }
  }
}

// 8-bit codes: one wave per 16-column x 64-deep block; lane l's four words
// hold its operands of the block's two 32-deep steps (words 2s, 2s+1).
__global__ __launch_bounds__(256) void dequant8_kernel(const uint32_t* __restrict__ Bp,
                                                       const _Float16* __restrict__ S,
                                                       _Float16* __restrict__ W,
                                                       int K, int N, int group) {
  const int KB = K / kBlockK8;
  const int64_t blocks = (int64_t)(N / kBlockN) * KB;
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t wstride = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t blk = wave0; blk < blocks; blk += wstride) {
    const int n16 = (int)(blk / KB);
    const int kb = (int)(blk % KB);
    const int n = n16 * kBlockN + (lane & 15);
    const uint4 words =
        *reinterpret_cast<const uint4*>(Bp + block_word_offset8(n16, kb, K) + lane * 4);
    const _Float16 s = S[(int64_t)(kb * kBlockK8 / group) * N + n];
    const half2_t s2 = {s, s};
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      Half8 h;
      h.v = unpack8_scale(st ? words.z : words.x, st ? words.w : words.y, s2);
      const int k0 = kb * kBlockK8 + 32 * st + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) W[(int64_t)(k0 + i) * N + n] = h.v[i];
    }
  }
}

// 2:4 sparsity: one wave per 768-byte block; lane l reads its two code
// words and its position word as the GEMM does, unpacks each code word with
// the GEMM's routine and writes its column's sixteen in-features of each
// 64-deep half: slot i's weight at position 4 (i / 2) + p_i, +0 at the two
// positions of each group of four that hold no slot.
__global__ __launch_bounds__(256) void dequant_sp24_kernel(const uint32_t* __restrict__ Bp,
                                                           const _Float16* __restrict__ S,
                                                           _Float16* __restrict__ W, int K,
                                                           int N, int group) {
  const int KB = K / kBlockK;
  const int64_t blocks = (int64_t)(N / kBlockN) * KB;
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t wstride = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t blk = wave0; blk < blocks; blk += wstride) {
    const int n16 = (int)(blk / KB);
    const int kb = (int)(blk % KB);
    const int n = n16 * kBlockN + (lane & 15);
    const uint32_t* base = Bp + block_word_offset_sp(n16, kb, K);
    const uint2 codes = *reinterpret_cast<const uint2*>(base + 2 * lane);
    const uint32_t pos = base[kCodeWordsSp + lane];
    const _Float16 s = S[(int64_t)(kb * kBlockK / group) * N + n];
    const half2_t s2 = {s, s};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      Half8 h;
      h.v = unpack_col<kFmtSp24>(t ? codes.y : codes.x, make_col<kFmtSp24>(s2, 8u));
      const uint32_t p = pos >> (16 * t);
      const int k0 = kb * kBlockK + 64 * t + 16 * (lane >> 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int plo = (p >> (4 * r)) & 3, phi = (p >> (4 * r + 2)) & 3;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const _Float16 v = plo == j ? h.v[2 * r] : phi == j ? h.v[2 * r + 1] : (_Float16)0.f;
          W[(int64_t)(k0 + 4 * r + j) * N + n] = v;
        }
      }
    }
  }
}

hipError_t launch_dequant_fmt(const uint32_t* Bp, const uint16_t* S, const uint8_t* Z,
                              uint16_t* W, int K, int N, int group, int fmt,
                              hipStream_t stream) {
  const int64_t blocks = (int64_t)(N / kBlockN) * (K / (fmt == kFmtW8 ? kBlockK8 : kBlockK));
  int64_t wgs = (blocks + 3) / 4;   // four waves per workgroup
  if (wgs > 65536) wgs = 65536;
  auto s = reinterpret_cast<const _Float16*>(S);
  auto w = reinterpret_cast<_Float16*>(W);
  const dim3 grid((unsigned)wgs), block(256);
  switch (fmt) {
    case kFmtF16:
      hipLaunchKernelGGL(dequant_kernel<kFmtF16>, grid, block, 0, stream, Bp, s, Z, w, K, N, group);
      break;
    case kFmtF16Zp:
      hipLaunchKernelGGL(dequant_kernel<kFmtF16Zp>, grid, block, 0, stream, Bp, s, Z, w, K, N,
                         group);
      break;
    case kFmtBf16:
      hipLaunchKernelGGL(dequant_kernel<kFmtBf16>, grid, block, 0, stream, Bp, s, Z, w, K, N,
                         group);
      break;
    case kFmtBf16Zp:
      hipLaunchKernelGGL(dequant_kernel<kFmtBf16Zp>, grid, block, 0, stream, Bp, s, Z, w, K, N,
                         group);
      break;
    case kFmtW8:
      hipLaunchKernelGGL(dequant8_kernel, grid, block, 0, stream, Bp, s, w, K, N, group);
      break;
    case kFmtSp24:
      hipLaunchKernelGGL(dequant_sp24_kernel, grid, block, 0, stream, Bp, s, w, K, N, group);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dequant(const uint32_t* Bp, const uint16_t* S, uint16_t* W,
                          int K, int N, int group, hipStream_t stream) {
  return launch_dequant_fmt(Bp, S, nullptr, W, K, N, group, kFmtF16, stream);
}

}  // namespace w4a16
