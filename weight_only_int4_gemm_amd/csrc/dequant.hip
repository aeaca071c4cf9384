// w4a16_dequant_debug's kernel: permuted words -> FP16 W[K][N].
//
// It runs the GEMM's own unpack-and-scale routine on every word, so W shows
// bit for bit the weights the GEMM feeds to the matrix instruction.  One
// wave handles one fragment block (16 columns x 128 in-features): lane l
// reads its four words (16 bytes) and the scale of its column, exactly as
// the GEMM does, and writes its 32 weights.
#include "internal.hpp"
#include "layout.hpp"
#include "unpack.hpp"

namespace w4a16 {

__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ Bp,
                                                      const _Float16* __restrict__ S,
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
    const _Float16 s = S[(int64_t)(kb * kBlockK / group) * N + n];
    const half2_t s2 = {s, s};
    const uint32_t w4[4] = {words.x, words.y, words.z, words.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Half8 h;
      h.v = unpack_scale(w4[j], s2);
      const int k0 = kb * kBlockK + 32 * j + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) W[(int64_t)(k0 + i) * N + n] = h.v[i];
    }
  }
}

hipError_t launch_dequant(const uint32_t* Bp, const uint16_t* S, uint16_t* W,
                          int K, int N, int group, hipStream_t stream) {
  const int64_t blocks = (int64_t)(N / kBlockN) * (K / kBlockK);
  int64_t wgs = (blocks + 3) / 4;   // four waves per workgroup
  if (wgs > 65536) wgs = 65536;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, Bp,
                     reinterpret_cast<const _Float16*>(S), reinterpret_cast<_Float16*>(W),
                     K, N, group);
  return hipGetLastError();
}

}  // namespace w4a16
