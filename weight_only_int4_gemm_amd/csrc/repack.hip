// w4a16_repack's kernel: canonical words -> permuted layout (version 1).
//
// Every permuted word holds the eight codes k0 .. k0+7 (k0 a multiple of 8)
// of one column, which are exactly the eight codes of one canonical word.
// So the permutation moves whole words and shuffles nibbles inside each
// word; one thread handles one canonical word.  It runs once per weight
// matrix, offline ("Quant Marlin kernel" explainer, the paragraph on the
// permuted weight layout).
#include "internal.hpp"
#include "layout.hpp"

namespace w4a16 {

// Canonical nibble i (code k0 + i) -> nibble nibble_of_code(i).
__device__ __forceinline__ uint32_t shuffle_nibbles(uint32_t w) {
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    out |= ((w >> (4 * i)) & 0xFu) << (4 * nibble_of_code(i));
  }
  return out;
}

__global__ __launch_bounds__(256) void repack_kernel(const uint32_t* __restrict__ Bq,
                                                     uint32_t* __restrict__ Bp,
                                                     int K, int N) {
  const int64_t total = (int64_t)(K / 8) * N;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += stride) {
    const int j = (int)(idx / N);   // canonical word row: codes 8j .. 8j+7
    const int n = (int)(idx % N);
    Bp[packed_word_of(8 * j, n, K)] = shuffle_nibbles(Bq[idx]);
  }
}

// 8 bits: canonical byte i (code k0 + i) -> byte byte_of_code8(i); every
// canonical word is exactly one permuted word.
__device__ __forceinline__ uint32_t shuffle_bytes(uint32_t w) {
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) out |= ((w >> (8 * i)) & 0xFFu) << (8 * byte_of_code8(i));
  return out;
}

__global__ __launch_bounds__(256) void repack8_kernel(const uint32_t* __restrict__ Bq,
                                                      uint32_t* __restrict__ Bp,
                                                      int K, int N) {
  const int64_t total = (int64_t)(K / 4) * N;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += stride) {
    const int j = (int)(idx / N);   // canonical word row: codes 4j .. 4j+3
    const int n = (int)(idx % N);
    Bp[packed_word_of8(4 * j, n, K)] = shuffle_bytes(Bq[idx]);
  }
}

hipError_t launch_repack8(const uint32_t* Bq, uint32_t* Bp, int K, int N,
                          hipStream_t stream) {
  const int64_t total = (int64_t)(K / 4) * N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(repack8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     Bq, Bp, K, N);
  return hipGetLastError();
}

hipError_t launch_repack(const uint32_t* Bq, uint32_t* Bp, int K, int N,
                         hipStream_t stream) {
  const int64_t total = (int64_t)(K / 8) * N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(repack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     Bq, Bp, K, N);
  return hipGetLastError();
}

}  // namespace w4a16
