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

// 2:4 sparsity: the two kept positions of one group of four in-features
// from its mask byte.  The set bits among bits 0..3, lowest first, then the
// unset ones, lowest first; the first two of that order are kept, lower
// position first.  A position taken from an unset bit (a group with fewer
// than two set bits) holds code 8, i.e. weight 0.
struct Kept {
  int lo, hi;
  bool vlo, vhi;  // from a set bit
};

__device__ __forceinline__ Kept kept_positions(uint32_t m) {
  m &= 0xFu;
  int p[2];
  bool v[2];
  int n = 0;
  for (int b = 0; b < 4 && n < 2; ++b)
    if ((m >> b) & 1u) { p[n] = b; v[n] = true; ++n; }
  for (int b = 0; b < 4 && n < 2; ++b)
    if (!((m >> b) & 1u)) { p[n] = b; v[n] = false; ++n; }
  Kept k;
  const bool swap = p[0] > p[1];
  k.lo = swap ? p[1] : p[0];
  k.hi = swap ? p[0] : p[1];
  k.vlo = swap ? v[1] : v[0];
  k.vhi = swap ? v[0] : v[1];
  return k;
}

// One thread per lane of a 2:4 block (layout.hpp): for each 64-deep half t
// it reads the sixteen canonical codes (two words) and the four mask bytes
// of its column's in-features 64t + 16 (lane / 16) .. +15 and writes the
// compressed code word and the 16 position bits.
__global__ __launch_bounds__(256) void repack_sp24_kernel(const uint32_t* __restrict__ Bq,
                                                          const uint8_t* __restrict__ mask,
                                                          uint32_t* __restrict__ Bp, int K,
                                                          int N) {
  const int KB = K / kBlockK;
  const int64_t total = (int64_t)(N / kBlockN) * KB * 64;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += stride) {
    const int lane = (int)(idx & 63);
    const int64_t blk = idx >> 6;
    const int n16 = (int)(blk / KB);
    const int kb = (int)(blk % KB);
    const int n = n16 * kBlockN + (lane & 15);
    uint32_t pos = 0;
    uint32_t* base = Bp + block_word_offset_sp(n16, kb, K);
    for (int t = 0; t < 2; ++t) {
      const int k0 = kb * kBlockK + 64 * t + 16 * (lane >> 4);  // multiple of 16
      const uint32_t w0 = Bq[(int64_t)(k0 / 8) * N + n];
      const uint32_t w1 = Bq[(int64_t)(k0 / 8 + 1) * N + n];
      uint32_t word = 0;
      for (int r = 0; r < 4; ++r) {
        const Kept kp = kept_positions(mask[(int64_t)(k0 / 4 + r) * N + n]);
        const uint32_t src = r < 2 ? w0 : w1;  // codes 4r .. 4r+3 of the sixteen
        const int sh = 16 * (r & 1);
        const uint32_t qlo = kp.vlo ? (src >> (sh + 4 * kp.lo)) & 0xFu : 8u;
        const uint32_t qhi = kp.vhi ? (src >> (sh + 4 * kp.hi)) & 0xFu : 8u;
        word |= qlo << (4 * nibble_of_code(2 * r));
        word |= qhi << (4 * nibble_of_code(2 * r + 1));
        pos |= (uint32_t)kp.lo << (16 * t + 4 * r);
        pos |= (uint32_t)kp.hi << (16 * t + 4 * r + 2);
      }
      base[2 * lane + t] = word;
    }
    base[kCodeWordsSp + lane] = pos;
  }
}

hipError_t launch_repack_sp24(const uint32_t* Bq, const uint8_t* mask, uint32_t* Bp, int K,
                              int N, hipStream_t stream) {
  const int64_t total = (int64_t)(N / kBlockN) * (K / kBlockK) * 64;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(repack_sp24_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, Bq, mask,
                     Bp, K, N);
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
