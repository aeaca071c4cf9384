// Index arithmetic of the permuted weight layout (version 1).
//
// The unit of the layout is a "fragment block": 16 output columns by 128
// in-features, 2048 codes, 1 KiB, 256 words.  Lane l (0..63) of a wave owns
// the four consecutive words 4l .. 4l+3 of a block.  Word j of lane l feeds
// the B operand of the j-th 32-deep step of the gfx950 16x16x32 FP16 matrix
// instruction: column l % 16, in-features 32j + 8*(l/16) + i for i = 0..7.
//
// Blocks are ordered column-block major, then along K:
//     block(n16, kb) = n16 * (K / 128) + kb
// so the blocks one column block streams along K are contiguous.
//
// Inside a word, code i of the fragment (i = 0..7 along K) sits at nibble
// kNibbleOfCode[i] = {0,4,1,5,2,6,3,7}[i]: shifting the word right by 4r and
// masking 0x000F000F leaves codes 2r and 2r+1 in the low and high 16-bit
// halves, the order the matrix instruction takes its FP16 pairs in.
#pragma once

#include <stdint.h>

namespace w4a16 {

constexpr int kLayoutVersion = 1;
constexpr int kBlockK = 128;        // in-features per fragment block
constexpr int kBlockN = 16;         // output columns per fragment block
constexpr int kWordsPerLane = 4;    // one 16-byte load per lane per block
constexpr int kWordsPerBlock = 256;

__host__ __device__ inline int nibble_of_code(int i) {
  // {0,4,1,5,2,6,3,7}: even codes to nibbles 0..3, odd codes to nibbles 4..7
  return (i >> 1) + ((i & 1) << 2);
}

// Word offset of fragment block (n16, kb).
__host__ __device__ inline int64_t block_word_offset(int n16, int kb, int K) {
  return ((int64_t)n16 * (K / kBlockK) + kb) * kWordsPerBlock;
}

// Word offset (within the whole buffer) that holds the eight codes
// k0 .. k0+7 of column n, for k0 a multiple of 8.
// 8-bit weights (layout version 1 for 8 bits): blocks of 16 columns x 64
// in-features, 1 KiB each, column-block-major then along K.  In a block,
// lane l = (n % 16) + 16 * ((k % 32) / 8) owns words 4l .. 4l+3, word
// 2 * ((k % 64) / 32) + (k % 8) / 4 holds codes k0 .. k0+3 (k0 a multiple
// of 4), code k0 + i at byte byte_of_code8(i).  A lane's 16-byte piece holds
// its operands of two 32-deep steps; a 128-deep K block is two pieces.
constexpr int kBlockK8 = 64;

__host__ __device__ inline int byte_of_code8(int i) {
  // {0,2,1,3}: codes k, k+1 in bytes 0 and 2 (one mask pairs them in the two
  // halves of a register), codes k+2, k+3 in bytes 1 and 3
  return (i >> 1) + ((i & 1) << 1);
}

__host__ __device__ inline int64_t block_word_offset8(int n16, int kb64, int K) {
  return ((int64_t)n16 * (K / kBlockK8) + kb64) * kWordsPerBlock;
}

__host__ __device__ inline int64_t packed_word_of8(int k0, int n, int K) {
  const int lane = (n % kBlockN) + kBlockN * ((k0 % 32) / 8);
  const int j = 2 * ((k0 % kBlockK8) / 32) + (k0 % 8) / 4;
  return block_word_offset8(n / kBlockN, k0 / kBlockK8, K) + lane * kWordsPerLane + j;
}

__host__ __device__ inline int64_t packed_word_of(int k0, int n, int K) {
  const int n16 = n / kBlockN;
  const int kb = k0 / kBlockK;
  const int j = (k0 % kBlockK) / 32;
  const int lane = (n % kBlockN) + kBlockN * ((k0 % 32) / 8);
  return block_word_offset(n16, kb, K) + lane * kWordsPerLane + j;
}

// 2:4-sparse 4-bit weights (layout version 1 for 2:4): blocks of 16 columns
// x 128 in-features as for 4 bits, column-block-major then along K, but
// 768 bytes (192 words) each: words 0 .. 127 hold the kept codes, words
// 128 .. 191 their positions.  Lane l of a block owns code words 2l, 2l+1
// (one per 64-deep half t of the block) and position word 128 + l.  Code
// word t of lane l holds, for column l % 16, the two kept codes of each of
// the four groups of four in-features 64t + 16 (l / 16) + 4r .. +3
// (r = 0..3; slots 2r, 2r+1, lower position first), slot i at nibble
// nibble_of_code(i); bits 16t + 2i .. +1 of the position word hold slot i's
// position (0..3) in its group.  So one 8-byte and one 4-byte read hand a
// lane the compressed sparse operand of both 64-deep steps of the block.
constexpr int kWordsPerBlockSp = 192;
constexpr int kCodeWordsSp = 128;  // code words at the start of a block

__host__ __device__ inline int64_t block_word_offset_sp(int n16, int kb, int K) {
  return ((int64_t)n16 * (K / kBlockK) + kb) * kWordsPerBlockSp;
}

}  // namespace w4a16
