// The W4A16 GEMM kernel: C[M x N] = A[M x K] . dequant(Bpacked)[K x N].
//
// Work decomposition ("Quant Marlin kernel" explainer, "The architecture:
// every piece explained", middle row, and "End-to-end flow"; split-K as in
// "Low-Precision Quantization Kernels in Production", section 3):
//  * grid.x walks output column tiles of 16*NB columns, grid.y row tiles of
//    16*MB rows, grid.z the K ranges ("splits") of one tile;
//  * the WK waves of a workgroup share its tile and its K range and take its
//    128-deep K blocks round-robin; their FP32 sums are added in wave order
//    through LDS;
//  * with splits > 1 each workgroup publishes its FP32 partial tile in the
//    workspace, and the last of a tile's workgroups to arrive (an atomic
//    counter per tile) adds the partials in split order 0, 1, ..., writes
//    the FP16 tile and sets the counter back to zero.  The order of every
//    addition is fixed, so results are bit-identical from run to run.
//
// The hand-off between workgroups uses device-coherent 16-byte stores and
// loads for the partials (coherent.hpp), a wait for those stores to complete
// before the arrival count, and no device-wide fence.
//
// 2:4-sparse weights (format 5) use the sparse 16x16x64 matrix instruction
// with the weights as its compressed operand: per K block and column block
// a lane loads its two code words and its position word (12 bytes instead
// of 16), and the accumulators hold C transposed (format.hpp, smma16).
//
// Per 128-deep K block a wave issues, for each of its NB column blocks, one
// 16-byte load per lane of permuted codes (the lane's own operand fragments
// for four 32-deep steps) and one scale load; it unpacks each word in
// registers (unpack.hpp) and issues 16x16x32 FP16 matrix instructions against
// activation fragments read straight from global memory (16 bytes per lane
// per 16-row block and 32-deep step).  Loads run one step ahead of the
// matrix instructions: the codes of the next K block and the activations of
// the next 32-deep step are in flight while the current ones are consumed.
//
// Batches of at most kAldsMaxRows rows with FP16 activations (ALDS; the
// rule is activations_lds_bytes): the workgroup first copies
// rows 0..M-1 of A over its K range into LDS (at most kAldsMaxBytes), once,
// while the first code loads are in flight, and each step reads its
// activation fragment from there.  A wave then issues two loads per K block
// and column block (codes and scale) instead of six, and a ring slot holds
// no activations.  Llama-2-7B qkv at M = 1: 8.5 against 9.5 us.
#include "coherent.hpp"
#include "epilogue.hpp"
#include "format.hpp"
#include "internal.hpp"
#include "layout.hpp"
#include "unpack.hpp"

namespace w4a16 {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef unsigned uint2_vt __attribute__((ext_vector_type(2)));

template <int MB, int NB, bool ZP, bool W8, bool SP = false>
struct Slot {
  uint4 b[NB];         // permuted codes: one 128-deep K block per column block
  half2_t s[NB];       // the group scale of this lane's column, in both halves
  half8_t a[MB][4];    // activation fragments, four 32-deep steps
};
// With zero points: the group zero point of this lane's column as well.
template <int MB, int NB>
struct Slot<MB, NB, true, false> {
  uint4 b[NB];
  half2_t s[NB];
  half8_t a[MB][4];
  uint32_t z[NB];
};
// 8-bit codes: a 128-deep K block is two 16-byte pieces per column block
// (b: steps 0 and 1, b2: steps 2 and 3).
template <int MB, int NB>
struct Slot<MB, NB, false, true> {
  uint4 b[NB];
  half2_t s[NB];
  half8_t a[MB][4];
  uint4 b2[NB];
};

// 2:4-sparse codes: the two compressed code words (64-deep halves 0 and 1)
// and the position word of this lane, per column block.
template <int MB, int NB>
struct Slot<MB, NB, false, false, true> {
  uint2 b[NB];
  half2_t s[NB];
  half8_t a[MB][4];
  uint32_t p[NB];
};

// FMT: the weight format (format.hpp); formats other than 0 are compiled
// without the fused epilogue.  A, S and C hold raw 16-bit values (FP16, or
// BF16 for formats 2 and 3); Z the zero points of formats 1 and 3.
// (BF16 without zero points: the compiler's own choice for the deepest
// variant kept one wave per SIMD; the hint asks for the two it gets in the
// other formats.)
template <int MB, int NB, int WK, int D, bool EPI, int FMT, bool ALDS = false>
__global__ __launch_bounds__(64 * WK)
__attribute__((amdgpu_waves_per_eu(FMT == kFmtBf16 ? 2 : 1))) void gemm_kernel(
    const _Float16* __restrict__ A, const uint32_t* __restrict__ Bp,
    const _Float16* __restrict__ S, _Float16* __restrict__ C, int M, int K, int N,
    uint64_t group_magic, int splits, unsigned* __restrict__ counters,
    float* __restrict__ partials, Epilogue ep, const uint8_t* __restrict__ Z) {
  static_assert(!EPI || FMT == kFmtF16, "the fused epilogue is FP16 only");
  constexpr bool ZP = Format<FMT>::kZp;
  constexpr bool W8 = Format<FMT>::kW8;
  constexpr bool SP = Format<FMT>::kSp;
  typedef Slot<MB, NB, ZP, W8, SP> SlotT;
  // FP16 formats 0 and 1: the scale is applied to FP32 sums (see compute).
  // Every variant compiled for them has a second column block or a second
  // wave per SIMD to cover the wait for those sums.
  constexpr bool kPostScale = FMT == kFmtF16 || FMT == kFmtF16Zp;
  static_assert(!ALDS || (MB == 1 && !SP), "activations in LDS: one row block, dense codes");
  // ALDS: rows 0..M-1 of the row tile over this workgroup's K range, row
  // after row, krange halfs each (the launch sizes it)
  extern __shared__ uint4 a_lds[];
  constexpr int TM = 16 * MB;
  constexpr int TN = 16 * NB;
  constexpr int LDT = TN + 4;  // padded LDS row (floats), keeps 16-byte alignment
  // The waves' partial tiles: one LDS slot per wave where they fit (one
  // barrier, then every thread adds the slots in wave order), else one slot
  // the waves add into in turn (a barrier per wave).  2:4-sparse codes keep
  // the second form: with the first, the compiler gave the 64-column
  // variant a shallower load schedule (the 18432 x 73728 layer at M = 1:
  // 159 against 107 us).
  constexpr bool SLOTS = !SP && (size_t)WK * TM * LDT * sizeof(float) <= 40 * 1024;
  __shared__ float red[(SLOTS ? WK : 1) * TM * LDT];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile_n = blockIdx.x;
  const int tile_m = blockIdx.y;
  const int split = blockIdx.z;
  const int KB = K / kBlockK;
  const int kb0 = (int)((int64_t)KB * split / splits);
  const int kb1 = (int)((int64_t)KB * (split + 1) / splits);
  const int l16 = lane & 15;
  const int lk = (lane >> 4) * 8;
  const int n16_0 = tile_n * NB;
  // column blocks of this tile inside N (ragged N: the rest are skipped)
  const int nvalid = N / kBlockN - n16_0 < NB ? N / kBlockN - n16_0 : NB;

  // Fused epilogue: the bias of the four columns this thread stores, read
  // now so that the load's latency hides behind the main loop.  Every
  // vector a thread stores (output stage below) starts at tile column
  // (threadIdx.x % (TN / 4)) * 4, since the block size is a multiple of TN / 4.
  static_assert((64 * WK) % (4 * NB) == 0, "a thread's output columns stay fixed");
  half4_t bias4 = {};
  if constexpr (EPI) {
    const int gc = tile_n * 16 * NB + (int)(threadIdx.x % (4 * NB)) * 4;
    if (ep.bias && gc < N) bias4 = *reinterpret_cast<const half4_t*>(ep.bias + gc);
  }

  float4_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = float4_t{0.f, 0.f, 0.f, 0.f};

  // Activation row of this lane in each 16-row block.  Rows >= M read row
  // M - 1 instead: their sums land in accumulator rows that are never
  // stored, so no load needs a mask.
  const _Float16* arow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = tile_m * TM + mb * 16 + l16;
    arow[mb] = A + (int64_t)(r < M ? r : M - 1) * K + lk;
  }
  // ALDS: halfs per LDS row, and this lane's row in LDS (rows past M read
  // the last row, as above)
  const int krange = (kb1 - kb0) * kBlockK;
  const int arow_l = tile_m * TM + l16 < M ? l16 : M - 1 - tile_m * TM;
  const uint32_t* bcol[NB];
  const _Float16* scol[NB];
  const uint8_t* zcol[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n16 = n16_0 + (nb < nvalid ? nb : nvalid - 1);
    if constexpr (SP)
      bcol[nb] = Bp + block_word_offset_sp(n16, 0, K);
    else
      bcol[nb] = Bp + (W8 ? block_word_offset8(n16, 0, K) : block_word_offset(n16, 0, K)) +
                 lane * kWordsPerLane;
    scol[nb] = S + n16 * kBlockN + l16;
    if constexpr (ZP) zcol[nb] = Z + n16 * kBlockN + l16;
  }

  // Scale row of K block kb: kb / group_blocks (group_magic = 0: a shift).
  // Scale row of K block kb: kb / (group / 128), as a multiply-high by
  // group_magic = ceil(2^32 / (group / 128)); no branch in the K loop.
  auto scale_row = [&](int kb) -> int {
    return (int)(((uint64_t)(uint32_t)kb * group_magic) >> 32);
  };
  auto load = [&](SlotT& sl, int kb) {
    const int srow = scale_row(kb) * N;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // Every code word is read exactly once (one row tile at the plans'
      // batch sizes): non-temporal loads, which keep the stream from
      // displacing the activations in the caches (the 18432 x 73728 layer
      // at M = 1..4: 119-123 us against 128-131 us).  The LDS kernel does
      // not use them: its row tiles share codes through the caches.
      if constexpr (SP) {
        const uint32_t* blk = bcol[nb] + kb * kWordsPerBlockSp;
        sl.b[nb] = __builtin_bit_cast(
            uint2, __builtin_nontemporal_load(reinterpret_cast<const uint2_vt*>(blk + 2 * lane)));
        sl.p[nb] = __builtin_nontemporal_load(blk + kCodeWordsSp + lane);
      } else if constexpr (W8) {
        // the two 64-deep blocks of this 128-deep K block
        sl.b[nb] = __builtin_bit_cast(
            uint4, __builtin_nontemporal_load(
                       reinterpret_cast<const uint4_vt*>(bcol[nb] + 2 * kb * kWordsPerBlock)));
        sl.b2[nb] = __builtin_bit_cast(
            uint4, __builtin_nontemporal_load(reinterpret_cast<const uint4_vt*>(
                       bcol[nb] + (2 * kb + 1) * kWordsPerBlock)));
      } else {
        sl.b[nb] = __builtin_bit_cast(
            uint4, __builtin_nontemporal_load(
                       reinterpret_cast<const uint4_vt*>(bcol[nb] + kb * kWordsPerBlock)));
      }
      const _Float16 sc = scol[nb][srow];
      sl.s[nb] = half2_t{sc, sc};
      if constexpr (ZP) sl.z[nb] = zcol[nb][srow];
    }
    if constexpr (!ALDS) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sl.a[mb][j] = *reinterpret_cast<const half8_t*>(arow[mb] + kb * kBlockK + 32 * j);
    }
  };
  // kbc: the K block the slot holds
  auto compute = [&](const SlotT& sl, int kbc) {
    half8_t al[4] = {};
    if constexpr (ALDS) {
      const _Float16* base = reinterpret_cast<const _Float16*>(a_lds) + arow_l * krange +
                             (kbc - kb0) * kBlockK + lk;
#pragma unroll
      for (int j = 0; j < 4; ++j) al[j] = *reinterpret_cast<const half8_t*>(base + 32 * j);
    }
    if constexpr (SP) {
      // two 64-deep sparse steps; the accumulators hold C transposed
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint32_t pos = t ? sl.p[nb] >> 16 : sl.p[nb];
          const half8_t w = unpack_scale(t ? sl.b[nb].y : sl.b[nb].x, sl.s[nb]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[mb][nb] = smma16(w, sl.a[mb][2 * t], sl.a[mb][2 * t + 1], pos, acc[mb][nb]);
        }
      }
    } else if constexpr (kPostScale) {
      // One group scale per lane and K block (the lane's column), so
      //   sum_k a_k * (q_k - z) * s = s * sum_k a_k * (q_k - z):
      // the four matrix instructions of a (row block, column block) take
      // the exact integers q - z, and their FP32 sum is scaled with one
      // multiply-add.  That drops the 4 packed multiplies per word (13 ->
      // 9 unpacking instructions) for 4 multiply-adds per 16 x 16 block:
      // the vector work, not HBM, limited this kernel (the 18432 x 73728
      // layer at M = 1..8: 4-6% faster; 28672 x 8192 and 4096 x 22016 at
      // M = 1: 7%).  The products are exact and the weights are never
      // rounded to FP16, so the result is the definition's up to FP32
      // summation order, closer to the float64 product than the rounded
      // weights are.  With one column block and one wave per SIMD the
      // multiply-adds would wait for the matrix unit (4096 x 4096 at
      // M = 16: 7.2 against 7.0 us with the weights scaled): that variant
      // is compiled only for the other formats, and the plans give FP16
      // eight waves or wider tiles there.
      float4_t blk[MB][NB];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint32_t w = j == 0 ? sl.b[nb].x : j == 1 ? sl.b[nb].y
                           : j == 2 ? sl.b[nb].z : sl.b[nb].w;
          uint32_t z = 8;
          if constexpr (ZP) z = sl.z[nb];
          const half8_t b = unpack_col_codes<FMT>(w, make_col<FMT>(sl.s[nb], z));
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const half8_t a = ALDS ? al[j] : sl.a[mb][j];
            if (j == 0)
              blk[mb][nb] = mma16<FMT>(a, b, float4_t{0.f, 0.f, 0.f, 0.f});
            else
              blk[mb][nb] = mma16<FMT>(a, b, blk[mb][nb]);
          }
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float s = (float)sl.s[nb].x;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[mb][nb][i] = __builtin_fmaf(blk[mb][nb][i], s, acc[mb][nb][i]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          // (column blocks past N recompute the last valid block; the store
          // drops them -- a branch here would stall the load pipeline)
          half8_t b;
          if constexpr (W8) {
            const uint4& pc = j < 2 ? sl.b[nb] : sl.b2[nb];
            b = unpack8_scale((j & 1) ? pc.z : pc.x, (j & 1) ? pc.w : pc.y, sl.s[nb]);
          } else {
            const uint32_t w = j == 0 ? sl.b[nb].x : j == 1 ? sl.b[nb].y
                             : j == 2 ? sl.b[nb].z : sl.b[nb].w;
            uint32_t z = 8;
            if constexpr (ZP) z = sl.z[nb];
            b = unpack_col<FMT>(w, make_col<FMT>(sl.s[nb], z));
          }
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            if constexpr (ALDS)
              acc[mb][nb] = mma16<FMT>(al[j], b, acc[mb][nb]);
            else
              acc[mb][nb] = mma16<FMT>(sl.a[mb][j], b, acc[mb][nb]);
          }
        }
      }
    }
  };

  // This wave's K blocks are first, first + WK, ...; D of them are in flight
  // (a ring of D register slots), the next load issued as soon as a slot has
  // been consumed.  Loads past the last block re-read the last block, which
  // keeps every load unconditional.
  const int first = kb0 + wave;
  const int nblk = first < kb1 ? (kb1 - first + WK - 1) / WK : 0;
  const int last = first + (nblk > 0 ? nblk - 1 : 0) * WK;
  SlotT slot[D];
  if (nblk > 0) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int kb = first + u * WK;
      load(slot[u], kb < last ? kb : last);
    }
  }
  if constexpr (ALDS) {
    // Rows 0..M-1 of this row tile over K blocks [kb0, kb1) into LDS, 16
    // bytes per thread and step, after the first code loads so that they
    // overlap.  Every wave takes part and meets the barrier, including
    // waves without K blocks.
    const int rows = M - tile_m * TM < TM ? M - tile_m * TM : TM;
    const int ppr = krange / 8;  // pieces per row
    const int pieces = rows * ppr;
    for (int v = threadIdx.x; v < pieces; v += blockDim.x) {
      const int r = v / ppr, c = v - r * ppr;
      a_lds[v] = *reinterpret_cast<const uint4*>(A + (int64_t)(tile_m * TM + r) * K +
                                                  kb0 * kBlockK + c * 8);
    }
    __syncthreads();
  }
  if (nblk > 0) {
    // Full rounds: straight-line code, so the wait before each slot's use
    // counts exactly the D - 1 slots of loads issued after it.  With two
    // slots and tiles of at most 32 columns the last full round is peeled
    // off and skips its loads past the wave's last block (which would
    // re-read it): a wave owns only 4 to 8 K blocks on the layers these
    // variants serve, and the re-reads were a third to a fifth of its loads
    // (4096 x 4096 at M = 16: 7.0 against 7.7 us; Llama-2-7B gate/up at
    // M = 1: 12.3 against 12.8 us).  The 64-column variant keeps the plain
    // loop: peeled, its 680 MB layer ran 25% slower.
    constexpr bool kPeel = D == 2 && NB <= 2;
    int t = 0;
    for (; t + (kPeel ? 2 * D : D) <= nblk; t += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        compute(slot[u], first + (t + u) * WK);
        const int kb = first + (t + u + D) * WK;
        load(slot[u], kb < last ? kb : last);
      }
    }
    if (kPeel && t + D <= nblk) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        compute(slot[u], first + (t + u) * WK);
        const int kb = first + (t + u + D) * WK;
        if (kb <= last) load(slot[u], kb);
      }
      t += D;
    }
    // The last, partial round: compute only.
#pragma unroll
    for (int u = 0; u < D - 1; ++u) {
      if (t + u < nblk) compute(slot[u], first + (t + u) * WK);
    }
  }

  // Sum the waves' tiles in LDS, wave 0 first.  Lane l holds rows
  // 4*(l/16) .. +3 of column l % 16 of each 16x16 block (with 2:4-sparse
  // weights: row l % 16, columns 4*(l/16) .. +3).
  auto red_index = [&](int mb, int nb, int i) {
    return SP ? (mb * 16 + l16) * LDT + nb * 16 + (lane >> 4) * 4 + i
              : (mb * 16 + (lane >> 4) * 4 + i) * LDT + nb * 16 + l16;
  };
  if constexpr (SLOTS) {
    float* mine = red + wave * TM * LDT;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[red_index(mb, nb, i)] = acc[mb][nb][i];
    __syncthreads();
  } else {
#pragma unroll 1
    for (int w = 0; w < WK; ++w) {
      if (wave == w) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float* p = &red[red_index(mb, nb, i)];
              *p = (w == 0) ? acc[mb][nb][i] : *p + acc[mb][nb][i];
            }
      }
      __syncthreads();
    }
  }
  // Four consecutive columns (c a multiple of 4) of row r of the summed
  // tile: the waves' values added in wave order 0, 1, ..., the same order
  // either way.
  auto tile_value = [&](int r, int c) -> float4_t {
    float4_t x = *reinterpret_cast<const float4_t*>(&red[r * LDT + c]);
    if constexpr (SLOTS) {
#pragma unroll
      for (int w = 1; w < WK; ++w)
        x = x + *reinterpret_cast<const float4_t*>(&red[w * TM * LDT + r * LDT + c]);
    }
    return x;
  };

  constexpr int VEC = 4;
  constexpr int VPR = TN / VEC;  // float4 vectors per tile row
  const int row0 = tile_m * TM;
  const int col0 = tile_n * TN;
  // Four consecutive columns of C (through the epilogue), rounded to the
  // output type.
  auto finish = [&](const float4_t& x) {
    half4_t h;
#pragma unroll
    for (int j = 0; j < VEC; ++j)
      h[j] = out16<FMT>(EPI ? epilogue_apply(ep, x[j], (float)bias4[j]) : x[j]);
    return h;
  };

  if (splits == 1) {
    for (int v = threadIdx.x; v < TM * VPR; v += blockDim.x) {
      const int r = v / VPR, c = (v % VPR) * VEC;
      const int gr = row0 + r, gc = col0 + c;
      if (gr < M && gc < N) {
        const float4_t x = tile_value(r, c);
        *reinterpret_cast<half4_t*>(C + (int64_t)gr * N + gc) = finish(x);
      }
    }
    return;
  }

  // Split-K: publish this workgroup's partial tile (rows < M, row-major,
  // 16 bytes per access, device-coherent), wait for the stores to complete,
  // then count the arrival.
  const int tile = tile_m * gridDim.x + tile_n;
  constexpr int TE = TM * TN;
  const int rows = M - row0 < TM ? M - row0 : TM;
  const float* tile_base = partials + (int64_t)tile * splits * TE;
  {
    const __amdgpu_buffer_rsrc_t mine = coherent_rsrc(tile_base + (int64_t)split * TE);
    for (int v = threadIdx.x; v < rows * VPR; v += blockDim.x) {
      const int r = v / VPR, c = (v % VPR) * VEC;
      store_coherent(mine, v, tile_value(r, c));
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(splits - 1);
  }
  __syncthreads();
  if (!s_last) return;

  // Add the partials in split order; up to eight splits' loads are in
  // flight at once.
  for (int v = threadIdx.x; v < rows * VPR; v += blockDim.x) {
    const int r = v / VPR, c = (v % VPR) * VEC;
    float4_t x = float4_t{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < splits; s0 += 8) {
      float4_t part[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = s0 + u < splits ? s0 + u : splits - 1;
        part[u] = load_coherent(coherent_rsrc(tile_base + (int64_t)s * TE), v);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (s0 + u < splits) x = (s0 + u == 0) ? part[u] : x + part[u];
      }
    }
    const int gc = col0 + c;
    if (gc < N) *reinterpret_cast<half4_t*>(C + (int64_t)(row0 + r) * N + gc) = finish(x);
  }
  if (threadIdx.x == 0)  // ready for the next call
    __hip_atomic_store(counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

size_t activations_lds_bytes(const Plan& p, int M, int K, int fmt) {
  // Not for the BF16 formats: with their longer unpacking the staged path
  // measured slower (Llama-2-7B down at M = 1: 12.7 against 10.5 us), and
  // not for 2:4, whose steps read activations in their own pattern.
  if (p.tile != 0 || p.mb != 1 || fmt == kFmtSp24 || fmt == kFmtBf16 || fmt == kFmtBf16Zp ||
      M < 1 || M > kAldsMaxRows)
    return 0;
  // M rows over the longest K range of a split (one row tile: M < 16)
  const int KB = K / kBlockK;
  const size_t bytes = (size_t)M * ((KB + p.splits - 1) / p.splits) * kBlockK * 2;
  return bytes <= kAldsMaxBytes ? bytes : 0;
}

template <int MB, int NB, int WK, int D, int FMT>
static hipError_t launch_one(const Plan& p, const uint16_t* A, const uint32_t* Bp,
                             const uint16_t* S, uint16_t* C, int M, int K, int N,
                             uint64_t gmagic, Epilogue ep, const uint8_t* Z, void* workspace,
                             hipStream_t stream) {
  unsigned* counters = nullptr;
  float* partials = nullptr;
  if (p.splits > 1) {
    counters = static_cast<unsigned*>(workspace);
    partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterHeaderBytes);
  }
  const dim3 grid(p.tiles_n, p.tiles_m, p.splits), block(64 * WK);
  auto a = reinterpret_cast<const _Float16*>(A);
  auto s = reinterpret_cast<const _Float16*>(S);
  auto c = reinterpret_cast<_Float16*>(C);
  // (the formats activations_lds_bytes admits; no staged kernel is compiled
  // for the others)
  constexpr bool kAldsVariant =
      MB == 1 && (FMT == kFmtF16 || FMT == kFmtF16Zp || FMT == kFmtW8);
  const size_t alds = kAldsVariant ? activations_lds_bytes(p, M, K, FMT) : 0;
  if constexpr (FMT == kFmtF16) {
    if (epilogue_needed(ep)) {
      if constexpr (kAldsVariant) {
        if (alds) {
          hipLaunchKernelGGL((gemm_kernel<MB, NB, WK, D, true, FMT, true>), grid, block, alds,
                             stream, a, Bp, s, c, M, K, N, gmagic, p.splits, counters, partials,
                             ep, Z);
          return hipGetLastError();
        }
      }
      hipLaunchKernelGGL((gemm_kernel<MB, NB, WK, D, true, FMT>), grid, block, 0, stream, a, Bp,
                         s, c, M, K, N, gmagic, p.splits, counters, partials, ep, Z);
      return hipGetLastError();
    }
  } else {
    if (epilogue_needed(ep)) return hipErrorInvalidValue;
  }
  if constexpr (kAldsVariant) {
    if (alds) {
      hipLaunchKernelGGL((gemm_kernel<MB, NB, WK, D, false, FMT, true>), grid, block, alds, stream,
                         a, Bp, s, c, M, K, N, gmagic, p.splits, counters, partials, ep, Z);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_kernel<MB, NB, WK, D, false, FMT>), grid, block, 0, stream, a, Bp, s,
                     c, M, K, N, gmagic, p.splits, counters, partials, ep, Z);
  return hipGetLastError();
}

// Compiled variants (MB, NB, WK, D): the plans' ones, for the formats 0 to
// 4 (FP16 and BF16 with or without zero points, 8-bit codes) ...
#define W4A16_VARIANTS(X) X(1, 1, 8, 2) X(1, 2, 8, 2) X(1, 4, 4, 2) X(1, 4, 4, 4)
// ... and, for the formats that scale the weights (2 to 4), 16-column tiles
// of four waves (the plans give the FP16 formats eight waves there).
#define W4A16_SCALED_WEIGHT_VARIANTS(X) X(1, 1, 4, 2)

// Variants compiled for 2:4-sparse weights (the plans keep two K blocks in
// flight).
#define W4A16_SP_VARIANTS(X) X(1, 1, 4, 2) X(1, 1, 8, 2) X(1, 2, 8, 2) X(1, 4, 4, 2)

bool sp_is_compiled(int mb, int nb, int wk, int depth) {
#define W4A16_SMATCH(MB_, NB_, WK_, D_) \
  if (mb == MB_ && nb == NB_ && wk == WK_ && depth == D_) return true;
  W4A16_SP_VARIANTS(W4A16_SMATCH)
#undef W4A16_SMATCH
  return false;
}

bool plan_is_compiled(int mb, int nb, int wk, int depth, int fmt) {
#define W4A16_MATCH(MB_, NB_, WK_, D_) \
  if (mb == MB_ && nb == NB_ && wk == WK_ && depth == D_) return true;
  W4A16_VARIANTS(W4A16_MATCH)
  if (fmt == kFmtBf16 || fmt == kFmtBf16Zp || fmt == kFmtW8) {
    W4A16_SCALED_WEIGHT_VARIANTS(W4A16_MATCH)
  }
#undef W4A16_MATCH
  return false;
}

hipError_t launch_gemm(const Plan& p, const uint16_t* A, const uint32_t* Bp,
                       const uint16_t* S, uint16_t* C, int M, int K, int N, int group,
                       Epilogue ep, WeightFormat wf, void* workspace, hipStream_t stream) {
  // Scale row of K block kb is kb / gb, gb = group / 128, computed in the
  // kernels as (kb * ceil(2^32 / gb)) >> 32: exact when gb is a power of two,
  // and for any gb as long as kb, gb < 2^16 (K < 2^23 is checked).
  const uint64_t gb = (uint64_t)(group / kBlockK);
  const uint64_t gmagic = (((uint64_t)1 << 32) + gb - 1) / gb;
  if (p.tile == 4)
    return launch_sk(p, A, Bp, S, C, M, K, N, gmagic, ep, wf, workspace, stream);
  if (p.tile == 2)
    return launch_lds(p, A, Bp, S, C, M, K, N, gmagic, ep, wf, workspace, stream);
  if (p.tile) return hipErrorInvalidValue;
#define W4A16_CASE(MB_, NB_, WK_, D_)                                                     \
  if (p.mb == MB_ && p.nb == NB_ && p.wk == WK_ && p.depth == D_) {                       \
    if (wf.fmt == kFmtF16)                                                                \
      return launch_one<MB_, NB_, WK_, D_, kFmtF16>(p, A, Bp, S, C, M, K, N, gmagic, ep,   \
                                                    nullptr, workspace, stream);          \
    if (wf.fmt == kFmtF16Zp)                                                              \
      return launch_one<MB_, NB_, WK_, D_, kFmtF16Zp>(p, A, Bp, S, C, M, K, N, gmagic, ep, \
                                                      wf.zeros, workspace, stream);       \
    if (wf.fmt == kFmtBf16)                                                               \
      return launch_one<MB_, NB_, WK_, D_, kFmtBf16>(p, A, Bp, S, C, M, K, N, gmagic, ep,  \
                                                     nullptr, workspace, stream);         \
    if (wf.fmt == kFmtBf16Zp)                                                             \
      return launch_one<MB_, NB_, WK_, D_, kFmtBf16Zp>(p, A, Bp, S, C, M, K, N, gmagic,   \
                                                       ep, wf.zeros, workspace, stream);  \
    if (wf.fmt == kFmtW8)                                                                 \
      return launch_one<MB_, NB_, WK_, D_, kFmtW8>(p, A, Bp, S, C, M, K, N, gmagic, ep,    \
                                                   nullptr, workspace, stream);           \
  }
  if (wf.fmt != kFmtSp24) {
    W4A16_VARIANTS(W4A16_CASE)
  }
#undef W4A16_CASE
#define W4A16_WCASE(MB_, NB_, WK_, D_)                                                    \
  if (p.mb == MB_ && p.nb == NB_ && p.wk == WK_ && p.depth == D_) {                       \
    if (wf.fmt == kFmtBf16)                                                               \
      return launch_one<MB_, NB_, WK_, D_, kFmtBf16>(p, A, Bp, S, C, M, K, N, gmagic, ep,  \
                                                     nullptr, workspace, stream);         \
    if (wf.fmt == kFmtBf16Zp)                                                             \
      return launch_one<MB_, NB_, WK_, D_, kFmtBf16Zp>(p, A, Bp, S, C, M, K, N, gmagic,   \
                                                       ep, wf.zeros, workspace, stream);  \
    if (wf.fmt == kFmtW8)                                                                 \
      return launch_one<MB_, NB_, WK_, D_, kFmtW8>(p, A, Bp, S, C, M, K, N, gmagic, ep,    \
                                                   nullptr, workspace, stream);           \
  }
  W4A16_SCALED_WEIGHT_VARIANTS(W4A16_WCASE)
#undef W4A16_WCASE
  if (wf.fmt == kFmtSp24) {
#define W4A16_SCASE(MB_, NB_, WK_, D_)                                                      \
  if (p.mb == MB_ && p.nb == NB_ && p.wk == WK_ && p.depth == D_)                           \
    return launch_one<MB_, NB_, WK_, D_, kFmtSp24>(p, A, Bp, S, C, M, K, N, gmagic, ep,     \
                                                   nullptr, workspace, stream);
    W4A16_SP_VARIANTS(W4A16_SCASE)
#undef W4A16_SCASE
  }
  return hipErrorInvalidValue;
}

}  // namespace w4a16
