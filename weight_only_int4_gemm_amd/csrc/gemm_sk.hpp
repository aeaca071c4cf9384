// The stream-K W4A16 GEMM (9 to 128 rows on large layers): C = A . dequant(Bpacked).
// (The kernel template; gemm_sk.hip and gemm_sk_fmt.hip instantiate it for
// the FP16 format and for the formats with zero points or BF16.)
//
// Work decomposition.  The output is cut into tiles of 16*MB rows x 16*NB*WN
// columns; a tile's K dimension into 128-deep K blocks.  The (tile, K block)
// iterations, tile-major and K-minor (row tiles of one column tile next to
// each other), are dealt out in G equal contiguous runs, one per workgroup,
// G about the number of compute units: every compute unit streams the same
// number of weight blocks, whatever the tile count ("Quant Marlin kernel"
// explainer, "The architecture", middle row: the split over the in-feature
// dimension with a global reduction, so that every SM has work; here the
// split points are placed so the work divides evenly -- the stream-K form).
// A tile whose iterations one workgroup runs alone is written straight to
// C; a tile split between workgroups is finished by whichever of them
// arrives last, adding the FP32 partials in K order (deterministic,
// "Low-Precision Quantization Kernels in Production", section 3, mechanism
// 1).  Workgroups are numbered so that consecutive runs land on one XCD
// (blocks are dealt to the 8 XCDs in turn), where row tiles of one column
// tile share their codes in the XCD's L2.
//
// Inside a workgroup: WN waves, one or two per SIMD.  Wave w owns the
// tile's columns 16*NB*w .. +16*NB and every row.  Per K block a pipeline
// stage in LDS holds the tile's activations and codes (each wave loads an
// equal share) and the scales (each wave those of its own columns), all
// brought in by the direct global -> LDS load NS - 1 K blocks ahead ("Quant
// Marlin kernel", "The architecture", top row: asynchronous copies of the
// next tiles into shared memory while the current one is multiplied).  With
// two waves per SIMD one wave's LDS reads and unpacking run while the
// other's matrix instructions do, and no weight is unpacked twice.
//
// Per 32-deep slice a wave reads MB activation fragments from LDS, unpacks
// NB code words (unpack.hpp) and issues MB x NB matrix instructions.  The
// slices are software-pipelined: the fragments and weights of the next
// slice are read and unpacked while the current slice's matrix instructions
// run, and the next K block's codes, scales and first activation fragments
// are read during the last slice of the current one.  One barrier per K
// block, placed before the last slice.
//
// Each tile runs KBP iterations, K / 128 rounded up to a multiple of NS, so
// runs can be cut at multiples of NS and every tile segment starts at stage
// 0: the hot loop is unrolled by NS with every stage known at compile time.
// The (at most NS - 1) padding iterations of a tile re-read its last K
// block with the scales taken as zero: their weights are exact zeros and
// add nothing to the sums.
//
// The weights are the matrix instruction's first operand and the
// activations its second, so a lane's four accumulators are four
// consecutive output columns of one row: each lane stores 8 bytes of FP16.
// The 16- and 32-row tiles of the FP16 formats swap the operands and scale each K
// block's sums instead of the weights (kPost below): a lane's four sums are
// then four rows of its own column, stored as four 2-byte values.
#pragma once

#include <type_traits>

#include "coherent.hpp"
#include "epilogue.hpp"
#include "format.hpp"
#include "internal.hpp"
#include "layout.hpp"
#include "tile_common.hpp"
#include "unpack.hpp"

namespace w4a16 {

namespace {

typedef _Float16 half4_sk_t __attribute__((ext_vector_type(4)));


// Logical run of this workgroup: runs g, g + 1, ... on one XCD when the
// grid is a multiple of the 8 XCDs (block b runs on XCD b % 8).
__device__ __forceinline__ int sk_run_index(int G) {
  const int b = blockIdx.x;
  if (G % 8 != 0) return b;
  return (b % 8) * (G / 8) + b / 8;
}

// Runs are cut in units of NS iterations (a tile is a whole number of
// units): first iteration of run g of G over U units, and the run holding
// iteration x.
template <int NS>
__device__ __forceinline__ int64_t sk_run_start(int64_t g, int64_t U, int64_t G) {
  return g * U / G * NS;
}
template <int NS>
__device__ __forceinline__ int sk_run_of(int64_t x, int64_t U, int64_t G) {
  return (int)(((x / NS + 1) * G - 1) / U);
}

}  // namespace

// FMT: the weight format (format.hpp), 0 to 3: FP16 or BF16, with or
// without zero points.  A, S and C hold raw 16-bit values; Z the zero points
// uint8[K/group][N] of formats 1 and 3.  The fused output stage is FP16 only.
// WN waves (4 or 8): one or two per SIMD.
template <int MB, int NB, int NS, int WN, bool EPI, int FMT>
__global__ __launch_bounds__(64 * WN) __attribute__((amdgpu_waves_per_eu(WN / 4, WN / 4))) void
gemm_sk_kernel(const _Float16* __restrict__ A, const uint32_t* __restrict__ Bp,
               const _Float16* __restrict__ S, _Float16* __restrict__ C, int M, int K, int N,
               uint64_t group_magic, int tiles_n, int tiles_m, unsigned* __restrict__ counters,
               float* __restrict__ partials, Epilogue ep, const uint8_t* __restrict__ Z) {
  static_assert(FMT >= 0 && FMT <= 3, "the 4-bit dense formats");
  static_assert(!EPI || FMT == kFmtF16, "the fused epilogue is FP16 only");
  constexpr bool ZP = Format<FMT>::kZp;
  static_assert(WN == 4 || WN == 8, "one or two waves per SIMD");
  constexpr int WAVES = WN;
  // Tiles of 128 rows: the step's instructions are interleaved one by one
  // (slice_order below, the unpacking in the form the scheduling groups see:
  // unpack_col<FMT, true>).  About two vector instructions co-issue with a
  // matrix instruction on gfx950, and these tiles have 1.6 unpacking
  // instructions per matrix instruction.  18432 x 73728 at M = 128: 2% faster
  // (three rounds, one box); the 64-row tile measured 2.6% slower with it,
  // and the smaller tiles keep the compiler's order as well.  FP16 weights
  // only: the zero-point and BF16 unpacking takes more instructions than
  // the pattern places (the same pattern cost the LDS kernel 4-8% there).
  constexpr bool kSched = FMT == kFmtF16 && MB >= 8;
  // One or two 16-row blocks, FP16 formats (kPost): the matrix instructions take the
  // exact integers q - z, with the activations as their first operand (a
  // lane's four sums are then four rows of its own column), and each K
  // block's FP32 sums are scaled with one multiply-add per sum: 9 unpacking
  // instructions per code word instead of 13.
  constexpr bool kPost = MB <= 2 && (FMT == kFmtF16 || FMT == kFmtF16Zp);
  constexpr int TM = 16 * MB;              // rows of the tile
  constexpr int TNW = 16 * NB;             // columns of one wave
  constexpr int TN = WN * TNW;             // columns of the tile
  constexpr int APIECES = TM * 16;         // 16-byte pieces of one stage's activations
  constexpr int ACHUNKS = APIECES / 64;         // 1 KiB wave-loads of activations
  // activation loads per wave; with fewer chunks than waves some chunks are
  // loaded twice (same bytes to the same place), so every wave issues the
  // same number of loads
  constexpr int ALOADS = (ACHUNKS + WAVES - 1) / WAVES;
  constexpr int CLOADS = NB;                    // code blocks each wave loads: its own
  static_assert(NB == 2 || NB == 4, "a wave's scales: one 2-byte direct load, one vector read");
  constexpr int LOADS = ALOADS + CLOADS + 1 + (ZP ? 1 : 0);  // direct loads per wave per stage
  static_assert(NS >= 2 && (NS - 1) * LOADS < 64, "vmcnt range");
  struct StagePlain {
    uint4 a[APIECES];               // activations, piece p of row r at slot p ^ (r & 15)
    uint4 b[WN * NB * 64];          // codes: block nb of wave column wn at 64 * (wn * NB + nb)
    uint32_t s[WN * 64];            // scales: wave column wn's 64 at 64 * wn, one per 32-bit word
  };
  struct StageZp {
    uint4 a[APIECES];
    uint4 b[WN * NB * 64];
    uint32_t s[WN * 64];
    uint32_t z[WN * 64];            // zero points, laid out like the scales
  };
  typedef typename std::conditional<ZP, StageZp, StagePlain>::type Stage;
  // One LDS object per stage: the compiler then knows that a direct load
  // into one stage does not write another, and waits for exactly the loads
  // a read depends on (one array of stages makes it wait for all of them).
  static_assert(NS <= 8, "at most eight stages");
  __shared__ Stage st0;
  __shared__ typename std::conditional<(NS > 1), Stage, char>::type st1;
  __shared__ typename std::conditional<(NS > 2), Stage, char>::type st2;
  __shared__ typename std::conditional<(NS > 3), Stage, char>::type st3;
  __shared__ typename std::conditional<(NS > 4), Stage, char>::type st4;
  __shared__ typename std::conditional<(NS > 5), Stage, char>::type st5;
  __shared__ typename std::conditional<(NS > 6), Stage, char>::type st6;
  __shared__ typename std::conditional<(NS > 7), Stage, char>::type st7;
  Stage* const st[8] = {&st0,
                        reinterpret_cast<Stage*>(&st1),
                        reinterpret_cast<Stage*>(&st2),
                        reinterpret_cast<Stage*>(&st3),
                        reinterpret_cast<Stage*>(&st4),
                        reinterpret_cast<Stage*>(&st5),
                        reinterpret_cast<Stage*>(&st6),
                        reinterpret_cast<Stage*>(&st7)};

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave;  // this wave's column block of the tile
  const int l16 = lane & 15;
  const int G = gridDim.x;
  const int run = sk_run_index(G);
  const int KB = K / kBlockK;
  const int KBP = (KB + NS - 1) / NS * NS;                      // iterations per tile
  const int64_t U = (int64_t)tiles_n * tiles_m * (KBP / NS);  // units of NS iterations
  const int64_t i0 = sk_run_start<NS>(run, U, G);
  const int64_t i1 = sk_run_start<NS>(run + 1, U, G);
  const int n16_last = N / kBlockN - 1;

  auto scale_row = [&](int kb) -> int {
    return (int)(((uint64_t)(uint32_t)kb * group_magic) >> 32);
  };

  // ---- the load stream: iteration il = (tile, kb), clamped to i1 - 1 ----
  // (loads past the run re-read its last iteration into a stage that is
  // never consumed again, which keeps the number of loads per stage fixed)
  // (all updates are selects: no branch may split the hot loop, or the
  // compiler's own waits before LDS reads turn conservative)
  int ld_tn, ld_tm;
  {
    const int t0 = (int)(i0 / KBP);
    ld_tn = t0 / tiles_m;
    ld_tm = t0 - ld_tn * tiles_m;
  }
  int ld_kb = (int)(i0 % KBP);
  int ld_left = (int)(i1 - i0) - 1;  // advances left before the clamp
  // Activation loads: a per-lane byte offset from the row tile's first row
  // (constant for the whole kernel), added to a scalar base that moves with
  // the K block, so the address costs one select instead of a 64-bit
  // multiply-add per load.  Two offsets per load: rows as they are, and rows
  // clamped to M - 1 for the last row tile (rows past M are never stored).
  // (TM - 1) * K * 2 + 256 < 2^32 under the API's K < 2^23.
  uint32_t a_off[ALOADS], a_off_last[ALOADS];
  {
    const int rlim = M - 1 - (tiles_m - 1) * TM;  // last valid row of the last row tile
#pragma unroll
    for (int q = 0; q < ALOADS; ++q) {
      const int chunk = (wave + WAVES * q) % ACHUNKS;
      const int r = 4 * chunk + (lane >> 4);
      const uint32_t piece = (uint32_t)(l16 ^ (r & 15));
      const int rl = r < rlim ? r : rlim;
      a_off[q] = (uint32_t)r * (uint32_t)K * 2u + piece * 16u;
      a_off_last[q] = (uint32_t)rl * (uint32_t)K * 2u + piece * 16u;
    }
  }
  auto load_stage = [&](Stage& sg) {
    const int tn = ld_tn;
    const int tm = ld_tm;
    const int kb = ld_kb < KB ? ld_kb : KB - 1;  // padding iterations re-read the last block
    // activations: chunk c = (wave + WAVES * q) % ACHUNKS holds rows 4c .. 4c + 3
    // (the empty asm keeps the base in scalar registers, where the load
    // takes it as its scalar address)
    {
      const char* abase = reinterpret_cast<const char*>(A) +
                          ((int64_t)tm * TM * K + (int64_t)kb * kBlockK) * 2;
      asm("" : "+s"(abase));
      const bool last_m = tm == tiles_m - 1;
#pragma unroll
      for (int q = 0; q < ALOADS; ++q) {
        const int chunk = (wave + WAVES * q) % ACHUNKS;
        const uint32_t off = last_m ? a_off_last[q] : a_off[q];
        __builtin_amdgcn_global_load_lds((global_ptr_t)(abase + off), (lds_ptr_t)&sg.a[64 * chunk],
                                         16, 0, 0);
      }
    }
    // the tile's code blocks wave * CLOADS .. + CLOADS - 1; non-temporal
    // (cache policy 2): the plans use a single row tile, so every code word
    // is read once, and the hint keeps the stream from evicting the
    // activations from L2 (18432 x 73728 at M = 64: 791 against 922 MB
    // fetched, 209 against 214 us)
#pragma unroll
    for (int q = 0; q < CLOADS; ++q) {
      const int blk = wave * CLOADS + q;
      const int n16 = tn * (WN * NB) + blk;
      const int n16c = n16 <= n16_last ? n16 : n16_last;  // columns past N: dropped at the store
      const uint32_t* src = Bp + block_word_offset(n16c, kb, K) + lane * kWordsPerLane;
      __builtin_amdgcn_global_load_lds((global_ptr_t)src, (lds_ptr_t)&sg.b[64 * blk], 16, 0, 2);
    }
    // the scales of this wave's 16*NB columns, one FP16 per lane; a 2-byte
    // direct load puts lane L's value in 32-bit word L of the destination.
    // Lane L loads column 16 (L % NB) + (L / NB) % 16, so the NB scales
    // lane l uses (columns 16 nb + l % 16) are words NB (l % 16) .. +NB-1:
    // one read.  (With NB = 2 lanes 32..63 load the same columns again
    // into words no lane reads.)
    {
      const int c0 = tn * TN + wn * TNW + 16 * (lane % NB) + (lane / NB) % 16;
      const int c = c0 <= N - 1 ? c0 : N - 1;
      const _Float16* src = S + (int64_t)scale_row(kb) * N + c;
      __builtin_amdgcn_global_load_lds((global_ptr_t)src, (lds_ptr_t)&sg.s[64 * wn], 2, 0, 0);
      if constexpr (ZP) {
        // the zero points the same way, one byte per lane and word
        const uint8_t* zsrc = Z + (int64_t)scale_row(kb) * N + c;
        __builtin_amdgcn_global_load_lds((global_ptr_t)zsrc, (lds_ptr_t)&sg.z[64 * wn], 1, 0, 0);
      }
    }
    // advance, clamped to the run's last iteration
    const int adv = ld_left > 0 ? 1 : 0;
    ld_left -= adv;
    const int kb_next = ld_kb + adv;
    const int wrap = kb_next == KBP ? 1 : 0;
    ld_kb = wrap ? 0 : kb_next;
    const int tm_next = ld_tm + wrap;
    const int wrap_m = tm_next == tiles_m ? 1 : 0;
    ld_tm = wrap_m ? 0 : tm_next;
    ld_tn += wrap_m;
  };

  // ---- per-wave registers ----
  float4_t acc[MB][NB];  // set by the first slice of every tile segment
  float4_t blk[kPost ? MB : 1][kPost ? NB : 1];  // kPost: the current K block's sums
  half2_t s_blk[kPost ? NB : 1];    // kPost: its scales
  half8_t af[2][MB];  // activation fragments, two slices
  half8_t bf[2][NB];  // unpacked weights, two slices
  uint4 cw[NB];       // this K block's code words (one per slice)
  ColParams cp[NB];   // this K block's scales (and zero points)

  auto read_a = [&](const Stage& sg, int j, half8_t* a) {
    const int lg = lane >> 4;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = mb * 16 + l16;
      a[mb] = __builtin_bit_cast(half8_t, sg.a[r * 16 + ((4 * j + lg) ^ (r & 15))]);
    }
  };
  // codes and scales of a K block; a padding block's scales are zero (a
  // mask, not a branch)
  auto read_codes = [&](const Stage& sg, bool pad) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) cw[nb] = sg.b[64 * (wn * NB + nb) + lane];
    const uint32_t keep = pad ? 0u : 0xFFFFu;
    uint32_t w[NB];
    uint32_t zp[NB];
    if constexpr (NB == 4) {
      const uint4 s4 = reinterpret_cast<const uint4*>(&sg.s[64 * wn])[l16];
      w[0] = s4.x & keep;
      w[1] = s4.y & keep;
      w[2] = s4.z & keep;
      w[3] = s4.w & keep;
    } else {
      const uint2 s2 = reinterpret_cast<const uint2*>(&sg.s[64 * wn])[l16];
      w[0] = s2.x & keep;
      w[1] = s2.y & keep;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) zp[nb] = 8u;
    if constexpr (ZP) {
      if constexpr (NB == 4) {
        const uint4 z4 = reinterpret_cast<const uint4*>(&sg.z[64 * wn])[l16];
        zp[0] = z4.x & 0xFFu;
        zp[1] = z4.y & 0xFFu;
        zp[2] = z4.z & 0xFFu;
        zp[3] = z4.w & 0xFFu;
      } else {
        const uint2 z2 = reinterpret_cast<const uint2*>(&sg.z[64 * wn])[l16];
        zp[0] = z2.x & 0xFFu;
        zp[1] = z2.y & 0xFFu;
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      cp[nb] = make_col<FMT>(__builtin_bit_cast(half2_t, w[nb] | (w[nb] << 16)), zp[nb]);
  };
  auto unpack = [&](int j, half8_t* b) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t w = j == 0 ? cw[nb].x : j == 1 ? cw[nb].y : j == 2 ? cw[nb].z : cw[nb].w;
      if constexpr (kPost)
        b[nb] = unpack_col_codes<FMT>(w, cp[nb]);
      else
        b[nb] = unpack_col<FMT, kSched>(w, cp[nb]);
    }
  };
  auto mma = [&](const half8_t* a, const half8_t* b) {
    if constexpr (kPost) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) blk[mb][nb] = mma16<FMT>(a[mb], b[nb], blk[mb][nb]);
      return;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[mb][nb] = mma16<FMT>(b[nb], a[mb], acc[mb][nb]);
  };
  // the first slice of a tile segment: the sums start from zero (an inline
  // constant operand, so no register is ever cleared)
  auto mma_first = [&](const half8_t* a, const half8_t* b) {
    if constexpr (kPost) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          blk[mb][nb] = mma16<FMT>(a[mb], b[nb], float4_t{0.f, 0.f, 0.f, 0.f});
      return;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[mb][nb] = mma16<FMT>(b[nb], a[mb], float4_t{0.f, 0.f, 0.f, 0.f});
  };
  // ---- the tile epilogue ----
  const int64_t G64 = G;
  auto finish_tile = [&](int tile, bool whole) {
    const int tn = tile / tiles_m;
    const int tm = tile - tn * tiles_m;
    const int row0 = tm * TM;
    const int col0 = tn * TN + wn * TNW;
    // fused output stage: the bias of the four columns this lane stores in
    // each column block, loaded together up front
    half4_sk_t bias4[NB] = {};
    if constexpr (EPI) {
      if (ep.bias) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int gc = col0 + nb * 16 + (lane >> 4) * 4;
          if (gc < N) bias4[nb] = *reinterpret_cast<const half4_sk_t*>(ep.bias + gc);
        }
      }
    }
    auto write_c = [&](int mb, int nb, const float4_t& x) {
      if constexpr (kPost) {
        // rows 16 mb + 4 (l / 16) .. +3 of column 16 nb + l % 16
        const int gc = col0 + nb * 16 + l16;
        if (gc >= N) return;
        float bias = 0.f;
        if constexpr (EPI) {
          if (ep.bias) bias = (float)ep.bias[gc];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gr = row0 + mb * 16 + (lane >> 4) * 4 + e;
          if (gr < M) {
            _Float16 h;
            if constexpr (EPI)
              h = (_Float16)epilogue_apply(ep, x[e], bias);
            else
              h = out16<FMT>(x[e]);
            C[(int64_t)gr * N + gc] = h;
          }
        }
        return;
      }
      const int gr = row0 + mb * 16 + l16;
      const int gc = col0 + nb * 16 + (lane >> 4) * 4;  // N % 16 == 0: all four or none
      if (gr < M && gc < N) {
        half4_sk_t h;
        if constexpr (EPI) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            h[e] = (_Float16)epilogue_apply(ep, x[e], (float)bias4[nb][e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = out16<FMT>(x[e]);
        }
        *reinterpret_cast<half4_sk_t*>(C + (int64_t)gr * N + gc) = h;
      }
    };
    if (whole) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) write_c(mb, nb, acc[mb][nb]);
      return;
    }
    // A tile shared with other runs: publish this wave's FP32 slice in the
    // run's slot (device-coherent 16-byte stores, fragment order), wait for
    // the stores, count the arrival on the tile's counter for this wave;
    // the last of the tile's runs to arrive adds every run's slice in run
    // (= K) order and writes C.  (The sums are identical whoever arrives
    // last: bit-identical results run to run.)
    constexpr int SLOT = TM * TN;  // floats per slot
    auto slot_of = [&](int g) -> int64_t {
      const int ft = (int)(sk_run_start<NS>(g, U, G64) / KBP);
      return 2 * (int64_t)g + (tile == ft ? 0 : 1);
    };
    const int frag0 = wave * MB * NB * 64 + lane;
    {
      const __amdgpu_buffer_rsrc_t mine = coherent_rsrc(partials + slot_of(run) * SLOT);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          store_coherent(mine, frag0 + (mb * NB + nb) * 64, acc[mb][nb]);
    }
    __builtin_amdgcn_s_waitcnt(0);
    const int g_first = sk_run_of<NS>((int64_t)tile * KBP, U, G64);
    const int g_last = sk_run_of<NS>((int64_t)tile * KBP + KBP - 1, U, G64);
    unsigned prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(counters + tile * WAVES + wave, 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != (unsigned)(g_last - g_first)) return;
    // Last to arrive: the sum in run order, every run's slice read back from
    // its slot (this wave's own too, so the order never depends on who
    // arrives last), eight fragments in flight at a time.
    {
      const __amdgpu_buffer_rsrc_t r0 = coherent_rsrc(partials + slot_of(g_first) * SLOT);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = load_coherent(r0, frag0 + (mb * NB + nb) * 64);
    }
    constexpr int MCH = MB < 2 ? MB : 2;  // row blocks per batch of loads
    for (int g = g_first + 1; g <= g_last; ++g) {
      const __amdgpu_buffer_rsrc_t rg = coherent_rsrc(partials + slot_of(g) * SLOT);
#pragma unroll
      for (int m0 = 0; m0 < MB; m0 += MCH) {
        float4_t p[MCH][NB];
#pragma unroll
        for (int mb = 0; mb < MCH; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            p[mb][nb] = load_coherent(rg, frag0 + ((m0 + mb) * NB + nb) * 64);
#pragma unroll
        for (int mb = 0; mb < MCH; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[m0 + mb][nb] = acc[m0 + mb][nb] + p[mb][nb];
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) write_c(mb, nb, acc[mb][nb]);
    if (lane == 0)  // ready for the next call
      __hip_atomic_store(counters + tile * WAVES + wave, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  };

  // ---- prologue: fill all NS stages, then the first block's operands ----
#pragma unroll
  for (int q = 0; q < NS; ++q) load_stage(*st[q]);
  stage_barrier<(NS - 1) * LOADS>();
  read_codes(*st[0], false);  // a run starts on a unit boundary: never a padding block
  read_a(*st[0], 0, af[0]);
  unpack(0, bf[0]);

  // ---- the compute stream ----
  // The run's iterations in tile segments: a segment's K blocks in the hot
  // loop, then the tile's epilogue.  Segments start on a unit boundary and
  // are whole units long, so the hot loop is unrolled by NS with stage
  // u = iteration % NS known at compile time, and the pipeline runs on
  // across segments.  One K block from stage u: slices 0..2 with the reads
  // and unpacking of the following slice; then the barrier (stage u + 1 has
  // landed, nobody reads stage u any more), the loads of the block NS ahead
  // into stage u, the reads of the next block's codes, scales and first
  // fragments from stage u + 1, and slice 3.
  // kSched: after each matrix instruction of a slice, one fragment read and
  // up to VPM unpacking instructions of the next slice; each slice fenced.
  constexpr int MM = MB * NB;
  constexpr int VPM = (NB * 13 + MM - 1) / MM;
  auto slice_order = [&](auto sid) {
    if constexpr (kSched) {
      constexpr int S = decltype(sid)::value;
#pragma unroll
      for (int i = 0; i < MM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, S);
        if (i < MB) __builtin_amdgcn_sched_group_barrier(0x100, 1, S);
        __builtin_amdgcn_sched_group_barrier(0x002, VPM, S);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto step = [&](Stage& cur, Stage& nxt, bool pad_next, auto first, auto read_next) {
    read_a(cur, 1, af[1]);
    unpack(1, bf[1]);
    if constexpr (decltype(first)::value || kPost)  // kPost: every K block's sums start at zero
      mma_first(af[0], bf[0]);
    else
      mma(af[0], bf[0]);
    slice_order(std::integral_constant<int, 1>());
    read_a(cur, 2, af[0]);
    unpack(2, bf[0]);
    mma(af[1], bf[1]);
    slice_order(std::integral_constant<int, 2>());
    read_a(cur, 3, af[1]);
    unpack(3, bf[1]);
    mma(af[0], bf[0]);
    slice_order(std::integral_constant<int, 3>());
    stage_barrier<(NS - 2) * LOADS>();
    if constexpr (kPost) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s_blk[nb] = cp[nb].s2;  // before the next block's
    }
    if constexpr (decltype(read_next)::value) {
      read_codes(nxt, pad_next);
      read_a(nxt, 0, af[0]);
    }
    load_stage(cur);
    mma(af[1], bf[1]);
    if constexpr (decltype(read_next)::value) unpack(0, bf[0]);
    if constexpr (kPost) {
      // the block's sums into the tile's, scaled (the next block's
      // unpacking above covers the matrix unit's latency)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float s = (float)s_blk[nb][0];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[mb][nb][e] = decltype(first)::value
                                 ? blk[mb][nb][e] * s
                                 : __builtin_fmaf(blk[mb][nb][e], s, acc[mb][nb][e]);
      }
    }
    if constexpr (kSched) {
      // after the barrier: the next block's code and scale reads first, then
      // per matrix instruction one fragment read, one direct load and the
      // first slice's unpacking
      if constexpr (decltype(read_next)::value) {
        __builtin_amdgcn_sched_group_barrier(0x100, NB + 1, 4);
#pragma unroll
        for (int i = 0; i < MM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 4);
          if (i < MB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 4);
          if (i < LOADS) __builtin_amdgcn_sched_group_barrier(0x010, 1, 4);
          __builtin_amdgcn_sched_group_barrier(0x002, VPM, 4);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const std::true_type first_step, read_next;
  const std::false_type later_step, segment_end;
  // A segment of n units: its first step (stage 0) starts the sums; then
  // n - 1 units rotated by one stage (stages 1 .. NS-1, 0), then stages
  // 1 .. NS-1.  Every stage index is a compile-time constant.  (NS >= 2, so
  // the segment's last step is a different step from its first.)
  int64_t i = i0;
  int tile = (int)(i0 / KBP);
  while (i < i1) {
    const int64_t tile_start = (int64_t)tile * KBP;
    const int64_t tile_end = tile_start + KBP;
    const int64_t seg_end = i1 < tile_end ? i1 : tile_end;
    const bool whole = i == tile_start && seg_end == tile_end;
    int kb = (int)(i - tile_start);  // K block of the step about to run
    auto pad = [&](int kbn) { return kbn >= KB && kbn < KBP; };  // is block kbn padding?
    step(*st[0], *st[1 % NS], pad(kb + 1), first_step, read_next);
    ++kb;
    const int64_t units = (seg_end - i) / NS;
    for (int64_t n = 1; n < units; ++n) {
#pragma unroll
      for (int q = 1; q < NS; ++q)
        step(*st[q], *st[(q + 1) % NS], pad(kb + q), later_step, read_next);
      step(*st[0], *st[1 % NS], pad(kb + NS), later_step, read_next);
      kb += NS;
    }
#pragma unroll
    for (int q = 1; q < NS - 1; ++q)
      step(*st[q], *st[(q + 1) % NS], pad(kb + q), later_step, read_next);
    // the segment's last step leaves the next segment's first operands
    // unread, so that the tile epilogue has the registers they would take
    step(*st[NS - 1], *st[0], false, later_step, segment_end);
    i = seg_end;
    finish_tile(tile, whole);
    ++tile;
    // the next segment starts on stage 0, at a tile's first K block
    read_codes(*st[0], false);
    read_a(*st[0], 0, af[0]);
    unpack(0, bf[0]);
  }
  // no direct load may still be landing in LDS when the workgroup ends
  __builtin_amdgcn_s_waitcnt(0);
}

// ---------------------------------------------------------------------------
// host side

// Compiled variants (MB, NB, NS, WN): the plans' ones (MB row blocks, NS
// stages, WN waves).
#define W4A16_SK_VARIANTS(X) X(1, 4, 4, 8) X(2, 4, 3, 8) X(4, 4, 3, 8) X(8, 2, 3, 8)

template <int MB, int NB, int NS, int WN, int FMT>
hipError_t launch_sk_one(const Plan& p, const uint16_t* A, const uint32_t* Bp, const uint16_t* S,
                         uint16_t* C, int M, int K, int N, uint64_t gmagic, Epilogue ep,
                         const uint8_t* Z, void* workspace, hipStream_t stream) {
  unsigned* counters = nullptr;
  float* partials = nullptr;
  if (p.workspace_bytes > 0) {
    counters = static_cast<unsigned*>(workspace);
    partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterHeaderBytes);
  }
  const dim3 grid(p.splits), block(64 * WN);
  auto a = reinterpret_cast<const _Float16*>(A);
  auto s = reinterpret_cast<const _Float16*>(S);
  auto c = reinterpret_cast<_Float16*>(C);
  if constexpr (FMT == kFmtF16) {
    if (epilogue_needed(ep)) {
      hipLaunchKernelGGL((gemm_sk_kernel<MB, NB, NS, WN, true, FMT>), grid, block, 0, stream, a, Bp, s,
                         c, M, K, N, gmagic, p.tiles_n, p.tiles_m, counters, partials, ep, Z);
      return hipGetLastError();
    }
  } else {
    if (epilogue_needed(ep)) return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL((gemm_sk_kernel<MB, NB, NS, WN, false, FMT>), grid, block, 0, stream, a, Bp, s, c,
                     M, K, N, gmagic, p.tiles_n, p.tiles_m, counters, partials, ep, Z);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_sk_fmt(const Plan& p, const uint16_t* A, const uint32_t* Bp, const uint16_t* S,
                         uint16_t* C, int M, int K, int N, uint64_t gmagic, Epilogue ep,
                         const uint8_t* Z, void* workspace, hipStream_t stream) {
#define W4A16_SKCASE(MB_, NB_, NS_, WN_)                                                     \
  if (p.mb == MB_ && p.nb == NB_ && p.depth == NS_ && p.wm == 1 && p.wk == WN_)               \
    return launch_sk_one<MB_, NB_, NS_, WN_, FMT>(p, A, Bp, S, C, M, K, N, gmagic, ep, Z,      \
                                                  workspace, stream);
  W4A16_SK_VARIANTS(W4A16_SKCASE)
#undef W4A16_SKCASE
  return hipErrorInvalidValue;
}

// Formats 1 to 3 (gemm_sk_fmt.hip).
hipError_t launch_sk_zp_bf16(const Plan& p, const uint16_t* A, const uint32_t* Bp,
                             const uint16_t* S, uint16_t* C, int M, int K, int N, uint64_t gmagic,
                             Epilogue ep, WeightFormat wf, void* workspace, hipStream_t stream);

}  // namespace w4a16
