// The W4A16 GEMM for all but the smallest batches (the plans in api.hip),
// with every operand staged through LDS: C = A . dequant(Bpacked).
//
// A workgroup of WM x WN waves owns an F*MB*WM x F*NB*WN output tile and one
// K range; wave (wm, wn) owns the F*MB x F*NB block at row block wm, column
// block wn.  With WM = 1 every wave spans all rows and each weight is
// unpacked once per workgroup; with WM > 1 each weight is unpacked by WM
// waves, but a wave reads only its own rows of the activation stage, which
// divides the LDS bytes read per matrix instruction (each wave re-reads its
// activation rows for every K block).
//
// Vector-memory loads of a wave complete in issue order, so if the codes
// went to registers and the activations to LDS, the wait for an activation
// stage would also wait for every code load issued before it, and the codes
// (which come from HBM) would never get more than a couple of K blocks of
// latency allowance however early they were issued.  Here one K block's
// activations, codes and scales form one LDS stage and are all brought in by
// the direct 16-byte global -> LDS load ("Quant Marlin kernel" explainer,
// "The architecture", top row: async copies of the next tile into shared
// memory while the current one is multiplied; "End-to-end flow": loads for
// the tile after next already in flight).  With NS stages, the loads of a
// stage are issued NS - 1 K blocks before the stage is consumed, and the
// single count-based wait before a step covers exactly the loads of that
// step's stage.
//
// Stage layout (per K block):
//  * activations: 16*MB rows x 16 pieces of 16 bytes, piece c of row r at
//    slot c ^ (r & 15) (conflict-free fragment reads);
//  * codes: the NB*WN (16-column) fragment blocks of the tile, 1 KiB each,
//    in the permuted layout's own order (lane l's four words at 16*l), so a
//    wave reads its fragments with one conflict-free 16-byte read per block;
//  * scales: the tile's 16*NB*WN FP16 scales of this K block's group.
//
// With 16 x 16 blocks the weights are the matrix instruction's first
// operand and the activations its second, so a lane's four accumulators are
// four consecutive output columns of one row and the output stage stores
// 8 bytes per lane and block (tile_common.hpp).  The 16- and 32-row tiles of
// the FP16 formats swap the operands and scale each K block's sums instead of
// the weights (kPost below): a lane's four sums are four rows of its own
// column.
//
// 2:4-sparse weights (format 5): a code block is 768 bytes (layout.hpp),
// brought in by one 16-byte direct load on lanes 0..47; a wave reads its
// two code words (8 bytes) and its position word from LDS and runs two
// sparse 16x16x64 matrix instructions per K block and 16 x 16 output block
// (format.hpp, smma16), whose results are likewise C transposed.
#include <type_traits>

#include "layout.hpp"
#include "tile_common.hpp"
#include "unpack.hpp"

namespace w4a16 {

// MB and NB count the 16-row and 16-column blocks of a wave's tile (the
// output block of v_mfma_f32_16x16x32_f16).
//
// FMT is the weight format (format.hpp): formats other than 0 have no fused
// epilogue; their zero points are one more part of each stage, loaded like
// the scales.
template <int MB, int NB, int WM, int WN, int NS, bool EPI, int FMT>
__global__ __launch_bounds__(64 * WM * WN) void gemm_lds_kernel(
    const _Float16* __restrict__ A, const uint32_t* __restrict__ Bp,
    const _Float16* __restrict__ S, _Float16* __restrict__ C, int M, int K, int N,
    uint64_t group_magic, int tiles_n, int head, int tail_tiles, int splits,
    unsigned* __restrict__ counters,
    float* __restrict__ partials, Epilogue ep, const uint8_t* __restrict__ Z) {
  static_assert(FMT == kFmtF16 || !EPI, "formats 1-5: no fused epilogue");
  constexpr bool ZP = Format<FMT>::kZp;
  constexpr bool SP = Format<FMT>::kSp;
  constexpr int BLOCK_PIECES = SP ? 48 : 64;     // 16-byte pieces of one code block
  constexpr int PPB = Format<FMT>::kW8 ? 2 : 1;  // 1 KiB pieces per code block and K block
  // Wave tiles of 128 rows, FP16 weights: the step's matrix instructions,
  // fragment reads and unpacking are interleaved one by one (see step
  // below).  Prefill 8192 x 28672 at M = 512 / 1024 / 4096: 1.2 / 2.2 / 1.7%
  // faster on one box.  The 64-row tiles measured up to 4% slower with it
  // (Llama-2-7B gate/up at M = 128), and so did the zero-point and BF16
  // formats, whose unpacking takes more instructions than the pattern
  // places (prefill at M = 1024: 4-8%); they keep the compiler's order.
  constexpr bool kSched = FMT == kFmtF16 && MB >= 8;
  // One or two 16-row blocks, FP16 formats with 4-bit codes (kPost): the matrix
  // instructions take the exact integers q - z with the activations as their
  // first operand (a lane's four sums are four rows of its own column), and
  // each K block's FP32 sums are scaled with one multiply-add per sum
  // instead of every weight: 9 unpacking instructions per code word, not 13.
  constexpr bool kPost = MB <= 2 && !SP && PPB == 1 && (FMT == kFmtF16 || FMT == kFmtF16Zp);
  constexpr int WAVES = WM * WN;
  constexpr int TM = 16 * MB * WM;
  constexpr int TN = 16 * NB * WN;
  constexpr int BLOCKS = NB * WN;              // 16-column code blocks of the tile
  constexpr int APIECES = TM * 16;             // 16-byte pieces of activations
  constexpr int ACHUNKS = APIECES / 64;        // 1 KiB wave-loads of activations
  // direct loads per wave of activation chunks and of code blocks; with
  // fewer chunks (blocks) than waves some are loaded twice (same bytes to
  // the same place), so every wave issues the same number of loads
  constexpr int ALOADS = (ACHUNKS + WAVES - 1) / WAVES;
  constexpr int BLOADS = (BLOCKS * PPB + WAVES - 1) / WAVES;
  constexpr int BPIECES = BLOCKS * PPB * BLOCK_PIECES;  // 16-byte pieces of codes
  constexpr int SDWORDS = TN / 2;              // scales of one K block, as 32-bit words
  constexpr int SLOADS = (SDWORDS + 63) / 64;  // 4-byte direct loads (every wave issues them)
  constexpr int ZLOADS = ZP ? (TN / 4 + 63) / 64 : 0;  // zero points: 4-byte loads, all waves
  constexpr int LOADS = ALOADS + BLOADS + SLOADS + ZLOADS;  // direct loads per wave per stage
  static_assert(NS >= 2 && NS <= 4, "two to four stages");
  struct StagePlain {
    uint4 a[APIECES];
    uint4 b[BPIECES];
    uint32_t s[64 * SLOADS];
  };
  struct StageZp {
    uint4 a[APIECES];
    uint4 b[BPIECES];
    uint32_t s[64 * SLOADS];
    uint32_t z[64 * (ZLOADS > 0 ? ZLOADS : 1)];  // the tile's zero points, one byte each
  };
  typedef typename std::conditional<ZP, StageZp, StagePlain>::type Stage;
  // one LDS object per stage: the compiler sees that a load into one stage
  // does not touch the others
  __shared__ Stage st0;
  __shared__ Stage st1;
  // stages 2 and 3 only where NS asks for them (a byte otherwise)
  __shared__ typename std::conditional<(NS > 2), Stage, char>::type st2;
  __shared__ typename std::conditional<(NS > 3), Stage, char>::type st3;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN;  // this wave's row block and column block
  const int wn = wave % WN;
  // Workgroup -> (tile, K range): the first `head` workgroups take whole
  // tiles; the remaining tail_tiles tiles are split `splits` ways, split
  // by split (all their first K ranges, then all their second, ...).
  // Tiles are numbered with the column tile fastest.
  const int b = blockIdx.x;
  int tile = b, split = 0, nsplit = 1;
  if (b >= head) {
    const int j = b - head;
    split = j / tail_tiles;
    tile = head + (j - split * tail_tiles);
    nsplit = splits;
  }
  const int tile_m = tile / tiles_n;
  const int tile_n = tile - tile_m * tiles_n;
  const int KB = K / kBlockK;
  const int kb0 = (int)((int64_t)KB * split / nsplit);
  const int kb1 = (int)((int64_t)KB * (split + 1) / nsplit);
  const int l16 = lane & 15;
  const int row0 = tile_m * TM;
  const int col0 = tile_n * TN;
  const int n16_last = N / kBlockN - 1;
  const int wrow0 = row0 + wm * 16 * MB;  // this wave's tile
  const int wcol0 = col0 + wn * 16 * NB;
  LaneBias4<NB, EPI> bias;
  bias.load(ep, wcol0, N);

  // Code pieces this wave loads: piece (wave + WAVES * i) % (BLOCKS * PPB)
  // of the stage for load i, i.e. tile block piece / PPB and, for 8-bit
  // codes, its 64-deep half piece % PPB (blocks past N re-read the last
  // valid one; their columns are dropped at the store).
  const uint32_t* bsrc[BLOADS];
  int bblk[BLOADS];
#pragma unroll
  for (int i = 0; i < BLOADS; ++i) {
    bblk[i] = (wave + WAVES * i) % (BLOCKS * PPB);
    const int n16 = tile_n * BLOCKS + bblk[i] / PPB;
    const int n16c = n16 <= n16_last ? n16 : n16_last;
    if constexpr (SP)
      bsrc[i] = Bp + block_word_offset_sp(n16c, 0, K) + lane * 4;
    else
      bsrc[i] = Bp +
                (PPB == 2 ? block_word_offset8(n16c, bblk[i] % 2, K) : block_word_offset(n16c, 0, K)) +
                lane * kWordsPerLane;
  }
  // Scale source: word i*64 + lane of the stage holds columns 2w, 2w+1.
  const _Float16* ssrc[SLOADS];
#pragma unroll
  for (int i = 0; i < SLOADS; ++i) {
    const int c = col0 + 2 * (64 * i + lane);
    ssrc[i] = S + (c <= N - 2 ? c : N - 2);
  }
  // Zero-point source: word i*64 + lane of the stage holds columns 4w .. 4w+3.
  const uint8_t* zsrc[ZLOADS > 0 ? ZLOADS : 1];
#pragma unroll
  for (int i = 0; i < ZLOADS; ++i) {
    const int c = col0 + 4 * (64 * i + lane);
    zsrc[i] = Z + (c <= N - 4 ? c : N - 4);
  }
  auto scale_row = [&](int kb) -> int {
    return (int)(((uint64_t)(uint32_t)kb * group_magic) >> 32);
  };

  auto load_stage = [&](Stage& sg, int kb) {
#pragma unroll
    for (int i = 0; i < ALOADS; ++i) {
      // activation load i of this wave: stage pieces 64 * chunk + lane
      const int chunk = (wave + WAVES * i) % ACHUNKS;
      const int r = 4 * chunk + (lane >> 4);
      const int piece = l16 ^ (r & 15);
      const int gr = row0 + r < M ? row0 + r : M - 1;  // rows past M: never stored
      const _Float16* src = A + (int64_t)gr * K + kb * kBlockK + piece * 8;
      __builtin_amdgcn_global_load_lds((global_ptr_t)src, (lds_ptr_t)&sg.a[64 * chunk], 16, 0,
                                       0);
    }
#pragma unroll
    for (int i = 0; i < BLOADS; ++i) {
      if constexpr (SP) {
        // a 768-byte block: lanes 0..47 move it (one load instruction still)
        if (lane < BLOCK_PIECES)
          __builtin_amdgcn_global_load_lds((global_ptr_t)(bsrc[i] + kb * kWordsPerBlockSp),
                                           (lds_ptr_t)&sg.b[BLOCK_PIECES * bblk[i]], 16, 0, 0);
      } else {
        __builtin_amdgcn_global_load_lds((global_ptr_t)(bsrc[i] + PPB * kb * kWordsPerBlock),
                                         (lds_ptr_t)&sg.b[64 * bblk[i]], 16, 0, 0);
      }
    }
    const int srow = scale_row(kb) * N;
#pragma unroll
    for (int i = 0; i < SLOADS; ++i) {
      __builtin_amdgcn_global_load_lds((global_ptr_t)(ssrc[i] + srow), (lds_ptr_t)&sg.s[64 * i],
                                       4, 0, 0);
    }
    if constexpr (ZP) {
#pragma unroll
      for (int i = 0; i < ZLOADS; ++i)
        __builtin_amdgcn_global_load_lds((global_ptr_t)(zsrc[i] + srow),
                                         (lds_ptr_t)&sg.z[64 * i], 4, 0, 0);
    }
  };

  float4_t acc[MB][NB];
  float4_t blk[kPost ? MB : 1][kPost ? NB : 1];  // kPost: the current K block's sums
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = float4_t{0.f, 0.f, 0.f, 0.f};

  // ---- 16 x 16 blocks: four 32-deep slices per K block -------------------
  // Lane l takes activation row l % 16, in-features 8(l/16) .. +7 of the
  // slice, and the code word j of its own 16-byte piece of the block.
  auto read_a = [&](const Stage& sg, int j, half8_t* a) {
    const int lg = lane >> 4;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = (wm * MB + mb) * 16 + l16;
      a[mb] = __builtin_bit_cast(half8_t, sg.a[r * 16 + ((4 * j + lg) ^ (r & 15))]);
    }
  };
  // Software-pipelined by one slice: while the matrix instructions of slice
  // j run, the activation fragments of slice j+1 are read and its codes
  // unpacked, so the vector ALU work has independent matrix work to overlap.
  auto compute16 = [&](const Stage& sg) {
    uint4 w[NB];
    uint4 w2[PPB == 2 ? NB : 1];  // 8-bit codes: the second 64-deep half
    ColParams cp[NB];
    const _Float16* sh = reinterpret_cast<const _Float16*>(sg.s);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      w[nb] = sg.b[64 * PPB * (wn * NB + nb) + lane];
      if constexpr (PPB == 2) w2[nb] = sg.b[64 * (2 * (wn * NB + nb) + 1) + lane];
      const int c = wn * 16 * NB + nb * 16 + l16;
      const _Float16 sc = sh[c];
      uint32_t z = 8;
      if constexpr (ZP) z = reinterpret_cast<const uint8_t*>(sg.z)[c];
      cp[nb] = make_col<FMT>(half2_t{sc, sc}, z);
    }
    auto unpack_slice = [&](int j, half8_t* bf) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (PPB == 2) {
          const uint4& pc = j < 2 ? w[nb] : w2[nb];
          bf[nb] = unpack8_scale((j & 1) ? pc.z : pc.x, (j & 1) ? pc.w : pc.y, cp[nb].s2);
        } else {
          const uint32_t word =
              j == 0 ? w[nb].x : j == 1 ? w[nb].y : j == 2 ? w[nb].z : w[nb].w;
          if constexpr (kPost)
            bf[nb] = unpack_col_codes<FMT>(word, cp[nb]);
          else
            bf[nb] = unpack_col<FMT, kSched>(word, cp[nb]);
        }
      }
    };
    half8_t a0[MB], a1[MB];
    half8_t b0[NB], b1[NB];
    read_a(sg, 0, a0);
    unpack_slice(0, b0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half8_t* cur = (j & 1) ? a1 : a0;
      half8_t* nxt = (j & 1) ? a0 : a1;
      half8_t* bcur = (j & 1) ? b1 : b0;
      half8_t* bnxt = (j & 1) ? b0 : b1;
      if (j < 3) {
        read_a(sg, j + 1, nxt);
        unpack_slice(j + 1, bnxt);
      }
      if constexpr (kPost) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            blk[mb][nb] = mma16<FMT>(cur[mb], bcur[nb],
                                     j == 0 ? float4_t{0.f, 0.f, 0.f, 0.f} : blk[mb][nb]);
      } else {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            acc[mb][nb] = mma16<FMT>(bcur[nb], cur[mb], acc[mb][nb]);
          }
      }
    }
    if constexpr (kPost) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float s = (float)cp[nb].s2[0];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[mb][nb][e] = __builtin_fmaf(blk[mb][nb][e], s, acc[mb][nb][e]);
      }
    }
  };

  // ---- 2:4-sparse codes: two 64-deep sparse steps per K block ------------
  // Step t multiplies the weights' compressed code word t (transposed: rows
  // are output columns) by the activation fragments of 32-deep slices 2t
  // and 2t+1 side by side; acc[mb][nb] holds C transposed.
  auto compute_sp = [&](const Stage& sg) {
    uint2 w[NB];
    uint32_t pos[NB];
    half2_t s2[NB];
    const _Float16* sh = reinterpret_cast<const _Float16*>(sg.s);
    const uint2* bw2 = reinterpret_cast<const uint2*>(sg.b);
    const uint32_t* bw = reinterpret_cast<const uint32_t*>(sg.b);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int blk = wn * NB + nb;
      w[nb] = bw2[(kWordsPerBlockSp / 2) * blk + lane];
      pos[nb] = bw[kWordsPerBlockSp * blk + kCodeWordsSp + lane];
      const _Float16 sc = sh[wn * 16 * NB + nb * 16 + l16];
      s2[nb] = half2_t{sc, sc};
    }
    half8_t a0[MB], a1[MB], a2[MB], a3[MB];
    half8_t b0[NB], b1[NB];
    read_a(sg, 0, a0);
    read_a(sg, 1, a1);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b0[nb] = unpack_scale(w[nb].x, s2[nb]);
    read_a(sg, 2, a2);
    read_a(sg, 3, a3);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b1[nb] = unpack_scale(w[nb].y, s2[nb]);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        acc[mb][nb] = smma16(b0[nb], a0[mb], a1[mb], pos[nb], acc[mb][nb]);
      }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        acc[mb][nb] = smma16(b1[nb], a2[mb], a3[mb], pos[nb] >> 16, acc[mb][nb]);
      }
  };
  auto compute = [&](const Stage& sg) {
    if constexpr (SP)
      compute_sp(sg);
    else
      compute16(sg);
  };

  // The pipeline: step t consumes stage t % NS; before it, once every wave
  // has passed the step's barrier (so the stage of block t - 1 is free), the
  // loads of block t + NS - 1 go into that stage.  The prologue fills stages
  // 0 .. NS-2.  Loads past the range are clamped to the last block
  // (harmless re-reads into a stage that is never consumed again).
  const int nblk = kb1 - kb0;  // >= 1: splits never exceed the K blocks
  const int last = kb1 - 1;
  auto clamp = [&](int kb) { return kb <= last ? kb : last; };
  Stage* const stages[4] = {&st0, &st1, NS > 2 ? reinterpret_cast<Stage*>(&st2) : &st0,
                            NS > 3 ? reinterpret_cast<Stage*>(&st3) : &st1};
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) load_stage(*stages[s], clamp(kb0 + s));
  // A wave issues in order, and a direct load waits at issue while the
  // address unit is busy with earlier ones (a burst of a dozen 1 KiB loads
  // from four waves stalls each wave for hundreds of cycles).  So the
  // step's loads are spread between its matrix instructions: one load
  // after every MFMA_PER_LOAD of them.
  constexpr int NMFMA = (SP ? 2 : 4) * MB * NB;
  constexpr int MFMA_PER_LOAD = NMFMA / (LOADS + 1) > 0 ? NMFMA / (LOADS + 1) : 1;
  constexpr int MM = MB * NB;                      // matrix instructions per slice
  constexpr int VPM = (NB * 13 + MM - 1) / MM;     // unpacking instructions per one
  auto step = [&](int u, int kb) {  // u = t % NS
    stage_barrier<(NS - 2) * LOADS>();
    load_stage(*stages[(u + NS - 1) % NS], clamp(kb + NS - 1));
    compute(*stages[u]);
    if constexpr (kSched) {
      // The first slice's operands (code words, scales, fragments and their
      // unpacking), then per matrix instruction of slice j one fragment
      // read and up to VPM unpacking instructions of slice j + 1, with the
      // step's direct loads spread as below.
      __builtin_amdgcn_sched_group_barrier(0x0100, MB + 2 * NB, 0);
      __builtin_amdgcn_sched_group_barrier(0x0002, NB * 13 + 2 * NB, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < MM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
          if (j < 3 && i < MB) __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);
          if (j < 3) __builtin_amdgcn_sched_group_barrier(0x0002, VPM, 0);
          if ((j * MM + i) % MFMA_PER_LOAD == MFMA_PER_LOAD - 1 &&
              (j * MM + i) / MFMA_PER_LOAD < LOADS)
            __builtin_amdgcn_sched_group_barrier(0x0010, 1, 0);
        }
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x0008, MFMA_PER_LOAD, 0);
        __builtin_amdgcn_sched_group_barrier(0x0010, 1, 0);
      }
    }
  };
  int t = 0;
  for (; t + NS <= nblk; t += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) step(u, kb0 + t + u);
  }
#pragma unroll
  for (int u = 0; u < NS - 1; ++u) {
    if (t + u < nblk) step(u, kb0 + t + u);
  }
  // No direct load may still be landing in LDS when the stages are reused
  // below or the workgroup ends.
  __builtin_amdgcn_s_waitcnt(0);

  store_output_tile<MB, NB, WAVES, EPI, FMT, kPost>(acc, C, M, N, wrow0, wcol0, split, nsplit,
                                             tile - head, counters, partials,
                                             reinterpret_cast<int*>(&st0.s[0]), ep, bias);
}

template <int MB, int NB, int WM, int WN, int NS, int FMT>
static hipError_t launch_lds_one(const Plan& p, const uint16_t* A, const uint32_t* Bp,
                                 const uint16_t* S, uint16_t* C, int M, int K, int N,
                                 uint64_t gmagic, Epilogue ep, const uint8_t* Z, void* workspace,
                                 hipStream_t stream) {
  unsigned* counters = nullptr;
  float* partials = nullptr;
  if (p.splits > 1) {
    counters = static_cast<unsigned*>(workspace);
    partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterHeaderBytes);
  }
  const int tiles = p.tiles_n * p.tiles_m;
  const int head = p.splits > 1 ? p.head : tiles;
  const int tail = tiles - head;
  const dim3 grid(head + tail * p.splits), block(64 * WM * WN);
  auto a = reinterpret_cast<const _Float16*>(A);
  auto s = reinterpret_cast<const _Float16*>(S);
  auto c = reinterpret_cast<_Float16*>(C);
  if constexpr (FMT == kFmtF16) {
    if (epilogue_needed(ep)) {
      hipLaunchKernelGGL((gemm_lds_kernel<MB, NB, WM, WN, NS, true, FMT>), grid, block, 0,
                         stream, a, Bp, s, c, M, K, N, gmagic, p.tiles_n, head, tail, p.splits,
                         counters, partials, ep, Z);
      return hipGetLastError();
    }
  } else {
    if (epilogue_needed(ep)) return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL((gemm_lds_kernel<MB, NB, WM, WN, NS, false, FMT>), grid, block, 0, stream,
                     a, Bp, s, c, M, K, N, gmagic, p.tiles_n, head, tail, p.splits, counters,
                     partials, ep, Z);
  return hipGetLastError();
}

// Compiled variants (MB, NB, WM, WN, NS): the plans' tiles, for the formats
// 0 to 4 (FP16 and BF16 with or without zero points, 8-bit codes).  WM = 1:
// every wave spans the tile's rows; WM > 1: a grid of WM x WN wave tiles.
#define W4A16_LDS_VARIANTS(X) \
  X(1, 2, 1, 8, 4) X(2, 2, 1, 8, 4) X(4, 1, 1, 8, 3) X(8, 2, 1, 8, 3) X(4, 2, 2, 4, 3)

bool lds_is_compiled(int mb, int nb, int wm, int wn, int ns) {
#define W4A16_LMATCH(MB_, NB_, WM_, WN_, NS_) \
  if (mb == MB_ && nb == NB_ && wm == WM_ && wn == WN_ && ns == NS_) return true;
  W4A16_LDS_VARIANTS(W4A16_LMATCH)
#undef W4A16_LMATCH
  return false;
}

// Variants compiled for 2:4-sparse codes: the plans' tiles (with half the
// matrix instructions per activation fragment, 32 < M <= 128 takes four
// waves of 64 x 32 rather than eight of 64 x 16).
#define W4A16_LDS_SP_VARIANTS(X) \
  X(1, 2, 1, 8, 4) X(2, 2, 1, 8, 4) X(8, 2, 1, 8, 3) X(4, 2, 1, 4, 3)

bool lds_sp_is_compiled(int mb, int nb, int wm, int wn, int ns) {
#define W4A16_LSMATCH(MB_, NB_, WM_, WN_, NS_) \
  if (mb == MB_ && nb == NB_ && wm == WM_ && wn == WN_ && ns == NS_) return true;
  W4A16_LDS_SP_VARIANTS(W4A16_LSMATCH)
#undef W4A16_LSMATCH
  return false;
}

// Stages for 8-bit codes, whose code pieces are twice the size: as many of
// the plan's NS as fit in the 160 KiB of LDS (the same tiles, splits and
// workspace; only the pipeline depth differs).
constexpr int w8_stages(int mb, int nb, int wm, int wn, int ns) {
  const int tm = 16 * mb * wm, tn = 16 * nb * wn;
  const int stage = tm * 256 + nb * wn * 2 * 1024 + (tn / 2 + 63) / 64 * 256;
  while (ns > 2 && ns * stage > 160 * 1024) --ns;
  return ns;
}

hipError_t launch_lds(const Plan& p, const uint16_t* A, const uint32_t* Bp,
                      const uint16_t* S, uint16_t* C, int M, int K, int N, uint64_t gmagic,
                      Epilogue ep, WeightFormat wf, void* workspace, hipStream_t stream) {
  if (wf.fmt == kFmtSp24) {
#define W4A16_LSCASE(MB_, NB_, WM_, WN_, NS_)                                                  \
  if (p.mb == MB_ && p.nb == NB_ && p.wm == WM_ && p.wk == WN_ && p.depth == NS_)              \
    return launch_lds_one<MB_, NB_, WM_, WN_, NS_, kFmtSp24>(p, A, Bp, S, C, M, K, N, gmagic, \
                                                             ep, nullptr, workspace, stream);
    W4A16_LDS_SP_VARIANTS(W4A16_LSCASE)
#undef W4A16_LSCASE
    return hipErrorInvalidValue;
  }
#define W4A16_LCASE(MB_, NB_, WM_, WN_, NS_)                                                  \
  if (p.mb == MB_ && p.nb == NB_ && p.wm == WM_ && p.wk == WN_ && p.depth == NS_) {           \
    if (wf.fmt == kFmtF16)                                                                    \
      return launch_lds_one<MB_, NB_, WM_, WN_, NS_, kFmtF16>(p, A, Bp, S, C, M, K, N, gmagic, \
                                                              ep, nullptr, workspace, stream); \
    if (wf.fmt == kFmtF16Zp)                                                                  \
      return launch_lds_one<MB_, NB_, WM_, WN_, NS_, kFmtF16Zp>(                              \
          p, A, Bp, S, C, M, K, N, gmagic, ep, wf.zeros, workspace, stream);                  \
    if (wf.fmt == kFmtBf16)                                                                   \
      return launch_lds_one<MB_, NB_, WM_, WN_, NS_, kFmtBf16>(                               \
          p, A, Bp, S, C, M, K, N, gmagic, ep, nullptr, workspace, stream);                   \
    if (wf.fmt == kFmtBf16Zp)                                                                 \
      return launch_lds_one<MB_, NB_, WM_, WN_, NS_, kFmtBf16Zp>(                             \
          p, A, Bp, S, C, M, K, N, gmagic, ep, wf.zeros, workspace, stream);                  \
    if (wf.fmt == kFmtW8)                                                                     \
      return launch_lds_one<MB_, NB_, WM_, WN_, w8_stages(MB_, NB_, WM_, WN_, NS_), kFmtW8>(  \
          p, A, Bp, S, C, M, K, N, gmagic, ep, nullptr, workspace, stream);                   \
  }
  W4A16_LDS_VARIANTS(W4A16_LCASE)
#undef W4A16_LCASE
  return hipErrorInvalidValue;
}

}  // namespace w4a16
