// A W4A16 GEMM for larger batches (forced plans only): C = A . dequant(Bpacked).
//
// Once a batch has dozens of rows the matrix instructions, not the weight
// stream, set the pace ("Quant Marlin kernel" explainer, "Why architecture
// matters here": with batching the same weights are reused and the kernel
// becomes compute-bound; "Low-Precision Quantization Kernels in Production",
// section 5, "Decoding Roofline Dynamics").  Two costs then matter:
// unpacking each weight as few times as possible, and feeding the matrix
// instructions their activation operands without saturating the caches.
//
// Work decomposition:
//  * a workgroup of WN waves owns an output tile of 16*MB rows by
//    16*NB*WN columns and one K range (grid.z splits K as in the streaming
//    kernel, with the same deterministic last-arriver reduction);
//  * each wave owns 16*NB columns and all 16*MB rows of the tile, so every
//    weight is loaded and unpacked exactly once per workgroup; its codes
//    come straight from global memory into registers (the permuted layout
//    hands each lane its own fragments), four K blocks ahead;
//  * the tile's activations for a 128-deep K block sit in LDS and are read
//    by every wave.  They are copied global -> LDS by the direct 16-byte
//    load of gfx950 (no staging registers), into one of two stages while
//    the other is being read ("Quant Marlin kernel" explainer, "End-to-end
//    flow": the next tile's loads go into the other half of a double buffer
//    before the first one is consumed).  Each 256-byte row of a stage holds
//    its sixteen 16-byte pieces in a row-dependent order (piece c of row r
//    at slot c ^ (r & 15)), so the sixteen rows a wave reads in one fragment
//    load fall in distinct banks.
#include "layout.hpp"
#include "tile_common.hpp"
#include "unpack.hpp"

namespace w4a16 {

namespace {

template <int NB>
struct BSlot {
  uint4 b[NB];
  // The scale's bits as loaded, one per register; they are broadcast to
  // both halves only where they are used, so no instruction right after the
  // load has to wait for it (that wait would drain every load in flight,
  // loads completing in order).
  uint32_t s[NB];
};

}  // namespace

template <int MB, int NB, int WN, int NS, int DB, bool EPI>
__global__ __launch_bounds__(64 * WN) void gemm_tile_kernel(
    const _Float16* __restrict__ A, const uint32_t* __restrict__ Bp,
    const _Float16* __restrict__ S, _Float16* __restrict__ C, int M, int K, int N,
    uint64_t group_magic, int splits, unsigned* __restrict__ counters,
    float* __restrict__ partials, Epilogue ep) {
  constexpr int TM = 16 * MB;
  constexpr int TN = 16 * NB * WN;
  constexpr int PIECES = TM * 16;          // 16-byte pieces of one activation stage
  constexpr int LOADS = PIECES / 64 / WN;  // direct loads per wave per stage
  static_assert(PIECES % (64 * WN) == 0, "stage must split evenly over the waves");
  constexpr int BLOADS = 2 * NB;           // code + scale loads per wave per K block
  static_assert(NS == 2 || NS == 4, "two or four activation stages");
  // Separate LDS objects (rather than one array) let the compiler see that
  // a direct load into one stage does not touch the others.
  __shared__ uint4 As0[PIECES];
  __shared__ uint4 As1[PIECES];
  __shared__ uint4 As2[NS > 2 ? PIECES : 1];
  __shared__ uint4 As3[NS > 2 ? PIECES : 1];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile_n = blockIdx.x;
  const int tile_m = blockIdx.y;
  const int split = blockIdx.z;
  const int KB = K / kBlockK;
  const int kb0 = (int)((int64_t)KB * split / splits);
  const int kb1 = (int)((int64_t)KB * (split + 1) / splits);
  const int l16 = lane & 15;
  const int row0 = tile_m * TM;
  const int n16_last = N / kBlockN - 1;
  const int n16_0 = tile_n * NB * WN + wave * NB;
  LaneBias<NB, 16, EPI> bias;
  bias.load(ep, tile_n * TN + wave * 16 * NB, N);

  // Direct load i of this wave fills stage pieces 64 * (wave + WN * i) + lane:
  // row r = 4 * (wave + WN * i) + lane / 16, slot lane % 16, which holds
  // piece (lane % 16) ^ (r & 15) of that row.  Rows past M read row M - 1
  // (their sums are never stored).
  auto load_a = [&](uint4* stage, int kb) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int r = 4 * (wave + WN * i) + (lane >> 4);
      const int piece = l16 ^ (r & 15);
      const int gr = row0 + r < M ? row0 + r : M - 1;
      const _Float16* src = A + (int64_t)gr * K + kb * kBlockK + piece * 8;
      __builtin_amdgcn_global_load_lds((global_ptr_t)src,
                                       (lds_ptr_t)&stage[64 * (wave + WN * i)], 16, 0, 0);
    }
  };
  const uint32_t* bcol[NB];
  const _Float16* scol[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    // blocks past N recompute the last valid one and are dropped at the store
    const int n16 = n16_0 + nb <= n16_last ? n16_0 + nb : n16_last;
    bcol[nb] = Bp + block_word_offset(n16, 0, K) + lane * kWordsPerLane;
    scol[nb] = S + n16 * kBlockN + l16;
  }
  // Scale row of K block kb: kb / (group / 128), as a multiply-high by
  // group_magic = ceil(2^32 / (group / 128)); no branch in the K loop.
  auto scale_row = [&](int kb) -> int {
    return (int)(((uint64_t)(uint32_t)kb * group_magic) >> 32);
  };
  auto load_b = [&](BSlot<NB>& sl, int kb) {
    const int srow = scale_row(kb) * N;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      sl.b[nb] = *reinterpret_cast<const uint4*>(bcol[nb] + kb * kWordsPerBlock);
      sl.s[nb] = reinterpret_cast<const uint16_t*>(scol[nb])[srow];
    }
  };

  float4_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = float4_t{0.f, 0.f, 0.f, 0.f};

  // One K block, four 32-deep steps.  The activation fragments of step j+1
  // are read from LDS before the matrix instructions of step j are issued,
  // so LDS latency hides behind them; the codes of step j are unpacked
  // just before they are used.
  auto read_a = [&](const uint4* stage, int j, half8_t* a) {
    const int lg = lane >> 4;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = mb * 16 + l16;
      a[mb] = __builtin_bit_cast(half8_t, stage[r * 16 + ((4 * j + lg) ^ (r & 15))]);
    }
  };
  auto compute = [&](const uint4* stage, const BSlot<NB>& sl) {
    half8_t a0[MB], a1[MB];
    read_a(stage, 0, a0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half8_t* cur = (j & 1) ? a1 : a0;
      half8_t* nxt = (j & 1) ? a0 : a1;
      if (j < 3) read_a(stage, j + 1, nxt);
      half8_t bf[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t w = j == 0 ? sl.b[nb].x : j == 1 ? sl.b[nb].y
                         : j == 2 ? sl.b[nb].z : sl.b[nb].w;
        const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)sl.s[nb]);
        bf[nb] = unpack_scale(w, half2_t{sc, sc});
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur[mb], bf[nb], acc[mb][nb], 0, 0, 0);
    }
  };

  // The pipeline.  Step t consumes K block kb0 + t from activation stage
  // t % NS and code slot t % DB.  Step s issues, in this order, the
  // activations of block s + NS - 1 (into the stage that block s - 1 used,
  // which every wave has finished with once it passed this step's barrier)
  // and the codes of block s + DB (into the slot step s has just consumed);
  // the prologue issues what steps -DB .. -1 would have.  So when step t
  // waits, the loads allowed to be still in flight are exactly the
  // activations of blocks t+1 .. t+NS-2 and the NS - 1 code loads issued
  // after A(t): the codes come from HBM DB blocks ahead, the activations
  // from L2 NS - 1 blocks ahead, and one barrier per step does.  Loads past
  // the range are clamped to the last block (harmless re-reads into stages
  // or slots that are never consumed again).
  static_assert(DB == 4 || DB == 8, "four or eight code slots");
  const int nblk = kb1 - kb0;  // >= 1: splits never exceed the K blocks
  const int last = kb1 - 1;
  auto clamp = [&](int kb) { return kb <= last ? kb : last; };
  uint4* const stages[4] = {As0, As1, NS > 2 ? As2 : As0, NS > 2 ? As3 : As1};
  BSlot<NB> slots[DB];
#pragma unroll
  for (int s = -DB; s < 0; ++s) {
    if (s + NS - 1 >= 0) load_a(stages[(s + NS - 1) % NS], clamp(kb0 + s + NS - 1));
    keep_load_order();
    load_b(slots[s + DB], clamp(kb0 + s + DB));
    keep_load_order();
  }
  constexpr int IN_FLIGHT = (NS - 2) * LOADS + (NS - 1) * BLOADS;

  auto step = [&](int u, int kb) {  // u = t % DB
    stage_barrier<IN_FLIGHT>();  // this block's stage has landed; block kb - 1's is free
    load_a(stages[(u + NS - 1) % NS], clamp(kb + NS - 1));
    keep_load_order();
    compute(stages[u % NS], slots[u]);
    load_b(slots[u], clamp(kb + DB));
  };
  int t = 0;
  for (; t + DB <= nblk; t += DB) {
#pragma unroll
    for (int u = 0; u < DB; ++u) step(u, kb0 + t + u);
  }
  // The last, partial round (fewer than DB blocks left).
#pragma unroll
  for (int u = 0; u < DB - 1; ++u) {
    if (t + u < nblk) step(u, kb0 + t + u);
  }
  // No direct load may still be landing in LDS when the stages are reused
  // below or the workgroup ends.
  __builtin_amdgcn_s_waitcnt(0);

  store_output_tile<MB, NB, WN, EPI>(acc, C, M, N, row0, tile_n * TN + wave * 16 * NB, split,
                                     splits, counters,
                                partials, reinterpret_cast<int*>(&As0[0]), ep, bias);
}

template <int MB, int NB, int WN, int NS, int DB>
static hipError_t launch_tile_one(const Plan& p, const uint16_t* A, const uint32_t* Bp,
                                  const uint16_t* S, uint16_t* C, int M, int K, int N,
                                  uint64_t gmagic, Epilogue ep, void* workspace,
                                  hipStream_t stream) {
  unsigned* counters = nullptr;
  float* partials = nullptr;
  if (p.splits > 1) {
    counters = static_cast<unsigned*>(workspace);
    partials = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        counters_bytes(p.tiles_n * p.tiles_m));
  }
  const dim3 grid(p.tiles_n, p.tiles_m, p.splits), block(64 * WN);
  auto a = reinterpret_cast<const _Float16*>(A);
  auto s = reinterpret_cast<const _Float16*>(S);
  auto c = reinterpret_cast<_Float16*>(C);
  if (epilogue_needed(ep))
    hipLaunchKernelGGL((gemm_tile_kernel<MB, NB, WN, NS, DB, true>), grid, block, 0, stream, a,
                       Bp, s, c, M, K, N, gmagic, p.splits, counters, partials, ep);
  else
    hipLaunchKernelGGL((gemm_tile_kernel<MB, NB, WN, NS, DB, false>), grid, block, 0, stream, a,
                       Bp, s, c, M, K, N, gmagic, p.splits, counters, partials, ep);
  return hipGetLastError();
}

// Compiled tile variants (MB, NB, WN, NS, DB).
#define W4A16_TILE_VARIANTS(X)                                                      \
  X(4, 2, 2, 4, 4) X(4, 2, 4, 2, 4) X(4, 2, 4, 2, 8) X(4, 2, 4, 4, 4) X(4, 2, 4, 4, 8) \
  X(4, 4, 2, 4, 4) X(4, 4, 4, 4, 4) X(8, 1, 4, 2, 4) X(8, 1, 4, 2, 8) X(8, 2, 2, 2, 4) \
  X(8, 2, 4, 2, 4) X(8, 4, 2, 2, 4) X(8, 4, 4, 2, 4) X(8, 4, 4, 4, 4)

bool tile_is_compiled(int mb, int nb, int wn, int ns, int db) {
#define W4A16_TMATCH(MB_, NB_, WN_, NS_, DB_) \
  if (mb == MB_ && nb == NB_ && wn == WN_ && ns == NS_ && db == DB_) return true;
  W4A16_TILE_VARIANTS(W4A16_TMATCH)
#undef W4A16_TMATCH
  return false;
}

hipError_t launch_tile(const Plan& p, const uint16_t* A, const uint32_t* Bp,
                       const uint16_t* S, uint16_t* C, int M, int K, int N,
                       uint64_t gmagic, Epilogue ep, void* workspace, hipStream_t stream) {
#define W4A16_TCASE(MB_, NB_, WN_, NS_, DB_)                                            \
  if (p.mb == MB_ && p.nb == NB_ && p.wk == WN_ && p.depth == NS_ && p.bdepth == DB_)   \
    return launch_tile_one<MB_, NB_, WN_, NS_, DB_>(p, A, Bp, S, C, M, K, N, gmagic,    \
                                                    ep, workspace, stream);
  W4A16_TILE_VARIANTS(W4A16_TCASE)
#undef W4A16_TCASE
  return hipErrorInvalidValue;
}

}  // namespace w4a16
