// Pieces of the LDS-staged GEMM kernel (gemm_lds.hip): address-space casts for the direct global -> LDS load, a
// count-based wait, and the output stage with its split-K hand-off.
#pragma once

#include "coherent.hpp"
#include "epilogue.hpp"
#include "format.hpp"
#include "internal.hpp"

namespace w4a16 {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* global_ptr_t;

// s_waitcnt that waits until at most n vector-memory operations of this
// wave are outstanding (and leaves the other counters alone).  Loads return
// in issue order, so this is "everything but the n most recent".
template <int n>
__device__ __forceinline__ void wait_vmem_at_most() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Keeps the compiler from moving memory operations across this point.  The
// count-based waits assume the loads leave in program order (direct loads
// into LDS and plain loads into registers touch different memory, so
// without it the scheduler may interleave them).
__device__ __forceinline__ void keep_load_order() { asm volatile("" ::: "memory"); }

// The barrier between two K blocks of a pipeline whose stages are filled by
// direct global -> LDS loads: wait until at most n of this wave's loads are
// outstanding and its LDS reads have returned, then meet the other waves.
// __syncthreads() would add a workgroup-scope release fence, and for the
// compiler a release fence has to wait for every direct load still writing
// LDS -- including the stages loaded for later K blocks, which would shrink
// the pipeline to a single K block.  The stages in flight are not ones any
// wave reads before a later barrier, so the count-based wait is all the
// ordering needed.  The empty asm keeps the compiler from moving LDS reads
// or writes across the barrier.
template <int n>
__device__ __forceinline__ void stage_barrier() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (0 << 8) | ((n >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  keep_load_order();
}


typedef _Float16 half4_tc_t __attribute__((ext_vector_type(4)));

// The bias of the columns this lane stores (fused epilogue only), loaded as
// raw FP16 at kernel start so that the load's latency hides behind the main
// loop; it is converted where the output stage uses it.  The count-based
// waits of the pipelines stay correct: this load is older than every stage
// load, and loads complete in order.  With transposed 16 x 16 blocks lane l
// stores columns wcol0 + 16 nb + 4 (l / 16) .. +3 of its NB column blocks:
// one 8-byte vector per block.
template <int NB, bool EPI>
struct LaneBias4 {
  half4_tc_t v[NB];
  __device__ __forceinline__ void load(const Epilogue& ep, int wcol0, int N) {
    if constexpr (EPI) {
      const int c = wcol0 + 4 * (int)((threadIdx.x & 63) >> 4);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        v[nb] = (ep.bias && c + 16 * nb < N)
                    ? *reinterpret_cast<const half4_tc_t*>(ep.bias + c + 16 * nb)
                    : half4_tc_t{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ float at(int nb, int e) const {
    if constexpr (EPI) return (float)v[nb][e];
    return 0.f;
  }
};

// Write a workgroup's output tile.  Each of its WAVES waves owns a
// 16*MB x 16*NB block of it starting at row wrow0, column wcol0; acc[mb][nb]
// holds block (mb, nb) of that wave tile transposed (the weights are the
// matrix instruction's first operand): lane l has row l % 16 and columns
// 4*(l/16) .. +3, stored as one 8-byte vector.
//
// With splits > 1 (slot: the tile's index among the split tiles, for its
// counter and partials): publish the partial tile with device-coherent stores,
// wait for them, count the arrival; the last workgroup of the tile adds the
// partials in split order and writes C.  A partial is kept in fragment
// order -- wave, 16-row block, 16-column block, lane, four values -- so each
// lane moves its four accumulators in one 16-byte access and the workgroup
// that sums finds its own fragments at the same places.  With COLS the
// blocks are not transposed (the activations were the first operand): lane
// l has rows 4*(l/16) .. +3 of column l % 16, stored as four 2-byte values.
// `flag` is an int in
// LDS no wave touches any more.  The epilogue is applied to the final sums
// only; FMT sets the output type (FP16, or BF16 for formats 2 and 3).
template <int MB, int NB, int WAVES, bool EPI, int FMT = kFmtF16, bool COLS = false>
__device__ __forceinline__ void store_output_tile(float4_t (&acc)[MB][NB],
                                                  _Float16* __restrict__ C, int M, int N,
                                                  int wrow0, int wcol0, int split, int splits,
                                                  int slot,
                                                  unsigned* __restrict__ counters,
                                                  float* __restrict__ partials, int* flag,
                                                  const Epilogue& ep,
                                                  const LaneBias4<NB, EPI>& bias) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  auto write_c = [&]() {
    if constexpr (COLS) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int gc = wcol0 + nb * 16 + (lane & 15);
        if (gc >= N) continue;
        const float b = (EPI && ep.bias) ? (float)ep.bias[gc] : 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int gr = wrow0 + mb * 16 + (lane >> 4) * 4 + e;
            const float x = acc[mb][nb][e];
            if (gr < M) C[(int64_t)gr * N + gc] = out16<FMT>(EPI ? epilogue_apply(ep, x, b) : x);
          }
      }
      return;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int gr = wrow0 + mb * 16 + (lane & 15);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        // N is a multiple of 16: four columns from a multiple of 4 fit
        const int gc = wcol0 + nb * 16 + (lane >> 4) * 4;
        if (gr < M && gc < N) {
          half4_tc_t h;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = acc[mb][nb][e];
            h[e] = out16<FMT>(EPI ? epilogue_apply(ep, x, bias.at(nb, e)) : x);
          }
          *reinterpret_cast<half4_tc_t*>(C + (int64_t)gr * N + gc) = h;
        }
      }
    }
  };
  if (splits == 1) {
    write_c();
    return;
  }

  constexpr int TE = WAVES * MB * NB * 256;  // elements of the tile
  const float* tile_base = partials + (int64_t)slot * splits * TE;
  const int frag0 = wave * MB * NB * 64 + lane;
  {
    const __amdgpu_buffer_rsrc_t mine = coherent_rsrc(tile_base + (int64_t)split * TE);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) store_coherent(mine, frag0 + (mb * NB + nb) * 64, acc[mb][nb]);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(counters + slot, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = prev == (unsigned)(splits - 1);
  }
  __syncthreads();
  if (!*flag) return;

  // Sum in split order 0, 1, ... into the (now free) accumulators.
  for (int s = 0; s < splits; ++s) {
    const __amdgpu_buffer_rsrc_t ps = coherent_rsrc(tile_base + (int64_t)s * TE);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float4_t x = load_coherent(ps, frag0 + (mb * NB + nb) * 64);
        acc[mb][nb] = s == 0 ? x : acc[mb][nb] + x;
      }
  }
  write_c();
  if (threadIdx.x == 0)
    __hip_atomic_store(counters + slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


}  // namespace w4a16
