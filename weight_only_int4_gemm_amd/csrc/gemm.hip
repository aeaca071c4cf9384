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
//  * with splits > 1 each workgroup stores its FP32 partial tile in the
//    workspace, and the last of a tile's workgroups to arrive (an atomic
//    counter per tile) adds the partials in split order 0, 1, ..., writes
//    the FP16 tile and sets the counter back to zero.  The order of every
//    addition is fixed, so results are bit-identical from run to run.
//
// Per 128-deep K block a wave issues, for each of its NB column blocks, one
// 16-byte load per lane of permuted codes (the lane's own operand fragments
// for four 32-deep steps) and one scale load; it unpacks each word in
// registers (unpack.hpp) and issues 16x16x32 FP16 matrix instructions against
// activation fragments read straight from global memory (16 bytes per lane
// per 16-row block and 32-deep step).
#include "internal.hpp"
#include "layout.hpp"
#include "unpack.hpp"

namespace w4a16 {

typedef float float4_t __attribute__((ext_vector_type(4)));

template <int MB, int NB, int WK>
__global__ __launch_bounds__(64 * WK) void gemm_kernel(
    const _Float16* __restrict__ A, const uint32_t* __restrict__ Bp,
    const _Float16* __restrict__ S, _Float16* __restrict__ C, int M, int K, int N,
    int group, int splits, unsigned* __restrict__ counters,
    float* __restrict__ partials) {
  constexpr int TM = 16 * MB;
  constexpr int TN = 16 * NB;
  constexpr int LDT = TN + 4;  // padded LDS row (floats), keeps 16-byte alignment
  __shared__ float red[TM * LDT];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tile_n = blockIdx.x;
  const int tile_m = blockIdx.y;
  const int split = blockIdx.z;
  const int KB = K / kBlockK;
  const int N16 = N / kBlockN;
  const int kb0 = (int)((int64_t)KB * split / splits);
  const int kb1 = (int)((int64_t)KB * (split + 1) / splits);
  const int l16 = lane & 15;
  const int lk = (lane >> 4) * 8;

  float4_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = float4_t{0.f, 0.f, 0.f, 0.f};

  // Activation rows of this lane (row l16 of each 16-row block); rows >= M
  // are never read and contribute zeros.
  const _Float16* arow[MB];
  bool aok[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = tile_m * TM + mb * 16 + l16;
    aok[mb] = r < M;
    arow[mb] = A + (int64_t)(aok[mb] ? r : 0) * K + lk;
  }
  // Column blocks of this wave; blocks past N (ragged N) are skipped.
  const uint32_t* bcol[NB];
  const _Float16* scol[NB];
  bool bok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n16 = tile_n * NB + nb;
    bok[nb] = n16 < N16;
    bcol[nb] = Bp + block_word_offset(bok[nb] ? n16 : 0, 0, K) + lane * kWordsPerLane;
    scol[nb] = S + (bok[nb] ? n16 * kBlockN + l16 : 0);
  }

  for (int kb = kb0 + wave; kb < kb1; kb += WK) {
    uint4 bw[NB];
    half2_t s2[NB];
    const int64_t srow = (int64_t)(kb * kBlockK / group) * N;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (bok[nb]) {
        bw[nb] = *reinterpret_cast<const uint4*>(bcol[nb] + (int64_t)kb * kWordsPerBlock);
        const _Float16 s = scol[nb][srow];
        s2[nb] = half2_t{s, s};
      } else {
        bw[nb] = uint4{0u, 0u, 0u, 0u};
        s2[nb] = half2_t{(_Float16)0.f, (_Float16)0.f};
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half8_t a[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if (aok[mb]) {
          a[mb] = *reinterpret_cast<const half8_t*>(arow[mb] + kb * kBlockK + 32 * j);
        } else {
          a[mb] = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (!bok[nb]) continue;
        const uint32_t w = j == 0 ? bw[nb].x : j == 1 ? bw[nb].y : j == 2 ? bw[nb].z : bw[nb].w;
        const half8_t b = unpack_scale(w, s2[nb]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mb], b, acc[mb][nb], 0, 0, 0);
        }
      }
    }
  }

  // Sum the waves' tiles in LDS, wave 0 first.  Lane l holds rows
  // 4*(l/16) .. +3 of column l % 16 of each 16x16 block.
#pragma unroll 1
  for (int w = 0; w < WK; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float* p = &red[(mb * 16 + (lane >> 4) * 4 + i) * LDT + nb * 16 + l16];
            *p = (w == 0) ? acc[mb][nb][i] : *p + acc[mb][nb][i];
          }
    }
    __syncthreads();
  }

  constexpr int VEC = 4;
  constexpr int VPR = TN / VEC;  // float4 vectors per tile row
  const int row0 = tile_m * TM;
  const int col0 = tile_n * TN;

  if (splits == 1) {
    for (int v = threadIdx.x; v < TM * VPR; v += blockDim.x) {
      const int r = v / VPR, c = (v % VPR) * VEC;
      const int gr = row0 + r, gc = col0 + c;
      if (gr < M && gc < N) {
        const float4_t x = *reinterpret_cast<const float4_t*>(&red[r * LDT + c]);
        typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
        const half4_t h = {(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
        *reinterpret_cast<half4_t*>(C + (int64_t)gr * N + gc) = h;
      }
    }
    return;
  }

  // Split-K: publish this workgroup's partial tile, then count arrivals.
  const int tile = tile_m * gridDim.x + tile_n;
  constexpr int TE = TM * TN;
  float* mine = partials + ((int64_t)tile * splits + split) * TE;
  for (int v = threadIdx.x; v < TM * VPR; v += blockDim.x) {
    const int r = v / VPR, c = (v % VPR) * VEC;
    *reinterpret_cast<float4_t*>(mine + r * TN + c) =
        *reinterpret_cast<const float4_t*>(&red[r * LDT + c]);
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counters + tile, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(splits - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  const float* base = partials + (int64_t)tile * splits * TE;
  for (int v = threadIdx.x; v < TM * VPR; v += blockDim.x) {
    const int r = v / VPR, c = (v % VPR) * VEC;
    const int gr = row0 + r, gc = col0 + c;
    if (gr < M && gc < N) {
      float4_t x = *reinterpret_cast<const float4_t*>(base + r * TN + c);
      for (int s = 1; s < splits; ++s) {
        x += *reinterpret_cast<const float4_t*>(base + (int64_t)s * TE + r * TN + c);
      }
      typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
      const half4_t h = {(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
      *reinterpret_cast<half4_t*>(C + (int64_t)gr * N + gc) = h;
    }
  }
  if (threadIdx.x == 0) counters[tile] = 0u;  // ready for the next call
}

template <int MB, int NB, int WK>
static hipError_t launch_one(const Plan& p, const uint16_t* A, const uint32_t* Bp,
                             const uint16_t* S, uint16_t* C, int M, int K, int N,
                             int group, void* workspace, hipStream_t stream) {
  unsigned* counters = nullptr;
  float* partials = nullptr;
  if (p.splits > 1) {
    counters = static_cast<unsigned*>(workspace);
    partials = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        counters_bytes(p.tiles_n * p.tiles_m));
  }
  hipLaunchKernelGGL((gemm_kernel<MB, NB, WK>), dim3(p.tiles_n, p.tiles_m, p.splits),
                     dim3(64 * WK), 0, stream, reinterpret_cast<const _Float16*>(A), Bp,
                     reinterpret_cast<const _Float16*>(S), reinterpret_cast<_Float16*>(C),
                     M, K, N, group, p.splits, counters, partials);
  return hipGetLastError();
}

bool plan_is_compiled(int mb, int nb, int wk) {
  return nb == 4 && wk == 4 && (mb == 1 || mb == 2 || mb == 4 || mb == 8);
}

hipError_t launch_gemm(const Plan& p, const uint16_t* A, const uint32_t* Bp,
                       const uint16_t* S, uint16_t* C, int M, int K, int N, int group,
                       void* workspace, hipStream_t stream) {
#define W4A16_CASE(MB_, NB_, WK_)                                                   \
  if (p.mb == MB_ && p.nb == NB_ && p.wk == WK_)                                    \
    return launch_one<MB_, NB_, WK_>(p, A, Bp, S, C, M, K, N, group, workspace, stream);
  W4A16_CASE(1, 4, 4)
  W4A16_CASE(2, 4, 4)
  W4A16_CASE(4, 4, 4)
  W4A16_CASE(8, 4, 4)
#undef W4A16_CASE
  return hipErrorInvalidValue;
}

}  // namespace w4a16
