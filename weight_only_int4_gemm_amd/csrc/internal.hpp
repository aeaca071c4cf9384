// Declarations shared by the library's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

// How one w4a16_gemm call is cut into work.
//  tile   0: the streaming kernel (small batches), 2: the LDS kernel
//         (every operand through LDS stages), 4: the stream-K kernel
//         (gemm_sk.hpp: wk waves of 16*mb x 16*nb, `splits` workgroups each
//         running an equal share of the (tile, K block) iterations)
//  mb     16-row blocks per wave (the workgroup's M tile is 16 * mb * wm)
//  nb     16-column blocks per wave
//  wk     waves per workgroup (LDS and stream-K kernels: waves along N).
//         Streaming kernel: they split the workgroup's K range (every wk-th
//         128-deep K block each) and their sums are added in wave order
//         through LDS; the N tile is 16 * nb.  LDS and stream-K kernels:
//         they split the N tile, which is 16 * nb * wk.
//  wm     LDS kernel: waves along M (1 elsewhere); the workgroup has
//         wm * wk waves
//  splits K ranges per output tile, one workgroup each; their FP32
//         partials go through the workspace and are added in split order
//         (stream-K kernel: the number of workgroups)
//  depth  streaming kernel: K blocks each wave keeps in flight; LDS and
//         stream-K kernels: stages of activations, codes and scales
struct Plan {
  int tile, mb, nb, wk, splits, depth, wm;
  int tm, tn;              // output tile of one workgroup
  int tiles_n, tiles_m;
  int head;                // LDS kernel with splits > 1: tiles run whole before the
                           // split ones (0: every tile is split)
  size_t workspace_bytes;  // 0 when splits == 1
};

// The operation the output stage applies to each FP32 sum before its one
// rounding to FP16: y = act(x + bias[col]).  bias null: no bias; act is a
// value of enum w4a16_activation.  Plain w4a16_gemm passes {nullptr, 0}.
struct Epilogue {
  const _Float16* bias;
  int act;
};

// The weight format of a call (format.hpp): 0 FP16, 1 FP16 with zero
// points, 2 BF16, 3 BF16 with zero points, 4 FP16 with 8-bit weights, 5 FP16
// with 2:4-sparse 4-bit weights;
// `zeros` are the zero points uint8[K/group][N] of formats 1 and 3 (null
// otherwise).
struct WeightFormat {
  int fmt;
  const uint8_t* zeros;
};

Plan make_plan(int M, int K, int N, int group, int cus, int fmt = 0);

// The streaming kernel with activations in LDS (gemm.hip): batches of at
// most kAldsMaxRows rows whose rows over one workgroup's K range take at
// most kAldsMaxBytes, in the FP16-activation formats (0, 1 and 4).  activations_lds_bytes: the LDS the launch of plan p
// gives them, 0 when the call reads its activations from global memory.
constexpr int kAldsMaxRows = 4;
constexpr size_t kAldsMaxBytes = 32768;
size_t activations_lds_bytes(const Plan& p, int M, int K, int fmt);
bool plan_is_compiled(int mb, int nb, int wk, int depth, int fmt);
bool sp_is_compiled(int mb, int nb, int wk, int depth);
bool lds_is_compiled(int mb, int nb, int wm, int wn, int ns);
bool lds_sp_is_compiled(int mb, int nb, int wm, int wn, int ns);
bool sk_is_compiled(int mb, int nb, int ns, int wm, int wn);
size_t sk_workspace_bytes(int wgs, int tm, int tn, int tiles, int KB, int ns);

hipError_t launch_repack(const uint32_t* Bq, uint32_t* Bp, int K, int N,
                         hipStream_t stream);
hipError_t launch_repack8(const uint32_t* Bq, uint32_t* Bp, int K, int N,
                          hipStream_t stream);
hipError_t launch_repack_sp24(const uint32_t* Bq, const uint8_t* mask, uint32_t* Bp, int K,
                              int N, hipStream_t stream);
hipError_t launch_dequant(const uint32_t* Bp, const uint16_t* S, uint16_t* W,
                          int K, int N, int group, hipStream_t stream);
hipError_t launch_lds(const Plan& p, const uint16_t* A, const uint32_t* Bp,
                      const uint16_t* S, uint16_t* C, int M, int K, int N, uint64_t gmagic,
                      Epilogue ep, WeightFormat wf, void* workspace, hipStream_t stream);
hipError_t launch_sk(const Plan& p, const uint16_t* A, const uint32_t* Bp, const uint16_t* S,
                     uint16_t* C, int M, int K, int N, uint64_t gmagic, Epilogue ep,
                     WeightFormat wf, void* workspace, hipStream_t stream);
hipError_t launch_gemm(const Plan& plan, const uint16_t* A, const uint32_t* Bp,
                       const uint16_t* S, uint16_t* C, int M, int K, int N,
                       int group, Epilogue ep, WeightFormat wf, void* workspace,
                       hipStream_t stream);
hipError_t launch_dequant_fmt(const uint32_t* Bp, const uint16_t* S, const uint8_t* Z,
                              uint16_t* W, int K, int N, int group, int fmt,
                              hipStream_t stream);

// Workspace layout for a plan with splits > 1: a fixed header of
// kMaxSplitTiles 32-bit arrival counters (one per output tile; 64 KiB
// whatever the shape), then the FP32 partial tiles
// [tile][split][tile rows][tile cols].  The header's size does not depend on
// the call, so the counters of one call never sit where an earlier call of
// another shape left partial sums: every call leaves the counters it used at
// zero, and a workspace zero-filled once serves calls of any shape in turn.
// Plans split K only when the output has at most kMaxSplitTiles tiles.
constexpr int kMaxSplitTiles = 16384;
// The stream-K kernel: the fewest iterations a workgroup is given.
constexpr int kSkMinIters = 8;
constexpr size_t kCounterHeaderBytes = (size_t)kMaxSplitTiles * sizeof(unsigned);

}  // namespace w4a16
