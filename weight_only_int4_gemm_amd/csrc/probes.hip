// Measurement probes (libw4a16_probes.so, include/w4a16_probes.h): what
// this chip sustains on the two resources that bound the W4A16 GEMM, to be
// reported beside the published peaks.
//  * w4a16_probe_read: a plain read of a device buffer with 16-byte
//    non-temporal loads, every byte once -- the HBM rate a weight stream
//    can reach.
//  * w4a16_probe_mfma: sixteen independent v_mfma_f32_16x16x32_f16 chains on
//    register operands in every wave of a full grid -- the FP16 matrix rate
//    with no memory traffic.
// Neither is part of the GEMM; bench.py times them with HIP events.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/w4a16_probes.h"

namespace {

typedef unsigned uint4_vt __attribute__((ext_vector_type(4)));
typedef _Float16 half8_vt __attribute__((ext_vector_type(8)));
typedef float float4_vt __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 512;
constexpr int kReadUnroll = 8;

// Each thread reads kReadUnroll 16-byte pieces per round, strided by the
// grid, and folds them into one word; the word is stored only if it equals
// a value no input is built to produce, so the loads stay live and the
// output traffic is nil.
__global__ __launch_bounds__(kReadThreads) void read_kernel(const uint4_vt* __restrict__ buf,
                                                            size_t pieces,
                                                            uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * stride < pieces; i += kReadUnroll * stride) {
    uint4_vt v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < pieces; i += stride) {
    const uint4_vt v = __builtin_nontemporal_load(buf + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

constexpr int kMfmaChains = 16;

// kMfmaChains independent accumulators per wave (enough to cover the
// instruction's latency), `iters` rounds; operands are built from the lane
// index so the compiler cannot fold them.
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* __restrict__ sink) {
  half8_vt a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(float)((threadIdx.x + i) & 7);
    b[i] = (_Float16)(float)((threadIdx.x * 3 + i) & 7);
  }
  // The first round starts from an inline zero accumulator: a zero-filled
  // array carried into the loop would have the compiler copy the
  // accumulators between registers on every trip.
  float4_vt acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, float4_vt{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  for (int it = 1; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) t += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (t == -1.f) sink[0] = t;
}

}  // namespace

extern "C" {

int w4a16_probe_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, void* stream) {
  if (!buf || !sink || bytes < 16 || (bytes & 15) || blocks <= 0) return -1;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return -1;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kReadThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4_vt*>(buf),
                     bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

double w4a16_probe_mfma_flops(int blocks, int iters) {
  // 4 waves per block, kMfmaChains instructions per round, 16*16*32*2 flops each
  return (double)blocks * 4 * iters * kMfmaChains * 16.0 * 16.0 * 32.0 * 2.0;
}

int w4a16_probe_mfma(float* sink, int blocks, int iters, void* stream) {
  if (!sink || blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
