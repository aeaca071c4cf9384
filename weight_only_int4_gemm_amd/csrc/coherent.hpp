// Device-coherent 16-byte stores and loads for the split-K hand-off.
//
// The workgroups of one output tile may run behind different XCDs, whose L2
// caches are not kept coherent with each other.  Their FP32 partials are
// therefore written with the device-scope cache policy (the store writes
// through to the device coherence point) and read back with it (the load
// does not trust a possibly stale L2 line).  A device-wide fence would do
// the same by writing back and invalidating the whole L2 of the XCD, which,
// done by hundreds of workgroups in flight, throws away the weights and
// activations the other workgroups are streaming.
//
// The accesses go through a raw buffer resource on the partials' base
// address (16-byte element offsets), so they are ordinary vector memory
// operations the compiler counts and waits for.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned uint4_vt __attribute__((ext_vector_type(4)));

// Cache-policy operand of the buffer intrinsics: device scope.
constexpr int kDeviceScope = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const float* base) {
  // raw (stride 0) resource over up to 2 GiB from base
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}

// Store v at base[4 * idx .. 4 * idx + 3].
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, int idx, float4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint4_vt, v), r, idx * 16, 0,
                                         kDeviceScope);
}

// Load base[4 * idx .. 4 * idx + 3].
__device__ __forceinline__ float4_t load_coherent(__amdgpu_buffer_rsrc_t r, int idx) {
  return __builtin_bit_cast(float4_t,
                            __builtin_amdgcn_raw_buffer_load_b128(r, idx * 16, 0, kDeviceScope));
}

}  // namespace w4a16
