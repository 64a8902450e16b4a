// Device-coherent accesses for the partial states that a tile kernel's
// work-groups hand to the work-group that merges them, which may run on
// another XCD: the XCDs' L2 caches are private, so these stores write
// through to the device-coherent level and these loads read from it (cache
// policy sc1, what the compiler emits for relaxed agent-scope atomics), with
// no cache flush. The merging side reads a wave's block of a partial state
// through a buffer resource, so that its many loads share one lane-offset
// register and a scalar offset each.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fi {

typedef unsigned int coh_u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent2(float* p, float a, float b) {
  const uint64_t u = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// `bytes` bytes from `base` as a raw buffer resource (in scalar registers
// when base is uniform); 0x20000 is the 32-bit data format every untyped
// access of gfx9 needs.
typedef __amdgpu_buffer_rsrc_t BufRes;
__device__ __forceinline__ BufRes buffer_of(const float* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, bytes, 0x00020000);
}
// 8 bytes at lane_off (a vector register) + run_off (uniform: a scalar
// register or constant), read from the coherent level
__device__ __forceinline__ coh_u32x2_t load_coherent_run(BufRes r, uint32_t lane_off, int run_off) {
  constexpr int kSc1 = 16;  // cache policy bit sc1
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)lane_off, run_off, kSc1);
}

}  // namespace fi
