// Streaming-read ceiling of the device, for the benchmark: the rate plain
// 16-byte nontemporal loads reach over a buffer larger than L2 and the
// Infinity Cache. A bandwidth-bound kernel reports its rate against the
// datasheet peak (8 TB/s on MI355X) and, beside it, against this practical
// bound measured on the same box. Not part of the attention library: it
// builds into its own shared object, which only bench.py loads.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fi_bench.h"

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves per work-group
constexpr int kUnroll = 8;     // independent 16-byte loads in flight per lane
constexpr int kGroups = 1024;  // 4 work-groups (16 waves) per CU on 256 CUs

// Work-group g reads tiles g, g + G, g + 2G, ... (G = grid size) of
// kThreads x kUnroll 16-byte words each, contiguous: lane t takes words
// tile * kThreads * kUnroll + j * kThreads + t for j < kUnroll, so every wave
// instruction covers 1 KiB and a work-group's loads of one tile cover 32 KiB
// in a row. The words are folded with XOR; a lane whose fold hits one
// arbitrary constant writes it to *sink, so no load can be dropped. A tail
// shorter than one tile is read word by word.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4_t* __restrict__ p,
                                                               int64_t n16, uint32_t* sink) {
  constexpr int64_t kTile = (int64_t)kThreads * kUnroll;
  const int64_t ntiles = n16 / kTile;
  uint32_t acc = 0;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const u32x4_t* b = p + tile * kTile + threadIdx.x;
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(b + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int64_t i = ntiles * kTile + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kThreads) {
    const u32x4_t v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) *sink = acc;
}

}  // namespace

extern "C" int fi_bench_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3(kGroups), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(buf),
                     (int64_t)(bytes / 16), sink);
  return (int)hipGetLastError();
}
