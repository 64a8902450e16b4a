// Merging attention states over disjoint token sets, for gfx950.
//
// The load-balanced scheduler of the FlashInfer paper explainer ("FlashInfer:
// Block-Sparse KV 캐시로 어텐션 병목을 해소하다", visionhong.com, benchmark
// section) cuts one request's softmax into several work units. Each unit
// leaves a state (v, s): v = its softmax-weighted average of V rows, s = the
// log of its softmax denominator. Softmax over the union of the units' token
// sets is the closed form
//     s = M + log sum_i e^(s_i - M),   v = sum_i e^(s_i - M) v_i / sum_i e^(s_i - M)
// with M = max_i s_i; an empty set has s = -inf and weight zero.
//
// merge_two_kernel is the standalone elementwise merge of two state arrays
// (natural-log LSE); each thread handles one 16-byte column of a row. (The
// decode, prefill and latent-attention runs merge their own partial states
// inside their kernels.)
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fi_bsr.h"
#include "kernels.h"

namespace fi {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// Elementwise merge of two state arrays. Thread = one 16-byte column of a row.
template <bool kBF16, int D>
__global__ __launch_bounds__(256) void merge_two_kernel(MergeTwoArgs a) {
  constexpr int kEB = kBF16 ? 2 : 4;
  constexpr int kCols = D * kEB / 16;  // 16-byte columns per row
  const int64_t total = a.num_rows * kCols;
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total;
       gid += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = gid / kCols;
    const int c = (int)(gid - r * kCols);
    const float sa = a.s_a[r], sb = a.s_b[r];
    const float M = fmaxf(sa, sb);
    const bool empty = M == -INFINITY;
    const float wa = (sa == -INFINITY || empty) ? 0.f : __builtin_amdgcn_exp2f((sa - M) * kLog2e);
    const float wb = (sb == -INFINITY || empty) ? 0.f : __builtin_amdgcn_exp2f((sb - M) * kLog2e);
    const float den = wa + wb;
    const float ia = empty ? 0.f : wa / den;
    const float ib = empty ? 0.f : wb / den;
    const int64_t off = r * (D * kEB) + c * 16;
    const uint4 va = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_a) + off);
    const uint4 vb = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_b) + off);
    uint4 vo;
    if constexpr (kBF16) {
      auto mix = [&](uint32_t x, uint32_t y) {
        const float x0 = __uint_as_float(x << 16), x1 = __uint_as_float(x & 0xFFFF0000u);
        const float y0 = __uint_as_float(y << 16), y1 = __uint_as_float(y & 0xFFFF0000u);
        return pack_bf16(ia * x0 + ib * y0, ia * x1 + ib * y1);
      };
      vo.x = mix(va.x, vb.x);
      vo.y = mix(va.y, vb.y);
      vo.z = mix(va.z, vb.z);
      vo.w = mix(va.w, vb.w);
    } else {
      auto mix = [&](uint32_t x, uint32_t y) {
        return __float_as_uint(ia * __uint_as_float(x) + ib * __uint_as_float(y));
      };
      vo.x = mix(va.x, vb.x);
      vo.y = mix(va.y, vb.y);
      vo.z = mix(va.z, vb.z);
      vo.w = mix(va.w, vb.w);
    }
    *reinterpret_cast<uint4*>(static_cast<char*>(a.v_out) + off) = vo;
    if (c == 0) a.s_out[r] = empty ? -INFINITY : M + __builtin_amdgcn_logf(den) * kLn2;
  }
}

}  // namespace

hipError_t launch_merge_two(const MergeTwoArgs& a, hipStream_t stream) {
  if (a.num_rows <= 0) return hipSuccess;
  const int eb = a.bf16 ? 2 : 4;
  const int64_t total = a.num_rows * (a.head_dim * eb / 16);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const dim3 grid((uint32_t)blocks), block(256);
  if (a.bf16) {
    if (a.head_dim == 128) hipLaunchKernelGGL((merge_two_kernel<true, 128>), grid, block, 0, stream, a);
    else if (a.head_dim == 64) hipLaunchKernelGGL((merge_two_kernel<true, 64>), grid, block, 0, stream, a);
    else return hipErrorInvalidValue;
  } else {
    if (a.head_dim == 128) hipLaunchKernelGGL((merge_two_kernel<false, 128>), grid, block, 0, stream, a);
    else if (a.head_dim == 64) hipLaunchKernelGGL((merge_two_kernel<false, 64>), grid, block, 0, stream, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fi
