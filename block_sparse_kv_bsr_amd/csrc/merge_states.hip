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
// decode run merges its own partial states inside the decode kernel.)
// prefill_merge_kernel folds the KV-chunk partials of cut prefill tiles
// (log2-unit LSE) into bf16 out and natural-log lse: a thread per (row, 4
// columns), the chunks' loads independent of each other, summed in slot
// order.
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

template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillArgs a) {
  constexpr int kTPR = D / 4;         // threads per row, 4 columns each
  constexpr int kRPB = 256 / kTPR;    // rows per workgroup
  const int32_t* m = a.merges + (int64_t)blockIdx.x * FI_QMERGE_STRIDE;
  const int rows = m[FI_QMERGE_NUM_QO] * a.group;
  const int r = blockIdx.y * kRPB + threadIdx.x / kTPR;
  if (r >= rows) return;
  const int qo_row = m[FI_QMERGE_QO_ROW];
  const int h = m[FI_QMERGE_KV_HEAD];
  const int64_t slot0 = m[FI_QMERGE_SLOT_BEGIN];
  const int k = m[FI_QMERGE_NUM_CHUNKS];
  const int c4 = 4 * (threadIdx.x % kTPR);
  const float* lse_r = a.part_lse + slot0 * FI_PREFILL_ROWS + r;
  float mx = -INFINITY;
#pragma unroll 8
  for (int c = 0; c < k; ++c) mx = fmaxf(mx, lse_r[(int64_t)c * FI_PREFILL_ROWS]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  if (mx != -INFINITY) {
#pragma unroll 4
    for (int c = 0; c < k; ++c) {
      const float s = lse_r[(int64_t)c * FI_PREFILL_ROWS];
      // a chunk the row attended nothing of has s = -inf and weight 0
      const float w = s == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s - mx);
      const float4 o = *reinterpret_cast<const float4*>(
          a.part_o + ((slot0 + c) * FI_PREFILL_ROWS + r) * D + c4);
      den += w;
      acc.x += w * o.x;
      acc.y += w * o.y;
      acc.z += w * o.z;
      acc.w += w * o.w;
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int64_t q_index =
      (int64_t)(qo_row + r / a.group) * a.num_qo_heads + (int64_t)h * a.group + r % a.group;
  uint2 packed;
  packed.x = pack_bf16(acc.x * inv, acc.y * inv);
  packed.y = pack_bf16(acc.z * inv, acc.w * inv);
  *reinterpret_cast<uint2*>(static_cast<__bf16*>(a.out) + q_index * D + c4) = packed;
  if (c4 == 0 && a.lse)
    a.lse[q_index] = den > 0.f ? (mx + __builtin_amdgcn_logf(den)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_prefill_merge(const PrefillArgs& a, hipStream_t stream) {
  if (a.num_merges <= 0) return hipSuccess;
  const uint32_t rpb = 256 / (a.head_dim / 4);
  const dim3 grid((uint32_t)a.num_merges, (FI_PREFILL_ROWS + rpb - 1) / rpb), block(256);
  if (a.head_dim == 128) hipLaunchKernelGGL((prefill_merge_kernel<128>), grid, block, 0, stream, a);
  else if (a.head_dim == 64) hipLaunchKernelGGL((prefill_merge_kernel<64>), grid, block, 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

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
