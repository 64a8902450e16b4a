// Shared-prefix attention on matrix cores, for gfx950 (bf16).
//
// Composable block-sparse formats (FlashInfer paper explainer, "FlashInfer:
// Block-Sparse KV 캐시로 어텐션 병목을 해소하다", visionhong.com, Block-Sparse
// section): a KV cache can be described by more than one block-sparse
// matrix. When many requests begin with the same pages, the common prefix is
// one block that all of their query rows share; computing it once per KV head
// for every row of the group turns a per-request vector problem (each request
// re-reading the prefix) into one matrix problem. The prefix state of each
// row, (o, lse) over the prefix tokens only, is later merged with the row's
// state over its own pages by the merge tree of the decode kernel (softmax
// over a disjoint union, the closed form of the explainer's scheduler split).
//
// One workgroup of 4 waves per prefix item = (group, KV head, <= 128 query
// rows, chunk of prefix pages). Wave w owns rows 32w .. 32w+31. K and V move
// through LDS in blocks of 32 tokens, double-buffered: the global loads of
// block i+1 are in flight while block i is computed (64-token blocks were
// measured slower: more staging registers cut occupancy). Per block:
//   S^T[token, row] = K . Q^T       v_mfma_f32_32x32x16_bf16, D/16 steps
//   online softmax per row (a lane owns one row: 16 tokens in the lane, the
//   other 16 in lane l^32)
//   O^T[d, row] += V^T . P^T        2 token steps x D/32 tiles
// Lane layout of v_mfma_f32_32x32x16_bf16 (A 32x16, B 16x32, C 32x32):
// A[m][k] in lane m + 32*(k/8), element k%8; B[k][n] in lane n + 32*(k/8);
// C[m][n] in lane n + 32*((m%8)/4), element 4*(m/8) + m%4.
// P^T comes straight from the S^T accumulators: the contraction index of the
// PV product enumerates the block's tokens in the order the S^T layout leaves
// them in the lanes, and V^T is read in that same order.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fi_bsr.h"
#include "kernels.h"

namespace fi {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kRows = 128;   // query rows per item (4 waves x 32)
constexpr int kBlock = 32;   // tokens staged per step (one 32-token matrix tile)
constexpr float kLog2e = 1.44269504088896340736f;

struct PrefixParams {
  const int32_t* pitems;
  const int32_t* members;
  const int32_t* prefix_slot;
  const int32_t* page_ids;
  const char* q;
  const char* k_pages;
  const char* v_pages;
  float* part_o;
  float* part_lse;
  int64_t page_stride;  // bytes between physical pages
  int64_t head_stride;  // bytes between KV heads within a page
  int num_qo_heads;
  int num_kv_heads;
  int page_size;
  int group;
  float scale_log2;     // sm_scale * log2(e)
};

__device__ __forceinline__ float max_with_partner32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// K and V pieces of one block of tokens, held in registers between their
// global load and their store to LDS.
template <int N>
struct Stage {
  uint4 k[N], v[N];
};

template <int kLoads, int kChunks, int kRowBytes>
__device__ __forceinline__ Stage<kLoads> load_stage(const PrefixParams& p, const int* s_pid,
                                                    int page_begin, int64_t head_off, int ntok,
                                                    int tok0, int tid) {
  Stage<kLoads> st;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int e = tid + 256 * i;
    const int t = e / kChunks, c = e % kChunks;
    const int tok = min(tok0 + t, ntok - 1);  // past the end: re-read the last token
    const int pid = s_pid[tok / p.page_size];
    const int64_t off = (int64_t)pid * p.page_stride + head_off +
                        (int64_t)(tok % p.page_size) * kRowBytes + c * 16;
    st.k[i] = *reinterpret_cast<const uint4*>(p.k_pages + off);
    st.v[i] = *reinterpret_cast<const uint4*>(p.v_pages + off);
  }
  return st;
}

// K row-major (padded rows); V transposed: element d = 8c + j of token t
// goes to row d, column t.
template <int kLoads, int kChunks, int kKStride, int kVtStride>
__device__ __forceinline__ void store_stage(const Stage<kLoads>& st, char* s_k, char* s_vt, int tid) {
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int e = tid + 256 * i;
    const int t = e / kChunks, c = e % kChunks;
    *reinterpret_cast<uint4*>(s_k + t * kKStride + c * 16) = st.k[i];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w = j < 2 ? st.v[i].x : j < 4 ? st.v[i].y : j < 6 ? st.v[i].z : st.v[i].w;
      *reinterpret_cast<uint16_t*>(s_vt + (8 * c + j) * kVtStride + t * 2) = (uint16_t)(w >> (16 * (j & 1)));
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void prefix_attend_kernel(PrefixParams p) {
  constexpr int kRowBytes = D * 2;
  constexpr int kKStride = kRowBytes + 16;     // K rows in LDS, padded
  constexpr int kVtStride = kBlock * 2 + 8;    // V^T rows (one per d), padded
  constexpr int kChunks = kRowBytes / 16;      // 16-byte pieces per token row
  constexpr int kLoads = kBlock * kChunks / 256;  // per thread per block, K and V each
  static_assert(kLoads >= 1 && kBlock * kChunks % 256 == 0, "block does not tile the workgroup");
  // two buffers: block i is computed from one while block i+1 is stored
  // into the other
  __shared__ __attribute__((aligned(16))) char s_k[2][kBlock * kKStride];
  __shared__ __attribute__((aligned(16))) char s_vt[2][D * kVtStride];
  // the item's page ids (at most FI_PREFIX_MAX_PAGES), read from LDS so a
  // block's K/V loads never wait on a page-table read
  __shared__ int s_pid[FI_PREFIX_MAX_PAGES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int32_t* it = p.pitems + (int64_t)blockIdx.x * FI_PITEM_STRIDE;
  const int h = it[FI_PITEM_KV_HEAD];
  const int member_base = it[FI_PITEM_MEMBER_BASE];
  const int row_begin = it[FI_PITEM_ROW_BEGIN];
  const int nrows = it[FI_PITEM_NUM_ROWS];
  const int chunk = it[FI_PITEM_CHUNK];
  const int page_begin = it[FI_PITEM_PAGE_BEGIN];
  const int npg = it[FI_PITEM_NUM_PAGES];
  const int ntok = npg * p.page_size;
  const int G = p.group;
  for (int i = tid; i < npg; i += 256) s_pid[i] = p.page_ids[page_begin + i];
  __syncthreads();

  // ---- this lane's query row (column n = lane % 32 of the wave's tiles)
  const int row = wave * 32 + (lane & 31);
  const bool row_ok = row < nrows;
  int b = 0, gi = 0;
  if (row_ok) {
    b = p.members[member_base + row_begin + row / G];
    gi = row % G;
  }
  const int half = lane >> 5;
  // Q^T as the B operand: lane holds Q[row][16s + 8*half .. +8] for step s
  bf16x8_t qf[D / 16];
  {
    const char* qrow = p.q + ((int64_t)b * p.num_qo_heads + (int64_t)h * G + gi) * kRowBytes;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qrow + (16 * s + 8 * half) * 2)
                             : make_uint4(0, 0, 0, 0);
      qf[s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // ---- staging: thread tid loads 16-byte pieces (token, piece) =
  // ((tid + 256 i) / kChunks, (tid + 256 i) % kChunks) of the K and V block.
  // The loads of block i+1 are issued before block i is computed and stored
  // to the other LDS buffer after it, so their latency hides behind the
  // matrix work.
  const int64_t head_off = (int64_t)h * p.head_stride;
  {
    const Stage<kLoads> st0 = load_stage<kLoads, kChunks, kRowBytes>(p, s_pid, page_begin, head_off, ntok, 0, tid);
    store_stage<kLoads, kChunks, kKStride, kVtStride>(st0, s_k[0], s_vt[0], tid);
  }
  __syncthreads();

  f32x16_t o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int nblocks = (ntok + kBlock - 1) / kBlock;
  for (int blk = 0; blk < nblocks; ++blk) {
    const int buf = blk & 1;
    // issued on every step (past the end it re-reads the last token), so the
    // staging registers never need a conditional path
    const Stage<kLoads> nxt =
        load_stage<kLoads, kChunks, kRowBytes>(p, s_pid, page_begin, head_off, ntok, (blk + 1) * kBlock, tid);
    const char* sk = s_k[buf];
    const char* svt = s_vt[buf];
    {
#pragma unroll
    for (int sub = 0; sub < kBlock / 32; ++sub) {
      // S^T = K . Q^T: A = K rows from LDS (row m = lane % 32, k 8*half .. +8)
      f32x16_t s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int q = 0; q < D / 16; ++q) {
        const uint4 kv = *reinterpret_cast<const uint4*>(sk + (32 * sub + (lane & 31)) * kKStride + (16 * q + 8 * half) * 2);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kv), qf[q], s, 0, 0, 0);
      }
      // element r holds token m = 4*half + 8*(r/4) + r%4 of the block
      const int tok0 = blk * kBlock + 32 * sub;
      float mb = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 4 * half + 8 * (r >> 2) + (r & 3);
        s[r] = tok0 + m < ntok ? s[r] * p.scale_log2 : -INFINITY;
        mb = fmaxf(mb, s[r]);
      }
      mb = max_with_partner32(mb);
      const float m_new = fmaxf(m_run, mb);  // finite: every block has a valid token
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = __builtin_amdgcn_exp2f(s[r] - m_new);  // masked tokens give 0
        ps += s[r];
      }
      l_run = l_run * alpha + sum_with_partner32(ps);
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] *= alpha;

      // O^T += V^T . P^T over two steps of 16 tokens. Step ks takes elements
      // 8ks .. 8ks+7 of s: contraction index 8*half + i is token
      // 4*half + 8*(2ks + i/4) + i%4 -- two runs of 4 consecutive tokens.
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8_t pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[i] = (__bf16)s[8 * ks + i];
        const int t0 = 32 * sub + 4 * half + 16 * ks;  // first run; the second starts 8 later
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          const char* vrow = svt + (32 * t + (lane & 31)) * kVtStride;
          const uint2 a0 = *reinterpret_cast<const uint2*>(vrow + t0 * 2);
          const uint2 a1 = *reinterpret_cast<const uint2*>(vrow + (t0 + 8) * 2);
          const uint4 av = make_uint4(a0.x, a0.y, a1.x, a1.y);
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av), pb, o[t], 0, 0, 0);
        }
      }
    }
    }
    store_stage<kLoads, kChunks, kKStride, kVtStride>(nxt, s_k[buf ^ 1], s_vt[buf ^ 1], tid);
    __syncthreads();
  }

  // ---- partial state of this row: o / l and lse (log2 units)
  if (!row_ok) return;
  const int slot = p.prefix_slot[(int64_t)b * p.num_kv_heads + h] + chunk;
  const int64_t prow = (int64_t)slot * G + gi;
  const float inv = 1.f / l_run;
  float* dst = p.part_o + prow * D;
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      // elements 4*q4 .. +3 are d = 32t + 8*q4 + 4*half .. +3
      const int d = 32 * t + 8 * q4 + 4 * half;
      *reinterpret_cast<float4*>(dst + d) =
          make_float4(o[t][4 * q4] * inv, o[t][4 * q4 + 1] * inv, o[t][4 * q4 + 2] * inv, o[t][4 * q4 + 3] * inv);
    }
  }
  if (half == 0) p.part_lse[prow] = m_run + __builtin_amdgcn_logf(l_run);
}

}  // namespace

hipError_t launch_prefix(const PrefixArgs& a, hipStream_t stream) {
  if (a.num_items <= 0) return hipSuccess;
  PrefixParams p;
  p.pitems = a.pitems;
  p.members = a.members;
  p.prefix_slot = a.prefix_slot;
  p.page_ids = a.page_ids;
  p.q = static_cast<const char*>(a.q);
  p.k_pages = static_cast<const char*>(a.k_pages);
  p.v_pages = static_cast<const char*>(a.v_pages);
  p.part_o = a.part_o;
  p.part_lse = a.part_lse;
  const int64_t row = (int64_t)a.head_dim * 2;
  p.head_stride = (int64_t)a.page_size * row;
  p.page_stride = (int64_t)a.num_kv_heads * a.page_size * row;
  p.num_qo_heads = a.num_qo_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.page_size = a.page_size;
  p.group = a.group;
  p.scale_log2 = a.sm_scale * kLog2e;
  const dim3 grid((uint32_t)a.num_items), block(256);
  if (a.head_dim == 128) hipLaunchKernelGGL(prefix_attend_kernel<128>, grid, block, 0, stream, p);
  else if (a.head_dim == 64) hipLaunchKernelGGL(prefix_attend_kernel<64>, grid, block, 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fi
