// Paged / BSR grouped-query decode attention for gfx950 (MI355X, CDNA4).
//
// What is computed: for each work item (request b, KV head kvh, chunk of whole
// pages) the G query heads kvh*G .. kvh*G+G-1 attend over the chunk's tokens;
// the page ids come from the request's block list, so blocks that are not
// listed are never touched (FlashInfer paper explainer, "FlashInfer:
// Block-Sparse KV 캐시로 어텐션 병목을 해소하다", section on the Block-Sparse
// format). Decode reads the whole KV history once per token generated and is
// bound by memory bandwidth (same page, section on the attention bottleneck),
// so the kernel is built around the page gather:
//
//  * One wave per item, 8 lanes per token row, 8 token rows per step: each
//    lane issues 16-byte loads at row offsets sub*16 + j*128, so one load
//    instruction covers eight whole 128-byte lines. Loads go straight to
//    VGPRs: a K/V row is used by exactly one wave, so LDS staging would add
//    traffic without reuse.
//  * GQA packing: each K/V row is loaded once per KV head and serves all G
//    query heads of the group (query heads kvh*G+i share KV head kvh).
//  * Scores: bf16 pairs go through v_dot2 (two products + accumulate into
//    fp32 per instruction); the 8 lanes of a token are summed with three DPP
//    row operations inside a half-row, with no LDS traffic.
//  * Softmax: each group of 8 lanes keeps its own running (max, sum,
//    accumulator) state in the log2 domain; the running max is only raised
//    when a score exceeds it by more than 8 (so exp2 stays <= 256), which
//    makes accumulator rescales rare. The eight per-lane-group states are
//    merged once at the end of the item.
//  * Prefetch: a ring of kDepth token steps (K and V) is kept in flight per
//    wave; the page-id window for 64 pages sits in one VGPR and is read with
//    ds_bpermute.
//  * Tokens past the request's length in the last page are excluded by
//    selection (score -inf, weight 0, V zeroed), never by multiplying by a
//    zero weight, so whatever those slots hold (NaN included) cannot leak.
//
// The result is written directly (bf16 rounded to nearest even, natural-log
// LSE) when the request is one chunk, else as an fp32 partial state (output
// already divided by its own sum, LSE in log2 units) for the merge kernel.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fi_bsr.h"
#include "kernels.h"

namespace fi {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
// The running max is raised only when a score exceeds it by more than this
// (log2 units), so unnormalised weights stay within [0, 2^8].
constexpr float kRescaleMargin = 8.0f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct DecodeParams {
  const int32_t* items;
  const int32_t* page_ids;
  const char* q;
  const char* k_pages;
  const char* v_pages;
  char* out;
  float* lse;
  float* part_o;
  float* part_lse;
  int64_t page_stride;  // bytes between consecutive physical pages
  int32_t head_stride;  // bytes between KV heads inside a page
  int32_t num_qo_heads;
  int32_t page_size;
  int32_t step_pages;   // 8 tokens = step_pages pages + step_slots slots
  int32_t step_slots;
  float scale_log2;     // sm_scale * log2(e)
};

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

// Sum over the 8 lanes of a half-row (lanes 8k .. 8k+7); all 8 get the total.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint4 load16(const char* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int w) {
  return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
}

template <bool kBF16, int D>
struct Row {
  static constexpr int kElemBytes = kBF16 ? 2 : 4;
  static constexpr int kBytes = D * kElemBytes;          // one token row
  static constexpr int kLoads = kBytes / 128;            // 16-byte loads per lane
  static constexpr int kWords = kLoads * 4;              // 32-bit words per lane
  static constexpr int kElems = D / 8;                   // elements per lane
  static constexpr int kPerLoad = 16 / kElemBytes;       // elements per load
  static_assert(kLoads >= 1, "row shorter than 128 bytes");
};

// Register plan per lane: accumulators G*NE, query words G*NW, a ring of
// kDepth (K, V) steps of 8*L words, plus ~80 for state, addressing and
// temporaries. Two waves per SIMD (<= 256 VGPRs) when that fits, else one
// wave (VGPRs + AGPRs, <= 512).
template <bool kBF16, int D, int G>
struct Tune {
  using R = Row<kBF16, D>;
  static constexpr int kBase = G * R::kElems + G * R::kWords + 2 * G + 80;
  static constexpr int kStage = 8 * R::kLoads;
  static constexpr int kWaves = kBase + 2 * kStage <= 240 ? 2 : 1;
  static constexpr int kBudget = kWaves == 2 ? 240 : 440;
  static constexpr int kDepth = kBase + 4 * kStage <= kBudget ? 4 : 2;
};

template <bool kBF16, int D, int G, int kDepth, int kWaves>
__global__ __launch_bounds__(64, kWaves) void decode_bsr_kernel(DecodeParams p) {
  using R = Row<kBF16, D>;
  constexpr int L = R::kLoads;
  constexpr int NW = R::kWords;
  constexpr int NE = R::kElems;

  const int lane = threadIdx.x;
  const int sub = lane & 7;   // 16-byte column within a 128-byte line
  const int tg = lane >> 3;   // token row within a step of 8
  const int32_t* it = p.items + (int64_t)blockIdx.x * FI_ITEM_STRIDE;
  const int b = it[FI_ITEM_REQUEST];
  const int kvh = it[FI_ITEM_KV_HEAD];
  const int pb = it[FI_ITEM_PAGE_BEGIN];
  const int ntok = it[FI_ITEM_NUM_TOKENS];
  const int slot = it[FI_ITEM_SLOT];
  const int npg = it[FI_ITEM_NUM_PAGES];
  const int P = p.page_size;

  // ---- query fragments of the G heads (same columns as the K/V fragments)
  const int64_t qrow0 = (int64_t)b * p.num_qo_heads + (int64_t)kvh * G;
  uint32_t qw[G][NW];
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const uint4 v = load16(p.q + (qrow0 + h) * R::kBytes + j * 128 + sub * 16);
      qw[h][j * 4 + 0] = v.x;
      qw[h][j * 4 + 1] = v.y;
      qw[h][j * 4 + 2] = v.z;
      qw[h][j * 4 + 3] = v.w;
    }
  }

  // ---- page-id window: lane i holds the id of page (wbase + i) of the chunk
  int wbase = 0;
  int win = lane < npg ? p.page_ids[pb + lane] : 0;

  // ---- load cursor: page-local index and slot of this lane's next token
  int cur_pl = tg / P;
  int cur_slot = tg - cur_pl * P;
  const int last_pl = (ntok - 1) / P;
  const int last_slot = (ntok - 1) - last_pl * P;
  const int ngroups = (ntok + 7) >> 3;
  const int64_t head_off = (int64_t)kvh * p.head_stride + sub * 16;

  uint4 kb[kDepth][L], vb[kDepth][L];

  auto issue = [&](int g, uint4 (&kr)[L], uint4 (&vr)[L]) {
    int pl = cur_pl, sl = cur_slot;
    if (g == ngroups - 1 && g * 8 + tg >= ntok) {  // past the end: re-read the last token
      pl = last_pl;
      sl = last_slot;
    }
    if (__builtin_amdgcn_readlane(pl, 63) - wbase >= 64) {
      wbase = __builtin_amdgcn_readfirstlane(pl);
      win = wbase + lane < npg ? p.page_ids[pb + wbase + lane] : 0;
    }
    const int pid = __shfl(win, pl - wbase);
    const int64_t off = (int64_t)pid * p.page_stride + head_off + (int64_t)sl * R::kBytes;
    const char* kp = p.k_pages + off;
    const char* vp = p.v_pages + off;
#pragma unroll
    for (int j = 0; j < L; ++j) kr[j] = load16(kp + j * 128);
#pragma unroll
    for (int j = 0; j < L; ++j) vr[j] = load16(vp + j * 128);
    cur_slot += p.step_slots;
    cur_pl += p.step_pages;
    if (cur_slot >= P) {
      cur_slot -= P;
      cur_pl += 1;
    }
  };

  float m[G], l[G], acc[G][NE];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[h][e] = 0.f;
  }

  auto consume = [&](const uint4 (&kr)[L], uint4 (&vr)[L], bool masked, bool valid) {
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const uint32_t kw = word(kr[w / 4], w % 4);
        if constexpr (kBF16) {
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kw),
                                              __builtin_bit_cast(bf16x2_t, qw[h][w]), d, false);
        } else {
          d = __builtin_fmaf(__uint_as_float(kw), __uint_as_float(qw[h][w]), d);
        }
      }
      s[h] = sum8(d) * p.scale_log2;
    }
    if (masked) {
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = valid ? s[h] : -INFINITY;
#pragma unroll
      for (int j = 0; j < L; ++j) {
        vr[j].x = valid ? vr[j].x : 0u;
        vr[j].y = valid ? vr[j].y : 0u;
        vr[j].z = valid ? vr[j].z : 0u;
        vr[j].w = valid ? vr[j].w : 0u;
      }
    }
    bool need = false;
#pragma unroll
    for (int h = 0; h < G; ++h) need |= s[h] > m[h] + kRescaleMargin;
    if (__any(need)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const bool up = s[h] > m[h] + kRescaleMargin;
        const float f = up ? exp2_fast(m[h] - s[h]) : 1.f;
        m[h] = up ? s[h] : m[h];
        l[h] *= f;
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[h][e] *= f;
      }
    }
    float pw[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      pw[h] = exp2_fast(s[h] - m[h]);
      if (masked) pw[h] = valid ? pw[h] : 0.f;
      l[h] += pw[h];
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t vw = word(vr[w / 4], w % 4);
      if constexpr (kBF16) {
        const float v0 = bf16_lo(vw), v1 = bf16_hi(vw);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h][2 * w] = __builtin_fmaf(pw[h], v0, acc[h][2 * w]);
          acc[h][2 * w + 1] = __builtin_fmaf(pw[h], v1, acc[h][2 * w + 1]);
        }
      } else {
        const float v0 = __uint_as_float(vw);
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h][w] = __builtin_fmaf(pw[h], v0, acc[h][w]);
      }
    }
  };

  // ---- main loop: ring of kDepth steps in flight
#pragma unroll
  for (int s = 0; s < kDepth; ++s)
    if (s < ngroups) issue(s, kb[s], vb[s]);
  const bool ragged = (ntok & 7) != 0;
  for (int g0 = 0; g0 < ngroups; g0 += kDepth) {
#pragma unroll
    for (int s = 0; s < kDepth; ++s) {
      const int g = g0 + s;
      if (g < ngroups) {
        if (ragged && g == ngroups - 1) consume(kb[s], vb[s], true, g * 8 + tg < ntok);
        else consume(kb[s], vb[s], false, true);
        if (g + kDepth < ngroups) issue(g + kDepth, kb[s], vb[s]);
      }
    }
  }

  // ---- merge the 8 lane-group states (lanes with equal `sub`)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = m[h];
    M = fmaxf(M, __shfl_xor(M, 8));
    M = fmaxf(M, __shfl_xor(M, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float f = m[h] == -INFINITY ? 0.f : exp2_fast(m[h] - M);
    float lh = l[h] * f;
    lh += __shfl_xor(lh, 8);
    lh += __shfl_xor(lh, 16);
    lh += __shfl_xor(lh, 32);
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      float a = acc[h][e] * f;
      a += __shfl_xor(a, 8);
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      acc[h][e] = a;
    }
    m[h] = M;
    l[h] = lh;
  }

  // ---- epilogue: lane group tg writes query head kvh*G + tg
  if (tg < G) {
    float o[NE];
    float mh = 0.f, lh = 1.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (tg == h) {
        mh = m[h];
        lh = l[h];
#pragma unroll
        for (int e = 0; e < NE; ++e) o[e] = acc[h][e];
      }
    }
    const float inv = 1.f / lh;
#pragma unroll
    for (int e = 0; e < NE; ++e) o[e] *= inv;
    const int64_t qrow = qrow0 + tg;
    if (slot < 0) {
      char* dst = p.out + qrow * R::kBytes + sub * 16;
#pragma unroll
      for (int j = 0; j < L; ++j) {
        uint4 v;
        if constexpr (kBF16) {
          v.x = pack_bf16(o[j * 8 + 0], o[j * 8 + 1]);
          v.y = pack_bf16(o[j * 8 + 2], o[j * 8 + 3]);
          v.z = pack_bf16(o[j * 8 + 4], o[j * 8 + 5]);
          v.w = pack_bf16(o[j * 8 + 6], o[j * 8 + 7]);
        } else {
          v.x = __float_as_uint(o[j * 4 + 0]);
          v.y = __float_as_uint(o[j * 4 + 1]);
          v.z = __float_as_uint(o[j * 4 + 2]);
          v.w = __float_as_uint(o[j * 4 + 3]);
        }
        *reinterpret_cast<uint4*>(dst + j * 128) = v;
      }
      if (sub == 0 && p.lse) p.lse[qrow] = (mh + log2_fast(lh)) * kLn2;
    } else {
      const int64_t prow = (int64_t)slot * p.num_qo_heads + (int64_t)kvh * G + tg;
      float* dst = p.part_o + prow * D;
#pragma unroll
      for (int j = 0; j < L; ++j) {
        // elements j*kPerLoad .. +kPerLoad-1 sit at dims j*(128/eb) + sub*kPerLoad
        constexpr int PL = R::kPerLoad;
        float* d0 = dst + j * (128 / R::kElemBytes) + sub * PL;
#pragma unroll
        for (int c = 0; c < PL; c += 4)
          *reinterpret_cast<float4*>(d0 + c) =
              make_float4(o[j * PL + c], o[j * PL + c + 1], o[j * PL + c + 2], o[j * PL + c + 3]);
      }
      if (sub == 0) p.part_lse[prow] = mh + log2_fast(lh);
    }
  }
}

template <bool kBF16, int D, int G>
hipError_t launch_typed(const DecodeParams& prm, int64_t num_items, hipStream_t stream) {
  using T = Tune<kBF16, D, G>;
  hipLaunchKernelGGL((decode_bsr_kernel<kBF16, D, G, T::kDepth, T::kWaves>),
                     dim3((uint32_t)num_items), dim3(64), 0, stream, prm);
  return hipGetLastError();
}

template <bool kBF16, int D>
hipError_t launch_group(const DecodeParams& prm, int64_t n, int G, hipStream_t s) {
  switch (G) {
    case 1: return launch_typed<kBF16, D, 1>(prm, n, s);
    case 2: return launch_typed<kBF16, D, 2>(prm, n, s);
    case 4: return launch_typed<kBF16, D, 4>(prm, n, s);
    case 8: return launch_typed<kBF16, D, 8>(prm, n, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_items <= 0) return hipSuccess;
  const int eb = a.bf16 ? 2 : 4;
  const int row = a.head_dim * eb;
  DecodeParams prm;
  prm.items = a.items;
  prm.page_ids = a.page_ids;
  prm.q = static_cast<const char*>(a.q);
  prm.k_pages = static_cast<const char*>(a.k_pages);
  prm.v_pages = static_cast<const char*>(a.v_pages);
  prm.out = static_cast<char*>(a.out);
  prm.lse = a.lse;
  prm.part_o = a.part_o;
  prm.part_lse = a.part_lse;
  prm.head_stride = a.page_size * row;
  prm.page_stride = (int64_t)a.num_kv_heads * a.page_size * row;
  prm.num_qo_heads = a.num_qo_heads;
  prm.page_size = a.page_size;
  prm.step_pages = 8 / a.page_size;
  prm.step_slots = 8 % a.page_size;
  prm.scale_log2 = a.sm_scale * kLog2e;
  if (a.bf16) {
    if (a.head_dim == 128) return launch_group<true, 128>(prm, a.num_items, a.group, stream);
    if (a.head_dim == 64) return launch_group<true, 64>(prm, a.num_items, a.group, stream);
  } else {
    if (a.head_dim == 128) return launch_group<false, 128>(prm, a.num_items, a.group, stream);
    if (a.head_dim == 64) return launch_group<false, 64>(prm, a.num_items, a.group, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fi
