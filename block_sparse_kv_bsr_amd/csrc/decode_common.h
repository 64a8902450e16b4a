// Pieces shared by the two decode kernels (the vector-ALU kernel in
// decode_bsr.hip and the matrix-core kernel in decode_mma.hip): kernel
// parameters, cache-policy and wait helpers, cross-lane reductions, the
// device-coherent accesses of partial states, and the in-kernel merge tree
// of cut requests. Each including file gets its own copy (anonymous
// namespace); nothing here is part of the library's interface.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
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
// Page ids of a chunk staged in LDS at a time (a wave reloads the window when
// it walks past it).
constexpr int kIdWindow = 256;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

struct DecodeParams {
  const int32_t* items;
  const int32_t* page_ids;
  const char* q;
  const char* k_pages;
  const char* v_pages;
  char* out;
  float* lse;
  float* part_o;        // [slots][G][D]
  float* part_lse;      // [slots][G], log2 units
  const int32_t* nodes; // merge nodes [num_nodes][FI_NODE_STRIDE]
  int32_t* counters;    // arrivals per merge node, 0 between runs
  int64_t page_stride;  // bytes between consecutive physical pages
  int32_t head_stride;  // bytes between KV heads inside a page
  int32_t num_qo_heads;
  int32_t page_size;
  int32_t step_pages;   // 8 tokens = step_pages pages + step_slots slots
  int32_t step_slots;
  float scale_log2;     // sm_scale * k_scale * log2(e)
  float v_scale;        // multiplies the output (V dequantisation)
  double rope_log2_theta;  // rotary embedding: log2(rope_theta)
  double rope_rev;         // 1 / (2 pi rope_scale): revolutions per radian, positions scaled
};

// Sine and cosine of the rotary angle of a dim pair at position `pos`. The
// pair's frequency is a 64-bit binary fraction of a revolution per position,
// so pos * freq mod 1 is exact integer arithmetic (no loss of phase at large
// positions); its top 32 bits give the angle for sincospif.
__device__ __forceinline__ void rope_sincos(uint64_t freq, int pos, float& c, float& s) {
  const uint64_t ph = (uint64_t)(uint32_t)pos * freq;
  const float rev = (float)(uint32_t)(ph >> 32) * 0x1p-32f;
  sincospif(2.f * rev, &s, &c);
}

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

// x *= f with the result tied to x's register. Used inside the rare rescale
// branch: a plain multiply there lets the compiler keep a second copy of
// every accumulator across the branch and copy them back on the common path.
__device__ __forceinline__ void scale_in_place(float& x, float f) {
  asm volatile("v_mul_f32 %0, %1, %0" : "+v"(x) : "v"(f));
}
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

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;

// Cache policy of the K/V loads. K/V rows are read once per decode step: the
// nontemporal policy (nt) streams them past the caches instead of allocating
// lines that will not be reused. When the plan lists a physical page for
// several requests (a shared prefix) the default policy keeps the re-reads
// cacheable in L2 / MALL.
template <bool kStream>
__device__ __forceinline__ void dma16(const char* src, void* lds_base) {
  constexpr int kAux = kStream ? 2 : 0;  // bit 1 = nt on gfx950
  __builtin_amdgcn_global_load_lds((global_void_t*)src, (lds_void_t*)lds_base, 16, 0, kAux);
}

// s_waitcnt vmcnt(n), leaving the other counters unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

// A 32-bit LDS read (a page id of the window) through inline asm, with its
// wait in the same block. In front of an ordinary LDS read the compiler
// waits for every direct-to-LDS load in flight (vmcnt(0)): it cannot tell
// that they never write this location, and the wait would drain the K/V
// loads a wave keeps in flight ahead of its work.
__device__ __forceinline__ int lds_read_id(const int* p) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}

// Read a ring stage back: n 16-byte chunks at the given LDS addresses, then
// wait for them. The wait is tied to the outputs so no use can move above it.
template <int N>
__device__ __forceinline__ void lds_read_stage(const uint32_t (&addr)[N], u32x4_t (&out)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("ds_read_b128 %0, %1" : "=v"(out[i]) : "v"(addr[i]) : "memory");
  if constexpr (N == 2) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(out[0]), "+v"(out[1]) :: "memory");
  } else if constexpr (N == 4) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(out[0]), "+v"(out[1]), "+v"(out[2]), "+v"(out[3]) :: "memory");
  } else {
    static_assert(N == 8, "stage of 2, 4 or 8 chunks");
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(out[0]), "+v"(out[1]), "+v"(out[2]), "+v"(out[3]), "+v"(out[4]),
                   "+v"(out[5]), "+v"(out[6]), "+v"(out[7])::"memory");
  }
}

// The rotary embedding over 128-byte K rows (fp8 at d 128, bf16 at d 64):
// this lane's rotate-half pairs are bytes 8 sub .. 8 sub + 7 and 64 + 8 sub
// .. of its token's row (two 8-byte reads at `ak` and ak + 64), packed as
// (x, y) = first half, (z, w) = second half; its V chunk is read as usual.
__device__ __forceinline__ void lds_read_k_halves(uint32_t ak, uint32_t av, u32x4_t& k, u32x4_t& v) {
  u32x2_t a, b;
  asm volatile("ds_read_b64 %0, %1" : "=v"(a) : "v"(ak) : "memory");
  asm volatile("ds_read_b64 %0, %1 offset:64" : "=v"(b) : "v"(ak) : "memory");
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(av) : "memory");
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(v) :: "memory");
  k = u32x4_t{a.x, a.y, b.x, b.y};
}

// The wait before reading ring stage s of the tail: stage s must have
// landed, while the kRing - 1 - s stages issued after it may still be in
// flight (s_waitcnt vmcnt(kPerStage * (kRing - 1 - s))). s is a constant once
// the tail loop is unrolled, so the switch folds to one wait.
template <int kPerStage, int kRing>
__device__ __forceinline__ void wait_stage(int s) {
  static_assert(kRing >= 1 && kRing <= 8, "tail waits cover rings of 1 to 8 stages");
  switch (s) {
    case 0: wait_vmcnt<kPerStage * (kRing - 1)>(); break;
    case 1: if constexpr (kRing > 1) wait_vmcnt<kPerStage * (kRing - 2)>(); break;
    case 2: if constexpr (kRing > 2) wait_vmcnt<kPerStage * (kRing - 3)>(); break;
    case 3: if constexpr (kRing > 3) wait_vmcnt<kPerStage * (kRing - 4)>(); break;
    case 4: if constexpr (kRing > 4) wait_vmcnt<kPerStage * (kRing - 5)>(); break;
    case 5: if constexpr (kRing > 5) wait_vmcnt<kPerStage * (kRing - 6)>(); break;
    case 6: if constexpr (kRing > 6) wait_vmcnt<kPerStage * (kRing - 7)>(); break;
    case 7: if constexpr (kRing > 7) wait_vmcnt<kPerStage * (kRing - 8)>(); break;
    default: break;
  }
}

__device__ __forceinline__ uint32_t word(const u32x4_t& v, int w) {
  return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
}

// Geometry of one token row. kKv = bytes per K/V element: 4 (fp32 cache, fp32
// q/out), 2 (bf16 cache, bf16 q/out) or 1 (fp8 e4m3 cache, bf16 q/out). Lane
// `sub` of a row holds the elements of dims j*kDimStride + sub*kPerLoad ..
// +kPerLoad-1 for j < kLoads: one 16-byte K/V load each, and the q elements of
// the same dims.
template <int kKv, int D>
struct Row {
  static constexpr bool kQoBF16 = kKv < 4;               // q and out in bf16
  static constexpr int kQoBytes = kQoBF16 ? 2 : 4;
  static constexpr int kBytes = D * kQoBytes;            // one q / out row
  static constexpr int kKvBytes = D * kKv;               // one K / V row
  static constexpr int kLoads = kKvBytes / 128;          // 16-byte K/V loads per lane
  static constexpr int kKvWords = kLoads * 4;            // K/V words per lane
  static constexpr int kElems = D / 8;                   // elements per lane
  static constexpr int kPerLoad = 16 / kKv;              // elements per K/V load
  static constexpr int kDimStride = 128 / kKv;           // dims between a lane's loads
  static constexpr int kWords = kElems * kQoBytes / 4;   // q words per lane
  static constexpr int kQLoads = kPerLoad * kQoBytes / 16;  // 16-byte q loads per K/V load
  static_assert(kLoads >= 1, "K/V row shorter than 128 bytes");
};

// Cross-lane exchanges over lane bits 5, 4 and 3 without the LDS path.
// permlane32_swap(x, y) swaps the upper 32 lanes of x with the lower 32 lanes
// of y; the sum of the two swapped registers is, in lanes 0..31, x + x's
// value in lane l+32, and in lanes 32..63, y + y's value in lane l-32.
// permlane16_swap does the same for odd and even 16-lane rows; a DPP row
// rotate by 8 reads lane l ^ 8.
__device__ __forceinline__ float swap_sum32(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_sum16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float row_ror8(float x) {
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), 0x128, 0xF, 0xF, false));
}
// max / sum over the 8 lanes l, l^8, l^16, ..., l^56 (the same `sub`)
__device__ __forceinline__ float group_max8(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  return fmaxf(x, row_ror8(x));
}
__device__ __forceinline__ float group_sum8(float x) {
  x = swap_sum32(x, x);
  x = swap_sum16(x, x);
  return x + row_ror8(x);
}

// Partial states cross XCDs, whose L2 caches are private. Every store and
// load of a partial is an agent-scope relaxed atomic, which gfx950 issues
// with the sc1 cache policy: the store writes through to the device-coherent
// level and the load reads from it, so no L2 writeback or invalidation
// (what an agent-scope fence costs, once per wave) is needed. Pairs of floats
// move as one 64-bit access.
__device__ __forceinline__ void store_shared(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_shared2(float* p, float a, float b) {
  const uint64_t u = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_shared(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_shared2(const float* p) {
  const uint64_t u = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32)));
}

// Completes the merge tree of a cut request after this wave wrote its chunk's
// partial state. Each node counts its children's arrivals (shared-prefix
// partials, written by an earlier kernel, are already in place and do not
// report); the wave whose arrival completes a node merges all of the node's
// children (in slot order, so the
// result does not depend on which wave arrives last), resets the counter for
// the next run, and reports the merged state to the parent, or writes the
// output at the root. Before its arrival is counted the wave waits for its
// partial stores to complete (vmcnt 0): write-through stores complete only
// once they are visible device-wide. The merging wave issues its loads only
// after the counter read that elected it has returned.
//
// The merge (the closed form for softmax over a union of disjoint token sets,
// in log2 units) is latency-bound and often the last thing a kernel does, so
// its loads go out in as few rounds as possible. Round one reads every
// child's LSE (value i = child * G + head in lane i % 64) together with the
// outputs of the first kB children; the per-head maximum and weight sum come
// from butterfly reductions over the lanes of one head (lanes equal mod G),
// and the weights go to LDS (s_w, FI_MERGE_FAN_IN * G floats; zero past the
// last child). Outputs move as float pairs: lane l takes floats 2l + 128c
// (c < NC) of a slot's G*D block, so each load covers 512 contiguous bytes.
// The wave is its whole work-group and a wave's LDS accesses execute in
// order, so the weights need only a compiler barrier, not s_barrier (whose
// fence would wait for the output loads still in flight).
template <int kKv, int D, int G>
__device__ void finish_split(const DecodeParams& p, int node, int lane, float* s_w) {
  constexpr int kF = G * D;                           // floats per slot
  constexpr int NC = (kF / 2 + 63) / 64;              // float pairs per lane
  constexpr int kV = (FI_MERGE_FAN_IN * G + 63) / 64; // LSE values per lane
  constexpr int kB = 64 / NC < 16 ? 64 / NC : 16;     // children in round one
  static_assert(kB <= FI_MERGE_FAN_IN, "round one reads past the weights");
  int hc[NC];  // query head (within the group) of each pair of this lane
#pragma unroll
  for (int c = 0; c < NC; ++c) hc[c] = (2 * lane + 128 * c) / D;
  for (;;) {
    // the node's fields are read-only: fetch them with the arrival
    const int32_t* nd = p.nodes + (int64_t)node * FI_NODE_STRIDE;
    const int count = nd[FI_NODE_COUNT];
    const int arrivals = nd[FI_NODE_ARRIVALS];  // children that report here
    const int sb = nd[FI_NODE_SLOT_BEGIN];
    const int parent = nd[FI_NODE_PARENT];
    const int out_slot = nd[FI_NODE_OUT_SLOT];
    const int b = nd[FI_NODE_REQUEST];
    const int kvh = nd[FI_NODE_KV_HEAD];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    int old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(p.counters + node, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != arrivals - 1) return;
    if (lane == 0) __hip_atomic_store(p.counters + node, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    float sv[kV];
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      const int i = lane + 64 * j;
      sv[j] = i < count * G ? load_shared(p.part_lse + (int64_t)sb * G + i) : -INFINITY;
    }
    float2 v[kB][NC];  // children past the last re-read it, with weight 0
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      const float* src = p.part_o + (int64_t)(sb + min(i, count - 1)) * kF;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int f = 2 * lane + 128 * c;
        v[i][c] = (kF >= 128 || f < kF) ? load_shared2(src + f) : make_float2(0.f, 0.f);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kV; ++j) mx = fmaxf(mx, sv[j]);
#pragma unroll
    for (int o = G; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float ws = 0.f;
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      const float w = sv[j] == -INFINITY ? 0.f : exp2_fast(sv[j] - mx);
      s_w[lane + 64 * j] = w;
      ws += w;
    }
#pragma unroll
    for (int o = G; o < 64; o <<= 1) ws += __shfl_xor(ws, o);
    asm volatile("" ::: "memory");
    // lane h < G now holds the maximum and weight sum of head h

    float2 acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = make_float2(0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kB; ++i) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float w = s_w[i * G + hc[c]];
        acc[c].x = __builtin_fmaf(w, v[i][c].x, acc[c].x);
        acc[c].y = __builtin_fmaf(w, v[i][c].y, acc[c].y);
      }
    }
#pragma unroll 8
    for (int i = kB; i < count; ++i) {
      const float* src = p.part_o + (int64_t)(sb + i) * kF;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int f = 2 * lane + 128 * c;
        if (kF >= 128 || f < kF) {
          const float w = s_w[i * G + hc[c]];
          const float2 x = load_shared2(src + f);
          acc[c].x = __builtin_fmaf(w, x.x, acc[c].x);
          acc[c].y = __builtin_fmaf(w, x.y, acc[c].y);
        }
      }
    }
    asm volatile("" ::: "memory");  // s_w is rewritten by the next level
    const float lse2 = mx + log2_fast(ws);  // valid in lanes h < G
    if (parent < 0) {
      const int64_t row0 = (int64_t)b * p.num_qo_heads + (int64_t)kvh * G;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int f = 2 * lane + 128 * c;
        const float inv = p.v_scale / __shfl(ws, hc[c]);
        if (kF >= 128 || f < kF) {
          if constexpr (Row<kKv, D>::kQoBF16)
            *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(p.out) + row0 * D + f) =
                pack_bf16(acc[c].x * inv, acc[c].y * inv);
          else
            *reinterpret_cast<float2*>(reinterpret_cast<float*>(p.out) + row0 * D + f) =
                make_float2(acc[c].x * inv, acc[c].y * inv);
        }
      }
      if (lane < G && p.lse) p.lse[row0 + lane] = lse2 * kLn2;
      return;
    }
    float* dst = p.part_o + (int64_t)out_slot * kF;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int f = 2 * lane + 128 * c;
      const float inv = 1.f / __shfl(ws, hc[c]);
      if (kF >= 128 || f < kF) store_shared2(dst + f, acc[c].x * inv, acc[c].y * inv);
    }
    if (lane < G) store_shared(p.part_lse + (int64_t)out_slot * G + lane, lse2);
    node = parent;
  }
}

// Kernel parameters from the launch arguments.
inline DecodeParams make_decode_params(const DecodeArgs& a) {
  const int row = a.head_dim * a.kv_bytes;  // one K/V row
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
  prm.nodes = a.nodes;
  prm.counters = a.counters;
  prm.head_stride = a.page_size * row;
  prm.page_stride = (int64_t)a.num_kv_heads * a.page_size * row;
  prm.num_qo_heads = a.num_qo_heads;
  prm.page_size = a.page_size;
  prm.step_pages = 8 / a.page_size;
  prm.step_slots = 8 % a.page_size;
  // the K dequantisation scale multiplies every score, the V one the output
  prm.scale_log2 = a.sm_scale * a.k_scale * kLog2e;
  prm.v_scale = a.v_scale;
  prm.rope_log2_theta = a.rope ? std::log2((double)a.rope_theta) : 0.0;
  prm.rope_rev = a.rope ? 1.0 / (2.0 * M_PI * (double)a.rope_scale) : 0.0;
  return prm;
}

}  // namespace
}  // namespace fi

