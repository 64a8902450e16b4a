// Multi-head latent attention (MLA) over a paged latent cache, on the matrix
// cores of gfx950 (bf16).
//
// FlashInfer 0.6.17 release write-up (llm-wiki.hwlabs.dev), section 2 on
// Blackwell and Kimi K3 MLA support: MLA caches one compressed latent vector
// per token; restoring per-head K and V from it by up-projection and writing
// them to shared memory before attention was the bottleneck, which the kernel
// removes by packing query-token rows and query-head rows into one tile, for
// any head count and several (speculative) query tokens per request. Here the
// up-projections are folded into the query (q_nope) and the output by the
// caller, so nothing is ever restored: every (query token, head) row scores
// a token as sm_scale (q_nope . c + q_pe . k_pe) against the cached latent c
// (512) and rotary key k_pe (64), and averages the latents. All rows of a
// request read the same cache rows, so one latent row in LDS serves them all.
//
// Work item: a tile of 32 (query token, head) rows of one request over one
// chunk of its tokens (whole pages). One workgroup of 4 waves, one per SIMD;
// each wave scores all 32 rows against every token of a block (the same
// scores and softmax state in every wave) and owns a quarter of the output,
// 128 latent dims. Per 32-token block and wave:
//   S^T[token, row] = K . Q^T     v_mfma_f32_32x32x16_bf16, 36 depth steps
//                                 (32 over the latent, 4 over the rotary key)
//   online softmax per row (a lane owns one row: 16 tokens in the lane, the
//   other 16 in lane l^32), running max raised lazily
//   O^T[d, row] += V^T . P^T      2 token steps x 4 tiles of 32 dims, P split
//                                 in two bf16 parts (hi + lo) for precision
// Lane layout of v_mfma_f32_32x32x16_bf16 (A 32x16, B 16x32, C 32x32):
// A[m][k] in lane m + 32*(k/8), element k%8; B[k][n] in lane n + 32*(k/8);
// C[m][n] in lane n + 32*((m%8)/4), element 4*(m/8) + m%4. P^T comes straight
// from the S^T accumulators (the PV contraction index enumerates the block's
// tokens in the order the S^T layout leaves them); V^T fragments come from
// the row-major latent rows through ds_read_b64_tr_b16 (within each 16-lane
// group, output lane 4p+q element k is element q of input lane 4k+p).
//
// LDS ring of 4 stages of 32 tokens, filled by direct-to-LDS loads: a
// latent row is one wave-wide 1 KiB load, placed at a row pitch of 1072
// bytes (48 bytes of padding: 268 words, 12 banks apart, so the 16 lanes of
// a K fragment read -- 16 rows, one 16-byte piece -- and of a transposed V
// read -- 4 rows x 32 bytes -- fall in distinct banks, and every fragment
// address is a lane base plus a compile-time offset); the rotary keys follow
// as 128-byte rows, eight per wave-wide load, their 16-byte pieces
// XOR-swizzled by (row / 2) mod 8.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "fi_bsr.h"
#include "kernels.h"

namespace fi {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;

constexpr int kDc = 512;                      // latent width
constexpr int kDr = 64;                       // rotary-key width
constexpr int kRows = FI_MLA_ROWS;            // rows per tile
constexpr int kWaves = 4;
constexpr int kDw = kDc / kWaves;             // output dims per wave
constexpr int kBlk = 32;                      // tokens per ring stage
constexpr int kStages = 4;
constexpr int kCRow = kDc * 2 + 48;           // LDS pitch of a latent row
constexpr int kCBytes = kBlk * kCRow;
constexpr int kPBytes = kBlk * kDr * 2;
constexpr int kStageBytes = kCBytes + kPBytes;
constexpr int kSteps = (kDc + kDr) / 16;      // depth steps of the score product
constexpr int kLoadsPerWave = kBlk / kWaves + 1;  // direct-to-LDS loads per wave and block
constexpr int kIds = FI_PREFILL_MAX_PAGES;    // page-id window
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kMargin = 8.0f;  // lazy-rescale margin, log2 units
static_assert(kWaves * 64 >= kIds, "one page id per thread");
static_assert(kBlk / kWaves == 8, "a wave loads eight latent rows and eight rotary-key rows");

struct MlaParams {
  const int32_t* items;     // [num_items][FI_QITEM_STRIDE]
  const int32_t* merges;    // [num_merges][FI_QMERGE_STRIDE]
  const int32_t* page_ids;  // the requests' page lists
  const char* q_nope;       // bf16 [N, H, 512]
  const char* q_pe;         // bf16 [N, H, 64]
  const char* ckv;          // bf16 [pages, P, 512]
  const char* kpe;          // bf16 [pages, P, 64]
  __bf16* out;              // bf16 [N, H, 512]
  float* lse;               // [N, H] natural log, or null
  float* part_o;            // [slots, kRows, 512]
  float* part_lse;          // [slots, kRows], log2 units
  int num_heads;
  int page_size;
  uint32_t page_magic;     // ceil(2^32 / page_size) mod 2^32
  uint32_t page_magic_hi;  // 1 when page_size is 1 (the quotient is then 2^32)
  int causal;
  float scale_log2;        // sm_scale * log2(e)
};

__device__ __forceinline__ uint32_t lds_u32(const void* p) { return (uint32_t)(uintptr_t)p; }

// LDS reads at a lane address plus a compile-time offset (the instruction's
// offset field), as inline asm: the compiler cannot tell which ring stage a
// direct-to-LDS load writes and would wait for every load in flight before a
// plain read. The waits are explicit instead.
template <int OFF>
__device__ __forceinline__ u32x4_t lds_b128(uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x4_t r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF) : "memory");
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2_t lds_tr_b64(uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF) : "memory");
  return r;
}
// One page id, read and waited for in one statement (the wait covers LDS
// operations only; the ring's loads are counted by vmcnt).
__device__ __forceinline__ int lds_id(const int* p) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_u32(p)) : "memory");
  return v;
}

// s_waitcnt vmcnt(n), leaving the other counters unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(CNT), then every register of r redefined by an empty asm
// statement ordered after the wait: no use of a value read can be scheduled
// above it.
template <int CNT, typename T, int N>
__device__ __forceinline__ void lgkm_wait_then(T (&r)[N]) {
  static_assert(CNT >= 0 && CNT < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(CNT) : "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(r[i]));
}

template <int I, int N>
struct StaticFor {
  template <class F>
  __device__ __forceinline__ static void run(F& f) {
    if constexpr (I < N) {
      f(std::integral_constant<int, I>{});
      StaticFor<I + 1, N>::run(f);
    }
  }
};
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  StaticFor<0, N>::run(f);
}

// Two floats rounded to a packed bf16 pair (nearest even), and the pair's
// rounding errors rounded to a second pair: hi + lo is within ~2^-16 of the
// inputs.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const f32x2_t f = {a, b};
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
  const f32x2_t r = {a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
}

__device__ __forceinline__ float max_with_partner32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__global__ __launch_bounds__(256, 1) void mla_attend_kernel(MlaParams p) {
  __shared__ __attribute__((aligned(1024))) char s_ring[kStages * kStageBytes];
  __shared__ int s_pid[kIds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int H = p.num_heads;
  const int d0 = kDw * wave;  // first output dim of this wave

  const int32_t* it = p.items + (int64_t)blockIdx.x * FI_QITEM_STRIDE;
  const int qo_row = it[FI_QITEM_QO_ROW];
  const int nqo = it[FI_QITEM_NUM_QO];
  const int kv_begin = it[FI_QITEM_KV_BEGIN];
  const int ntok = it[FI_QITEM_NUM_KV];
  const int visible = it[FI_QITEM_VISIBLE];
  const int page_begin = it[FI_QITEM_PAGE_BEGIN];
  const int slot = it[FI_QITEM_SLOT];
  const int head_begin = it[FI_QITEM_HEAD_BEGIN];

  // this lane's row (column n = lane % 32 of the tiles): (query token, head)
  // number head_begin + lane % 32, token-major from the tile's first token
  const int row = lane & 31;
  const int f = head_begin + row;
  const bool row_ok = f < nqo * H;
  const int qi = row_ok ? f / H : 0;
  const int64_t q_index = (int64_t)(qo_row + qi) * H + (row_ok ? f - qi * H : 0);
  // tokens of the chunk this row attends (may be <= 0)
  const int lim = min(visible + (p.causal ? qi : 0) - kv_begin, ntok);

  if (ntok == 0) {
    // a tile that attends nothing (no mask, a request with no pages):
    // out = 0, lse = -inf, no cache read at all
    if (row_ok) {
      __bf16* dst = p.out + q_index * kDc + d0;
      for (int d = 4 * half; d < kDw; d += 8) *reinterpret_cast<uint2*>(dst + d) = make_uint2(0u, 0u);
      if (wave == 0 && half == 0 && p.lse) p.lse[q_index] = -INFINITY;
    }
    return;
  }

  // ---- the chunk's pages (it starts on a page boundary; at most kIds)
  const int P = p.page_size;
  const int npg = (ntok + P - 1) / P;
  if (tid < kIds) s_pid[tid] = p.page_ids[page_begin + min(tid, npg - 1)];

  // Q^T as the B operand: lane holds Q[row][16s + 8*half .. +8] for depth
  // step s (latent part for s < 32, rotary part after); a padding row loads
  // the tile's first row and zeroes it, so the loads are unconditional
  bf16x8_t qf[kSteps];
  {
    const char* qn = p.q_nope + q_index * (kDc * 2);
    const char* qp = p.q_pe + q_index * (kDr * 2);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      uint4 v = s < kDc / 16 ? *reinterpret_cast<const uint4*>(qn + (16 * s + 8 * half) * 2)
                             : *reinterpret_cast<const uint4*>(qp + (16 * (s - kDc / 16) + 8 * half) * 2);
      if (!row_ok) v = make_uint4(0, 0, 0, 0);
      qf[s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  // q and the page ids are in before any ring load is issued, so the vmcnt
  // waits below count ring loads only
  wait_vmcnt<0>();
  __syncthreads();

  // ---- direct-to-LDS loads of block j into stage st. Wave w loads rows
  // 8w .. 8w+7 of the block: their rotary keys with one wave-wide load (lane
  // l: row 8w + l/8, swizzled piece l%8 from the global piece it stands
  // for), and each latent row with one wave-wide load (lane l: bytes 16l ..
  // +15) whose pool row comes from lane 8i. Rows past the chunk's end
  // re-read its last token (the same number of loads on every path, so the
  // vmcnt waits are exact). The latent rows are read by every tile of the
  // chunk, so the loads stay cacheable.
  const uint32_t pmag = p.page_magic, pmag_hi = p.page_magic_hi;
  const uint32_t psz = (uint32_t)P;
  const int my_t = 8 * wave + (lane >> 3);
  const int kslot = (lane & 7) ^ ((my_t >> 1) & 7);
  auto issue = [&](int j, int st) {
    const uint32_t tok = (uint32_t)min(j * kBlk + my_t, ntok - 1);
    const uint32_t pg = __umulhi(tok, pmag) + tok * pmag_hi;
    const uint32_t rip = tok - pg * psz;
    const int64_t prow = (int64_t)lds_id(&s_pid[pg]) * P + rip;  // row of the pools
    char* stage = s_ring + st * kStageBytes;
    __builtin_amdgcn_global_load_lds((global_void_t*)(p.kpe + prow * (kDr * 2) + kslot * 16),
                                     (lds_void_t*)(stage + kCBytes + 8 * wave * (kDr * 2)), 16, 0, 0);
    const uint32_t rlo = (uint32_t)prow, rhi = (uint32_t)((uint64_t)prow >> 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint64_t r = ((uint64_t)__builtin_amdgcn_readlane(rhi, 8 * i) << 32) |
                         __builtin_amdgcn_readlane(rlo, 8 * i);
      __builtin_amdgcn_global_load_lds((global_void_t*)(p.ckv + r * (kDc * 2) + lane * 16),
                                       (lds_void_t*)(stage + (8 * wave + i) * kCRow), 16, 0, 0);
    }
  };

  // LDS byte offsets that depend only on the lane. K fragment of depth step
  // s < 32: token row lane % 32, latent piece 2s + half (lane base + 32 s);
  // rotary steps: piece 2(s-32) + half of the swizzled 128-byte row. V^T
  // fragment of tile t, token step ks and run r (input role: token 16 ks +
  // 8 r + 4 (g16/2) + v_k, dims d0 + 32 t + 16 (g16%2) + 4 v_p .. +3): lane
  // base plus (16 ks + 8 r) rows and 64 t bytes.
  const int m = lane & 31;
  const uint32_t kbase = m * kCRow + 16 * half;
  uint32_t pbase[kDr / 16];
#pragma unroll
  for (int s = 0; s < kDr / 16; ++s) pbase[s] = kCBytes + m * (kDr * 2) + 16 * ((2 * s + half) ^ ((m >> 1) & 7));
  const int g16 = lane >> 4, L16 = lane & 15;
  const uint32_t vbase = (4 * (g16 >> 1) + (L16 >> 2)) * kCRow + 2 * (d0 + 16 * (g16 & 1) + 4 * (L16 & 3));

  f32x16_t o[kDw / 32];
#pragma unroll
  for (int t = 0; t < kDw / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int nblocks = (ntok + kBlk - 1) / kBlk;
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) issue(s, s);

  // Scores stay unscaled; exp2(c * s - c * m) is one fma and an exp. The
  // running max is raised only when a block's max passes it by more than
  // kMargin in log2 units (weights stay <= 2^kMargin), so the accumulators
  // are rescaled rarely after the first block.
  const float c = p.scale_log2;
  const float margin = kMargin / c;
  const uint32_t ring = lds_u32(s_ring);

  for (int j = 0; j < nblocks; ++j) {
    const int st = j % kStages;
    // this wave's loads of block j have landed (later blocks may be in flight)
    wait_vmcnt<kLoadsPerWave * (kStages - 2)>();
    // every wave's loads of block j have landed, and every wave is done
    // reading block j-1, whose stage is refilled below
    __builtin_amdgcn_s_barrier();
    const uint32_t sb = ring + st * kStageBytes;

    // ---- S^T = K . Q^T: 36 depth steps, fragments read in groups of 4,
    // the next group requested before the current one's products
    f32x16_t sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
    u32x4_t kf[2][4];
    auto read_group = [&](auto G, u32x4_t(&dst)[4]) {
      constexpr int g = decltype(G)::value;
      if constexpr (g < kDc / 64) {
        dst[0] = lds_b128<32 * (4 * g + 0)>(sb + kbase);
        dst[1] = lds_b128<32 * (4 * g + 1)>(sb + kbase);
        dst[2] = lds_b128<32 * (4 * g + 2)>(sb + kbase);
        dst[3] = lds_b128<32 * (4 * g + 3)>(sb + kbase);
      } else {
        dst[0] = lds_b128<0>(sb + pbase[0]);
        dst[1] = lds_b128<0>(sb + pbase[1]);
        dst[2] = lds_b128<0>(sb + pbase[2]);
        dst[3] = lds_b128<0>(sb + pbase[3]);
      }
    };
    read_group(std::integral_constant<int, 0>{}, kf[0]);
    static_for<kSteps / 4>([&](auto G) {
      constexpr int g = decltype(G)::value;
      if constexpr (g + 1 < kSteps / 4) {
        read_group(std::integral_constant<int, g + 1>{}, kf[(g + 1) & 1]);
        lgkm_wait_then<4>(kf[g & 1]);
      } else {
        lgkm_wait_then<0>(kf[g & 1]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[g & 1][i]),
                                                     qf[4 * g + i], sc, 0, 0, 0);
    });

    // the loads of a later block go out while the products run
    issue(j + kStages - 1, (j + kStages - 1) % kStages);

    // ---- V^T fragments of both 16-token steps, requested now so that they
    // arrive during the softmax step below
    u32x2_t va[2][kDw / 32][2];
    static_for<2>([&](auto KS) {
      constexpr int ks = decltype(KS)::value;
      static_for<kDw / 32>([&](auto T) {
        constexpr int t = decltype(T)::value;
        va[ks][t][0] = lds_tr_b64<(16 * ks) * kCRow + 64 * t>(sb + vbase);
        va[ks][t][1] = lds_tr_b64<(16 * ks + 8) * kCRow + 64 * t>(sb + vbase);
      });
    });

    // ---- online softmax over the block; element r holds token
    // 4*half + 8*(r/4) + r%4 of the block
    const int tok0 = j * kBlk;
    if (__builtin_amdgcn_ballot_w64(tok0 + kBlk > lim)) {  // some row stops in here
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (tok0 + 4 * half + 8 * (r >> 2) + (r & 3) >= lim) sc[r] = -INFINITY;
    }
    float mb = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mb = fmaxf(mb, sc[r]);
    mb = max_with_partner32(mb);  // -inf if the row attends none of these tokens
    const bool up = mb > m_run + margin;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float alpha = up ? __builtin_amdgcn_exp2f((m_run - mb) * c) : 1.f;  // 0 at first
      l_run *= alpha;
      if (j > 0) {  // the accumulators are still zero on the first block
#pragma unroll
        for (int t = 0; t < kDw / 32; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
      }
      m_run = up ? mb : m_run;
    }
    // a row with no token yet has m = -inf and only masked scores: weight 0
    const float mc = m_run == -INFINITY ? 0.f : m_run * c;

    lgkm_wait_then<0>(va[0][0]);
    lgkm_wait_then<0>(va[0][1]);
    lgkm_wait_then<0>(va[0][2]);
    lgkm_wait_then<0>(va[0][3]);
    lgkm_wait_then<0>(va[1][0]);
    lgkm_wait_then<0>(va[1][1]);
    lgkm_wait_then<0>(va[1][2]);
    lgkm_wait_then<0>(va[1][3]);

    // ---- P = exp2(c s - c m), then O^T += V^T . P^T. Step ks takes
    // elements 8ks .. 8ks+7: contraction index 8*half + i is token
    // 4*half + 16ks + 8*(i/4) + i%4 of the block. P is multiplied as two
    // bf16 parts, hi = P rounded to bf16 and lo = the rounding error rounded
    // again: P alone in bf16 carries a relative error up to 2^-8, which a row
    // that attends few tokens does not average away.
    float ps = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint32_t phw[4], plw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(sc[8 * ks + 2 * i], c, -mc));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(sc[8 * ks + 2 * i + 1], c, -mc));
        ps += e0 + e1;
        split_bf16x2(e0, e1, phw[i], plw[i]);
      }
      const bf16x8_t ph = __builtin_bit_cast(bf16x8_t, u32x4_t{phw[0], phw[1], phw[2], phw[3]});
      const bf16x8_t pl = __builtin_bit_cast(bf16x8_t, u32x4_t{plw[0], plw[1], plw[2], plw[3]});
      bf16x8_t vfr[kDw / 32];
#pragma unroll
      for (int t = 0; t < kDw / 32; ++t)
        vfr[t] = __builtin_bit_cast(bf16x8_t, u32x4_t{va[ks][t][0][0], va[ks][t][0][1],
                                                      va[ks][t][1][0], va[ks][t][1][1]});
#pragma unroll
      for (int t = 0; t < kDw / 32; ++t) o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[t], ph, o[t], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < kDw / 32; ++t) o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[t], pl, o[t], 0, 0, 0);
    }
    l_run += sum_with_partner32(ps);
  }
  // loads past the end may still be landing in the ring
  wait_vmcnt<0>();

  // ---- this row's state over the wave's 128 dims: o / l and lse; a row
  // that attended nothing has o = 0 and lse = -inf
  if (!row_ok) return;
  const bool empty = l_run == 0.f;
  const float inv = empty ? 0.f : 1.f / l_run;
  const float lse2 = empty ? -INFINITY : m_run * c + __builtin_amdgcn_logf(l_run);
  if (slot < 0) {
    __bf16* dst = p.out + q_index * kDc + d0;
#pragma unroll
    for (int t = 0; t < kDw / 32; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // elements 4*q4 .. +3 are dims 32t + 8*q4 + 4*half .. +3
        const bf16x4_t v = {(__bf16)(o[t][4 * q4] * inv), (__bf16)(o[t][4 * q4 + 1] * inv),
                            (__bf16)(o[t][4 * q4 + 2] * inv), (__bf16)(o[t][4 * q4 + 3] * inv)};
        *reinterpret_cast<bf16x4_t*>(dst + 32 * t + 8 * q4 + 4 * half) = v;
      }
    if (wave == 0 && half == 0 && p.lse) p.lse[q_index] = lse2 * kLn2;
    return;
  }
  float* dst = p.part_o + ((int64_t)slot * kRows + row) * kDc + d0;
#pragma unroll
  for (int t = 0; t < kDw / 32; ++t)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<float4*>(dst + 32 * t + 8 * q4 + 4 * half) =
          make_float4(o[t][4 * q4] * inv, o[t][4 * q4 + 1] * inv, o[t][4 * q4 + 2] * inv,
                      o[t][4 * q4 + 3] * inv);
  if (wave == 0 && half == 0) p.part_lse[(int64_t)slot * kRows + row] = lse2;
}

// Folds the chunk states of cut tiles (log2-unit lse) into bf16 out and
// natural-log lse: the closed form of softmax over a disjoint union of token
// sets (FlashInfer paper explainer, visionhong.com, benchmark section: the
// split scheduler's pieces are merged). A thread per (row, 4 dims), two rows
// per workgroup; the chunks are summed in slot order.
__global__ __launch_bounds__(256) void mla_merge_kernel(MlaParams p) {
  const int32_t* mg = p.merges + (int64_t)blockIdx.x * FI_QMERGE_STRIDE;
  const int r = blockIdx.y * 2 + (threadIdx.x >> 7);
  const int H = p.num_heads;
  const int f = mg[FI_QMERGE_HEAD_BEGIN] + r;
  if (f >= mg[FI_QMERGE_NUM_QO] * H) return;
  const int qi = f / H;
  const int64_t q_index = (int64_t)(mg[FI_QMERGE_QO_ROW] + qi) * H + (f - qi * H);
  const int64_t slot0 = mg[FI_QMERGE_SLOT_BEGIN];
  const int k = mg[FI_QMERGE_NUM_CHUNKS];
  const int c4 = 4 * (threadIdx.x & 127);
  const float* lse_r = p.part_lse + slot0 * kRows + r;
  float mx = -INFINITY;
  for (int ch = 0; ch < k; ++ch) mx = fmaxf(mx, lse_r[(int64_t)ch * kRows]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  if (mx != -INFINITY) {
#pragma unroll 4
    for (int ch = 0; ch < k; ++ch) {
      const float s = lse_r[(int64_t)ch * kRows];
      // a chunk the row attended nothing of has s = -inf and weight 0
      const float w = s == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s - mx);
      const float4 v = *reinterpret_cast<const float4*>(p.part_o + ((slot0 + ch) * kRows + r) * kDc + c4);
      den += w;
      acc.x += w * v.x;
      acc.y += w * v.y;
      acc.z += w * v.z;
      acc.w += w * v.w;
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const bf16x4_t v = {(__bf16)(acc.x * inv), (__bf16)(acc.y * inv), (__bf16)(acc.z * inv),
                      (__bf16)(acc.w * inv)};
  *reinterpret_cast<bf16x4_t*>(p.out + q_index * kDc + c4) = v;
  if (c4 == 0 && p.lse) p.lse[q_index] = den > 0.f ? (mx + __builtin_amdgcn_logf(den)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_mla(const MlaArgs& a, hipStream_t stream) {
  if (a.num_items <= 0) return hipSuccess;
  MlaParams p{};
  p.items = a.items;
  p.merges = a.merges;
  p.page_ids = a.page_ids;
  p.q_nope = static_cast<const char*>(a.q_nope);
  p.q_pe = static_cast<const char*>(a.q_pe);
  p.ckv = static_cast<const char*>(a.ckv);
  p.kpe = static_cast<const char*>(a.kpe);
  p.out = static_cast<__bf16*>(a.out);
  p.lse = a.lse;
  p.part_o = a.part_o;
  p.part_lse = a.part_lse;
  p.num_heads = a.num_heads;
  p.page_size = a.page_size;
  const uint64_t mg = ((1ull << 32) + (uint64_t)a.page_size - 1) / (uint64_t)a.page_size;
  p.page_magic = (uint32_t)mg;
  p.page_magic_hi = (uint32_t)(mg >> 32);
  p.causal = a.causal;
  p.scale_log2 = a.sm_scale * kLog2e;
  hipLaunchKernelGGL(mla_attend_kernel, dim3((uint32_t)a.num_items), dim3(64 * kWaves), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_merges <= 0) return e;
  hipLaunchKernelGGL(mla_merge_kernel, dim3((uint32_t)a.num_merges, kRows / 2), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fi
