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
// chunk of its tokens (whole pages). One workgroup of 4 waves and 80 KiB of
// LDS, so two workgroups share a CU (two waves per SIMD, independent of each
// other). Wave w takes rows 16 (w/2) .. +15 of the tile and output dims
// 256 (w%2) .. +255. The two waves of a row half score one 16-token tile of
// each block each, over the full depth, and swap the raw scores through LDS,
// so both hold the block's 32 scores per row and the same softmax state.
// Per 32-token block and wave:
//   S^T[token, row] = K . Q^T     v_mfma_f32_16x16x32_bf16: the wave's token
//                                 tile x 18 depth steps (16 over the latent,
//                                 2 over the rotary key), then the partner's
//                                 tile from LDS
//   online softmax per row (lane n + 16g holds row n and tokens 4g .. 4g+3 of
//   each tile: the row's maximum is a lane-local maximum and two lane swaps;
//   every lane keeps its own running sum), running max raised lazily
//   O^T[d, row] += V^T . P^T      16 dim tiles x 1 token step of 32, P split
//                                 in two bf16 parts (hi + lo) for precision
// Lane layout of v_mfma_f32_16x16x32_bf16: A[m][k] in lane m + 16 (k/8),
// element k%8; B[k][n] in lane n + 16 (k/8), element k%8; C[m][n] in lane
// n + 16 (m/4), element m%4. P^T comes straight from the S^T accumulators:
// contraction slot 8g + e is token 4g + e of tile 0 (e < 4) or 4g + e - 4 of
// tile 1. V^T fragments come from the row-major latent rows through
// ds_read_b64_tr_b16 (within each 16-lane group, output lane 4p+q element k
// is element q of input lane 4k+p), two per tile: tokens 4g .. 4g+3 and
// 16 + 4g .. +3.
//
// A tile whose tokens are cut into several chunks (items) merges in this
// kernel: each chunk writes its partial state and counts its arrival at the
// tile's merge; the chunk that completes the count merges all of them.
//
// LDS ring of 2 stages of 32 tokens, filled by direct-to-LDS loads; a
// block's loads go out as soon as every wave is done with the stage they
// refill, one block ahead. A latent row is one wave-wide 1 KiB load, placed
// at a row pitch of 1072 bytes (48 bytes of padding, 268 words) in a
// permuted row order (lds_row), so K fragment reads and transposed V reads
// are free of bank conflicts and every fragment address is a lane base plus
// a compile-time offset; the rotary keys follow as 128-byte rows, eight per
// wave-wide load, their 16-byte pieces XOR-swizzled by (row / 2) mod 8.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "coherent.h"
#include "fi_bsr.h"
#include "kernels.h"

namespace fi {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;

constexpr int kDc = 512;                      // latent width
constexpr int kDr = 64;                       // rotary-key width
constexpr int kRows = FI_MLA_ROWS;            // rows per tile
constexpr int kWaves = 4;
constexpr int kRw = 16;                       // rows per wave
constexpr int kDw = kDc / 2;                  // output dims per wave
constexpr int kBlk = 32;                      // tokens per ring stage
constexpr int kStages = 2;
constexpr int kCRow = kDc * 2 + 48;           // LDS pitch of a latent row
constexpr int kCBytes = kBlk * kCRow;
constexpr int kPBytes = kBlk * kDr * 2;
constexpr int kStageBytes = kCBytes + kPBytes;
constexpr int kSteps = (kDc + kDr) / 32;      // depth steps of the score product
constexpr int kLatSteps = kDc / 32;
constexpr int kIds = FI_MLA_MAX_PAGES;        // page-id window
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kMargin = 8.0f;  // lazy-rescale margin, log2 units
static_assert(kWaves * 64 >= kIds, "one page id per thread");
static_assert(kRows == 2 * kRw, "a tile is two row halves");
static_assert(kBlk == 8 * kWaves, "each wave loads eight rows of a block");
static_assert(kStages * kStageBytes + kIds * 4 + kWaves * 64 * 16 <= 80 * 1024,
              "two workgroups share a CU's LDS");

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
  int32_t* counters;        // [merges] arrivals, 0 between runs
  float* part_o;            // [slots][kRows * 512] in the kernel's register order
  float* part_lse;          // [slots, kRows], log2 units
  int num_heads;
  int page_size;
  uint32_t page_magic;     // ceil(2^32 / page_size) mod 2^32
  uint32_t page_magic_hi;  // 1 when page_size is 1 (the quotient is then 2^32)
  int causal;
  float scale_log2;        // sm_scale * log2(e)
};

__device__ __forceinline__ uint32_t lds_u32(const void* p) { return (uint32_t)(uintptr_t)p; }

// LDS row of token t of a block: within each 16-token half, tokens 0..7 take
// the even rows and 8..15 the odd ones. At a pitch of 268 words (12 banks mod
// 64) the 16 rows a K fragment read touches (one half) still fall on 16
// distinct 4-bank slots, and the 8 rows a transposed V read of two 16-lane
// groups touches (8 consecutive tokens) on rows 8 banks apart, so neither
// read conflicts on 64 banks.
__device__ __forceinline__ constexpr int lds_row(int t) { return (t & ~15) | ((t & 7) << 1) | ((t >> 3) & 1); }

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
// LDS write of registers a matrix instruction has just written. The
// hardware does not hold an LDS instruction back until an MFMA's results
// are in its destination registers, and the compiler pads only its own
// instructions for that, not inline asm: so the write waits 24 wait states
// itself (more than the longest MFMA needs before its results may be read
// by an LDS instruction).
__device__ __forceinline__ void lds_w128_after_mfma(uint32_t a, u32x4_t v) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\tds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory");
}
// One page id, read and waited for in one statement (the wait covers LDS
// operations only; the ring's loads are counted by vmcnt).
__device__ __forceinline__ int lds_id(const int* p) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_u32(p)) : "memory");
  return v;
}

// A wave's block of a partial state (kRw x kDw floats, 16 KiB) as a buffer
// resource.
__device__ __forceinline__ BufRes wave_partial(const float* part_o, int64_t slot, int wave) {
  return buffer_of(part_o + slot * (kRows * kDc) + wave * (kRw * kDw), kRw * kDw * 4);
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

// The same for V^T fragment pairs.
template <int CNT, int N>
__device__ __forceinline__ void lgkm_wait_then(u32x2_t (&r)[N][2]) {
  static_assert(CNT >= 0 && CNT < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(CNT) : "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(r[i][0]), "+v"(r[i][1]));
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

// maximum / sum over lanes l, l^16, l^32, l^48 (the four lanes of a row)
__device__ __forceinline__ float row_max4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_sum4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__global__ __launch_bounds__(64 * kWaves, 2) void mla_attend_kernel(MlaParams p) {
  __shared__ __attribute__((aligned(1024))) char s_ring[kStages * kStageBytes];
  __shared__ int s_pid[kIds];
  // each wave's token tile of scores, [wave][lane] x 16 bytes
  __shared__ __attribute__((aligned(16))) float s_x[kWaves * 64 * 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rh = wave >> 1;   // row half
  const int dh = wave & 1;    // output-dim half
  const int n = lane & 15;    // this lane's row within the wave's 16
  const int g = lane >> 4;    // 16-lane group
  const int H = p.num_heads;
  const int d0 = kDw * dh;    // first output dim of this wave

  const int32_t* it = p.items + (int64_t)blockIdx.x * FI_QITEM_STRIDE;
  const int qo_row = it[FI_QITEM_QO_ROW];
  const int nqo = it[FI_QITEM_NUM_QO];
  const int kv_begin = it[FI_QITEM_KV_BEGIN];
  const int ntok = it[FI_QITEM_NUM_KV];
  const int visible = it[FI_QITEM_VISIBLE];
  const int page_begin = it[FI_QITEM_PAGE_BEGIN];
  const int slot = it[FI_QITEM_SLOT];
  const int head_begin = it[FI_QITEM_HEAD_BEGIN];

  // this lane's row: (query token, head) number head_begin + row,
  // token-major from the tile's first token
  const int row = kRw * rh + n;
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
      for (int d = 4 * g; d < kDw; d += 16) *reinterpret_cast<uint2*>(dst + d) = make_uint2(0u, 0u);
      if (dh == 0 && g == 0 && p.lse) p.lse[q_index] = -INFINITY;
    }
    return;
  }
  // a row half of padding rows loads and waits like the others but computes
  // nothing
  const bool rows_on = head_begin + kRw * rh < nqo * H;

  // ---- the chunk's pages (it starts on a page boundary; at most kIds)
  const int P = p.page_size;
  const int npg = (ntok + P - 1) / P;
  if (tid < kIds) s_pid[tid] = p.page_ids[page_begin + min(tid, npg - 1)];

  // Q^T as the B operand: lane n + 16g holds Q[row n][32s + 8g .. +8] for
  // depth step s (latent part for s < 16, rotary part after); a padding row
  // loads the tile's first row and zeroes it, so the loads are
  // unconditional. The loads stay in flight while the first block is
  // requested.
  bf16x8_t qf[kSteps];
  {
    const char* qn = p.q_nope + q_index * (kDc * 2);
    const char* qp = p.q_pe + q_index * (kDr * 2);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const uint4 v = s < kLatSteps ? *reinterpret_cast<const uint4*>(qn + (32 * s + 8 * g) * 2)
                                    : *reinterpret_cast<const uint4*>(qp + (32 * (s - kLatSteps) + 8 * g) * 2);
      qf[s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  // the page ids are in LDS before any ring load is issued (q may still be
  // on its way)
  __syncthreads();

  // ---- direct-to-LDS loads of block j into stage st. Wave w loads rows
  // 8w .. 8w+7 of the block: their rotary keys with one wave-wide load (lane
  // l: row 8w + l/8, swizzled piece l%8 from the global piece it stands
  // for), and each latent row with one wave-wide load (lane l: bytes 16l ..
  // +15) whose pool row comes from lane 8i (which looked up row 8w + i). The
  // latent rows are read by every tile of the chunk, so the loads stay
  // cacheable.
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
    static_for<8>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const uint64_t r = ((uint64_t)__builtin_amdgcn_readlane(rhi, 8 * i) << 32) |
                         __builtin_amdgcn_readlane(rlo, 8 * i);
      __builtin_amdgcn_global_load_lds((global_void_t*)(p.ckv + r * (kDc * 2) + lane * 16),
                                       (lds_void_t*)(stage + lds_row(8 * wave + i) * kCRow), 16, 0, 0);
    });
  };

  // LDS byte offsets that depend only on the lane. K fragment of depth step
  // s < 16 of this wave's token tile (tokens 16 dh ..): token row 16 dh + n,
  // latent piece 4s + g (lane base + 64 s); rotary steps: piece 4(s-16) + g
  // of the swizzled 128-byte row (one base per step). V^T fragment of dim
  // tile td (input role: token 4g + L16/4 (+16 for the second read), dims
  // d0 + 16 td + 4 (L16%4) .. +3): lane base + 32 td bytes (+ 16 rows).
  const int kt = 16 * dh + n;  // this lane's token of the K fragments
  const uint32_t kbase = lds_row(kt) * kCRow + 16 * g;
  uint32_t pbase[kSteps - kLatSteps];
#pragma unroll
  for (int s = 0; s < kSteps - kLatSteps; ++s)
    pbase[s] = kCBytes + kt * (kDr * 2) + 16 * ((4 * s + g) ^ ((kt >> 1) & 7));
  const uint32_t xme = lds_u32(s_x) + 1024 * wave + 16 * lane;           // this wave's scores
  const uint32_t xpart = lds_u32(s_x) + 1024 * (wave ^ 1) + 16 * lane;   // the partner's
  const int L16 = lane & 15;
  // (the second read's tokens are 16 later: lds_row adds 16 rows)
  const uint32_t vbase = lds_row(4 * g + (L16 >> 2)) * kCRow + 2 * (d0 + 4 * (L16 & 3));

  f32x4_t o[kDw / 16];
#pragma unroll
  for (int t = 0; t < kDw / 16; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;  // l_run: this lane's share of the row sum

  const int nblocks = (ntok + kBlk - 1) / kBlk;
  issue(0, 0);
  // q (issued before block 0's loads) is in: vector memory loads complete in
  // order, so at most block 0's nine loads remain; from here on only ring
  // loads are in flight
  wait_vmcnt<9>();
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
    if (!row_ok) qf[s] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));

  // Scores stay unscaled; exp2(c * s - c * m) is one fma and an exp. The
  // running max is raised only when a block's max passes it by more than
  // kMargin in log2 units (weights stay <= 2^kMargin), so the accumulators
  // are rescaled rarely after the first block.
  const float c = p.scale_log2;
  const float margin = kMargin / c;
  const uint32_t ring = lds_u32(s_ring);

  for (int j = 0; j < nblocks; ++j) {
    const int st = j & 1;
    // this wave's loads of block j have landed
    wait_vmcnt<0>();
    // every wave's loads of block j have landed, and every wave is done
    // reading block j-1, whose stage the next block's loads refill now
    __builtin_amdgcn_s_barrier();
    if (j + 1 < nblocks) issue(j + 1, st ^ 1);
    if (!rows_on) {
      __builtin_amdgcn_s_barrier();  // the score swap's barrier, kept in step
      continue;
    }
    const uint32_t sb = ring + st * kStageBytes;

    // ---- S^T = K . Q^T for this wave's 16-token tile, 18 depth steps;
    // fragments read six steps at a time, the next group requested before
    // the current group's products
    f32x4_t sme = {0.f, 0.f, 0.f, 0.f};
    u32x4_t kf[2][6];
    auto read_group = [&](auto G, u32x4_t(&dst)[6]) {
      constexpr int gi = decltype(G)::value;
      static_for<6>([&](auto I) {
        constexpr int s = 6 * gi + decltype(I)::value;
        if constexpr (s < kLatSteps)
          dst[decltype(I)::value] = lds_b128<64 * s>(sb + kbase);
        else
          dst[decltype(I)::value] = lds_b128<0>(sb + pbase[s - kLatSteps]);
      });
    };
    read_group(std::integral_constant<int, 0>{}, kf[0]);
    static_for<kSteps / 6>([&](auto G) {
      constexpr int gi = decltype(G)::value;
      if constexpr (gi + 1 < kSteps / 6) {
        read_group(std::integral_constant<int, gi + 1>{}, kf[(gi + 1) & 1]);
        lgkm_wait_then<6>(kf[gi & 1]);
      } else {
        lgkm_wait_then<0>(kf[gi & 1]);
      }
      static_for<6>([&](auto I) {
        constexpr int i = decltype(I)::value;
        sme = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[gi & 1][i]),
                                                      qf[6 * gi + i], sme, 0, 0, 0);
      });
    });
    // swap tiles with the partner wave of the row half (same lanes, same
    // rows): after the barrier both waves hold the block's 32 scores
    lds_w128_after_mfma(xme, u32x4_t{__float_as_uint(sme[0]), __float_as_uint(sme[1]),
                                     __float_as_uint(sme[2]), __float_as_uint(sme[3])});
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    f32x4_t sc[2];
    {
      u32x4_t xo[1];
      xo[0] = lds_b128<0>(xpart);
      lgkm_wait_then<0>(xo);
      const f32x4_t spart = {__uint_as_float(xo[0][0]), __uint_as_float(xo[0][1]), __uint_as_float(xo[0][2]),
                             __uint_as_float(xo[0][3])};
      sc[0] = dh == 0 ? sme : spart;
      sc[1] = dh == 0 ? spart : sme;
    }

    // ---- V^T fragments of the first four dim tiles, requested now so that
    // they arrive during the softmax step below
    u32x2_t va[2][4][2];
    auto read_v = [&](auto H4, u32x2_t(&dst)[4][2]) {
      constexpr int h4 = decltype(H4)::value;
      static_for<4>([&](auto T) {
        constexpr int td = 4 * h4 + decltype(T)::value;
        dst[decltype(T)::value][0] = lds_tr_b64<32 * td>(sb + vbase);
        dst[decltype(T)::value][1] = lds_tr_b64<16 * kCRow + 32 * td>(sb + vbase);
      });
    };
    read_v(std::integral_constant<int, 0>{}, va[0]);

    // ---- online softmax over the block; element e of tile tt holds token
    // 16 tt + 4g + e of the block
    const int tok0 = j * kBlk;
    if (__builtin_amdgcn_ballot_w64(tok0 + kBlk > lim)) {  // some row stops in here
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (tok0 + 16 * tt + 4 * g + e >= lim) sc[tt][e] = -INFINITY;
    }
    float mb = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mb = row_max4(mb);  // -inf if the row attends none of these tokens
    const bool up = mb > m_run + margin;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float alpha = up ? __builtin_amdgcn_exp2f((m_run - mb) * c) : 1.f;  // 0 at first
      l_run *= alpha;
      if (j > 0) {  // the accumulators are still zero on the first block
#pragma unroll
        for (int t = 0; t < kDw / 16; ++t) o[t] *= alpha;
      }
      m_run = up ? mb : m_run;
    }
    // a row with no token yet has m = -inf and only masked scores: weight 0
    const float mc = m_run == -INFINITY ? 0.f : m_run * c;

    // ---- P^T = exp2(c s - c m) as hi + lo bf16 parts (P alone in bf16
    // carries a relative error up to 2^-8, which a row that attends few
    // tokens does not average away), then O^T += V^T . P^T
    float pv[8];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[4 * tt + e] = __builtin_amdgcn_exp2f(fmaf(sc[tt][e], c, -mc));
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      l_run += pv[2 * i] + pv[2 * i + 1];
      split_bf16x2(pv[2 * i], pv[2 * i + 1], hw[i], lw[i]);
    }
    const bf16x8_t ph = __builtin_bit_cast(bf16x8_t, u32x4_t{hw[0], hw[1], hw[2], hw[3]});
    const bf16x8_t pl = __builtin_bit_cast(bf16x8_t, u32x4_t{lw[0], lw[1], lw[2], lw[3]});
    // four groups of four dim tiles, the next group's fragments requested
    // before the current group's products
    static_for<kDw / 64>([&](auto H4) {
      constexpr int h4 = decltype(H4)::value;
      if constexpr (h4 + 1 < kDw / 64) {
        read_v(std::integral_constant<int, h4 + 1>{}, va[(h4 + 1) & 1]);
        lgkm_wait_then<8>(va[h4 & 1]);
      } else {
        lgkm_wait_then<0>(va[h4 & 1]);
      }
      bf16x8_t vt[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        vt[t] = __builtin_bit_cast(bf16x8_t, u32x4_t{va[h4 & 1][t][0][0], va[h4 & 1][t][0][1],
                                                     va[h4 & 1][t][1][0], va[h4 & 1][t][1][1]});
#pragma unroll
      for (int t = 0; t < 4; ++t)
        o[4 * h4 + t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[t], ph, o[4 * h4 + t], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        o[4 * h4 + t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[t], pl, o[4 * h4 + t], 0, 0, 0);
    });
  }
  // the last block's loads may still be landing in the ring
  wait_vmcnt<0>();

  // ---- this row's state over the wave's 256 dims: o / l and lse; a row
  // that attended nothing has o = 0 and lse = -inf
  const float l_tot = row_sum4(l_run);
  const bool empty = l_tot == 0.f;
  const float inv = empty ? 0.f : 1.f / l_tot;
  const float lse2 = empty ? -INFINITY : m_run * c + __builtin_amdgcn_logf(l_tot);
  // lane n + 16g holds O^T[16 td + 4g + e][n], e = 0 .. 3
  if (slot < 0) {
    if (row_ok) {
      __bf16* dst = p.out + q_index * kDc + d0 + 4 * g;
#pragma unroll
      for (int t = 0; t < kDw / 16; ++t) {
        const bf16x4_t v = {(__bf16)(o[t][0] * inv), (__bf16)(o[t][1] * inv), (__bf16)(o[t][2] * inv),
                            (__bf16)(o[t][3] * inv)};
        *reinterpret_cast<bf16x4_t*>(dst + 16 * t) = v;
      }
      if (dh == 0 && g == 0 && p.lse) p.lse[q_index] = lse2 * kLn2;
    }
    return;
  }

  // ---- a cut tile: this chunk's state goes to its partial slot in the
  // order the registers hold it (wave w's 16 x 256 floats as 32 runs of 512
  // bytes, run 2 td + h holding elements 2h, 2h + 1 of dim tile td of every
  // lane), written through to the device-coherent level; then the chunk
  // counts its arrival, and the chunk that arrives last merges the tile.
  const int merge = it[FI_QITEM_MERGE];
  const int32_t* mg = p.merges + (int64_t)merge * FI_QMERGE_STRIDE;
  const int nch = mg[FI_QMERGE_NUM_CHUNKS];
  const int64_t slot0 = mg[FI_QMERGE_SLOT_BEGIN];
  constexpr int kWaveFloats = kRw * kDw;  // 4096
  if (row_ok) {
    float* dst = p.part_o + (int64_t)slot * (kRows * kDc) + wave * kWaveFloats + 2 * lane;
#pragma unroll
    for (int t = 0; t < kDw / 16; ++t) {
      store_coherent2(dst + (2 * t) * 128, o[t][0] * inv, o[t][1] * inv);
      store_coherent2(dst + (2 * t + 1) * 128, o[t][2] * inv, o[t][3] * inv);
    }
    if (dh == 0 && g == 0) store_coherent(p.part_lse + (int64_t)slot * kRows + row, lse2);
  }
  // Each wave's stores are complete (acknowledged by the coherent level)
  // before the barrier, so every store of the work-group is before the
  // arrival that thread 0 issues after it. The page-id window is free now
  // (every wave has left the block loop) and carries the election.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(p.counters + merge, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == nch - 1;
    if (last) __hip_atomic_store(p.counters + merge, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_pid[0] = last;
  }
  __syncthreads();
  if (!s_pid[0] || !row_ok) return;

  // ---- the merge (closed form of softmax over a disjoint union of token
  // sets; FlashInfer paper explainer, visionhong.com, benchmark section: the
  // split scheduler's pieces are merged): each lane folds its own elements
  // of every chunk, in chunk order (so the result does not depend on which
  // chunk finished last), in two passes over half of its runs each, four
  // chunks' loads in flight, the running maximum raised per group of four
  // (a chunk the row attended nothing of has lse = -inf and weight 0).
  // Every load reads the coherent level.
  const float* lse0 = p.part_lse + slot0 * kRows + row;
  __bf16* dst = p.out + q_index * kDc + d0 + 4 * g;
  float mx = -INFINITY, den = 0.f;
  static_for<2>([&](auto PASS) {
    constexpr int kHalf = kDw / 16;  // runs per pass
    constexpr int r0 = decltype(PASS)::value * kHalf;
    constexpr int kK = 4;            // chunks per group
    f32x2_t acc[kHalf];
#pragma unroll
    for (int i = 0; i < kHalf; ++i) acc[i] = f32x2_t{0.f, 0.f};
    mx = -INFINITY;
    den = 0.f;
    for (int c0 = 0; c0 < nch; c0 += kK) {
      float sv[kK];
      coh_u32x2_t v[kK][kHalf];
#pragma unroll
      for (int k = 0; k < kK; ++k) {
        const int ch = min(c0 + k, nch - 1);  // a short group re-reads its last chunk, weight 0
        sv[k] = load_coherent(lse0 + (int64_t)ch * kRows);
        const BufRes r = wave_partial(p.part_o, slot0 + ch, wave);
#pragma unroll
        for (int i = 0; i < kHalf; ++i) v[k][i] = load_coherent_run(r, 8u * lane, 512 * (r0 + i));
      }
#pragma unroll
      for (int k = 1; k < kK; ++k)
        if (c0 + k >= nch) sv[k] = -INFINITY;
      const float mn = fmaxf(mx, fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
      if (mn == -INFINITY) continue;
      const float a = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx - mn);
      float w[kK];
#pragma unroll
      for (int k = 0; k < kK; ++k) w[k] = sv[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[k] - mn);
      den = den * a + ((w[0] + w[1]) + (w[2] + w[3]));
#pragma unroll
      for (int i = 0; i < kHalf; ++i) {
        float x = acc[i][0] * a, y = acc[i][1] * a;
#pragma unroll
        for (int k = 0; k < kK; ++k) {
          x = fmaf(w[k], __uint_as_float(v[k][i][0]), x);
          y = fmaf(w[k], __uint_as_float(v[k][i][1]), y);
        }
        acc[i] = f32x2_t{x, y};
      }
      mx = mn;
    }
    // run 2 td + h holds dims d0 + 16 td + 4g + 2h, +1 of the row
    const float rinv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
    for (int t = r0 / 2; t < (r0 + kHalf) / 2; ++t) {
      const int i = 2 * t - r0;
      const bf16x4_t o4 = {(__bf16)(acc[i][0] * rinv), (__bf16)(acc[i][1] * rinv),
                           (__bf16)(acc[i + 1][0] * rinv), (__bf16)(acc[i + 1][1] * rinv)};
      *reinterpret_cast<bf16x4_t*>(dst + 16 * t) = o4;
    }
  });
  if (dh == 0 && g == 0 && p.lse)
    p.lse[q_index] = den > 0.f ? (mx + __builtin_amdgcn_logf(den)) * kLn2 : -INFINITY;
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
  p.counters = a.counters;
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
  return hipGetLastError();
}

}  // namespace fi
