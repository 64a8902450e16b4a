// Attention of many query rows against one run of paged K/V, on the matrix
// cores of gfx950 (bf16). Two uses: shared prefixes (cascade) and prefill /
// append (several query tokens per request, causal).
//
// Composable block-sparse formats (FlashInfer paper explainer, "FlashInfer:
// Block-Sparse KV 캐시로 어텐션 병목을 해소하다", visionhong.com, Block-Sparse
// section): a KV cache can be described by more than one block-sparse
// matrix. When many requests begin with the same pages, that prefix is one
// block all of their query rows share; computing it once per KV head for
// every row of the group turns each request re-reading the prefix into one
// matrix problem. Each row's prefix state (o, lse) is merged with the row's
// state over its own pages by the decode kernel's merge tree (softmax over a
// disjoint union, the closed form behind the explainer's split scheduler).
//
// Prefill (same explainer, section on where the attention bottleneck lies:
// prefill attends all prompt tokens at once and is bound by arithmetic): a
// tile is up to 256 query rows of one request and KV head -- 256 / G query
// tokens times the G query heads of the KV head -- over one chunk of the
// request's pages. The queries are the request's newest cached tokens, so
// with the causal mask row r attends the first VISIBLE + r / G tokens of the
// request; the mask is a per-row token limit. A tile with one chunk writes
// bf16 out and lse itself; a cut tile writes partial states that the merge
// kernel combines.
//
// One workgroup of 8 waves per item, two per SIMD. Shared prefix: wave w
// owns query rows 32(w%4) .. +31 and the tokens 32(w/4) .. +31 of every
// 64-token block; the two partial softmax states of a row are merged through
// LDS at the end. Prefill: wave w owns rows 32w .. +31 and both 32-token
// halves of every block, so a K/V block serves 256 rows. Per block a wave
// requests all its K fragments and issues each sub-block's S^T products as
// soon as that sub-block's fragments are in, then the loads of a later
// block and its V^T fragment reads, takes one online-softmax step over its
// tokens (the running max moves at most once per block) while those reads
// land, and runs one branch-free stretch of exponentials, P splits and PV
// products that the scheduler interleaves. K/V blocks stream into
// an LDS ring of kStages stages with gfx950's direct-to-LDS loads (no
// staging registers), one barrier per block. Per 32 tokens of a wave:
//   S^T[token, row] = K . Q^T     v_mfma_f32_32x32x16_bf16, D/16 steps
//   online softmax per row (a lane owns one row: 16 tokens in the lane, the
//   other 16 in lane l^32)
//   O^T[d, row] += V^T . P^T      2 token steps x D/32 tiles, P split in
//                                 two bf16 parts (hi + lo) for precision
// Lane layout of v_mfma_f32_32x32x16_bf16 (A 32x16, B 16x32, C 32x32):
// A[m][k] in lane m + 32*(k/8), element k%8; B[k][n] in lane n + 32*(k/8);
// C[m][n] in lane n + 32*((m%8)/4), element 4*(m/8) + m%4.
// P^T comes straight from the S^T accumulators: the PV contraction index
// enumerates the block's tokens in the order the S^T layout leaves them in
// the lanes. V^T fragments come from the row-major V tile through
// ds_read_b64_tr_b16: within each 16-lane group, output lane 4p+q element k
// is element q of input lane 4k+p, so input lanes pointing at
// V[tok_k][d0 + 4p] hand every output lane four tokens of one column.
// 16-byte pieces of each K and V row are XOR-swizzled in LDS (through the
// source address of the direct-to-LDS loads) so both reads stay at or below
// two-way bank conflicts.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "coherent.h"
#include "fi_bsr.h"
#include "kernels.h"

namespace fi {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;

constexpr int kWaves = 8;
constexpr int kBlock = 64;   // tokens per ring stage (32 per wave half)
constexpr int kIds = FI_PREFILL_MAX_PAGES;  // page-id window
static_assert(FI_PREFIX_MAX_PAGES <= kIds && kIds <= 512, "page-id window: one id per thread");
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kMargin = 8.0f;  // lazy-rescale margin, log2 units

struct TileParams {
  const int32_t* pitems;       // prefix items, or prefill items (FI_QITEM_*)
  const int32_t* members;
  const int32_t* prefix_slot;
  __bf16* out;                 // prefill: [N, num_qo_heads, D]
  float* lse;                  // prefill: [N, num_qo_heads] natural log, or null
  const int32_t* page_ids;
  const char* q;
  const char* k_pages;
  const char* v_pages;
  float* part_o;
  float* part_lse;
  const int32_t* merges;  // prefill: merges of cut tiles (FI_QMERGE_*)
  int32_t* counters;      // prefill: their arrival counts, 0 between runs
  int64_t page_stride;  // bytes between physical pages
  int64_t head_stride;  // bytes between KV heads within a page
  int num_qo_heads;
  int num_kv_heads;
  int page_size;
  uint32_t page_magic;     // ceil(2^32 / page_size) mod 2^32
  uint32_t page_magic_hi;  // 1 when page_size is 1 (the quotient is then 2^32)
  int group;
  int causal;           // prefill: row r attends VISIBLE + r / G tokens
  float scale_log2;     // sm_scale * k_scale * log2(e)
  float v_scale;        // multiplies every output and partial state (V dequantisation)
  double rope_log2_theta;  // rotary embedding: log2(rope_theta)
  double rope_rev;         // 1 / (2 pi rope_scale): revolutions per radian, positions scaled
};

template <int D, int kKv = 2>
struct Geom {
  static constexpr int kRowBytes = D * kKv;               // bf16 (kKv 2) or fp8 E4M3 (kKv 1)
  static constexpr int kPieces = kRowBytes / 16;          // 16-byte pieces per row
  static constexpr int kBlockBytes = kBlock * kRowBytes;  // one K (or V) block
  static constexpr int kRowsPerDma = 1024 / kRowBytes;    // rows one wave-wide load covers
  static constexpr int kDmaPerWave = kBlockBytes / 1024 / kWaves;
  // 96 / 80 KiB of bf16 K+V in flight; fp8 blocks are half the bytes
  static constexpr int kStages = kKv == 1 ? 4 : (D == 128 ? 3 : 5);
  static_assert(kDmaPerWave >= 1, "block does not cover the workgroup");
  static_assert(kKv == 2 || D == 128, "the fp8 tile is built for head_dim 128");
  // piece swizzles: bf16 K is read 16 rows x 1 piece, V 8 rows x 4 pieces at
  // a time; fp8 K 16 rows x half a piece, V 8 rows (two runs of four, eight
  // apart) x 1 piece
  static __device__ __forceinline__ int swz_k(int t) {
    if constexpr (kKv == 1) return (t >> 1) & 7;
    else return t % kPieces;
  }
  static_assert(kStages * 2 * kBlockBytes >= 4 * 32 * D * 4, "ring too small for the final merge");
  static __device__ __forceinline__ int swz_v(int t) {
    if constexpr (kKv == 1) return (t & 7) ^ (((t >> 3) & 1) << 2);
    else return (4 * (t % 4)) % kPieces;
  }
};

__device__ __forceinline__ uint32_t lds_u32(const void* p) { return (uint32_t)(uintptr_t)p; }

// LDS reads at a lane address plus a compile-time immediate offset (the
// instruction's 16-bit offset field), as inline asm: the compiler cannot tell
// which ring stage a direct-to-LDS load writes, and would otherwise wait for
// every load in flight before each read. The waits are explicit instead.
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

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1, so that I can
// appear in template arguments (immediate offsets) inside f.
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

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats rounded to a packed bf16 pair (nearest even), and the pair's
// rounding errors rounded to a second pair: hi + lo is within ~2^-16 of the
// inputs.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const f32x2_t f = {a, b};
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
  const f32x2_t r = {a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
}

// s_waitcnt vmcnt(n), leaving the other counters unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) with the registers the inline-asm LDS reads wrote as
// operands, so no use of them can be scheduled above the wait.
template <int N>
__device__ __forceinline__ void lgkm_wait_tied(u32x4_t (&r)[N]) {
  if constexpr (N == 4) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3])::"memory");
  } else {
    static_assert(N == 8, "4 or 8 fragments");
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]),
                   "+v"(r[7])::"memory");
  }
}
// s_waitcnt lgkmcnt(CNT): the reads of r are done once at most CNT LDS
// operations issued after them are still in flight (LDS returns in order).
template <int CNT, int N>
__device__ __forceinline__ void lgkm_wait_tied_n(u32x4_t (&r)[N]) {
  static_assert(CNT >= 0 && CNT < 16, "lgkmcnt range");
  if constexpr (N == 4) {
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]) : "i"(CNT) : "memory");
  } else {
    static_assert(N == 8, "4 or 8 fragments");
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]),
                   "+v"(r[7])
                 : "i"(CNT)
                 : "memory");
  }
}
template <int N>
__device__ __forceinline__ void lgkm_wait_tied(u32x2_t (&r)[N][2]) {
  if constexpr (N == 2) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r[0][0]), "+v"(r[0][1]), "+v"(r[1][0]), "+v"(r[1][1])::"memory");
  } else {
    static_assert(N == 4, "2 or 4 tiles");
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(r[0][0]), "+v"(r[0][1]), "+v"(r[1][0]), "+v"(r[1][1]), "+v"(r[2][0]), "+v"(r[2][1]),
                   "+v"(r[3][0]), "+v"(r[3][1])::"memory");
  }
}

// s_waitcnt lgkmcnt(CNT), then every register of r redefined by an empty
// asm statement ordered after the wait: no use of a value read can be
// scheduled above it.
template <int CNT, typename T, int N>
__device__ __forceinline__ void lgkm_wait_then(T (&r)[N]) {
  static_assert(CNT >= 0 && CNT < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(CNT) : "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(r[i]));
}

// s_waitcnt lgkmcnt(CNT) tied to fp8 K fragments (see lgkm_wait_tied_n).
template <int CNT>
__device__ __forceinline__ void lgkm_wait_tied_n8(u32x2_t (&r)[8]) {
  static_assert(CNT >= 0 && CNT < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]),
                 "+v"(r[7])
               : "i"(CNT)
               : "memory");
}
__device__ __forceinline__ void lgkm_wait_tied4(u32x2_t (&r)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3])::"memory");
}
template <int OFF>
__device__ __forceinline__ u32x2_t lds_b64(uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x2_t r;
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF) : "memory");
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2_t lds_tr8_b64(uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF) : "memory");
  return r;
}
template <int OFF>
__device__ __forceinline__ void lds_w128(uint32_t a, u32x4_t v) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(a), "v"(v), "i"(OFF) : "memory");
}
__device__ __forceinline__ void lds_w64(uint32_t a, u32x2_t v) {
  asm volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(v) : "memory");
}

// Cosine and sine of the rotary angle of a dim pair at position pos: the
// pair's frequency is a 64-bit binary fraction of a revolution per position,
// so pos * freq mod 1 is exact integer arithmetic; its top 32 bits give the
// angle for sincospif.
__device__ __forceinline__ void rot_sincos(uint64_t freq, uint32_t pos, float& c, float& s) {
  const uint64_t ph = (uint64_t)pos * freq;
  const float rev = (float)(uint32_t)(ph >> 32) * 0x1p-32f;
  sincospif(2.f * rev, &s, &c);
}

// Eight fp8 (E4M3) codes widened to eight bf16 values (exact) in code order.
__device__ __forceinline__ bf16x8_t widen8(u32x2_t w) {
  const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false));
  const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true));
  const uint32_t c = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false));
  const uint32_t d = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true));
  return __builtin_bit_cast(bf16x8_t, u32x4_t{a, b, c, d});
}

__device__ __forceinline__ float max_with_partner32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave roles. Shared prefixes: 4 row groups of 32 rows (128 rows); the two
// waves of a row group take the two 32-token halves of every block and merge
// their states at the end. Prefill: 8 row groups (256 rows); each wave takes
// both halves of every block itself, as two sub-blocks whose products are
// independent accumulation chains; one softmax step covers the wave's whole
// block, and the exponentials of one 16-token step overlap the products of
// the previous one.
template <bool kPrefill, bool kRope = false>
struct Roles {
  // a rope tile (prefill with the rotary embedding) takes the split layout:
  // its waves hold the queries' lo parts too, so each takes half a block
  static constexpr bool kSplit = !kPrefill || kRope;
  static constexpr int kRowGroups = kSplit ? 4 : 8;
  static constexpr int kSub = kSplit ? 1 : 2;  // 32-token sub-blocks per wave and block
};
static_assert(FI_PREFILL_ROWS == 32 * 8, "a prefill tile is 8 row groups of 32 rows");

template <int D, bool kPrefill, int kKv = 2, bool kRope = false>
__global__ __launch_bounds__(512) void tile_attend_kernel(TileParams p) {
  static_assert(kKv == 2 || kPrefill, "shared-prefix items read bf16 caches");
  static_assert(!kRope || (kPrefill && kKv == 2 && D == 128), "rope tiles: bf16 prefill, d 128");
  using Gm = Geom<D, kKv>;
  using R = Roles<kPrefill, kRope>;
  constexpr int NS = Gm::kStages;
  constexpr int kRB = Gm::kRowBytes;
  __shared__ __attribute__((aligned(1024))) char s_ring[NS][2][Gm::kBlockBytes];
  __shared__ uint32_t s_pid[kIds];  // page byte offsets (page + head) / 128
  // rotary embedding: each pair's frequency (a 64-bit fraction of a
  // revolution per position), the rotations of the 64 rows of a block
  // relative to its first token, [row][pair] (cos, sin), the rotation of the
  // block's first token (two blocks, by parity), and the lo bf16 parts of the
  // rotated K block (its hi parts replace K in the ring stage)
  __shared__ uint64_t s_freq[kRope ? D / 2 : 1];
  __shared__ __attribute__((aligned(16))) float2 s_rrow[kRope ? kBlock * D / 2 : 1];
  __shared__ __attribute__((aligned(16))) float2 s_rbase[kRope ? 2 * D / 2 : 1];
  __shared__ __attribute__((aligned(1024))) char s_klo[kRope ? Gm::kBlockBytes : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wrow = R::kSplit ? (wave & 3) : wave;  // row group of this wave
  const int wtok = R::kSplit ? (wave >> 2) : 0;    // first 32-token half it takes
  const int half = lane >> 5;
  const int G = p.group;
  // this lane's query row (column n = lane % 32 of the wave's tiles)
  const int row = wrow * 32 + (lane & 31);

  int h, nrows, page_begin, npg, ntok;
  int tok_off = 0;      // slot of the chunk's first token in its first page
  int kv_pos = 0, q_pos = 0;  // rope: positions of the chunk's first token and of the tile's first query
  int lim;              // tokens of the chunk this row attends (may be <= 0)
  int64_t q_index;      // row of q (and, for prefill, of out / lse) x heads + head
  // prefix: partial row = prefix_slot[b][h] + chunk; prefill: slot (-1 = direct)
  int slot_base;
  int gi;
  bool row_ok;
  if constexpr (!kPrefill) {
    const int32_t* it = p.pitems + (int64_t)blockIdx.x * FI_PITEM_STRIDE;
    h = it[FI_PITEM_KV_HEAD];
    const int member_base = it[FI_PITEM_MEMBER_BASE];
    const int row_begin = it[FI_PITEM_ROW_BEGIN];
    nrows = it[FI_PITEM_NUM_ROWS];
    const int chunk = it[FI_PITEM_CHUNK];
    page_begin = it[FI_PITEM_PAGE_BEGIN];
    npg = it[FI_PITEM_NUM_PAGES];  // <= FI_PREFIX_MAX_PAGES = kIds
    tok_off = it[FI_PITEM_TOKEN_BEGIN];
    ntok = it[FI_PITEM_NUM_TOKENS];  // tok_off + ntok <= npg * page_size
    row_ok = row < nrows;
    const int b = p.members[member_base + row_begin + (row_ok ? row / G : 0)];
    gi = row_ok ? row % G : 0;
    q_index = (int64_t)b * p.num_qo_heads + (int64_t)h * G + gi;
    lim = ntok;
    slot_base = row_ok ? p.prefix_slot[(int64_t)b * p.num_kv_heads + h] + chunk : 0;
  } else {
    const int32_t* it = p.pitems + (int64_t)blockIdx.x * FI_QITEM_STRIDE;
    h = it[FI_QITEM_KV_HEAD];
    const int qo_row = it[FI_QITEM_QO_ROW];
    nrows = it[FI_QITEM_NUM_QO] * G;
    const int kv_begin = it[FI_QITEM_KV_BEGIN];
    ntok = it[FI_QITEM_NUM_KV];
    const int visible = it[FI_QITEM_VISIBLE];
    if constexpr (kRope) {
      kv_pos = kv_begin;
      q_pos = it[FI_QITEM_Q_POS];
    }
    page_begin = it[FI_QITEM_PAGE_BEGIN];
    slot_base = it[FI_QITEM_SLOT];
    npg = (ntok + p.page_size - 1) / p.page_size;  // <= FI_PREFILL_MAX_PAGES = kIds, ntok <= 2^20
    row_ok = row < nrows;
    const int qi = row_ok ? row / G : 0;
    gi = row_ok ? row % G : 0;
    q_index = (int64_t)(qo_row + qi) * p.num_qo_heads + (int64_t)h * G + gi;
    lim = visible + (p.causal ? qi : 0) - kv_begin;
    if (ntok == 0) {
      // a tile that attends nothing (a request with no pages, no mask):
      // out = 0, lse = -inf, and no K/V read at all
      if (wtok == 0 && row_ok) {
        __bf16* dst = p.out + q_index * D;
        for (int d = 4 * half; d < D; d += 8)
          *reinterpret_cast<uint2*>(dst + d) = make_uint2(0u, 0u);
        if (half == 0 && p.lse) p.lse[q_index] = -INFINITY;
      }
      return;
    }
  }
  lim = min(lim, ntok);

  // ---- the item's pages (one window: an item has at most kIds pages) as
  // byte offsets of the page's rows of this KV head in 128-byte units: every
  // page and head stride is a multiple of 128 bytes, and 2^32 such units
  // (512 GiB) exceed any device's memory
  const int64_t head_off = (int64_t)h * p.head_stride;
  if (tid < kIds)
    s_pid[tid] = (uint32_t)(((int64_t)p.page_ids[page_begin + min(tid, npg - 1)] * p.page_stride + head_off) >> 7);

  // Q^T as the B operand: lane holds Q[row][16s + 8*half .. +8] for step s
  // (a padding row loads the tile's first row and zeroes it, so the loads
  // are unconditional). Without the rotary embedding the loads stay in
  // flight while the first K/V blocks are requested (they are waited for,
  // and padding rows zeroed, after those requests).
  bf16x8_t qf[D / 16];
  {
    const char* qrow = p.q + q_index * (D * 2);  // q is bf16 whatever the cache holds
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      uint4 v = *reinterpret_cast<const uint4*>(qrow + (16 * s + 8 * half) * 2);
      if constexpr (kRope)
        if (!row_ok) v = make_uint4(0, 0, 0, 0);
      qf[s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  // rope: frequencies, the row table and block 0's base rotation; the
  // lane's query row turned at its position and split into hi (qf) and lo
  // (ql) bf16 parts. Pairs (i, i + 64) sit in steps s and s + 4 of one lane.
  bf16x8_t ql[kRope ? D / 16 : 1];
  if constexpr (kRope) {
    if (tid < D / 2) {
      double fq = exp2(-(2.0 * tid / D) * p.rope_log2_theta) * p.rope_rev;
      fq -= floor(fq);
      s_freq[tid] = (uint64_t)ldexp(fq, 64);
    }
    __syncthreads();
    for (int e = tid; e < kBlock * D / 2; e += 512) {
      float cs, sn;
      rot_sincos(s_freq[e % (D / 2)], (uint32_t)(e / (D / 2)), cs, sn);
      s_rrow[e] = make_float2(cs, sn);
    }
    if (tid < D / 2) {
      float cs, sn;
      rot_sincos(s_freq[tid], (uint32_t)kv_pos, cs, sn);
      s_rbase[tid] = make_float2(cs, sn);
    }
    const uint32_t qp = (uint32_t)(q_pos + (row_ok ? row / G : 0));
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      float x[8], y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = (float)qf[s][e];
        y[e] = (float)qf[s + D / 32][e];
      }
      uint32_t xh[4], xl[4], yh[4], yl[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float c0, s0, c1, s1;
        rot_sincos(s_freq[16 * s + 8 * half + e], qp, c0, s0);
        rot_sincos(s_freq[16 * s + 8 * half + e + 1], qp, c1, s1);
        split_bf16x2(x[e] * c0 - y[e] * s0, x[e + 1] * c1 - y[e + 1] * s1, xh[e / 2], xl[e / 2]);
        split_bf16x2(y[e] * c0 + x[e] * s0, y[e + 1] * c1 + x[e + 1] * s1, yh[e / 2], yl[e / 2]);
      }
      qf[s] = __builtin_bit_cast(bf16x8_t, u32x4_t{xh[0], xh[1], xh[2], xh[3]});
      ql[s] = __builtin_bit_cast(bf16x8_t, u32x4_t{xl[0], xl[1], xl[2], xl[3]});
      qf[s + D / 32] = __builtin_bit_cast(bf16x8_t, u32x4_t{yh[0], yh[1], yh[2], yh[3]});
      ql[s + D / 32] = __builtin_bit_cast(bf16x8_t, u32x4_t{yl[0], yl[1], yl[2], yl[3]});
    }
  }
  // the page ids are in LDS before any K/V load is issued (q may still be on
  // its way)
  __syncthreads();  // s_pid is written

  // ---- direct-to-LDS loads of block j into stage st: wave-wide load i of
  // wave w fills rows (w*kDmaPerWave + i) * kRowsPerDma + lane / kPieces,
  // piece lane % kPieces of the swizzled layout, from the global piece it
  // stands for. Blocks past the end re-read the last token (same count of
  // loads on every path, so the vmcnt waits below are exact). Prefix K/V is
  // read once per row block (one, unless a group holds over 128 query
  // rows), so those loads carry the nontemporal policy (aux bit 1 = nt on
  // gfx950) and stream past the caches; prefill tiles of one request and KV
  // head read the same K/V, so theirs stay cacheable.
  constexpr int kAux = kPrefill ? 0 : 2;
  const int dma_row = lane / Gm::kPieces;
  const int dma_piece = lane % Gm::kPieces;
  // tok / page_size as a multiply-high: tok < 2^20 (a prefill chunk holds at
  // most 2^20 tokens, a prefix item at most 256 pages of at most 4096) and the
  // reciprocal ceil(2^32 / P) is too large by less than 1, so the quotient is
  // off by less than 2^-12 < 1 / P -- exact for every P < 4096, and powers of
  // two are exact anyway
  const uint32_t pmag = p.page_magic, pmag_hi = p.page_magic_hi;
  const uint32_t psz = (uint32_t)p.page_size;
  auto issue = [&](int j, int st) {
#pragma unroll
    for (int i = 0; i < Gm::kDmaPerWave; ++i) {
      const int t = (wave * Gm::kDmaPerWave + i) * Gm::kRowsPerDma + dma_row;
      const uint32_t tok = (uint32_t)(min(j * kBlock + t, ntok - 1) + tok_off);
      const uint32_t pg = __umulhi(tok, pmag) + tok * pmag_hi;
      const uint32_t row_in_page = tok - pg * psz;
      const uint64_t page_off = (uint64_t)s_pid[pg] << 7;
      const int kp = dma_piece ^ Gm::swz_k(t);
      const int vp = dma_piece ^ Gm::swz_v(t);
      const uint32_t krow = row_in_page * kRB + kp * 16;
      const uint32_t vrow = row_in_page * kRB + vp * 16;
      char* kdst = &s_ring[st][0][(wave * Gm::kDmaPerWave + i) * 1024];
      char* vdst = &s_ring[st][1][(wave * Gm::kDmaPerWave + i) * 1024];
      __builtin_amdgcn_global_load_lds((global_void_t*)(p.k_pages + (page_off + krow)),
                                       (lds_void_t*)kdst, 16, 0, kAux);
      __builtin_amdgcn_global_load_lds((global_void_t*)(p.v_pages + (page_off + vrow)),
                                       (lds_void_t*)vdst, 16, 0, kAux);
    }
  };

  f32x16_t o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int nblocks = (ntok + kBlock - 1) / kBlock;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s, s);
  // q (issued before the ring loads) is in: vector memory loads complete in
  // order, so at most this stage-filling's loads remain. From here on only
  // ring loads are in flight, which the waits in the loop count.
  wait_vmcnt<2 * Gm::kDmaPerWave * (NS - 1)>();
  if constexpr (!kRope) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      if (!row_ok) qf[s] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
  }

  // LDS byte offsets that depend only on the lane. K fragment q of token row
  // kt = 32 (wtok + sb) + lane % 32 sits at kt * kRB + piece * 16 with the
  // piece swizzled by kt % kPieces = lane % kPieces (32 rows are a whole
  // number of swizzle periods), so the sub-block moves it by a constant. V
  // fragment t of the transposed read (input role: token 4 (g16/2) + v_k of
  // a 16-token step, columns 32t + 16 (g16%2) + 4 v_p .. +3) is swizzled by
  // tok % 4 = v_k, so sub-block, step and run move it by constants too: those
  // go into the reads' immediate offsets.
  const int g16 = lane >> 4, L16 = lane & 15;
  const int v_k = L16 >> 2, v_p = L16 & 3;  // this lane's input role in a transposed read
  uint32_t kb[D / 16], vb[D / 32];
  if constexpr (kKv == 1) {
    // fp8: K fragment q is half a piece (8 codes, dims 16q + 8 half ..) of
    // row kt; one transposed byte read per step and tile hands each lane 8
    // tokens of one column: input lane 2 jj + pp of group g16 points at token
    // 4 (g16/2) + 8 (jj/4) + jj%4 of the step, columns 32t + 16 (g16%2) +
    // 8 pp .. +7. Both rows' swizzles are step- and sub-block-invariant.
    const int kt = 32 * wtok + (lane & 31);
#pragma unroll
    for (int q = 0; q < D / 16; ++q) kb[q] = kt * kRB + ((q ^ Gm::swz_k(kt)) * 16) + 8 * half;
    const int jj = L16 >> 1, pp = L16 & 1;
    const int vt = 32 * wtok + 4 * (g16 >> 1) + 8 * (jj >> 2) + (jj & 3);
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
      vb[t] = vt * kRB + (((2 * t + (g16 & 1)) ^ Gm::swz_v(vt)) * 16) + 8 * pp;
  } else {
    const int kt = 32 * wtok + (lane & 31);
#pragma unroll
    for (int q = 0; q < D / 16; ++q) kb[q] = kt * kRB + (((2 * q + half) ^ Gm::swz_k(kt)) * 16);
    const int vt = 32 * wtok + 4 * (g16 >> 1) + v_k;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      const int d = 32 * t + 16 * (g16 & 1) + 4 * v_p;
      vb[t] = vt * kRB + (((d >> 3) ^ Gm::swz_v(vt)) * 16) + (d & 7) * 2;
    }
  }
  // Scores stay unscaled; exp2(c * s - c * m) is one fma and an exp. The
  // running max m is raised only when a sub-block's max passes it by more
  // than kMargin in log2 units (weights stay <= 2^kMargin), so the
  // accumulators, which cost a read, a multiply and a write each, are
  // rescaled rarely after the first block.
  const float c = p.scale_log2;
  const float margin = kMargin / c;

  for (int j = 0; j < nblocks; ++j) {
    const int st = j % NS;
    // this wave's loads of block j have landed (later blocks may be in flight)
    wait_vmcnt<2 * Gm::kDmaPerWave * (NS - 2)>();
    // every wave's loads of block j have landed, and every wave is done
    // reading block j-1, whose stage is refilled next
    __builtin_amdgcn_s_barrier();

    const uint32_t kst = lds_u32(s_ring[st][0]);
    const uint32_t vst = lds_u32(s_ring[st][1]);
    f32x16_t sc[R::kSub];
    if constexpr (kRope) {
      // ---- turn block j's K rows: thread t takes row t / 8 and pairs
      // 8 (t % 8) .. +7 (dims i and i + 64), at position kv_pos + 64 j + row
      // (the block's base rotation times the row's, both from exact
      // phases), in fp32; the hi bf16 parts replace K in the stage, the lo
      // parts go to s_klo, at the same swizzled places
      const int rr = tid >> 3, gg = tid & 7;
      const int sw = Gm::swz_k(rr);
      const uint32_t pa = rr * kRB + ((gg ^ sw) * 16), pb = rr * kRB + (((gg + 8) ^ sw) * 16);
      const uint32_t klo = lds_u32(s_klo);
      const uint32_t rra = lds_u32(&s_rrow[rr * (D / 2) + 8 * gg]);
      const uint32_t rba = lds_u32(&s_rbase[(j & 1) * (D / 2) + 8 * gg]);
      u32x4_t kx[2], rt[8];
      kx[0] = lds_b128<0>(kst + pa);
      kx[1] = lds_b128<0>(kst + pb);
      rt[0] = lds_b128<0>(rra);
      rt[1] = lds_b128<16>(rra);
      rt[2] = lds_b128<32>(rra);
      rt[3] = lds_b128<48>(rra);
      rt[4] = lds_b128<0>(rba);
      rt[5] = lds_b128<16>(rba);
      rt[6] = lds_b128<32>(rba);
      rt[7] = lds_b128<48>(rba);
      lgkm_wait_then<0>(kx);
      lgkm_wait_then<0>(rt);
      // the next block's base rotation, read after the next barrier (its
      // buffer was last read before this block's barrier)
      if (tid < D / 2) {
        u32x2_t fw[1];
        fw[0] = lds_b64<0>(lds_u32(&s_freq[tid]));
        lgkm_wait_then<0>(fw);
        float cs, sn;
        rot_sincos(((uint64_t)fw[0].y << 32) | fw[0].x, (uint32_t)(kv_pos + (j + 1) * kBlock), cs,
                   sn);
        lds_w64(lds_u32(&s_rbase[((j + 1) & 1) * (D / 2) + tid]),
                u32x2_t{__float_as_uint(cs), __float_as_uint(sn)});
      }
      uint32_t xh[4], xl[4], yh[4], yl[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float cs[2], sn[2], x[2], y[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int k = e + u;  // pair 8 gg + k: float2 k of the row and base tables
          const float rc = __uint_as_float(rt[k / 2][2 * (k % 2)]);
          const float rs = __uint_as_float(rt[k / 2][2 * (k % 2) + 1]);
          const float bc = __uint_as_float(rt[4 + k / 2][2 * (k % 2)]);
          const float bs = __uint_as_float(rt[4 + k / 2][2 * (k % 2) + 1]);
          cs[u] = bc * rc - bs * rs;
          sn[u] = bs * rc + bc * rs;
          const uint32_t wx = kx[0][k / 2], wy = kx[1][k / 2];
          x[u] = __uint_as_float(k % 2 ? (wx & 0xFFFF0000u) : (wx << 16));
          y[u] = __uint_as_float(k % 2 ? (wy & 0xFFFF0000u) : (wy << 16));
        }
        split_bf16x2(x[0] * cs[0] - y[0] * sn[0], x[1] * cs[1] - y[1] * sn[1], xh[e / 2], xl[e / 2]);
        split_bf16x2(y[0] * cs[0] + x[0] * sn[0], y[1] * cs[1] + x[1] * sn[1], yh[e / 2], yl[e / 2]);
      }
      lds_w128<0>(kst + pa, u32x4_t{xh[0], xh[1], xh[2], xh[3]});
      lds_w128<0>(kst + pb, u32x4_t{yh[0], yh[1], yh[2], yh[3]});
      lds_w128<0>(klo + pa, u32x4_t{xl[0], xl[1], xl[2], xl[3]});
      lds_w128<0>(klo + pb, u32x4_t{yl[0], yl[1], yl[2], yl[3]});
      // every wave's rotated rows are in place before any fragment is read
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();

      // ---- S^T = Kh.Qh + Kh.Ql + Kl.Qh (one sub-block per wave)
      u32x4_t kh[D / 16], kl[D / 16];
#pragma unroll
      for (int q = 0; q < D / 16; ++q) {
        kh[q] = lds_b128<0>(kst + kb[q]);
        kl[q] = lds_b128<0>(klo + kb[q]);
      }
      lgkm_wait_then<0>(kh);
      lgkm_wait_then<0>(kl);
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[0][r] = 0.f;
#pragma unroll
      for (int q = 0; q < D / 16; ++q) {
        const bf16x8_t h8 = __builtin_bit_cast(bf16x8_t, kh[q]);
        sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h8, qf[q], sc[0], 0, 0, 0);
        sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h8, ql[q], sc[0], 0, 0, 0);
        sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kl[q]), qf[q],
                                                        sc[0], 0, 0, 0);
      }
    } else {
    // ---- S^T = K . Q^T of every sub-block (independent chains). All K
    // fragments are requested first; each sub-block's products start as soon
    // as its own fragments are in, and the scheduling barriers keep the
    // first sub-block's products ahead of the second's wait.
    u32x4_t kv[kKv == 2 ? R::kSub : 1][D / 16];   // bf16 fragments
    u32x2_t kv8[kKv == 1 ? R::kSub : 1][D / 16];  // fp8 fragments (widened to bf16 for the product)
    static_for<R::kSub>([&](auto SB) {
      constexpr int sb = decltype(SB)::value;
#pragma unroll
      for (int q = 0; q < D / 16; ++q) {
        if constexpr (kKv == 1)
          kv8[sb][q] = lds_b64<32 * sb * kRB>(kst + kb[q]);
        else
          kv[sb][q] = lds_b128<32 * sb * kRB>(kst + kb[q]);
      }
    });
    static_for<R::kSub>([&](auto SB) {
      constexpr int sb = decltype(SB)::value;
      if constexpr (kKv == 1)
        lgkm_wait_tied_n8<(R::kSub - 1 - sb) * (D / 16)>(kv8[sb]);
      else
        lgkm_wait_tied_n<(R::kSub - 1 - sb) * (D / 16)>(kv[sb]);
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[sb][r] = 0.f;
#pragma unroll
      for (int q = 0; q < D / 16; ++q) {
        bf16x8_t kf;
        if constexpr (kKv == 1)
          kf = widen8(kv8[sb][q]);
        else
          kf = __builtin_bit_cast(bf16x8_t, kv[sb][q]);
        sc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[q], sc[sb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    }  // kRope
    // the loads of a later block go out while the products run
    issue(j + NS - 1, (j + NS - 1) % NS);

    // ---- V^T fragments of every 16-token step, requested now so that they
    // arrive during the softmax step below. Step (sb, ks) covers tokens
    // 32 sb + 16 ks .. +15; this lane's A fragment (d = 32t + lane%32) comes
    // from two transposed reads: tokens 4*half + 0..3 of the step, then +8.
    u32x2_t va[kKv == 2 ? R::kSub * 2 : 1][D / 32][2];
    u32x2_t va8[kKv == 1 ? R::kSub * 2 : 1][D / 32];  // fp8: one byte-transposed read per tile
    static_for<R::kSub * 2>([&](auto STEP) {
      constexpr int step = decltype(STEP)::value;
      constexpr int kOff = 16 * step * kRB;
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        if constexpr (kKv == 1) {
          va8[step][t] = lds_tr8_b64<kOff>(vst + vb[t]);
        } else {
          va[step][t][0] = lds_tr_b64<kOff>(vst + vb[t]);
          va[step][t][1] = lds_tr_b64<kOff + 8 * kRB>(vst + vb[t]);
        }
      }
    });

    // ---- online softmax over the wave's tokens of the block; element r of
    // sub-block sb holds token 32 (wtok + sb) + 4*half + 8*(r/4) + r%4
    const int tok0 = j * kBlock + 32 * wtok;
    if (__builtin_amdgcn_ballot_w64(tok0 + 32 * R::kSub > lim)) {  // some row stops in here
#pragma unroll
      for (int sb = 0; sb < R::kSub; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 32 * sb + 4 * half + 8 * (r >> 2) + (r & 3);
          if (tok0 + m >= lim) sc[sb][r] = -INFINITY;
        }
    }
    float mb = sc[0][0];
#pragma unroll
    for (int sb = 0; sb < R::kSub; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mb = fmaxf(mb, sc[sb][r]);
    mb = max_with_partner32(mb);  // -inf if the row attends none of these tokens
    const bool up = mb > m_run + margin;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float alpha = up ? __builtin_amdgcn_exp2f((m_run - mb) * c) : 1.f;  // 0 at first
      l_run *= alpha;
      if (j > 0) {  // the accumulators are still zero on the first block
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
      }
      m_run = up ? mb : m_run;
    }
    // a row with no token yet has m = -inf and only masked scores: weight 0
    const float mc = m_run == -INFINITY ? 0.f : m_run * c;

    // every V^T fragment is in: the exponentials, the P split and the PV
    // products below form one branch-free stretch the scheduler can
    // interleave (one step's products run while the next step's weights are
    // computed)
    if constexpr (kKv == 1) {
#pragma unroll
      for (int step = 0; step < R::kSub * 2; ++step) lgkm_wait_tied4(va8[step]);
    } else {
      lgkm_wait_tied<D / 32>(va[0]);
#pragma unroll
      for (int step = 1; step < R::kSub * 2; ++step) lgkm_wait_tied<D / 32>(va[step]);
    }

    // ---- P = exp2(c s - c m), then O^T += V^T . P^T. Step ks of a sub-block
    // takes elements 8ks .. 8ks+7: contraction index 8*half + i is token
    // 4*half + 16ks + 8*(i/4) + i%4 of the sub-block. P is multiplied as two
    // bf16 parts, hi = P rounded to bf16 and lo = the rounding error rounded
    // again: P alone in bf16 carries a relative error up to 2^-8, which a row
    // that attends few tokens does not average away; hi + lo is within about
    // 2^-16 of P.
    float ps = 0.f;
#pragma unroll
    for (int sb = 0; sb < R::kSub; ++sb) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint32_t phw[4], plw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e0 = __builtin_amdgcn_exp2f(fmaf(sc[sb][8 * ks + 2 * i], c, -mc));
          const float e1 = __builtin_amdgcn_exp2f(fmaf(sc[sb][8 * ks + 2 * i + 1], c, -mc));
          ps += e0 + e1;
          split_bf16x2(e0, e1, phw[i], plw[i]);
        }
        const u32x4_t ph = {phw[0], phw[1], phw[2], phw[3]};
        const u32x4_t pl = {plw[0], plw[1], plw[2], plw[3]};
        const int step = 2 * sb + ks;
        bf16x8_t vfr[D / 32];
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          if constexpr (kKv == 1) {
            vfr[t] = widen8(va8[step][t]);
          } else {
            const u32x4_t av = {va[step][t][0][0], va[step][t][0][1], va[step][t][1][0], va[step][t][1][1]};
            vfr[t] = __builtin_bit_cast(bf16x8_t, av);
          }
        }
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[t], __builtin_bit_cast(bf16x8_t, ph), o[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[t], __builtin_bit_cast(bf16x8_t, pl), o[t], 0, 0, 0);
      }
    }
    l_run += sum_with_partner32(ps);
  }
  // loads past the end may still be landing in the ring
  wait_vmcnt<0>();

  // waves that hand their state on (the second token half of a split tile)
  // stay until the last barrier of a cut prefill tile, idle
  bool holds = true;
  if constexpr (R::kSplit) {
  // ---- merge the two token halves of each row: waves 4..7 hand (m, l, o)
  // to waves 0..3 through the (drained) ring, lane-for-lane
  __syncthreads();
  float* xo = reinterpret_cast<float*>(&s_ring[0][0][0]);  // [4 waves][D/32][16][64]
  __shared__ float s_ml[4][2][64];
  if (wtok == 1) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[((wrow * (D / 32) + t) * 16 + r) * 64 + lane] = o[t][r];
    s_ml[wrow][0][lane] = m_run;
    s_ml[wrow][1][lane] = l_run;
  }
  __syncthreads();
  holds = wtok == 0;
  if (!kPrefill && !holds) return;
  if (holds) {
    // either half may have attended nothing (m = -inf, l = 0, o = 0)
    const float m2 = s_ml[wrow][0][lane], l2 = s_ml[wrow][1][lane];
    const float mm = fmaxf(m_run, m2);
    const float a1 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - mm) * c);
    const float a2 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m2 - mm) * c);
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        o[t][r] = o[t][r] * a1 + xo[((wrow * (D / 32) + t) * 16 + r) * 64 + lane] * a2;
    l_run = l_run * a1 + l2 * a2;
    m_run = mm;
  }
  }  // kSplit

  // ---- this row's state: o / l and lse; a row that attended nothing has
  // o = 0 and lse = -inf
  const bool mine = holds && row_ok;  // this lane holds a row of the tile
  const bool empty = l_run == 0.f;
  // V's dequantisation scale (1 for bf16) multiplies outputs and partial
  // states alike: the merge of partials is linear in them
  const float inv = empty ? 0.f : p.v_scale / l_run;
  // log2 units of the scaled scores (m_run is an unscaled score)
  const float lse2 = empty ? -INFINITY : m_run * c + __builtin_amdgcn_logf(l_run);
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  if constexpr (!kPrefill) {
    // prefix rows: partial state to slot prefix_slot[b][h] + chunk (G rows
    // per slot), merged by the decode kernel's trees
    if (!mine) return;
    float* dst = p.part_o + ((int64_t)slot_base * G + gi) * D;
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
    if (half == 0) p.part_lse[(int64_t)slot_base * G + gi] = lse2;
    return;
  } else {
  if (slot_base < 0) {
    // the tile's only chunk: bf16 out and natural-log lse of the row
    if (!mine) return;
    __bf16* dst = p.out + q_index * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * t + 8 * q4 + 4 * half;
        const bf16x4_t v = {(__bf16)(o[t][4 * q4] * inv), (__bf16)(o[t][4 * q4 + 1] * inv),
                            (__bf16)(o[t][4 * q4 + 2] * inv), (__bf16)(o[t][4 * q4 + 3] * inv)};
        *reinterpret_cast<bf16x4_t*>(dst + d) = v;
      }
    }
    if (half == 0 && p.lse) p.lse[q_index] = lse2 * kLn2;
    return;
  }

  // ---- a cut tile: this chunk's state goes to its partial slot in the
  // order the registers hold it (row group w's 32 rows x D floats as D / 4
  // runs of 512 bytes, run 8t + j holding elements 2j, 2j + 1 of tile t of
  // every lane), written through to the device-coherent level; then the
  // chunk counts its arrival at the tile's merge, and the chunk that
  // arrives last merges the tile (closed form of softmax over a disjoint
  // union of token sets; FlashInfer paper explainer, visionhong.com,
  // benchmark section: the split scheduler's pieces are merged).
  constexpr int kRuns = D / 4;
  constexpr int kBlockFloats = 32 * D;  // one row group's state
  const int merge = p.pitems[(int64_t)blockIdx.x * FI_QITEM_STRIDE + FI_QITEM_MERGE];
  const int32_t* mg = p.merges + (int64_t)merge * FI_QMERGE_STRIDE;
  const int nch = mg[FI_QMERGE_NUM_CHUNKS];
  const int64_t slot0 = mg[FI_QMERGE_SLOT_BEGIN];
  constexpr int64_t kSlotFloats = (int64_t)FI_PREFILL_ROWS * D;
  if (mine) {
    float* dst = p.part_o + (int64_t)slot_base * kSlotFloats + wrow * kBlockFloats + 2 * lane;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int jp = 0; jp < 8; ++jp)
        store_coherent2(dst + (8 * t + jp) * 128, o[t][2 * jp] * inv, o[t][2 * jp + 1] * inv);
    if (half == 0) store_coherent(p.part_lse + (int64_t)slot_base * FI_PREFILL_ROWS + row, lse2);
  }
  // Each wave's stores are complete (acknowledged by the coherent level)
  // before the barrier, so every store of the work-group precedes the
  // arrival thread 0 issues after it. The page-id window is free now (every
  // wave has left the block loop) and carries the election.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(p.counters + merge, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == nch - 1;
    if (last) __hip_atomic_store(p.counters + merge, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_pid[0] = (uint32_t)last;
  }
  __syncthreads();
  if (!s_pid[0] || !mine) return;

  // ---- the merge: each lane folds its own elements of every chunk in
  // chunk order (so the result does not depend on which chunk finished
  // last), 16 runs per pass with four chunks' loads in flight, the running
  // maximum raised per group of four (a chunk the row attended nothing of
  // has lse = -inf and weight 0). Every load reads the coherent level.
  const float* lse0 = p.part_lse + slot0 * FI_PREFILL_ROWS + row;
  __bf16* out_row = p.out + q_index * D;
  float mx = -INFINITY, den = 0.f;
  static_for<kRuns / 16>([&](auto PASS) {
    constexpr int r0 = decltype(PASS)::value * 16;
    constexpr int kK = 4;  // chunks per group
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    f32x2_t acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = f32x2_t{0.f, 0.f};
    mx = -INFINITY;
    den = 0.f;
    for (int c0 = 0; c0 < nch; c0 += kK) {
      float sv[kK];
      coh_u32x2_t v[kK][16];
#pragma unroll
      for (int k = 0; k < kK; ++k) {
        const int ch = min(c0 + k, nch - 1);  // a short group re-reads its last chunk, weight 0
        sv[k] = load_coherent(lse0 + (int64_t)ch * FI_PREFILL_ROWS);
        const BufRes rs = buffer_of(p.part_o + (slot0 + ch) * kSlotFloats + wrow * kBlockFloats,
                                    kBlockFloats * 4);
#pragma unroll
        for (int i = 0; i < 16; ++i) v[k][i] = load_coherent_run(rs, 8u * lane, 512 * (r0 + i));
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
      for (int i = 0; i < 16; ++i) {
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
    // runs 8t + 2q4 and 8t + 2q4 + 1 hold dims 32t + 8q4 + 4half .. +3
    const float rinv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const int run = r0 + i;
      const int d = 32 * (run / 8) + 8 * ((run % 8) / 2) + 4 * half;
      const bf16x4_t o4 = {(__bf16)(acc[i][0] * rinv), (__bf16)(acc[i][1] * rinv),
                           (__bf16)(acc[i + 1][0] * rinv), (__bf16)(acc[i + 1][1] * rinv)};
      *reinterpret_cast<bf16x4_t*>(out_row + d) = o4;
    }
  });
  if (half == 0 && p.lse)
    p.lse[q_index] = den > 0.f ? (mx + __builtin_amdgcn_logf(den)) * kLn2 : -INFINITY;
  }  // kPrefill
}

// ceil(2^32 / page_size), split into its low word and the 2^32 bit
void set_page_magic(TileParams& p) {
  const uint64_t m = ((1ull << 32) + (uint64_t)p.page_size - 1) / (uint64_t)p.page_size;
  p.page_magic = (uint32_t)m;
  p.page_magic_hi = (uint32_t)(m >> 32);
}

}  // namespace

hipError_t launch_prefix(const PrefixArgs& a, hipStream_t stream) {
  if (a.num_items <= 0) return hipSuccess;
  TileParams p{};
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
  set_page_magic(p);
  p.group = a.group;
  p.scale_log2 = a.sm_scale * kLog2e;
  p.v_scale = 1.f;
  const dim3 grid((uint32_t)a.num_items), block(64 * kWaves);
  if (a.head_dim == 128) hipLaunchKernelGGL((tile_attend_kernel<128, false>), grid, block, 0, stream, p);
  else if (a.head_dim == 64) hipLaunchKernelGGL((tile_attend_kernel<64, false>), grid, block, 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.num_items <= 0) return hipSuccess;
  TileParams p{};
  p.pitems = a.items;
  p.page_ids = a.page_ids;
  p.out = static_cast<__bf16*>(a.out);
  p.lse = a.lse;
  p.q = static_cast<const char*>(a.q);
  p.k_pages = static_cast<const char*>(a.k_pages);
  p.v_pages = static_cast<const char*>(a.v_pages);
  p.part_o = a.part_o;
  p.part_lse = a.part_lse;
  p.merges = a.merges;
  p.counters = a.counters;
  const int64_t row = (int64_t)a.head_dim * a.kv_bytes;
  p.head_stride = (int64_t)a.page_size * row;
  p.page_stride = (int64_t)a.num_kv_heads * a.page_size * row;
  p.num_qo_heads = a.num_qo_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.page_size = a.page_size;
  set_page_magic(p);
  p.group = a.group;
  p.causal = a.causal;
  // K's dequantisation scale multiplies every score, V's the outputs
  p.scale_log2 = a.sm_scale * a.k_scale * kLog2e;
  p.v_scale = a.v_scale;
  const dim3 grid((uint32_t)a.num_items), block(64 * kWaves);
  if (a.rope) {
    if (a.head_dim != 128 || a.kv_bytes != 2) return hipErrorInvalidValue;
    p.rope_log2_theta = std::log2((double)a.rope_theta);
    p.rope_rev = 1.0 / (2.0 * M_PI * (double)a.rope_scale);
    hipLaunchKernelGGL((tile_attend_kernel<128, true, 2, true>), grid, block, 0, stream, p);
  } else if (a.kv_bytes == 1) {
    if (a.head_dim != 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL((tile_attend_kernel<128, true, 1>), grid, block, 0, stream, p);
  } else if (a.head_dim == 128) {
    hipLaunchKernelGGL((tile_attend_kernel<128, true>), grid, block, 0, stream, p);
  } else if (a.head_dim == 64) {
    hipLaunchKernelGGL((tile_attend_kernel<64, true>), grid, block, 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fi
