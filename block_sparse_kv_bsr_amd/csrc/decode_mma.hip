// Paged / BSR grouped-query decode attention on the matrix cores of gfx950,
// for the variants whose vector work bounds the vector-ALU kernel
// (decode_bsr.hip): an fp8 (E4M3) KV cache, whose bytes per token are half
// of bf16's for the same arithmetic, and eight query heads per KV head.
//
// What is computed is the same as decode_bsr.hip (FlashInfer paper
// explainer, "FlashInfer: Block-Sparse KV 캐시로 어텐션 병목을 해소하다",
// sections on the attention bottleneck and the Block-Sparse format): per
// work item (request, KV head, chunk of whole pages) the G query heads of
// the KV head attend over the chunk's tokens, whose pages come from the
// request's block list; the quantised cache is dequantised in the kernel
// (same page, JIT section). The work is laid out for the matrix cores:
//
//  * One wave per item. Blocks of BT tokens (32 for fp8, 16 for bf16, 4 KiB
//    of K and 4 KiB of V either way) stream into a 2-stage LDS ring with
//    gfx950's direct-to-LDS loads; a stage is refilled as soon as its
//    fragments are in registers, so two blocks are in flight while one is
//    computed. Loads past the item's last token re-read that token (in
//    bounds, finite), so the products never see a padding slot.
//  * Scores: S^T[token][head] = K . Q^T with v_mfma_f32_16x16x32_bf16, one
//    16-token tile per product chain over d = 128 (4 products). Q^T is the
//    B operand (16 columns, the G heads and zero padding); the fp8 K codes
//    are widened to bf16 (exact) on the way into the A operand.
//  * Online softmax on the accumulators: lane n + 16g holds head n and
//    tokens 4g .. 4g+3 of each tile, so the per-head block maximum is a
//    lane-local maximum plus two lane swaps (lanes n, n^16, n^32, n^48);
//    the running maximum is raised lazily (weights stay <= 2^8), each lane
//    keeps its own running sum.
//  * PV: O^T[d][head] += V^T . P^T with P^T straight from the score
//    accumulators (the contraction index enumerates tokens in the order the
//    score layout leaves them), V^T fragments from gfx950's transposing LDS
//    reads (ds_read_b64_tr_b8 for fp8 over 32 tokens with
//    v_mfma_f32_16x16x32_bf16, ds_read_b64_tr_b16 for bf16 over 16 tokens
//    with v_mfma_f32_16x16x16bf16_1k). P is multiplied as two bf16 parts,
//    hi = bf16(P) and lo = bf16(P - hi), so P's rounding (2^-9 relative in
//    bf16 alone) stays far below the output tolerance.
//  * 16-byte pieces of each K and V row are XOR-swizzled in LDS (through the
//    source addresses of the direct-to-LDS loads) so the fragment reads stay
//    at or below two-way bank conflicts.
//  * Rotary embedding (same page, JIT section: fused into the kernel; the
//    cache holds keys before it): a lane's K and q values already form whole
//    rotate-half pairs (dims i and i + 64 sit in slices s and s + 2), so each
//    lane turns its own K rows in fp32 and feeds them as hi + lo bf16 parts,
//    with q turned once and split the same way: S = Kh.Qh + Kh.Ql + Kl.Qh.
//
// Lane layouts (checked on the GPU with in-bounds probes): for
// v_mfma_f32_16x16x32_bf16, A[m][k] sits in lane m + 16 (k/8), element k%8;
// B[k][n] in lane n + 16 (k/8), element k%8; C[m][n] in lane n + 16 (m/4),
// element m%4. v_mfma_f32_16x16x16bf16_1k: the same with k/4 and k%4.
// ds_read_b64_tr_b8: within each 16-lane group, output lane 8p + q receives
// as byte j byte q of input lane 2j + p. ds_read_b64_tr_b16: output lane
// 4p + q receives as element k element q of input lane 4k + p.
//
// The epilogue is the vector kernel's: bf16 output and natural-log LSE for a
// request in one chunk, else an fp32 partial state that the request's merge
// tree folds in this kernel (finish_split).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "decode_common.h"
#include "fi_bsr.h"
#include "kernels.h"

namespace fi {
namespace {

typedef __bf16 mma_bf16x8_t __attribute__((ext_vector_type(8)));
typedef short mma_s16x4_t __attribute__((ext_vector_type(4)));
typedef float mma_f32x4_t __attribute__((ext_vector_type(4)));

// Geometry of a block of the ring for a K/V element of kKv bytes, d = 128.
template <int kKv>
struct Mma {
  static constexpr int D = 128;
  static constexpr int kRowBytes = D * kKv;              // 128 (fp8) or 256 (bf16)
  static constexpr int kBT = kKv == 1 ? 32 : 16;         // tokens per block
  static constexpr int kTiles = kBT / 16;                // score tiles per block
  static constexpr int kBlockBytes = kBT * kRowBytes;    // K (or V) of a block: 4 KiB
  static constexpr int kLoads = kBlockBytes / 1024;      // wave-wide 16-byte loads per block
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;  // 8 (fp8) or 4 (bf16)
  static constexpr int kPieces = kRowBytes / 16;         // 16-byte pieces per row
  static constexpr int kStageBytes = 2 * kBlockBytes;    // K then V
  static_assert(kLoads == 4 && kTiles * 16 == kBT, "block geometry");
  // Piece swizzle of block row r: LDS piece c of row r holds global piece
  // c ^ swz(r). fp8 K reads take one half-piece of 16 consecutive rows, V
  // reads whole pieces of rows 4g .. 4g+3 and 16 + 4g .. +3; bf16 K reads one
  // piece of 16 rows, V reads two pieces of rows 4g .. 4g+3.
  static __device__ __forceinline__ int swz(int r) {
    if constexpr (kKv == 1)
      return ((r >> 1) & 7) ^ (((r >> 4) & 1) << 2);
    else
      return ((r << 1) | (r >> 3)) & 15;
  }
};

template <int OFF>
__device__ __forceinline__ u32x2_t mma_lds_b64(uint32_t a) {
  u32x2_t r;
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF) : "memory");
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x4_t mma_lds_b128(uint32_t a) {
  u32x4_t r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF) : "memory");
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2_t mma_lds_tr8(uint32_t a) {
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF) : "memory");
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2_t mma_lds_tr16(uint32_t a) {
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF) : "memory");
  return r;
}

// s_waitcnt lgkmcnt(0) with the fragments as operands, so no use of them
// can be scheduled above the wait.
__device__ __forceinline__ void mma_wait_tied(u32x2_t (&a)[8], u32x2_t (&b)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]),
                 "+v"(a[7]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(b[4]), "+v"(b[5]),
                 "+v"(b[6]), "+v"(b[7])::"memory");
}
__device__ __forceinline__ void mma_wait_tied(u32x4_t (&a)[4], u32x2_t (&b)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]),
                 "+v"(b[3]), "+v"(b[4]), "+v"(b[5]), "+v"(b[6]), "+v"(b[7])::"memory");
}

// Eight fp8 (E4M3) codes, two words, widened to eight bf16 values (exact:
// every E4M3 value is a bf16 value) in code order.
__device__ __forceinline__ mma_bf16x8_t widen_fp8x8(u32x2_t w) {
  const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false));
  const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true));
  const uint32_t c = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false));
  const uint32_t d = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true));
  return __builtin_bit_cast(mma_bf16x8_t, u32x4_t{a, b, c, d});
}

// Two floats rounded to a packed bf16 pair (nearest even), and the pair's
// rounding errors rounded to a second pair.
__device__ __forceinline__ void mma_split(float x, float y, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(x, y);
  lo = pack_bf16(x - __uint_as_float(hi << 16), y - __uint_as_float(hi & 0xFFFF0000u));
}

// Eight floats as two bf16x8 fragments, hi = bf16(x) and lo = bf16(x - hi):
// hi + lo is within ~2^-17 of x.
__device__ __forceinline__ void split_x8(const float (&x)[8], mma_bf16x8_t& hi, mma_bf16x8_t& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) mma_split(x[2 * i], x[2 * i + 1], h[i], l[i]);
  hi = __builtin_bit_cast(mma_bf16x8_t, u32x4_t{h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(mma_bf16x8_t, u32x4_t{l[0], l[1], l[2], l[3]});
}

__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int kKv, int G, bool kStream, bool kRope>
__global__ __launch_bounds__(64, 2) void decode_mma_kernel(DecodeParams p) {
  using M = Mma<kKv>;
  constexpr int D = 128;
  constexpr int BT = M::kBT;
  constexpr int RB = M::kRowBytes;
  constexpr int SB = M::kStageBytes;
  static_assert(G >= 1 && G <= 16, "the heads of a KV head fill at most 16 columns");

  const int lane = threadIdx.x;
  const int g = lane >> 4, n = lane & 15;
  const int32_t* it = p.items + (int64_t)blockIdx.x * FI_ITEM_STRIDE;
  const int b = it[FI_ITEM_REQUEST];
  const int kvh = it[FI_ITEM_KV_HEAD];
  const int pb = it[FI_ITEM_PAGE_BEGIN];
  const int ntok = it[FI_ITEM_NUM_TOKENS];
  const int slot = it[FI_ITEM_SLOT];
  const int npg = it[FI_ITEM_NUM_PAGES];
  const int node = it[FI_ITEM_MERGE_NODE];
  const int P = p.page_size;  // a multiple of 16: a 16-token half never straddles pages
  const int64_t qrow0 = (int64_t)b * p.num_qo_heads + (int64_t)kvh * G;

  if (ntok == 0) {  // a request with no pages: out = 0, lse = -inf
    const int h = lane >> 3, sub = lane & 7;
    if (h < G) {
      char* dst = p.out + (qrow0 + h) * (D * 2) + sub * 32;
      *reinterpret_cast<uint4*>(dst) = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(0, 0, 0, 0);
      if (sub == 0 && p.lse) p.lse[qrow0 + h] = -INFINITY;
    }
    return;
  }

  __shared__ int s_ids[kIdWindow];
  __shared__ __attribute__((aligned(1024))) char s_ring[2][SB];

  // ---- page-id window: entry i is the id of page wbase + i of the chunk
  int wbase = 0;
  auto fill_window = [&](int base) {
    int w[kIdWindow / 64];
#pragma unroll
    for (int i = 0; i < kIdWindow / 64; ++i) w[i] = p.page_ids[pb + min(base + i * 64 + lane, npg - 1)];
#pragma unroll
    for (int i = 0; i < kIdWindow / 64; ++i) s_ids[i * 64 + lane] = w[i];
    __syncthreads();
  };
  fill_window(0);

  // ---- rotary embedding (K and q stored before it): this lane's K and q
  // values are dims 32 s + 8 g + e (s < 4, e < 8), and dims i and i + 64 form
  // a rotate-half pair, so the lane holds 16 whole pairs, i = 32 s + 8 g + e
  // for s < 2. Pair i turns by pos * freq_i revolutions; freq_i is kept in
  // LDS as a 64-bit binary fraction of a revolution per position (lane i
  // computes it in double precision), so pos * freq_i mod 1 is exact.
  __shared__ uint64_t s_freq[kRope ? 64 : 1];
  int kv_pos0 = 0;
  if constexpr (kRope) {
    double fq = exp2(-(2.0 * lane / D) * p.rope_log2_theta) * p.rope_rev;
    fq -= floor(fq);
    s_freq[lane] = (uint64_t)ldexp(fq, 64);
    __syncthreads();
    kv_pos0 = it[FI_ITEM_KV_POS];
  }

  // ---- Q^T, the B operand of the score products: lane n + 16g holds
  // q[head n][32 s + 8 g .. +7] for s = 0..3 (zero columns past G). With the
  // rotary embedding q is turned at the query position in fp32 and carried
  // as two bf16 parts, qb (hi) and qbl (lo).
  mma_bf16x8_t qb[4], qbl[kRope ? 4 : 1];
  {
    const char* qr = p.q + (qrow0 + (n < G ? n : 0)) * (D * 2);
    uint4 raw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      raw[s] = load16(qr + (32 * s + 8 * g) * 2);
      if (n >= G) raw[s] = make_uint4(0, 0, 0, 0);
    }
    if constexpr (!kRope) {
#pragma unroll
      for (int s = 0; s < 4; ++s) qb[s] = __builtin_bit_cast(mma_bf16x8_t, raw[s]);
    } else {
      float x[4][8];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t w[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[s][2 * i] = bf16_lo(w[i]);
          x[s][2 * i + 1] = bf16_hi(w[i]);
        }
      }
      const int qpos = it[FI_ITEM_Q_POS];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float cq, sq;
          rope_sincos(s_freq[32 * s + 8 * g + e], qpos, cq, sq);
          const float a = x[s][e], b = x[s + 2][e];
          x[s][e] = a * cq - b * sq;
          x[s + 2][e] = b * cq + a * sq;
        }
#pragma unroll
      for (int s = 0; s < 4; ++s) split_x8(x[s], qb[s], qbl[s]);
    }
  }
  // rotation of this lane's 16 pairs at its token of the current score tile
  // (position kv_pos0 + 16 t + n for the t-th tile of the item), advanced by
  // 16 positions per tile and recomputed exactly every 32 tiles
  float rc[kRope ? 2 : 1][8], rs[kRope ? 2 : 1][8], dc[kRope ? 2 : 1][8], dsn[kRope ? 2 : 1][8];
  if constexpr (kRope) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) rope_sincos(s_freq[32 * s + 8 * g + e], 16, dc[s][e], dsn[s][e]);
  }

  // ---- direct-to-LDS loads. Wave-wide load i of a block covers rows
  // i * kRowsPerLoad .. of the block (one 16-row half, so one page): this
  // lane fills LDS piece dma_c of row r_i with global piece dma_c ^ swz(r_i)
  // of token row (first token of the half + row in half), clamped to the
  // item's last token.
  const int dma_row = lane / M::kPieces;
  const int dma_c = lane % M::kPieces;
  int rih[M::kLoads];   // row within its 16-row half
  int poff[M::kLoads];  // byte offset of the fetched piece within a row
  int doff[M::kLoads];  // byte offset from the half's first row (no clamp)
#pragma unroll
  for (int i = 0; i < M::kLoads; ++i) {
    const int r = i * M::kRowsPerLoad + dma_row;
    rih[i] = r & 15;
    poff[i] = (dma_c ^ M::swz(r)) * 16;
    doff[i] = rih[i] * RB + poff[i];
  }
  const int64_t kvh_off = (int64_t)kvh * p.head_stride;
  const int last_pl = npg - 1;
  const int last_slot = (ntok - 1) - last_pl * P;
  int cur_pl = 0, cur_slot = 0;      // page and slot of the next half to issue
  int cached_pl = -1;
  int64_t cached_base = 0;
  auto page_base = [&](int pl) -> int64_t {
    if (pl != cached_pl) {
      if (pl - wbase >= kIdWindow) {  // rare: slide the window
        __syncthreads();
        wbase = pl;
        fill_window(wbase);
      }
      const int pid = __builtin_amdgcn_readfirstlane(lds_read_id(&s_ids[pl - wbase]));
      cached_base = (int64_t)pid * p.page_stride + kvh_off;
      cached_pl = pl;
    }
    return cached_base;
  };
  // Issues block j into ring stage ST; blocks are issued in order, once each.
  auto issue = [&](int j, auto ST) {
    constexpr int st = decltype(ST)::value;
#pragma unroll
    for (int hh = 0; hh < M::kTiles; ++hh) {
      const int tok_h = j * BT + 16 * hh;
      int pl, sl, lim;
      if (tok_h < ntok) {
        pl = cur_pl;
        sl = cur_slot;
        lim = min(15, ntok - 1 - tok_h);
      } else {  // the whole half past the end: every row re-reads the last token
        pl = last_pl;
        sl = last_slot;
        lim = 0;
      }
      cur_slot += 16;
      if (cur_slot == P) {
        cur_slot = 0;
        cur_pl += 1;
      }
      const int64_t base = page_base(pl) + (int64_t)sl * RB;
      const char* kp = p.k_pages + base;
      const char* vp = p.v_pages + base;
      constexpr int kPerHalf = 16 / M::kRowsPerLoad;  // loads per 16-row half
      if (lim == 15) {
#pragma unroll
        for (int u = 0; u < kPerHalf; ++u) {
          const int i = hh * kPerHalf + u;
          dma16<kStream>(kp + doff[i], &s_ring[st][i * 1024]);
          dma16<kStream>(vp + doff[i], &s_ring[st][M::kBlockBytes + i * 1024]);
        }
      } else {  // the item's last half: rows past its last token re-read it
#pragma unroll
        for (int u = 0; u < kPerHalf; ++u) {
          const int i = hh * kPerHalf + u;
          const int off = min(rih[i], lim) * RB + poff[i];
          dma16<kStream>(kp + off, &s_ring[st][i * 1024]);
          dma16<kStream>(vp + off, &s_ring[st][M::kBlockBytes + i * 1024]);
        }
      }
    }
  };

  // ---- LDS read addresses (lane constants; the stage is an immediate
  // offset). K: tile T, d-slice s; V: d-tile dt.
  constexpr int NKR = kKv == 1 ? 8 : 4;
  uint32_t ka[NKR], va[8];
  const uint32_t ring0 = lds_addr(&s_ring[0][0]);
  if constexpr (kKv == 1) {
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int t = 16 * T + n;
        const int gp = 2 * s + (g >> 1);
        ka[T * 4 + s] = ring0 + t * RB + ((gp ^ M::swz(t)) << 4) + ((g & 1) << 3);
      }
    // transposed read of group g: input lane 2j + p points at row
    // pi_g(j) = 4g + j (j < 4) or 16 + 4g + j - 4, half p of piece dt
    const int jj = n >> 1, pp = n & 1;
    const int row = jj < 4 ? 4 * g + jj : 16 + 4 * g + (jj - 4);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      va[dt] = ring0 + M::kBlockBytes + row * RB + ((dt ^ M::swz(row)) << 4) + (pp << 3);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int gp = 4 * s + g;
      ka[s] = ring0 + n * RB + ((gp ^ M::swz(n)) << 4);
    }
    // input lane 4k + pq points at row 4g + k, columns 16 dt + 4 pq .. +3
    const int kk = n >> 2, pq = n & 3;
    const int row = 4 * g + kk;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int gp = 2 * dt + (pq >> 1);
      va[dt] = ring0 + M::kBlockBytes + row * RB + ((gp ^ M::swz(row)) << 4) + ((pq & 1) << 3);
    }
  }

  mma_f32x4_t o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = mma_f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.scale_log2;
  const float margin = kRescaleMargin / c;
  const int nblocks = (ntok + BT - 1) / BT;

  issue(0, std::integral_constant<int, 0>{});
  if (nblocks > 1) issue(1, std::integral_constant<int, 1>{});

  auto body = [&](int j, auto ST) {
    constexpr int st = decltype(ST)::value;
    constexpr int kOff = st * SB;
    // block j has landed; block j + 1 may still be in flight
    if (j + 1 < nblocks)
      wait_vmcnt<2 * M::kLoads>();
    else
      wait_vmcnt<0>();
    mma_f32x4_t sc[M::kTiles];
    u32x2_t vr[8];
    if constexpr (kRope) {
      // K of each tile in fp32, turned at its tokens' positions, then as hi +
      // lo bf16 parts: S = Kh.Qh + Kh.Ql + Kl.Qh (the dropped Kl.Ql is below
      // 2^-18 of |K||q|)
      u32x2_t kr8[kKv == 1 ? 8 : 1];
      u32x4_t kr16[kKv == 1 ? 1 : 4];
      if constexpr (kKv == 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) kr8[i] = mma_lds_b64<kOff>(ka[i]);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) vr[dt] = mma_lds_tr8<kOff>(va[dt]);
        mma_wait_tied(kr8, vr);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) kr16[i] = mma_lds_b128<kOff>(ka[i]);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) vr[dt] = mma_lds_tr16<kOff>(va[dt]);
        mma_wait_tied(kr16, vr);
      }
      if (j + 2 < nblocks) issue(j + 2, ST);
#pragma unroll
      for (int T = 0; T < M::kTiles; ++T) {
        const int tile = j * M::kTiles + T;
        if ((tile & 31) == 0) {  // exact rotation every 32 tiles
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              rope_sincos(s_freq[32 * s + 8 * g + e], kv_pos0 + 16 * tile + n, rc[s][e], rs[s][e]);
        }
        float x[4][8];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if constexpr (kKv == 1) {
            const u32x2_t w = kr8[T * 4 + s];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const uint32_t ww = h2 ? w.y : w.x;
              const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(ww, false);
              const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(ww, true);
              x[s][4 * h2 + 0] = lo.x;
              x[s][4 * h2 + 1] = lo.y;
              x[s][4 * h2 + 2] = hi.x;
              x[s][4 * h2 + 3] = hi.y;
            }
          } else {
            const uint32_t w[4] = {kr16[s].x, kr16[s].y, kr16[s].z, kr16[s].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              x[s][2 * i] = bf16_lo(w[i]);
              x[s][2 * i + 1] = bf16_hi(w[i]);
            }
          }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float a = x[s][e], b = x[s + 2][e];
            x[s][e] = a * rc[s][e] - b * rs[s][e];
            x[s + 2][e] = b * rc[s][e] + a * rs[s][e];
            // advance to the next tile's token (16 positions on)
            const float c2 = rc[s][e] * dc[s][e] - rs[s][e] * dsn[s][e];
            rs[s][e] = rs[s][e] * dc[s][e] + rc[s][e] * dsn[s][e];
            rc[s][e] = c2;
          }
        mma_f32x4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          mma_bf16x8_t kh, kl;
          split_x8(x[s], kh, kl);
          sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qb[s], sa, 0, 0, 0);
          sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qbl[s], sb, 0, 0, 0);
          sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qb[s], sb, 0, 0, 0);
        }
        sc[T] = sa + sb;
      }
    } else if constexpr (kKv == 1) {
      u32x2_t kr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) kr[i] = mma_lds_b64<kOff>(ka[i]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) vr[dt] = mma_lds_tr8<kOff>(va[dt]);
      mma_wait_tied(kr, vr);
      if (j + 2 < nblocks) issue(j + 2, ST);  // this stage's fragments are in registers
      // the two tiles' product chains alternate (independent accumulators)
      sc[0] = mma_f32x4_t{0.f, 0.f, 0.f, 0.f};
      sc[1] = mma_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int T = 0; T < 2; ++T)
          sc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen_fp8x8(kr[T * 4 + s]), qb[s], sc[T], 0, 0, 0);
    } else {
      u32x4_t kr[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) kr[s] = mma_lds_b128<kOff>(ka[s]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) vr[dt] = mma_lds_tr16<kOff>(va[dt]);
      mma_wait_tied(kr, vr);
      if (j + 2 < nblocks) issue(j + 2, ST);
      sc[0] = mma_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mma_bf16x8_t, kr[s]), qb[s], sc[0], 0, 0, 0);
    }

    // ---- online softmax; element e of tile T is token j BT + 16 T + 4 g + e
    const int tok0 = j * BT;
    if (tok0 + BT > ntok) {  // the item's last block: tokens past the end get weight 0
#pragma unroll
      for (int T = 0; T < M::kTiles; ++T)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (tok0 + 16 * T + 4 * g + e >= ntok) sc[T][e] = -INFINITY;
    }
    float mb = sc[0][0];
#pragma unroll
    for (int T = 0; T < M::kTiles; ++T)
#pragma unroll
      for (int e = 0; e < 4; ++e) mb = fmaxf(mb, sc[T][e]);
    mb = xor32_max(xor16_max(mb));  // block maximum of head n (finite: token j BT is valid)
    const bool up = mb > m_run + margin;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float alpha = up ? exp2_fast((m_run - mb) * c) : 1.f;  // 0 on the first block
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[dt][e] *= alpha;
      m_run = up ? mb : m_run;
    }
    const float mc = m_run * c;

    // ---- P^T (B operand) as hi + lo bf16 parts, then O^T += V^T . P^T
    if constexpr (kKv == 1) {
      // contraction slot 8g + j: tile 0 token 4g + j (j < 4), tile 1 token 4g + j - 4
      float pv[8];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[4 * T + e] = exp2_fast(fmaf(sc[T][e], c, -mc));
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        l_run += pv[2 * i] + pv[2 * i + 1];
        mma_split(pv[2 * i], pv[2 * i + 1], hw[i], lw[i]);
      }
      const mma_bf16x8_t ph = __builtin_bit_cast(mma_bf16x8_t, u32x4_t{hw[0], hw[1], hw[2], hw[3]});
      const mma_bf16x8_t pl = __builtin_bit_cast(mma_bf16x8_t, u32x4_t{lw[0], lw[1], lw[2], lw[3]});
      // all hi products, then all lo ones: consecutive products are independent
      mma_bf16x8_t vt[8];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        vt[dt] = widen_fp8x8(vr[dt]);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[dt], ph, o[dt], 0, 0, 0);
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[dt], pl, o[dt], 0, 0, 0);
    } else {
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[e] = exp2_fast(fmaf(sc[0][e], c, -mc));
      uint32_t hw[2], lw[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        l_run += pv[2 * i] + pv[2 * i + 1];
        mma_split(pv[2 * i], pv[2 * i + 1], hw[i], lw[i]);
      }
      const mma_s16x4_t ph = __builtin_bit_cast(mma_s16x4_t, u32x2_t{hw[0], hw[1]});
      const mma_s16x4_t pl = __builtin_bit_cast(mma_s16x4_t, u32x2_t{lw[0], lw[1]});
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(mma_s16x4_t, vr[dt]), ph,
                                                          o[dt], 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(mma_s16x4_t, vr[dt]), pl,
                                                          o[dt], 0, 0, 0);
    }
  };
  for (int j = 0; j < nblocks; j += 2) {
    body(j, std::integral_constant<int, 0>{});
    if (j + 1 < nblocks) body(j + 1, std::integral_constant<int, 1>{});
  }
  wait_vmcnt<0>();  // nothing is in flight past the last block; kept for the exit

  // ---- epilogue: the sum of head n is spread over lanes n + 16g
  float lt = l_run;
  lt += __shfl_xor(lt, 16);
  lt += __shfl_xor(lt, 32);
  const float lse2 = m_run * c + log2_fast(lt);  // log2 units of the scaled scores
  // lane n + 16g holds O^T[16 dt + 4g + e][n]
  if (slot < 0) {
    if (n < G) {
      const float inv = p.v_scale / lt;
      __bf16* dst = reinterpret_cast<__bf16*>(p.out) + (qrow0 + n) * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<uint2*>(dst + 16 * dt) =
            make_uint2(pack_bf16(o[dt][0] * inv, o[dt][1] * inv), pack_bf16(o[dt][2] * inv, o[dt][3] * inv));
      if (g == 0 && p.lse) p.lse[qrow0 + n] = lse2 * kLn2;
    }
    return;
  }
  // Partial state: staged in the drained ring as [head][d] and written out as
  // float pairs (lane l takes floats 2l + 128c), whole 512-byte runs per
  // store, since these stores write through to HBM. One wave is the whole
  // work-group and its LDS accesses execute in order.
  float* stage = reinterpret_cast<float*>(&s_ring[0][0]);
  static_assert(sizeof(s_ring) >= sizeof(float) * G * D, "ring too small to stage a partial");
  if (n < G) {
    const float inv = 1.f / lt;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<float4*>(stage + n * D + 16 * dt + 4 * g) =
          make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
    if (g == 0) store_shared(p.part_lse + (int64_t)slot * G + n, lse2);
  }
  asm volatile("" ::: "memory");
  constexpr int kF = G * D;
  float* dstp = p.part_o + (int64_t)slot * kF;
#pragma unroll
  for (int cc = 0; cc < (kF / 2 + 63) / 64; ++cc) {
    const int f = 2 * lane + 128 * cc;
    if (kF >= 128 || f < kF) {
      const float2 x = *reinterpret_cast<const float2*>(stage + f);
      store_shared2(dstp + f, x.x, x.y);
    }
  }
  static_assert(kIdWindow >= FI_MERGE_FAN_IN * G, "merge weights reuse the page-id window");
  finish_split<kKv, D, G>(p, node, lane, reinterpret_cast<float*>(s_ids));
}

template <int kKv, int G, bool kRope>
hipError_t launch_mma_typed(const DecodeParams& prm, int64_t num_items, bool stream_kv,
                            hipStream_t stream) {
  if (stream_kv)
    hipLaunchKernelGGL((decode_mma_kernel<kKv, G, true, kRope>), dim3((uint32_t)num_items),
                       dim3(64), 0, stream, prm);
  else
    hipLaunchKernelGGL((decode_mma_kernel<kKv, G, false, kRope>), dim3((uint32_t)num_items),
                       dim3(64), 0, stream, prm);
  return hipGetLastError();
}

template <int kKv, bool kRope>
hipError_t launch_mma_group(const DecodeParams& prm, int64_t n, int G, bool st, hipStream_t s) {
  switch (G) {
    case 1: return launch_mma_typed<kKv, 1, kRope>(prm, n, st, s);
    case 2: return launch_mma_typed<kKv, 2, kRope>(prm, n, st, s);
    case 4: return launch_mma_typed<kKv, 4, kRope>(prm, n, st, s);
    case 8: return launch_mma_typed<kKv, 8, kRope>(prm, n, st, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_mma_supported(const DecodeArgs& a) {
  return a.head_dim == 128 && (a.kv_bytes == 1 || a.kv_bytes == 2) && a.page_size % 16 == 0 &&
         (a.group == 1 || a.group == 2 || a.group == 4 || a.group == 8);
}

hipError_t launch_decode_mma(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_items <= 0) return hipSuccess;
  if (!decode_mma_supported(a)) return hipErrorInvalidValue;
  const DecodeParams prm = make_decode_params(a);
  if (a.rope)
    return a.kv_bytes == 1 ? launch_mma_group<1, true>(prm, a.num_items, a.group, a.stream_kv, stream)
                           : launch_mma_group<2, true>(prm, a.num_items, a.group, a.stream_kv, stream);
  return a.kv_bytes == 1 ? launch_mma_group<1, false>(prm, a.num_items, a.group, a.stream_kv, stream)
                         : launch_mma_group<2, false>(prm, a.num_items, a.group, a.stream_kv, stream);
}

}  // namespace fi
