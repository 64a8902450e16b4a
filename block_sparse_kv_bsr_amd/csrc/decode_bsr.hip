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
//    lane fetches 16 bytes at row offset sub*16 + j*128, so one load
//    instruction covers eight whole 128-byte lines.
//  * The loads go to LDS with gfx950's direct-to-LDS loads
//    (global_load_lds_dwordx4): a ring of kRing steps per wave stays in
//    flight without holding VGPRs, which is what keeps enough bytes in
//    flight per CU to stream HBM. Each lane reads back exactly the 16 bytes
//    it fetched (ds_read_b128 at lane*16), so LDS sees no bank conflicts.
//  * GQA packing: each K/V row is loaded once per KV head and serves all G
//    query heads of the group (query heads kvh*G+i share KV head kvh). The
//    query words live in registers, or at G = 8 in LDS, read per head and
//    step (Tune::kQLds), which keeps that variant at two waves per SIMD.
//  * Scores: bf16 pairs go through v_dot2 (two products + accumulate into
//    fp32 per instruction); the 8 lanes of a token are summed with three DPP
//    row operations inside a half-row, with no LDS traffic.
//  * Softmax: each group of 8 lanes keeps its own running (max, sum,
//    accumulator) state in the log2 domain; the running max is only raised
//    when a score exceeds it by more than 8 (so exp2 stays <= 256), which
//    makes accumulator rescales rare. The eight per-lane-group states are
//    merged once at the end of the item.
//  * The ring reads use inline ds_read_b128 behind explicit vmcnt waits
//    (loads retire in issue order, so "all but the last N loads done" is a
//    count). The compiler cannot tell which ring slot a direct-to-LDS load
//    writes and would otherwise wait for every load in flight before each
//    LDS read. Page ids of a chunk sit in an LDS window.
//  * Tokens past the request's length in the last page are excluded by
//    selection (score -inf, weight 0, V zeroed), never by multiplying by a
//    zero weight, so whatever those slots hold (NaN included) cannot leak.
//
// The result is written directly (bf16 rounded to nearest even, natural-log
// LSE) when the request is one chunk, else as an fp32 partial state (output
// already divided by its own sum, LSE in log2 units) that the request's merge
// tree folds inside this same kernel (finish_split).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "decode_common.h"
#include "fi_bsr.h"
#include "kernels.h"

namespace fi {
namespace {

// Occupancy and ring depth. Streamed (nontemporal) K/V uses a 2-stage ring
// (8 KiB of K/V per wave at bf16, d 128), read back and refilled together:
// deeper rings were measured slower on MI355X there, since with 4 stages
// (16 KiB per wave) more requests queue at the memory controllers and the
// skewed batch lost ~4% bandwidth. When pages are shared between requests
// the loads go through the caches, whose hits return early; a 4-stage ring
// keeps enough bytes in flight for the misses and was ~20% faster on a
// shared-prefix batch.
// VGPRs per lane: accumulators G*NE, query words G*NW, two stages read back
// from LDS (16*L), softmax state and ~48 for addressing and temporaries.
// LDS per wave: kRing stages of 2*L KiB plus the page-id window. Waves per SIMD:
// as many as both budgets allow, at most 3.
template <int kKv, int D, int G, bool kStream, bool kRope = false>
struct Tune {
  using R = Row<kKv, D>;
  // An fp8 stage holds half the bytes of a bf16 one and its waves spend less
  // time per step; 8 stages (16 KiB in flight per wave, the most that still
  // fits 2 waves per SIMD in LDS) measured 17% faster than 4 on the skewed
  // batch. With the rotary embedding the fp8 waves are bound by their vector
  // work, and 4 stages measured 3% faster than 8.
  static constexpr int kRing = kKv == 1 ? (kRope ? 4 : 8) : (kStream ? 2 : 4);
  static_assert(kRing % 2 == 0, "the main loop reads ring stages two at a time");
  // At G = 8 the query words stay in LDS and are read per head and step
  // (the 8 lanes of a column read the same 16 bytes, one broadcast): in
  // registers they would take the wave past 256 and to one wave per SIMD.
  static constexpr bool kQLds = G == 8 && !kRope && D == 128 && kKv <= 2;
  // the rotary embedding keeps q in fp32 (G * kElems) and 4 x D/16 rotation terms
  static constexpr int kRegs =
      G * R::kElems + (kRope ? G * R::kElems + D / 4 : (kQLds ? R::kWords : G * R::kWords)) +
      16 * R::kLoads + 2 * G + 48;
  static constexpr int kByRegs = kRegs <= 168 ? 3 : (kRegs <= 240 ? 2 : 1);
  static constexpr int kLdsPerWave =
      kRing * 2 * R::kLoads * 1024 + kIdWindow * 4 + (kQLds ? G * 8 * R::kWords * 4 : 0);
  static constexpr int kByLds = (160 * 1024) / (4 * kLdsPerWave);
  static constexpr int kWaves = kByRegs < kByLds ? kByRegs : (kByLds >= 1 ? kByLds : 1);
};

template <int kKv, int D, int G, int kRing, int kWaves, bool kStream, bool kUniform, bool kRope>
__global__ __launch_bounds__(64, kWaves) void decode_bsr_kernel(DecodeParams p) {
  using R = Row<kKv, D>;
  static_assert(!kRope || (kKv <= 2 && D == 128) || (kKv == 2 && D == 64),
                "the rotary embedding is built for bf16 (d 128 or 64) and fp8 (d 128)");
  constexpr int L = R::kLoads;
  constexpr bool kQLds = Tune<kKv, D, G, kStream, kRope>::kQLds;
  // With the rotary embedding a lane holds kPairs rotate-half pairs. Where a
  // K row is one 128-byte line (fp8 at d 128, bf16 at d 64), the pairs of a
  // lane sit in two lanes' chunks, and the row is read back from LDS as two
  // 8-byte halves instead (kHalves).
  constexpr int kPairs = D / 16;
  constexpr bool kHalves = kRope && L == 1;
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
  const int first_pid = it[FI_ITEM_FIRST_PAGE];
  const int node = it[FI_ITEM_MERGE_NODE];
  const int P = p.page_size;

  if (ntok == 0) {  // a request with no pages: out = 0, lse = -inf
    if (tg < G) {
      const int64_t qrow = (int64_t)b * p.num_qo_heads + (int64_t)kvh * G + tg;
#pragma unroll
      for (int j = 0; j < R::kBytes / 128; ++j)
        *reinterpret_cast<uint4*>(p.out + qrow * R::kBytes + j * 128 + sub * 16) = make_uint4(0, 0, 0, 0);
      if (sub == 0 && p.lse) p.lse[qrow] = -INFINITY;
    }
    return;
  }

  // ---- page-id window in LDS: entry i is the id of page (wbase + i) of the
  // chunk. Reading ids from LDS keeps the id lookup off the vector-memory
  // counter, so fetching an id never waits for the K/V loads in flight.
  // Every lane loads and stores unconditionally (indices clamped to the
  // chunk), so the wait for these loads is the same on every path.
  __shared__ int s_ids[kIdWindow];
  int wbase = 0;
  int wreg[kIdWindow / 64];
  auto load_window = [&](int base) {
#pragma unroll
    for (int i = 0; i < kIdWindow / 64; ++i)
      wreg[i] = p.page_ids[pb + min(base + i * 64 + lane, npg - 1)];
  };
  auto store_window = [&]() {
#pragma unroll
    for (int i = 0; i < kIdWindow / 64; ++i) s_ids[i * 64 + lane] = wreg[i];
    __syncthreads();
  };
  auto fill_window = [&](int base) {
    load_window(base);
    store_window();
  };
  load_window(0);  // stored below, after the first K/V loads are on their way

  // ---- query fragments of the G heads (same columns as the K/V fragments)
  const int64_t qrow0 = (int64_t)b * p.num_qo_heads + (int64_t)kvh * G;
  uint32_t qw[G][NW];
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int j = 0; j < L; ++j) {
#pragma unroll
      for (int x = 0; x < R::kQLoads; ++x) {
        // the rotary embedding over 128-byte K rows takes the rows' halves
        // (dims kPairs sub .. + kPairs - 1 and D/2 + kPairs sub ..), and q
        // the same dims: two 16-byte loads at d 128, two 8-byte ones at d 64
        if constexpr (kHalves && D == 64) {
          const char* qr = p.q + (qrow0 + h) * R::kBytes + sub * 8;
          const uint2 a = *reinterpret_cast<const uint2*>(qr);
          const uint2 c = *reinterpret_cast<const uint2*>(qr + 64);
          qw[h][0] = a.x;
          qw[h][1] = a.y;
          qw[h][2] = c.x;
          qw[h][3] = c.y;
        } else {
          const int off = kHalves
                              ? (x * (D / 2) + sub * 8) * R::kQoBytes
                              : (j * R::kDimStride + sub * R::kPerLoad) * R::kQoBytes + x * 16;
          const uint4 v = load16(p.q + (qrow0 + h) * R::kBytes + off);
          const int w0 = (j * R::kQLoads + x) * 4;
          qw[h][w0 + 0] = v.x;
          qw[h][w0 + 1] = v.y;
          qw[h][w0 + 2] = v.z;
          qw[h][w0 + 3] = v.w;
        }
      }
    }
  }

  // q words of every head in LDS, [head][sub][word] (see Tune::kQLds)
  __shared__ __attribute__((aligned(16))) uint32_t s_q[kQLds ? G : 1][8][kQLds ? NW : 1];
  if constexpr (kQLds) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int w = 0; w < NW; ++w) s_q[h][sub][w] = qw[h][w];
    __syncthreads();
  }

  // ---- rotary embedding (K stored before it): lane `sub` holds dims
  // kPairs sub + e and D/2 + kPairs sub + e (e < kPairs) of q and of every
  // K row (a bf16 d-128 row's two 16-byte chunks; a 128-byte row read back
  // from LDS as two 8-byte halves), which are exactly the rotate-half pairs
  // i = kPairs sub + e. Pair i's frequency, as a 64-bit fraction of a
  // revolution per position, goes to LDS (lane i computes it in double
  // precision); q turns at the query position here, K rows as they are read
  // (consume). q words: the first kPairs / 2 hold the pairs' first dims.
  __shared__ uint64_t s_freq[kRope ? 64 : 1];
  float qf[kRope ? G : 1][2 * kPairs];
  float rc[kPairs], rs[kPairs], dc[kPairs], ds[kPairs];  // current and per-step rotation
  int rope_step = 0;
  int rope_pos0 = 0;
  if constexpr (kRope) {
    double g = exp2(-(2.0 * lane / D) * p.rope_log2_theta) * p.rope_rev;
    g -= floor(g);
    s_freq[lane] = (uint64_t)ldexp(g, 64);
    __syncthreads();
    const int qpos = it[FI_ITEM_Q_POS];
    rope_pos0 = it[FI_ITEM_KV_POS] + tg;
#pragma unroll
    for (int e = 0; e < kPairs; ++e) {
      const uint64_t f = s_freq[kPairs * sub + e];
      float cq, sq;
      rope_sincos(f, qpos, cq, sq);
      rope_sincos(f, 8, dc[e], ds[e]);  // a step advances 8 positions
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint32_t w1 = qw[h][e >> 1], w2 = qw[h][kPairs / 2 + (e >> 1)];
        const float x1 = (e & 1) ? bf16_hi(w1) : bf16_lo(w1);
        const float x2 = (e & 1) ? bf16_hi(w2) : bf16_lo(w2);
        qf[h][e] = x1 * cq - x2 * sq;
        qf[h][kPairs + e] = x2 * cq + x1 * sq;
      }
    }
  }

  // ---- load cursor: page-local index and slot of this lane's next token
  int cur_pl = tg / P;
  int cur_slot = tg - cur_pl * P;
  const int last_pl = (ntok - 1) / P;
  const int last_slot = (ntok - 1) - last_pl * P;
  const int ngroups = (ntok + 7) >> 3;
  const int nfull = ntok >> 3;
  const int64_t head_off = (int64_t)kvh * p.head_stride + sub * 16;

  // LDS ring: stage s holds the K rows (chunks 0..L-1) and V rows (chunks
  // L..2L-1) of one step, 64 lanes x 16 bytes per chunk.
  __shared__ __attribute__((aligned(16))) uint4 s_ring[kRing][2 * L][64];

  // Issue the K/V loads of step g into ring stage `stage`. Loads are issued
  // on every path (a step past the end re-reads the item's last token, which
  // is cached) so every stage is refilled exactly once per consume and the
  // vmcnt counts below are exact.
  auto issue = [&](int g, int stage) {
    const bool real = g < ngroups;
    int pl = real ? cur_pl : last_pl;
    int sl = real ? cur_slot : last_slot;
    if (g == ngroups - 1 && g * 8 + tg >= ntok) {  // ragged last step: clamp to the last token
      pl = last_pl;
      sl = last_slot;
    }
    if (__builtin_amdgcn_readlane(pl, 63) - wbase >= kIdWindow) {  // rare: slide the window
      __syncthreads();
      wbase = __builtin_amdgcn_readfirstlane(pl);
      fill_window(wbase);
    }
    const int pid = lds_read_id(&s_ids[pl - wbase]);
    const int64_t off = (int64_t)pid * p.page_stride + head_off + (int64_t)sl * R::kKvBytes;
    const char* kp = p.k_pages + off;
    const char* vp = p.v_pages + off;
#pragma unroll
    for (int j = 0; j < L; ++j) dma16<kStream>(kp + j * 128, &s_ring[stage][j][0]);
#pragma unroll
    for (int j = 0; j < L; ++j) dma16<kStream>(vp + j * 128, &s_ring[stage][L + j][0]);
    if (real) {
      cur_slot += p.step_slots;
      cur_pl += p.step_pages;
      if (cur_slot >= P) {
        cur_slot -= P;
        cur_pl += 1;
      }
    }
  };

  // Page sizes that are multiples of 8: the 8 rows of a step always sit in
  // one page, so the page id and the row base are wave-uniform (scalar
  // registers) and each lane adds a fixed offset (row tg, column sub). A
  // ragged last step reads the whole 8 rows of its page (in bounds; the
  // extra rows are masked in consume); a step past the end re-reads the last
  // step.
  const int last_step = ngroups - 1;
  const int u_last_pl = (last_step * 8) / P;
  const int u_last_slot = last_step * 8 - u_last_pl * P;
  const int lane_off = tg * R::kKvBytes + sub * 16;
  const int64_t kvh_off = (int64_t)kvh * p.head_stride;
  int u_pl = 0, u_slot = 0, u_cached_pl = 0, u_pid = first_pid;
  auto issue_uniform = [&](int g, int stage) {
    const bool real = g < ngroups;
    const int pl = real ? u_pl : u_last_pl;
    const int sl = real ? u_slot : u_last_slot;
    if (pl != u_cached_pl) {
      if (pl - wbase >= kIdWindow) {  // rare: slide the window
        __syncthreads();
        wbase = pl;
        fill_window(wbase);
      }
      u_pid = __builtin_amdgcn_readfirstlane(lds_read_id(&s_ids[pl - wbase]));
      u_cached_pl = pl;
    }
    const int64_t base = (int64_t)u_pid * p.page_stride + kvh_off + (int64_t)sl * R::kKvBytes;
    const char* kp = p.k_pages + base;
    const char* vp = p.v_pages + base;
#pragma unroll
    for (int j = 0; j < L; ++j) dma16<kStream>(kp + lane_off + j * 128, &s_ring[stage][j][0]);
#pragma unroll
    for (int j = 0; j < L; ++j) dma16<kStream>(vp + lane_off + j * 128, &s_ring[stage][L + j][0]);
    if (real) {
      u_slot += 8;
      if (u_slot == P) {
        u_slot = 0;
        u_pl += 1;
      }
    }
  };

  auto read_stage = [&](int stage, u32x4_t (&kr)[L], u32x4_t (&vr)[L]) {
    if constexpr (kHalves) {
      // K row of this lane's token: chunks 8 tg .. 8 tg + 7 of the stage
      lds_read_k_halves(lds_addr(&s_ring[stage][0][8 * tg]) + 8 * sub,
                        lds_addr(&s_ring[stage][1][lane]), kr[0], vr[0]);
      return;
    }
    uint32_t addr[2 * L];
    u32x4_t v[2 * L];
#pragma unroll
    for (int j = 0; j < 2 * L; ++j) addr[j] = lds_addr(&s_ring[stage][j][lane]);
    lds_read_stage<2 * L>(addr, v);
#pragma unroll
    for (int j = 0; j < L; ++j) {
      kr[j] = v[j];
      vr[j] = v[L + j];
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

  auto consume = [&](const u32x4_t (&kr)[L], u32x4_t (&vr)[L], bool masked, bool valid) {
    float s[G];
    if constexpr (kRope) {
      // this lane's token of the step sits at rope_pos0 + 8 * step; the
      // rotation is recomputed exactly every 32 steps and advanced by one
      // step's rotation in between (error ~ 32 fp32 roundings)
      if ((rope_step & 31) == 0) {
#pragma unroll
        for (int e = 0; e < kPairs; ++e)
          rope_sincos(s_freq[kPairs * sub + e], rope_pos0 + 8 * rope_step, rc[e], rs[e]);
      }
      float d[G];
#pragma unroll
      for (int h = 0; h < G; ++h) d[h] = 0.f;
      // pair e of this lane: x1 = dim kPairs sub + e, x2 = dim D/2 + kPairs sub + e
      float x1v[kPairs], x2v[kPairs];
      if constexpr (kKv == 1) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const f32x2_t a0 = __builtin_amdgcn_cvt_pk_f32_fp8(word(kr[0], u), false);
          const f32x2_t a1 = __builtin_amdgcn_cvt_pk_f32_fp8(word(kr[0], u), true);
          const f32x2_t b0 = __builtin_amdgcn_cvt_pk_f32_fp8(word(kr[0], 2 + u), false);
          const f32x2_t b1 = __builtin_amdgcn_cvt_pk_f32_fp8(word(kr[0], 2 + u), true);
          x1v[4 * u] = a0[0];
          x1v[4 * u + 1] = a0[1];
          x1v[4 * u + 2] = a1[0];
          x1v[4 * u + 3] = a1[1];
          x2v[4 * u] = b0[0];
          x2v[4 * u + 1] = b0[1];
          x2v[4 * u + 2] = b1[0];
          x2v[4 * u + 3] = b1[1];
        }
      } else if constexpr (kHalves) {  // bf16, d 64: (x, y) first dims, (z, w) second
#pragma unroll
        for (int e = 0; e < kPairs; ++e) {
          const uint32_t w1 = word(kr[0], e >> 1), w2 = word(kr[0], 2 + (e >> 1));
          x1v[e] = (e & 1) ? bf16_hi(w1) : bf16_lo(w1);
          x2v[e] = (e & 1) ? bf16_hi(w2) : bf16_lo(w2);
        }
      } else {
#pragma unroll
        for (int e = 0; e < kPairs; ++e) {
          const uint32_t w1 = word(kr[0], e >> 1), w2 = word(kr[1], e >> 1);
          x1v[e] = (e & 1) ? bf16_hi(w1) : bf16_lo(w1);
          x2v[e] = (e & 1) ? bf16_hi(w2) : bf16_lo(w2);
        }
      }
#pragma unroll
      for (int e = 0; e < kPairs; ++e) {
        const float x1 = x1v[e], x2 = x2v[e];
        const float k1 = x1 * rc[e] - x2 * rs[e];
        const float k2 = x2 * rc[e] + x1 * rs[e];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          d[h] = __builtin_fmaf(k1, qf[h][e], d[h]);
          d[h] = __builtin_fmaf(k2, qf[h][kPairs + e], d[h]);
        }
        const float c2 = rc[e] * dc[e] - rs[e] * ds[e];
        rs[e] = rs[e] * dc[e] + rc[e] * ds[e];
        rc[e] = c2;
      }
      ++rope_step;
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = sum8(d[h]) * p.scale_log2;
    } else {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      // this head's query words: registers, or LDS (Tune::kQLds)
      uint32_t qh[kQLds ? NW : 1];
      if constexpr (kQLds) {
#pragma unroll
        for (int w = 0; w < NW; w += 4) {
          const uint4 t = *reinterpret_cast<const uint4*>(&s_q[h][sub][w]);
          qh[w] = t.x;
          qh[w + 1] = t.y;
          qh[w + 2] = t.z;
          qh[w + 3] = t.w;
        }
      }
      auto qword = [&](int w) -> uint32_t {
        if constexpr (kQLds) return qh[w];
        else return qw[h][w];
      };
      float d = 0.f;
      if constexpr (kKv == 1) {
        // 4 fp8 per K word, widened exactly to two bf16 pairs (converted
        // once per word and reused by all G heads)
#pragma unroll
        for (int w = 0; w < R::kKvWords; ++w) {
          const uint32_t kw = word(kr[w / 4], w % 4);
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw, 1.0f, false),
                                              __builtin_bit_cast(bf16x2_t, qword(2 * w)), d, false);
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw, 1.0f, true),
                                              __builtin_bit_cast(bf16x2_t, qword(2 * w + 1)), d, false);
        }
      } else {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const uint32_t kw = word(kr[w / 4], w % 4);
          if constexpr (kKv == 2) {
            d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kw),
                                                __builtin_bit_cast(bf16x2_t, qword(w)), d, false);
          } else {
            d = __builtin_fmaf(__uint_as_float(kw), __uint_as_float(qword(w)), d);
          }
        }
      }
      s[h] = sum8(d) * p.scale_log2;
    }
    }  // kRope
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
    // rescale only when some score passes its running max by the margin
    float over = s[0] - m[0];
#pragma unroll
    for (int h = 1; h < G; ++h) over = fmaxf(over, s[h] - m[h]);
    if (__any(over > kRescaleMargin)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const bool up = s[h] > m[h] + kRescaleMargin;
        const float f = up ? exp2_fast(m[h] - s[h]) : 1.f;
        m[h] = up ? s[h] : m[h];
        scale_in_place(l[h], f);
#pragma unroll
        for (int e = 0; e < NE; ++e) scale_in_place(acc[h][e], f);
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
    for (int w = 0; w < R::kKvWords; ++w) {
      const uint32_t vw = word(vr[w / 4], w % 4);
      if constexpr (kKv == 1) {
        const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(vw, false);
        const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(vw, true);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h][4 * w] = __builtin_fmaf(pw[h], lo[0], acc[h][4 * w]);
          acc[h][4 * w + 1] = __builtin_fmaf(pw[h], lo[1], acc[h][4 * w + 1]);
          acc[h][4 * w + 2] = __builtin_fmaf(pw[h], hi[0], acc[h][4 * w + 2]);
          acc[h][4 * w + 3] = __builtin_fmaf(pw[h], hi[1], acc[h][4 * w + 3]);
        }
      } else if constexpr (kKv == 2) {
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

  // ---- main loop: a ring of kRing steps in flight. Steps [0, nfull) are
  // whole (8 valid tokens); only step ngroups-1 can be ragged. The loop
  // consumes whole steps; the tail pass consumes what is left (<= kRing
  // steps, all already in flight) with per-lane masking. Before stage s is
  // read, exactly the loads of the stages issued after it may be pending.
  constexpr int kPerStage = 2 * L;
  // The first kRing steps lie in the chunk's first page when the page holds
  // them all: issue them from the inline page id before the window is
  // stored, so the item's first K/V loads overlap the page-table read.
  if constexpr (kUniform) {
    if (kRing * 8 <= P) {
#pragma unroll
      for (int s = 0; s < kRing; ++s) issue_uniform(s, s);
      store_window();
    } else {
      store_window();
#pragma unroll
      for (int s = 0; s < kRing; ++s) issue_uniform(s, s);
    }
  } else {
    store_window();
#pragma unroll
    for (int s = 0; s < kRing; ++s) issue(s, s);
  }
  int g0 = 0;
  for (; g0 + kRing <= nfull; g0 += kRing) {
    // Stages are read back and refilled two at a time: the refill then asks
    // DRAM for both halves of a 4 KiB K page (and of its V page) back to
    // back, which keeps DRAM row hits high; refilling one 2 KiB half per
    // step, with the arithmetic in between, let other waves' requests land
    // in between and cost about a tenth of the bandwidth.
#pragma unroll
    for (int s = 0; s < kRing; s += 2) {
      u32x4_t kr0[L], vr0[L], kr1[L], vr1[L];
      wait_vmcnt<kPerStage * (kRing - 1)>();
      read_stage(s, kr0, vr0);
      wait_vmcnt<kPerStage * (kRing - 2)>();
      read_stage(s + 1, kr1, vr1);
      if constexpr (kUniform) {
        issue_uniform(g0 + s + kRing, s);
        issue_uniform(g0 + s + 1 + kRing, s + 1);
      } else {
        issue(g0 + s + kRing, s);
        issue(g0 + s + 1 + kRing, s + 1);
      }
      consume(kr0, vr0, false, true);
      consume(kr1, vr1, false, true);
    }
  }
#pragma unroll
  for (int s = 0; s < kRing; ++s) {
    const int g = g0 + s;
    u32x4_t kr[L], vr[L];
    wait_stage<kPerStage, kRing>(s);
    if (g < ngroups) {
      read_stage(s, kr, vr);
      consume(kr, vr, true, g * 8 + tg < ntok);
    }
  }
  // Loads past the end may still be in flight into the ring; let them land
  // before the wave can exit and its LDS is handed to another workgroup.
  wait_vmcnt<0>();

  // ---- combine the 8 lane groups (lanes with equal `sub` hold the same
  // columns, for different tokens). The per-head maximum and sum are
  // all-reduced over lane bits 3..5. The G x NE accumulators are then
  // reduce-scattered: each stage hands half of the remaining values to the
  // partner lane and keeps the other half plus the partner's copy of it, so
  // after the stages over lane bits 5, 4 and 3, lane group tg holds the tg-th
  // eighth of the flattened (head, element) block, fully summed. That eighth
  // is exactly what the lane writes out.
  float* stage = reinterpret_cast<float*>(&s_ring[0][0][0]);
  static_assert(sizeof(s_ring) >= sizeof(float) * G * D, "ring too small to stage a partial");
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = group_max8(m[h]);
    const float f = m[h] == -INFINITY ? 0.f : exp2_fast(m[h] - M);
    l[h] = group_sum8(l[h] * f);
    m[h] = M;
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[h][e] *= f;
  }
  constexpr int V = G * NE;   // values per lane before the reduce-scatter
  constexpr int VB = V / 8;   // and after
  static_assert(VB <= NE && NE % VB == 0, "a lane's eighth must lie in one head");
  float* a = &acc[0][0];
#pragma unroll
  for (int i = 0; i < V / 2; ++i) a[i] = swap_sum32(a[i], a[i + V / 2]);
#pragma unroll
  for (int i = 0; i < V / 4; ++i) a[i] = swap_sum16(a[i], a[i + V / 4]);
  {
    const bool hi = (lane & 8) != 0;
#pragma unroll
    for (int i = 0; i < VB; ++i) {
      const float send = hi ? a[i] : a[i + VB];
      const float keep = hi ? a[i + VB] : a[i];
      a[i] = keep + row_ror8(send);
    }
  }

  // ---- epilogue: lane (sub, tg) holds elements e0 .. e0+VB-1 of head hq
  {
    constexpr int PL = R::kPerLoad;
    constexpr int SEG = VB < PL ? VB : PL;  // elements per contiguous piece
    static_assert(SEG <= 4 || SEG % 8 == 0 || !R::kQoBF16, "bf16 pieces are 1, 2, 4 or 8k elements");
    const int hq = tg * VB / NE;
    const int e0 = tg * VB % NE;
    float mh = 0.f, lh = 1.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (h == hq) {
        mh = m[h];
        lh = l[h];
      }
    }
    // V's dequantisation scale is applied once, where a final output is
    // written (here, or at the root of a merge tree); partials stay unscaled
    const float inv = (slot < 0 ? p.v_scale : 1.f) / lh;
#pragma unroll
    for (int i = 0; i < VB; ++i) a[i] *= inv;
    const int64_t qrow = qrow0 + hq;
    const bool lse_lane = e0 == 0 && sub == 0;
#pragma unroll
    for (int sgi = 0; sgi < VB / SEG; ++sgi) {
      const int e = e0 + sgi * SEG;
      // element e sits at dim (e / PL) * kDimStride + sub * PL + e % PL
      const int dim = (e / PL) * R::kDimStride + sub * PL + e % PL;
      const float* x = a + sgi * SEG;
      if (slot < 0) {
        char* dst = p.out + qrow * R::kBytes + dim * R::kQoBytes;
        if constexpr (R::kQoBF16) {
          if constexpr (SEG == 1) {
            *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(pack_bf16(x[0], 0.f) & 0xFFFFu);
          } else if constexpr (SEG == 2) {
            *reinterpret_cast<uint32_t*>(dst) = pack_bf16(x[0], x[1]);
          } else if constexpr (SEG == 4) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]));
          } else {
#pragma unroll
            for (int c = 0; c < SEG; c += 8)
              *reinterpret_cast<uint4*>(dst + 2 * c) =
                  make_uint4(pack_bf16(x[c], x[c + 1]), pack_bf16(x[c + 2], x[c + 3]),
                             pack_bf16(x[c + 4], x[c + 5]), pack_bf16(x[c + 6], x[c + 7]));
          }
        } else {
          if constexpr (SEG == 1) *reinterpret_cast<float*>(dst) = x[0];
          else if constexpr (SEG == 2) *reinterpret_cast<float2*>(dst) = make_float2(x[0], x[1]);
          else *reinterpret_cast<float4*>(dst) = make_float4(x[0], x[1], x[2], x[3]);
        }
      } else {
        // stage the G x D partial in the drained ring (row hq = head hq)
        float* d0 = stage + hq * D + dim;
        if constexpr (SEG == 1) *d0 = x[0];
        else if constexpr (SEG == 2) *reinterpret_cast<float2*>(d0) = make_float2(x[0], x[1]);
        else {
#pragma unroll
          for (int c = 0; c < SEG; c += 4)
            *reinterpret_cast<float4*>(d0 + c) = make_float4(x[c], x[c + 1], x[c + 2], x[c + 3]);
        }
      }
    }
    if (lse_lane) {
      if (slot < 0) {
        if (p.lse) p.lse[qrow] = (mh + log2_fast(lh)) * kLn2;
      } else {
        store_shared(p.part_lse + (int64_t)slot * G + hq, mh + log2_fast(lh));
      }
    }
  }
  if (slot >= 0) {
    // Write the staged partial out as float pairs, lane l taking floats
    // 2l + 128c: each store covers 512 contiguous bytes, whole lines, which
    // matters because these stores write through to HBM (partial lines would
    // cost a read-modify-write each). One wave is the whole work-group and
    // its LDS accesses execute in order, so a compiler barrier suffices.
    asm volatile("" ::: "memory");
    constexpr int kF = G * D;
    float* dst = p.part_o + (int64_t)slot * kF;
#pragma unroll
    for (int c = 0; c < (kF / 2 + 63) / 64; ++c) {
      const int f = 2 * lane + 128 * c;
      if (kF >= 128 || f < kF) {
        const float2 x = *reinterpret_cast<const float2*>(stage + f);
        store_shared2(dst + f, x.x, x.y);
      }
    }
    static_assert(kIdWindow >= FI_MERGE_FAN_IN * G, "merge weights reuse the page-id window");
    finish_split<kKv, D, G>(p, node, lane, reinterpret_cast<float*>(s_ids));
  }
}

template <int kKv, int D, int G, bool kStream, bool kRope>
hipError_t launch_variant(const DecodeParams& prm, int64_t num_items, hipStream_t stream) {
  using T = Tune<kKv, D, G, kStream, kRope>;
  if (prm.page_size % 8 == 0)
    hipLaunchKernelGGL((decode_bsr_kernel<kKv, D, G, T::kRing, T::kWaves, kStream, true, kRope>),
                       dim3((uint32_t)num_items), dim3(64), 0, stream, prm);
  else
    hipLaunchKernelGGL((decode_bsr_kernel<kKv, D, G, T::kRing, T::kWaves, kStream, false, kRope>),
                       dim3((uint32_t)num_items), dim3(64), 0, stream, prm);
  return hipGetLastError();
}

template <int kKv, int D, int G, bool kRope>
hipError_t launch_typed(const DecodeParams& prm, int64_t num_items, bool stream_kv,
                        hipStream_t stream) {
  return stream_kv ? launch_variant<kKv, D, G, true, kRope>(prm, num_items, stream)
                   : launch_variant<kKv, D, G, false, kRope>(prm, num_items, stream);
}

template <int kKv, int D, bool kRope = false>
hipError_t launch_group(const DecodeParams& prm, int64_t n, int G, bool st, hipStream_t s) {
  switch (G) {
    case 1: return launch_typed<kKv, D, 1, kRope>(prm, n, st, s);
    case 2: return launch_typed<kKv, D, 2, kRope>(prm, n, st, s);
    case 4: return launch_typed<kKv, D, 4, kRope>(prm, n, st, s);
    case 8: return launch_typed<kKv, D, 8, kRope>(prm, n, st, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_items <= 0) return hipSuccess;
  if (a.mma) return launch_decode_mma(a, stream);
  const DecodeParams prm = make_decode_params(a);
  if (a.rope) {
    if (a.kv_bytes == 2 && a.head_dim == 128)
      return launch_group<2, 128, true>(prm, a.num_items, a.group, a.stream_kv, stream);
    if (a.kv_bytes == 1 && a.head_dim == 128)
      return launch_group<1, 128, true>(prm, a.num_items, a.group, a.stream_kv, stream);
    if (a.kv_bytes == 2 && a.head_dim == 64)
      return launch_group<2, 64, true>(prm, a.num_items, a.group, a.stream_kv, stream);
    return hipErrorInvalidValue;
  }
  if (a.kv_bytes == 2) {
    if (a.head_dim == 128) return launch_group<2, 128>(prm, a.num_items, a.group, a.stream_kv, stream);
    if (a.head_dim == 64) return launch_group<2, 64>(prm, a.num_items, a.group, a.stream_kv, stream);
  } else if (a.kv_bytes == 4) {
    if (a.head_dim == 128) return launch_group<4, 128>(prm, a.num_items, a.group, a.stream_kv, stream);
    if (a.head_dim == 64) return launch_group<4, 64>(prm, a.num_items, a.group, a.stream_kv, stream);
  } else if (a.kv_bytes == 1) {
    if (a.head_dim == 128) return launch_group<1, 128>(prm, a.num_items, a.group, a.stream_kv, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fi
