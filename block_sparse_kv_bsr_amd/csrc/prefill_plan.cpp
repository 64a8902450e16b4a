// Work list for prefill / append attention over a paged / BSR KV cache.
//
// FlashInfer paper explainer ("FlashInfer: Block-Sparse KV 캐시로 어텐션 병목을
// 해소하다", visionhong.com), section on where the attention bottleneck lies:
// prefill attends every token of a prompt at once and is bound by arithmetic.
// The query tokens of a request are its newest cached tokens; with the causal
// mask query i of n over L cached tokens attends the first L - n + i + 1.
//
// A tile is up to FI_PREFILL_ROWS query rows of one (request, KV head): its
// FI_PREFILL_ROWS / G query tokens times the G query heads that share the KV
// head, so every K/V row a workgroup loads serves all of them (a matrix
// problem for the matrix cores). A tile attends the tokens its last query
// sees. The same load-balancing idea as the decode planner (explainer,
// benchmark section: cut long work into units and interleave them with
// short ones) applies: a tile whose range is long is cut into KV chunks of
// whole pages, and a merge pass combines the chunks' partial states. The
// tiles of one (request, KV head) read the same K/V, so they are kept on one
// L2 domain (XCD) of the chip: pairs are dealt to per-XCD bins by the
// longest-processing-time rule and the bins interleaved in the order the
// dispatcher deals workgroups to XCDs.
//
// Plain C++17 with no HIP dependency: the planner is tested on CPU-only hosts.
#include <algorithm>
#include <cstring>
#include <memory>
#include <new>
#include <string>

#include "plan.h"

namespace fi {

void plan_free_host(fi_prefill_plan* p) { delete p; }

namespace {

fi_status fail(fi_status st, const std::string& msg) {
  set_error(msg);
  return st;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace
}  // namespace fi

namespace fi {
namespace {

// The planner of both call families. mla: multi-head latent attention, one
// latent "KV head" shared by num_qo_heads query heads, tiles of FI_MLA_ROWS
// (query token, head) rows.
fi_status build_tile_plan(const int32_t* qo_indptr, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* kv_last_page_len,
                          int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t page_size, int64_t num_pool_pages,
                          fi_dtype dtype, int32_t causal, const fi_prefill_opts* opts, bool mla,
                          fi_prefill_plan** out_plan) {
  try {
    if (!out_plan) return fail(FI_ERR_INVALID_ARG, "out_plan is NULL");
    *out_plan = nullptr;
    if (batch < 0) return fail(FI_ERR_INVALID_ARG, "batch < 0");
    if (!qo_indptr) return fail(FI_ERR_INVALID_ARG, "qo_indptr is NULL");
    if (num_qo_heads <= 0 || num_kv_heads <= 0)
      return fail(FI_ERR_INVALID_ARG, "head counts must be positive");
    if (num_qo_heads % num_kv_heads != 0)
      return fail(FI_ERR_INVALID_ARG, "num_qo_heads is not a multiple of num_kv_heads");
    const int32_t group = num_qo_heads / num_kv_heads;
    if (!mla && group > FI_PREFILL_ROWS)
      return fail(FI_ERR_UNSUPPORTED, "GQA group size above " + std::to_string(FI_PREFILL_ROWS));
    if (!mla && head_dim != 64 && head_dim != 128)
      return fail(FI_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (dtype != FI_DTYPE_BF16 && dtype != FI_DTYPE_FP8_E4M3)
      return fail(FI_ERR_UNSUPPORTED, "prefill needs FI_DTYPE_BF16 or FI_DTYPE_FP8_E4M3");
    if (dtype == FI_DTYPE_FP8_E4M3 && head_dim != 128)
      return fail(FI_ERR_UNSUPPORTED, "fp8 prefill is built for head_dim 128");
    const bool rope = opts && opts->rope;
    if (mla && rope)
      return fail(FI_ERR_UNSUPPORTED, "MLA plans take rotated q_pe and k_pe (fi_prefill_opts.rope "
                                      "must be 0)");
    if (rope && (dtype != FI_DTYPE_BF16 || head_dim != 128))
      return fail(FI_ERR_UNSUPPORTED, "prefill with the rotary embedding is built for bf16, head_dim 128");
    if (rope && group > FI_PREFILL_ROWS / 2)
      return fail(FI_ERR_UNSUPPORTED, "prefill with the rotary embedding needs G <= " +
                                          std::to_string(FI_PREFILL_ROWS / 2));
    std::vector<int64_t> kvlen;
    {
      const fi_status st = fi::check_page_table(kv_indptr, kv_indices, kv_last_page_len, batch,
                                                page_size, num_pool_pages, &kvlen);
      if (st != FI_OK) return st;
    }
    if (qo_indptr[0] != 0) return fail(FI_ERR_INVALID_ARG, "qo_indptr[0] != 0");
    for (int32_t b = 0; b < batch; ++b) {
      if (qo_indptr[b + 1] < qo_indptr[b])
        return fail(FI_ERR_INVALID_ARG, "qo_indptr is not non-decreasing at request " +
                                            std::to_string(b));
      if ((causal || rope) && qo_indptr[b + 1] - qo_indptr[b] > kvlen[b])
        return fail(FI_ERR_INVALID_ARG, "request " + std::to_string(b) +
                                            " has more query tokens than cached tokens "
                                            "(causal or rotated queries are the newest cached "
                                            "tokens)");
    }
    const int64_t total_qo = batch > 0 ? qo_indptr[batch] : 0;
    if (total_qo * (int64_t)num_qo_heads > INT32_MAX)
      return fail(FI_ERR_INVALID_ARG, "query rows x heads exceed 2^31-1");
    fi_prefill_opts o{};
    if (opts) o = *opts;
    if (o.num_cus < 0 || o.items_per_cu < 0 || o.fixed_chunk_tokens < 0 || o.num_xcds < 0)
      return fail(FI_ERR_INVALID_ARG, "negative planner option");
    const int64_t num_cus = o.num_cus ? o.num_cus : 256;
    // 2 items per CU: fewer cut tiles (append batch 794.6 against 816.7 us at
    // 4, its fp8 twin 785.3 against 805.7; a prompt batch, whose tiles are
    // not cut, is the same plan either way; latent attention 139 against
    // 191 at 1 and 151 at 3)
    const int64_t items_per_cu = o.items_per_cu ? o.items_per_cu : 2;
    const int64_t num_xcds = o.num_xcds ? o.num_xcds : 8;

    auto p = std::make_unique<fi_prefill_plan>();
    p->batch = batch;
    p->num_qo_heads = num_qo_heads;
    p->num_kv_heads = num_kv_heads;
    p->head_dim = head_dim;
    p->page_size = page_size;
    p->group = group;
    p->causal = causal ? 1 : 0;
    p->dtype = dtype;
    p->num_pool_pages = num_pool_pages;
    p->total_qo = total_qo;
    p->rope = rope ? 1 : 0;
    p->mla = mla ? 1 : 0;
    // query tokens per tile: a rope tile is half as tall (its kernel keeps
    // the queries' lo parts in registers too); an MLA tile holds FI_MLA_ROWS
    // rows, whole query tokens or one token's heads in blocks
    const int64_t T = mla ? std::max(1, FI_MLA_ROWS / group)
                          : (rope ? FI_PREFILL_ROWS / 2 : FI_PREFILL_ROWS) / group;
    const int32_t head_blocks = mla && group > FI_MLA_ROWS ? (group + FI_MLA_ROWS - 1) / FI_MLA_ROWS : 1;
    p->tokens_per_tile = (int32_t)T;

    // ---- tiles: (request, KV head, block of T query tokens, and for MLA
    // with more than FI_MLA_ROWS heads a block of heads); the range a tile
    // attends is what its last query sees
    struct Tile {
      int32_t b, qo_row, nqo, head_begin;
      int64_t visible, range, qpos;
    };
    std::vector<Tile> tiles;
    int64_t work = 0;
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t n = qo_indptr[b + 1] - qo_indptr[b], L = kvlen[b];
      p->total_kv += L;
      for (int64_t i = 0; i < n; ++i) p->visible_pairs += causal ? L - n + i + 1 : L;
      for (int64_t t0 = 0; t0 < n; t0 += T) {
        const int64_t nq = std::min<int64_t>(T, n - t0);
        const int64_t vis = causal ? L - n + t0 + 1 : L;
        const int64_t range = causal ? vis + nq - 1 : L;
        for (int32_t hb = 0; hb < head_blocks; ++hb) {
          tiles.push_back({b, (int32_t)(qo_indptr[b] + t0), (int32_t)nq, hb * FI_MLA_ROWS, vis,
                           range, L - n + t0});
          work += range * num_kv_heads;
        }
      }
    }
    p->num_tiles = (int64_t)tiles.size() * num_kv_heads;

    // ---- one chunk length C (whole pages, at most the kernel's page-id
    // window; a prefill chunk also at most 2^20 tokens, the range over which
    // the tile kernel's reciprocal division by the page size is exact). The
    // longer prefill window measured 2.1-2.8% faster on the append batches
    // than 256 pages (fewer cut tiles).
    const int64_t cap_pages = mla ? (int64_t)FI_MLA_MAX_PAGES
                                  : std::min<int64_t>(FI_PREFILL_MAX_PAGES, (int64_t(1) << 20) / page_size);
    const int64_t cap = cap_pages * page_size;
    int64_t C;
    if (o.fixed_chunk_tokens > 0) {
      C = ceil_div(o.fixed_chunk_tokens, page_size) * page_size;
    } else {
      // an MLA partial state is FI_MLA_ROWS x 512 floats (64 KiB), as many
      // bytes as 57 cached latent rows: its chunks stay long
      const int64_t want = std::max<int64_t>(ceil_div(work, num_cus * items_per_cu), mla ? 1024 : 512);
      C = ceil_div(want, page_size) * page_size;
    }
    C = std::min(C, cap);

    // ---- items, longest chunk first
    {
      int64_t n_items = 0;
      for (const Tile& t : tiles) n_items += std::max<int64_t>(1, ceil_div(t.range, C));
      p->items.reserve((size_t)(n_items * num_kv_heads * FI_QITEM_STRIDE));
    }
    int32_t longest = 0;
    for (const Tile& t : tiles) {
      const int64_t k = std::max<int64_t>(1, ceil_div(t.range, C));
      for (int32_t h = 0; h < num_kv_heads; ++h) {
        const int64_t slot0 = k > 1 ? p->num_slots : -1;
        if (k > 1) {
          int32_t m[FI_QMERGE_STRIDE] = {0};
          m[FI_QMERGE_QO_ROW] = t.qo_row;
          m[FI_QMERGE_NUM_QO] = t.nqo;
          m[FI_QMERGE_KV_HEAD] = h;
          m[FI_QMERGE_SLOT_BEGIN] = (int32_t)slot0;
          m[FI_QMERGE_NUM_CHUNKS] = (int32_t)k;
          m[FI_QMERGE_HEAD_BEGIN] = t.head_begin;
          p->merges.insert(p->merges.end(), m, m + FI_QMERGE_STRIDE);
          p->num_slots += k;
        }
        for (int64_t c = 0; c < k; ++c) {
          const int64_t begin = c * C;
          const int64_t len = std::min<int64_t>(C, t.range - begin);
          int32_t f[FI_QITEM_STRIDE] = {0};
          f[FI_QITEM_REQUEST] = t.b;
          f[FI_QITEM_KV_HEAD] = h;
          f[FI_QITEM_QO_ROW] = t.qo_row;
          f[FI_QITEM_NUM_QO] = t.nqo;
          f[FI_QITEM_KV_BEGIN] = (int32_t)begin;
          f[FI_QITEM_NUM_KV] = (int32_t)std::max<int64_t>(len, 0);
          f[FI_QITEM_VISIBLE] = (int32_t)t.visible;
          f[FI_QITEM_PAGE_BEGIN] = (int32_t)(kv_indptr[t.b] + begin / page_size);
          f[FI_QITEM_SLOT] = k > 1 ? (int32_t)(slot0 + c) : -1;
          f[FI_QITEM_CHUNK] = (int32_t)c;
          f[FI_QITEM_Q_POS] = (int32_t)t.qpos;
          f[FI_QITEM_HEAD_BEGIN] = t.head_begin;
          f[FI_QITEM_MERGE] = k > 1 ? (int32_t)(p->num_merges() - 1) : -1;
          longest = std::max(longest, f[FI_QITEM_NUM_KV]);
          p->items.insert(p->items.end(), f, f + FI_QITEM_STRIDE);
        }
      }
    }
    p->chunk_tokens = longest;

    // ---- order: (request, KV head) pairs dealt to num_xcds bins, heaviest
    // first into the least loaded bin; bins interleaved item by item
    {
      const int64_t n = p->num_items();
      const int32_t* it = p->items.data();
      auto key = [&](int64_t i, int f) { return it[i * FI_QITEM_STRIDE + f]; };
      // items of each pair, longest chunk first; ties in (query row, chunk)
      // order, which is the order the items of a pair were made in, so the
      // item index breaks them (keys sorted, not items). MLA: chunk order
      // (the tiles of one chunk, which read the same latent rows, adjacent).
      // (Keeping a cut tile's chunks together instead, so that its merge in
      // the kernel comes earlier, measured 1-5% slower: the longest-first
      // order balances the CUs better.)
      struct SortKey {
        uint32_t req, head, shorter, index;
        bool operator<(const SortKey& o) const {
          if (req != o.req) return req < o.req;
          if (head != o.head) return head < o.head;
          if (shorter != o.shorter) return shorter < o.shorter;
          return index < o.index;
        }
      };
      std::vector<SortKey> keys((size_t)n);
      for (int64_t i = 0; i < n; ++i)
        keys[(size_t)i] = {(uint32_t)key(i, FI_QITEM_REQUEST), (uint32_t)key(i, FI_QITEM_KV_HEAD),
                           (uint32_t)(mla ? key(i, FI_QITEM_KV_BEGIN)
                                          : INT32_MAX - key(i, FI_QITEM_NUM_KV)),
                           (uint32_t)i};
      std::sort(keys.begin(), keys.end());
      std::vector<int64_t> order(n);
      for (int64_t i = 0; i < n; ++i) order[i] = keys[(size_t)i].index;
      struct Pair {
        int64_t begin, end, work;
      };
      std::vector<Pair> pairs;
      for (int64_t i = 0; i < n;) {
        int64_t j = i, w = 0;
        while (j < n && key(order[j], FI_QITEM_REQUEST) == key(order[i], FI_QITEM_REQUEST) &&
               key(order[j], FI_QITEM_KV_HEAD) == key(order[i], FI_QITEM_KV_HEAD)) {
          // a chunk's blocks of 64 tokens, plus one for the item's fixed costs
          w += (key(order[j], FI_QITEM_NUM_KV) + 63) / 64 + 1;
          ++j;
        }
        pairs.push_back({i, j, w});
        i = j;
      }
      std::vector<int64_t> by_work(pairs.size());
      for (size_t i = 0; i < pairs.size(); ++i) by_work[i] = (int64_t)i;
      std::stable_sort(by_work.begin(), by_work.end(),
                       [&](int64_t a, int64_t b) { return pairs[a].work > pairs[b].work; });
      std::vector<std::vector<int64_t>> bins((size_t)num_xcds);
      std::vector<int64_t> load((size_t)num_xcds, 0);
      for (int64_t pi : by_work) {
        const size_t x = (size_t)(std::min_element(load.begin(), load.end()) - load.begin());
        load[x] += pairs[pi].work;
        for (int64_t j = pairs[pi].begin; j < pairs[pi].end; ++j) bins[x].push_back(order[j]);
      }
      std::vector<int32_t> sorted;
      sorted.reserve(p->items.size());
      for (size_t j = 0, left = (size_t)n; left > 0; ++j)
        for (auto& bin : bins)
          if (j < bin.size()) {
            sorted.insert(sorted.end(), it + bin[j] * FI_QITEM_STRIDE,
                          it + (bin[j] + 1) * FI_QITEM_STRIDE);
            --left;
          }
      p->items.swap(sorted);
    }

    // ---- workspace layout and host image of its uploaded part
    const int64_t nnz = batch > 0 ? kv_indptr[batch] : 0;
    auto& ws = p->ws;
    int64_t off = 0;
    ws.items = off;
    off = fi::align_up(off + (int64_t)p->items.size() * 4, 256);
    ws.merges = off;
    off = fi::align_up(off + (int64_t)p->merges.size() * 4, 256);
    ws.page_ids = off;
    off = fi::align_up(off + nnz * 4, 256);
    // the merges' arrival counters, uploaded as zeros (the chunk that
    // completes a merge sets its counter back to 0)
    ws.counters = off;
    off = fi::align_up(off + p->num_merges() * 4, 256);
    ws.image_bytes = off;
    ws.part_o = off;
    const int64_t slot_rows = mla ? FI_MLA_ROWS : FI_PREFILL_ROWS;
    off = fi::align_up(off + p->num_slots * slot_rows * (int64_t)head_dim * 4, 256);
    ws.part_lse = off;
    off = fi::align_up(off + p->num_slots * slot_rows * 4, 256);
    ws.total_bytes = std::max<int64_t>(off, 256);
    p->image.assign(ws.image_bytes, 0);
    if (!p->items.empty()) std::memcpy(p->image.data() + ws.items, p->items.data(), p->items.size() * 4);
    if (!p->merges.empty())
      std::memcpy(p->image.data() + ws.merges, p->merges.data(), p->merges.size() * 4);
    if (nnz > 0) std::memcpy(p->image.data() + ws.page_ids, kv_indices, nnz * 4);

    *out_plan = p.release();
    return FI_OK;
  } catch (const std::bad_alloc&) {
    return fail(FI_ERR_NOMEM, "host allocation failed in the prefill / MLA planner");
  } catch (...) {
    return fail(FI_ERR_INVALID_ARG, "unexpected error in the prefill / MLA planner");
  }
}

}  // namespace
}  // namespace fi

extern "C" {

fi_status fi_prefill_plan_create(const int32_t* qo_indptr, const int32_t* kv_indptr,
                                 const int32_t* kv_indices, const int32_t* kv_last_page_len,
                                 int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t page_size, int64_t num_pool_pages,
                                 fi_dtype dtype, int32_t causal, const fi_prefill_opts* opts,
                                 fi_prefill_plan** out_plan) {
  return fi::build_tile_plan(qo_indptr, kv_indptr, kv_indices, kv_last_page_len, batch,
                             num_qo_heads, num_kv_heads, head_dim, page_size, num_pool_pages,
                             dtype, causal, opts, false, out_plan);
}

fi_status fi_mla_plan_create(const int32_t* qo_indptr, const int32_t* kv_indptr,
                             const int32_t* kv_indices, const int32_t* kv_last_page_len,
                             int32_t batch, int32_t num_heads, int32_t head_dim_ckv,
                             int32_t head_dim_kpe, int32_t page_size, int64_t num_pool_pages,
                             int32_t causal, const fi_prefill_opts* opts,
                             fi_prefill_plan** out_plan) {
  if (out_plan) *out_plan = nullptr;
  if (head_dim_ckv != 512 || head_dim_kpe != 64)
    return fi::fail(FI_ERR_UNSUPPORTED, "MLA is built for a 512-wide latent and a 64-wide "
                                        "rotary key");
  if (num_heads <= 0 || num_heads > 4096)
    return fi::fail(FI_ERR_INVALID_ARG, "num_heads must be in 1 .. 4096");
  const fi_status st = fi::build_tile_plan(qo_indptr, kv_indptr, kv_indices, kv_last_page_len,
                                           batch, num_heads, 1, head_dim_ckv, page_size,
                                           num_pool_pages, FI_DTYPE_BF16, causal, opts, true,
                                           out_plan);
  if (st == FI_OK) (*out_plan)->head_dim_kpe = head_dim_kpe;
  return st;
}

fi_status fi_prefill_plan_get_info(const fi_prefill_plan* p, fi_prefill_info* info) {
  if (!p || !info) return fi::fail(FI_ERR_INVALID_ARG, "NULL plan or info");
  fi_prefill_info r{};
  r.num_items = p->num_items();
  r.num_tiles = p->num_tiles;
  r.num_merges = p->num_merges();
  r.num_partial_slots = p->num_slots;
  r.workspace_bytes = p->ws.total_bytes;
  r.total_qo_tokens = p->total_qo;
  r.total_kv_tokens = p->total_kv;
  r.visible_pairs = p->visible_pairs;
  r.tokens_per_tile = p->tokens_per_tile;
  r.chunk_tokens = p->chunk_tokens;
  r.batch = p->batch;
  r.num_qo_heads = p->num_qo_heads;
  r.num_kv_heads = p->num_kv_heads;
  r.head_dim = p->head_dim;
  r.page_size = p->page_size;
  r.causal = p->causal;
  r.dtype = p->dtype;
  r.rope = p->rope;
  r.mla = p->mla;
  r.head_dim_kpe = p->head_dim_kpe;
  *info = r;
  return FI_OK;
}

fi_status fi_prefill_plan_work_list(const fi_prefill_plan* p, const int32_t** items,
                                    int64_t* num_items) {
  if (!p || !items || !num_items) return fi::fail(FI_ERR_INVALID_ARG, "NULL argument");
  *items = p->items.data();
  *num_items = p->num_items();
  return FI_OK;
}

fi_status fi_prefill_plan_merges(const fi_prefill_plan* p, const int32_t** merges,
                                 int64_t* num_merges) {
  if (!p || !merges || !num_merges) return fi::fail(FI_ERR_INVALID_ARG, "NULL argument");
  *merges = p->merges.data();
  *num_merges = p->num_merges();
  return FI_OK;
}

}  // extern "C"
