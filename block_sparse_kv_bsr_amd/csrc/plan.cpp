// Load-balanced split-KV planner for paged / BSR decode attention.
//
// FlashInfer paper explainer ("FlashInfer: Block-Sparse KV 캐시로 어텐션 병목을
// 해소하다", visionhong.com), benchmark section: in a skewed batch (lengths of
// 32 and 4096 side by side) one workgroup per sequence leaves most
// workgroups idle while the long sequences finish. The scheduler instead cuts
// sequences into smaller work units, splits the long ones into several, and
// interleaves them with the short ones so the GPU stays busy.
//
// Here a work unit is (request, KV head, chunk of whole pages). One chunk
// length serves the whole batch: the smallest that keeps the unit count within
// a budget of (compute units x items per CU); a request of n pages is cut into
// k = ceil(n / C) chunks of near-equal page counts. Units are ordered longest
// first -- the longest-processing-time rule -- so that the hardware dispatcher,
// which starts workgroups in grid order, places long chunks first and short
// requests into the gaps; and since it hands consecutive workgroups to the
// CUs in turn, every other layer of num_cus units is reversed (a snake
// order), so a CU that took a layer's longest unit takes the next layer's
// shortest. Requests cut into several chunks
// write partial (output, log-sum-exp) states; per KV head a small tree of
// merge nodes (fan-in at most FI_MERGE_FAN_IN) combines them inside the same
// kernel.
//
// Plain C++17 with no HIP dependency: the planner is tested on CPU-only hosts.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <memory>
#include <new>
#include <numeric>
#include <string>

#include "plan.h"

namespace fi {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

void plan_free_host(fi_plan* p) { delete p; }

namespace {

fi_status fail(fi_status st, const std::string& msg) {
  set_error(msg);
  return st;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Number of items a chunk length of `c` pages produces.
int64_t count_items(const std::vector<int64_t>& npages, int64_t c, int64_t heads) {
  int64_t n = 0;
  for (int64_t x : npages) n += ceil_div(x, c);
  return n * heads;
}

}  // namespace

fi_status check_page_table(const int32_t* kv_indptr, const int32_t* kv_indices,
                           const int32_t* kv_last_page_len, int32_t batch, int32_t page_size,
                           int64_t num_pool_pages, std::vector<int64_t>* tokens) {
  if (!kv_indptr) return fail(FI_ERR_INVALID_ARG, "kv_indptr is NULL");
  if (batch > 0 && !kv_last_page_len) return fail(FI_ERR_INVALID_ARG, "kv_last_page_len is NULL");
  if (page_size < 1 || page_size > 4096)
    return fail(FI_ERR_INVALID_ARG, "page_size must be in [1, 4096]");
  if (num_pool_pages < 0) return fail(FI_ERR_INVALID_ARG, "num_pool_pages < 0");
  if (kv_indptr[0] != 0) return fail(FI_ERR_INVALID_ARG, "kv_indptr[0] != 0");
  for (int32_t b = 0; b < batch; ++b)
    if (kv_indptr[b + 1] < kv_indptr[b])
      return fail(FI_ERR_INVALID_ARG, "kv_indptr is not non-decreasing at request " +
                                          std::to_string(b));
  const int64_t nnz = batch > 0 ? kv_indptr[batch] : 0;
  if (nnz > 0 && !kv_indices) return fail(FI_ERR_INVALID_ARG, "kv_indices is NULL");
  for (int64_t j = 0; j < nnz; ++j)
    if (kv_indices[j] < 0 || kv_indices[j] >= num_pool_pages)
      return fail(FI_ERR_INVALID_ARG, "kv_indices[" + std::to_string(j) +
                                          "] outside [0, num_pool_pages)");
  tokens->assign(batch, 0);
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t npages = kv_indptr[b + 1] - kv_indptr[b];
    const int32_t ell = kv_last_page_len[b];
    if (npages > 0) {
      if (ell < 1 || ell > page_size)
        return fail(FI_ERR_INVALID_ARG, "kv_last_page_len[" + std::to_string(b) +
                                            "] outside [1, page_size]");
      (*tokens)[b] = (npages - 1) * (int64_t)page_size + ell;
    } else if (ell < 0 || ell > page_size) {
      return fail(FI_ERR_INVALID_ARG, "kv_last_page_len[" + std::to_string(b) +
                                          "] outside [0, page_size]");
    }
    if ((*tokens)[b] > INT32_MAX) return fail(FI_ERR_INVALID_ARG, "request longer than 2^31-1 tokens");
  }
  return FI_OK;
}

namespace {

// The prefix cache of a composed plan (fi_plan_create_composed).
struct Composed {
  const int32_t* indptr;
  const int32_t* indices;
  const int32_t* last;
  int32_t num_prefixes;
  const int32_t* prefix_of;
  int32_t page_size;
  int64_t num_pool_pages;
};

fi_status create_plan(const int32_t* kv_indptr, const int32_t* kv_indices,
                      const int32_t* kv_last_page_len, int32_t batch, int32_t num_qo_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                      int64_t num_pool_pages, fi_dtype dtype, const fi_plan_opts* opts,
                      const Composed* comp, fi_plan** out_plan);

}  // namespace
}  // namespace fi

extern "C" {

const char* fi_last_error(void) { return fi::g_last_error.c_str(); }

fi_status fi_plan_create(const int32_t* kv_indptr, const int32_t* kv_indices,
                         const int32_t* kv_last_page_len, int32_t batch,
                         int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t page_size, int64_t num_pool_pages, fi_dtype dtype,
                         const fi_plan_opts* opts, fi_plan** out_plan) {
  return fi::create_plan(kv_indptr, kv_indices, kv_last_page_len, batch, num_qo_heads,
                         num_kv_heads, head_dim, page_size, num_pool_pages, dtype, opts, nullptr,
                         out_plan);
}

fi_status fi_plan_create_composed(const int32_t* kv_indptr, const int32_t* kv_indices,
                                  const int32_t* kv_last_page_len, int32_t batch,
                                  const int32_t* prefix_indptr, const int32_t* prefix_indices,
                                  const int32_t* prefix_last_page_len, int32_t num_prefixes,
                                  const int32_t* prefix_of, int32_t num_qo_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                  int64_t num_pool_pages, int32_t prefix_page_size,
                                  int64_t num_prefix_pool_pages, fi_dtype dtype,
                                  const fi_plan_opts* opts, fi_plan** out_plan) {
  const fi::Composed c{prefix_indptr, prefix_indices, prefix_last_page_len, num_prefixes,
                       prefix_of, prefix_page_size, num_prefix_pool_pages};
  return fi::create_plan(kv_indptr, kv_indices, kv_last_page_len, batch, num_qo_heads,
                         num_kv_heads, head_dim, page_size, num_pool_pages, dtype, opts, &c,
                         out_plan);
}

}  // extern "C"

namespace fi {
namespace {

fi_status create_plan(const int32_t* kv_indptr, const int32_t* kv_indices,
                      const int32_t* kv_last_page_len, int32_t batch, int32_t num_qo_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                      int64_t num_pool_pages, fi_dtype dtype, const fi_plan_opts* opts,
                      const Composed* comp, fi_plan** out_plan) {
  try {
    if (!out_plan) return fail(FI_ERR_INVALID_ARG, "out_plan is NULL");
    *out_plan = nullptr;
    if (batch < 0) return fail(FI_ERR_INVALID_ARG, "batch < 0");
    if (!kv_indptr) return fail(FI_ERR_INVALID_ARG, "kv_indptr is NULL");
    if (batch > 0 && !kv_last_page_len)
      return fail(FI_ERR_INVALID_ARG, "kv_last_page_len is NULL");
    if (num_qo_heads <= 0 || num_kv_heads <= 0)
      return fail(FI_ERR_INVALID_ARG, "head counts must be positive");
    if (num_qo_heads % num_kv_heads != 0)
      return fail(FI_ERR_INVALID_ARG, "num_qo_heads is not a multiple of num_kv_heads");
    const int32_t group = num_qo_heads / num_kv_heads;
    // Children per merge node: as many as the merging wave reads in its first
    // round of loads (64 / float pairs per lane of one partial state, at most
    // 16), so a merge costs one round trip: 16 up to G * head_dim = 512, 8
    // at 1024 (64 query / 8 KV heads at d 128, whose merges cost 21 us of 189
    // at fan-in 32 on the skewed batch, measured).
    const int64_t pairs_per_lane = ((int64_t)group * head_dim / 2 + 63) / 64;
    const int64_t fan_in =
        std::max<int64_t>(2, std::min<int64_t>({(int64_t)FI_MERGE_FAN_IN, 16, 64 / pairs_per_lane}));
    if (group != 1 && group != 2 && group != 4 && group != 8)
      return fail(FI_ERR_UNSUPPORTED, "GQA group size must be 1, 2, 4 or 8");
    if (head_dim != 64 && head_dim != 128)
      return fail(FI_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (dtype != FI_DTYPE_F32 && dtype != FI_DTYPE_BF16 && dtype != FI_DTYPE_FP8_E4M3)
      return fail(FI_ERR_UNSUPPORTED, "dtype must be FI_DTYPE_F32, FI_DTYPE_BF16 or FI_DTYPE_FP8_E4M3");
    if (dtype == FI_DTYPE_FP8_E4M3 && head_dim != 128)
      return fail(FI_ERR_UNSUPPORTED, "an fp8 KV cache needs head_dim 128");
    std::vector<int64_t> ntok;
    {
      const fi_status st = fi::check_page_table(kv_indptr, kv_indices, kv_last_page_len, batch,
                                                page_size, num_pool_pages, &ntok);
      if (st != FI_OK) return st;
    }
    const int64_t nnz = batch > 0 ? kv_indptr[batch] : 0;
    // composed: tokens of each prefix, and of the prefix each request begins with
    std::vector<int64_t> pre_tok, lead(batch, 0);
    int64_t pre_nnz = 0;
    if (comp) {
      if (dtype != FI_DTYPE_BF16) return fail(FI_ERR_UNSUPPORTED, "composed formats need FI_DTYPE_BF16");
      if (comp->num_prefixes < 0) return fail(FI_ERR_INVALID_ARG, "num_prefixes < 0");
      const fi_status st = check_page_table(comp->indptr, comp->indices, comp->last,
                                            comp->num_prefixes, comp->page_size,
                                            comp->num_pool_pages, &pre_tok);
      if (st != FI_OK) return fail(st, "prefix table: " + g_last_error);
      pre_nnz = comp->num_prefixes > 0 ? comp->indptr[comp->num_prefixes] : 0;
      if (batch > 0 && !comp->prefix_of) return fail(FI_ERR_INVALID_ARG, "prefix_of is NULL");
      for (int32_t b = 0; b < batch; ++b) {
        const int32_t g = comp->prefix_of[b];
        if (g < -1 || g >= comp->num_prefixes)
          return fail(FI_ERR_INVALID_ARG, "prefix_of[" + std::to_string(b) +
                                              "] outside [-1, num_prefixes)");
        if (g >= 0) lead[b] = pre_tok[g];
        if (lead[b] > 0 && ntok[b] == 0)
          return fail(FI_ERR_INVALID_ARG, "request " + std::to_string(b) +
                                              " has a prefix but no token of its own");
        if (lead[b] + ntok[b] > INT32_MAX)
          return fail(FI_ERR_INVALID_ARG, "request longer than 2^31-1 tokens");
      }
    }
    std::vector<int64_t> npages(batch);
    int64_t total_tokens = 0;
    for (int32_t b = 0; b < batch; ++b) {
      npages[b] = kv_indptr[b + 1] - kv_indptr[b];
      total_tokens += lead[b] + ntok[b];
    }
    fi_plan_opts o{};
    if (opts) o = *opts;
    if (o.num_cus < 0 || o.items_per_cu < 0 || o.min_chunk_tokens < 0 ||
        o.max_chunk_tokens < 0 || o.fixed_chunk_tokens < 0)
      return fail(FI_ERR_INVALID_ARG, "negative planner option");
    if (o.cascade < -1 || o.cascade > 1) return fail(FI_ERR_INVALID_ARG, "cascade must be -1, 0 or 1");
    if (o.decode_kernel < FI_DECODE_KERNEL_AUTO || o.decode_kernel > FI_DECODE_KERNEL_MATRIX)
      return fail(FI_ERR_INVALID_ARG, "decode_kernel must be one of FI_DECODE_KERNEL_*");
    if (o.decode_kernel == FI_DECODE_KERNEL_MATRIX &&
        (head_dim != 128 || dtype == FI_DTYPE_F32 || page_size % 16 != 0))
      return fail(FI_ERR_UNSUPPORTED,
                  "the matrix-core decode kernel needs head_dim 128, bf16 or fp8 K/V and a page "
                  "size that is a multiple of 16");
    // The matrix-core kernel was measured faster for fp8 caches and for eight
    // query heads per KV head (both bound by vector work in the other kernel).
    const bool mma_fits = head_dim == 128 && dtype != FI_DTYPE_F32 && page_size % 16 == 0;
    const bool mma =
        o.decode_kernel == FI_DECODE_KERNEL_MATRIX ||
        (o.decode_kernel == FI_DECODE_KERNEL_AUTO && mma_fits &&
         (dtype == FI_DTYPE_FP8_E4M3 || num_qo_heads == 8 * num_kv_heads));
    const int64_t num_cus = o.num_cus ? o.num_cus : 256;
    // Items per CU: 8 keeps every item resident from the start (two waves per
    // SIMD) and was measured best for the vector kernel (with the rotary
    // embedding too: 179.9 against 206.2 us at 12); the matrix kernel
    // without the embedding moves more per item for the same fixed costs
    // and measured faster with 6 (fp8 skewed batch 91.0 against 93.7 us,
    // 64 / 8 heads 168.6 against 171.5); with it, bound by vector work, it
    // measured best at 16 (fp8 skewed batch 129.0 against 133.4 at 8, 130.2
    // at 20, 134.9 at 24, 168.4 at 6).
    const int64_t items_per_cu = o.items_per_cu ? o.items_per_cu : (mma ? (o.rope ? 16 : 6) : 8);
    // The floor matters only for batches too small to fill the budget with
    // whole requests, which are latency-bound: there shorter chunks finish
    // sooner (tiny batch 17.7 -> 9.4 us, shared-prefix batch 44.4 -> 39.1 us
    // at 32 against 256 tokens, measured); larger batches cut at the budget.
    const int64_t min_chunk_tokens = o.min_chunk_tokens ? o.min_chunk_tokens : 32;

    // ---- shared-prefix groups: requests (of two pages or more) whose lists
    // start with the same physical page; the group's prefix is the longest
    // run of leading pages all members share, never a member's last page
    struct Group {
      int64_t member_base, members, lcp, chunks, row_blocks;
      int32_t first;  // a member; its first lcp pages are the prefix
      // the prefix's tokens, its first page as an index into the uploaded
      // page ids, and the size of its pages
      int64_t tokens, page_base, psize;
    };
    std::vector<Group> groups;
    std::vector<int32_t> members;
    std::vector<int32_t> group_of(batch, -1);
    std::vector<int64_t> pre_pages(batch, 0);
    const int64_t kPrefixRows = 128;
    if (comp) {
      // one group per prefix with members, in prefix order; members in
      // batch order
      std::vector<std::vector<int32_t>> mem((size_t)comp->num_prefixes);
      for (int32_t b = 0; b < batch; ++b)
        if (lead[b] > 0) mem[(size_t)comp->prefix_of[b]].push_back(b);
      for (int32_t g = 0; g < comp->num_prefixes; ++g) {
        if (mem[(size_t)g].empty()) continue;
        Group gr{};
        gr.member_base = (int64_t)members.size();
        gr.members = (int64_t)mem[(size_t)g].size();
        gr.lcp = comp->indptr[g + 1] - comp->indptr[g];
        gr.first = mem[(size_t)g][0];
        gr.row_blocks = fi::ceil_div(gr.members * group, kPrefixRows);
        gr.tokens = pre_tok[(size_t)g];
        gr.page_base = nnz + comp->indptr[g];
        gr.psize = comp->page_size;
        for (int32_t b : mem[(size_t)g]) {
          members.push_back(b);
          group_of[b] = (int32_t)groups.size();
        }
        groups.push_back(gr);
      }
    } else if (o.cascade >= 0 && dtype == FI_DTYPE_BF16 && batch >= 2) {
      std::vector<std::pair<int32_t, int32_t>> firsts;  // (first page, request)
      for (int32_t b = 0; b < batch; ++b)
        if (npages[b] >= 2) firsts.emplace_back(kv_indices[kv_indptr[b]], b);
      std::sort(firsts.begin(), firsts.end());
      for (size_t i = 0; i < firsts.size();) {
        size_t j = i;
        while (j < firsts.size() && firsts[j].first == firsts[i].first) ++j;
        if (j - i >= 2) {
          const int32_t b0 = firsts[i].second;
          int64_t lcp = npages[b0] - 1;
          for (size_t t = i + 1; t < j; ++t) {
            const int32_t b = firsts[t].second;
            const int64_t lim = std::min<int64_t>(lcp, npages[b] - 1);
            int64_t q = 0;
            while (q < lim && kv_indices[kv_indptr[b] + q] == kv_indices[kv_indptr[b0] + q]) ++q;
            lcp = q;
          }
          lcp = std::min<int64_t>(lcp, (fan_in - 1) * FI_PREFIX_MAX_PAGES);
          const int64_t saved = (int64_t)(j - i - 1) * lcp * page_size * head_dim * 4 * num_kv_heads;
          if (lcp >= 1 && (o.cascade == 1 || saved >= (int64_t(8) << 20))) {
            Group g{};
            g.member_base = (int64_t)members.size();
            g.members = (int64_t)(j - i);
            g.lcp = lcp;
            g.first = b0;
            g.row_blocks = fi::ceil_div(g.members * group, kPrefixRows);
            g.tokens = lcp * page_size;
            g.page_base = kv_indptr[b0];
            g.psize = page_size;
            for (size_t t = i; t < j; ++t) {
              const int32_t b = firsts[t].second;
              members.push_back(b);
              group_of[b] = (int32_t)groups.size();
              pre_pages[b] = lcp;
            }
            groups.push_back(g);
          }
        }
        i = j;
      }
    }
    // prefix chunks per group: about num_cus prefix items in all, at most
    // fan_in - 1 per tree so every tree's first node still has a decode
    // child (nodes complete only inside the decode kernel). Shared pages of
    // the requests' own lists are cut at page boundaries; a composed prefix
    // into near-equal token ranges (of at least 64 tokens), each touching at
    // most FI_PREFIX_MAX_PAGES pages.
    {
      int64_t blocks = 0;
      for (const Group& g : groups) blocks += g.row_blocks;
      for (size_t gi = 0; gi < groups.size(); ++gi) {
        Group& g = groups[gi];
        const int64_t want = fi::ceil_div(num_cus, std::max<int64_t>(1, blocks * num_kv_heads));
        if (comp) {
          g.chunks = std::max<int64_t>(
              1, std::min<int64_t>({want, fan_in - 1, fi::ceil_div(g.tokens, 64)}));
          g.chunks = std::max<int64_t>(
              g.chunks, fi::ceil_div(g.tokens, (FI_PREFIX_MAX_PAGES - 1) * g.psize));
          if (g.chunks > fan_in - 1)
            return fail(FI_ERR_UNSUPPORTED,
                        "prefix " + std::to_string(comp->prefix_of[g.first]) + " holds " +
                            std::to_string(g.tokens) + " tokens, more than " +
                            std::to_string(fan_in - 1) + " chunks of " +
                            std::to_string((FI_PREFIX_MAX_PAGES - 1) * g.psize) + " cover");
        } else {
          g.chunks = std::max<int64_t>(1, std::min<int64_t>({want, g.lcp, fan_in - 1}));
          // no prefix item spans more than FI_PREFIX_MAX_PAGES pages
          g.chunks = std::max<int64_t>(g.chunks, fi::ceil_div(g.lcp, FI_PREFIX_MAX_PAGES));
        }
      }
    }
    std::vector<int64_t> dpages(batch);  // pages left to the decode items
    for (int32_t b = 0; b < batch; ++b) dpages[b] = npages[b] - pre_pages[b];

    // ---- chunk length (pages) of the decode items
    const int64_t max_n = batch > 0 ? *std::max_element(dpages.begin(), dpages.end()) : 0;
    int64_t C = std::max<int64_t>(1, max_n);
    if (o.fixed_chunk_tokens > 0) {
      C = std::max<int64_t>(1, fi::ceil_div(o.fixed_chunk_tokens, page_size));
    } else if (max_n > 0) {
      const int64_t budget = num_cus * items_per_cu;
      const int64_t cmin = std::max<int64_t>(1, fi::ceil_div(min_chunk_tokens, page_size));
      if (cmin < max_n && fi::count_items(dpages, max_n, num_kv_heads) <= budget) {
        int64_t lo = cmin, hi = max_n;  // count_items is non-increasing in C
        while (lo < hi) {
          const int64_t mid = lo + (hi - lo) / 2;
          if (fi::count_items(dpages, mid, num_kv_heads) <= budget) hi = mid;
          else lo = mid + 1;
        }
        C = lo;
      }
      if (o.max_chunk_tokens > 0)
        C = std::min<int64_t>(C, std::max<int64_t>(1, o.max_chunk_tokens / page_size));
    }
    if (C > INT32_MAX) C = INT32_MAX;

    std::unique_ptr<fi_plan> p(new fi_plan());
    p->decode_kernel = o.decode_kernel;
    p->merge_fan_in = (int32_t)fan_in;
    p->resolved_kernel = mma ? FI_DECODE_KERNEL_MATRIX : FI_DECODE_KERNEL_VECTOR;
    p->batch = batch;
    p->num_qo_heads = num_qo_heads;
    p->num_kv_heads = num_kv_heads;
    p->head_dim = head_dim;
    p->page_size = page_size;
    p->group = group;
    p->dtype = dtype;
    p->num_pool_pages = num_pool_pages;
    p->chunk_pages = (int32_t)C;
    p->total_tokens = total_tokens;
    p->num_groups = (int32_t)groups.size();
    p->prefix_rows = (int32_t)kPrefixRows;
    p->composed = comp != nullptr;
    p->prefix_page_size = comp ? comp->page_size : 0;
    p->num_prefix_pool_pages = comp ? comp->num_pool_pages : 0;
    p->members = members;
    {
      // physical pages that the decode items read more than once (several
      // requests, or one request twice; a cascade's prefix pages are read by
      // the prefix items instead): a bitmap over the pool when it is not
      // much larger than the page lists, else a sort
      if (num_pool_pages <= 64 * nnz + 65536) {
        std::vector<uint64_t> seen((size_t)(num_pool_pages + 63) / 64, 0), twice(seen.size(), 0);
        for (int32_t b = 0; b < batch; ++b) {
          for (int64_t j = kv_indptr[b] + pre_pages[b]; j < kv_indptr[b + 1]; ++j) {
            const int32_t id = kv_indices[j];
            const uint64_t bit = 1ull << (id & 63);
            uint64_t& w = seen[(size_t)(id >> 6)];
            if (w & bit) twice[(size_t)(id >> 6)] |= bit;
            w |= bit;
          }
        }
        for (uint64_t w : twice) p->shared_pages += __builtin_popcountll(w);
      } else {
        std::vector<int32_t> ids;
        ids.reserve((size_t)nnz);
        for (int32_t b = 0; b < batch; ++b)
          for (int64_t j = kv_indptr[b] + pre_pages[b]; j < kv_indptr[b + 1]; ++j)
            ids.push_back(kv_indices[j]);
        std::sort(ids.begin(), ids.end());
        for (size_t j = 1; j < ids.size(); ++j)
          if (ids[j] == ids[j - 1] && (j == 1 || ids[j - 1] != ids[j - 2])) ++p->shared_pages;
      }
    }

    // ---- items, partial slots, merge trees
    struct Item { int32_t f[FI_ITEM_STRIDE]; };
    std::vector<Item> items;
    {
      int64_t n_items = 0;
      for (int32_t b = 0; b < batch; ++b)
        n_items += num_kv_heads * std::max<int64_t>(1, dpages[b] > 0 ? fi::ceil_div(dpages[b], C) : 0);
      items.reserve((size_t)n_items);
    }
    std::vector<int32_t>& nodes = p->nodes;
    std::vector<int32_t>& pslot = p->prefix_slot;
    if (!groups.empty()) pslot.assign((size_t)batch * num_kv_heads, -1);
    int64_t slot = 0;
    int32_t max_chunks = 0, min_split = 0;
    auto new_node = [&](int32_t count, int32_t arrivals, int64_t slot_begin, int64_t out_slot,
                        int32_t b, int32_t h, int32_t level) {
      const int32_t id = (int32_t)(nodes.size() / FI_NODE_STRIDE);
      int32_t f[FI_NODE_STRIDE] = {0};
      f[FI_NODE_COUNT] = count;
      f[FI_NODE_SLOT_BEGIN] = (int32_t)slot_begin;
      f[FI_NODE_PARENT] = -1;
      f[FI_NODE_OUT_SLOT] = (int32_t)out_slot;
      f[FI_NODE_REQUEST] = b;
      f[FI_NODE_KV_HEAD] = h;
      f[FI_NODE_LEVEL] = level;
      f[FI_NODE_ARRIVALS] = arrivals;
      nodes.insert(nodes.end(), f, f + FI_NODE_STRIDE);
      return id;
    };
    std::vector<int32_t> leaf_node, prev;  // per merge tree, reused
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t n = dpages[b];
      const int64_t pre = pre_pages[b];
      const int64_t k = n > 0 ? fi::ceil_div(n, C) : 0;
      const int64_t cpre = group_of[b] >= 0 ? groups[group_of[b]].chunks : 0;
      max_chunks = std::max<int32_t>(max_chunks, (int32_t)k);
      if (k >= 2) min_split = min_split == 0 ? (int32_t)k : std::min<int32_t>(min_split, (int32_t)k);
      if (k == 0) {  // no pages: one item per KV head writes out = 0, lse = -inf
        for (int32_t h = 0; h < num_kv_heads; ++h) {
          Item it{};
          it.f[FI_ITEM_REQUEST] = b;
          it.f[FI_ITEM_KV_HEAD] = h;
          it.f[FI_ITEM_PAGE_BEGIN] = kv_indptr[b];
          it.f[FI_ITEM_SLOT] = -1;
          it.f[FI_ITEM_MERGE_NODE] = -1;
          items.push_back(it);
        }
        continue;
      }
      const int64_t nchild = cpre + k;
      for (int32_t h = 0; h < num_kv_heads; ++h) {
        // merge tree of (b, h): leaves take the cpre prefix partials, then
        // the k chunk partials, in slots [leaf_base, leaf_base + nchild);
        // each level groups fan_in children
        const int64_t leaf_base = slot;
        leaf_node.assign((size_t)nchild, -1);
        if (nchild >= 2) {
          slot += nchild;
          if (cpre > 0) pslot[(size_t)b * num_kv_heads + h] = (int32_t)leaf_base;
          int64_t child_begin = leaf_base, nch = nchild;
          int32_t level = 0;
          prev.clear();
          for (;;) {
            const int64_t ngroups = fi::ceil_div(nch, fan_in);
            const bool root = ngroups == 1;
            const int64_t out_base = root ? -1 : slot;
            if (!root) slot += ngroups;
            const int32_t first = (int32_t)(nodes.size() / FI_NODE_STRIDE);
            for (int64_t g = 0; g < ngroups; ++g) {
              const int64_t c0 = g * fan_in;
              const int64_t cnt = std::min<int64_t>(fan_in, nch - c0);
              // prefix partials (level 0, children [0, cpre)) do not report
              const int64_t quiet = level == 0 ? std::max<int64_t>(0, std::min(cpre, c0 + cnt) - c0) : 0;
              new_node((int32_t)cnt, (int32_t)(cnt - quiet), child_begin + c0,
                       root ? -1 : out_base + g, b, h, level);
            }
            for (size_t i = 0; i < prev.size(); ++i)
              nodes[(size_t)prev[i] * FI_NODE_STRIDE + FI_NODE_PARENT] =
                  first + (int32_t)(i / fan_in);
            if (level == 0)
              for (int64_t c = 0; c < nchild; ++c) leaf_node[c] = first + (int32_t)(c / fan_in);
            prev.clear();
            for (int64_t g = 0; g < ngroups; ++g) prev.push_back(first + (int32_t)g);
            if (root) break;
            child_begin = out_base;
            nch = ngroups;
            ++level;
          }
        }
        int64_t page0 = 0;
        for (int64_t c = 0; c < k; ++c) {
          // near-equal cut: the first (n % k) chunks get one page more
          const int64_t np = n / k + (c < n % k ? 1 : 0);
          const bool has_last = page0 + np == n;
          const int64_t tok = has_last ? (np - 1) * page_size + kv_last_page_len[b]
                                       : np * (int64_t)page_size;
          Item it{};
          it.f[FI_ITEM_REQUEST] = b;
          it.f[FI_ITEM_KV_HEAD] = h;
          it.f[FI_ITEM_PAGE_BEGIN] = (int32_t)(kv_indptr[b] + pre + page0);
          it.f[FI_ITEM_NUM_TOKENS] = (int32_t)tok;
          it.f[FI_ITEM_SLOT] = nchild == 1 ? -1 : (int32_t)(leaf_base + cpre + c);
          it.f[FI_ITEM_CHUNK] = (int32_t)c;
          it.f[FI_ITEM_NUM_PAGES] = (int32_t)np;
          it.f[FI_ITEM_FIRST_PAGE] = kv_indices[kv_indptr[b] + pre + page0];
          it.f[FI_ITEM_MERGE_NODE] = leaf_node[cpre + c];
          it.f[FI_ITEM_KV_POS] = (int32_t)(lead[b] + (pre + page0) * page_size);
          it.f[FI_ITEM_Q_POS] = (int32_t)(lead[b] + ntok[b] - 1);
          items.push_back(it);
          page0 += np;
        }
      }
    }
    if (slot > INT32_MAX) return fail(FI_ERR_UNSUPPORTED, "too many partial states");
    // longest first; ties in (request, KV head, chunk) order, which is the
    // order the items were made in: sort 64-bit keys (token count, then
    // that index) rather than the items themselves
    std::vector<uint64_t> order(items.size());
    for (size_t i = 0; i < items.size(); ++i)
      order[i] = ((uint64_t)(uint32_t)(INT32_MAX - items[i].f[FI_ITEM_NUM_TOKENS]) << 32) | i;
    std::sort(order.begin(), order.end());
    // snake: layers of num_cus units alternate longest-first and
    // shortest-first (dealt in turn, each CU then sums long and short)
    {
      const size_t layer = (size_t)std::max<int64_t>(1, num_cus);
      for (size_t b0 = layer; b0 < order.size(); b0 += 2 * layer)
        std::reverse(order.begin() + (std::ptrdiff_t)b0,
                     order.begin() + (std::ptrdiff_t)std::min(order.size(), b0 + layer));
    }
    p->items.resize(items.size() * FI_ITEM_STRIDE);
    for (size_t i = 0; i < order.size(); ++i)
      std::memcpy(&p->items[i * FI_ITEM_STRIDE], items[(uint32_t)order[i]].f, sizeof(Item));
    p->num_slots = slot;
    p->max_chunks = max_chunks;
    p->min_chunks_split = min_split;

    // ---- shared-prefix items: (group, KV head, block of members, chunk)
    for (int64_t gi = 0; gi < (int64_t)groups.size(); ++gi) {
      const Group& g = groups[gi];
      const int64_t per_block = kPrefixRows / group;
      for (int64_t c = 0, page0 = 0; c < g.chunks; ++c) {
        // the chunk's tokens [t0, t0 + nt) of the prefix
        int64_t t0, nt;
        if (comp) {
          t0 = c * g.tokens / g.chunks;
          nt = (c + 1) * g.tokens / g.chunks - t0;
        } else {
          const int64_t np = g.lcp / g.chunks + (c < g.lcp % g.chunks ? 1 : 0);
          t0 = page0 * page_size;
          nt = np * page_size;
          page0 += np;
        }
        const int64_t tok_off = t0 % g.psize;
        const int64_t npg = fi::ceil_div(tok_off + nt, g.psize);
        for (int32_t h = 0; h < num_kv_heads; ++h) {
          for (int64_t rb = 0; rb < g.row_blocks; ++rb) {
            const int64_t m0 = rb * per_block;
            const int64_t nm = std::min<int64_t>(per_block, g.members - m0);
            int32_t f[FI_PITEM_STRIDE] = {0};
            f[FI_PITEM_GROUP] = (int32_t)gi;
            f[FI_PITEM_KV_HEAD] = h;
            f[FI_PITEM_MEMBER_BASE] = (int32_t)g.member_base;
            f[FI_PITEM_ROW_BEGIN] = (int32_t)m0;
            f[FI_PITEM_NUM_ROWS] = (int32_t)(nm * group);
            f[FI_PITEM_CHUNK] = (int32_t)c;
            f[FI_PITEM_PAGE_BEGIN] = (int32_t)(g.page_base + t0 / g.psize);
            f[FI_PITEM_NUM_PAGES] = (int32_t)npg;
            f[FI_PITEM_TOKEN_BEGIN] = (int32_t)tok_off;
            f[FI_PITEM_NUM_TOKENS] = (int32_t)nt;
            p->pitems.insert(p->pitems.end(), f, f + FI_PITEM_STRIDE);
          }
        }
      }
    }

    // ---- workspace layout and host image of its uploaded part
    fi::WorkspaceLayout& ws = p->ws;
    const int64_t nn = p->num_nodes();
    int64_t off = 0;
    ws.items = off;
    off = fi::align_up(off + (int64_t)p->items.size() * 4, 256);
    ws.nodes = off;
    off = fi::align_up(off + (int64_t)nodes.size() * 4, 256);
    ws.counters = off;
    off = fi::align_up(off + nn * 4, 256);
    ws.page_ids = off;
    off = fi::align_up(off + (nnz + pre_nnz) * 4, 256);
    ws.pitems = off;
    off = fi::align_up(off + (int64_t)p->pitems.size() * 4, 256);
    ws.members = off;
    off = fi::align_up(off + (int64_t)members.size() * 4, 256);
    ws.prefix_slot = off;
    off = fi::align_up(off + (int64_t)pslot.size() * 4, 256);
    ws.image_bytes = off;
    ws.part_o = off;
    off = fi::align_up(off + p->num_slots * group * (int64_t)head_dim * 4, 256);
    ws.part_lse = off;
    off = fi::align_up(off + p->num_slots * group * 4, 256);
    ws.total_bytes = std::max<int64_t>(off, 256);
    p->image.assign(ws.image_bytes, 0);  // counters start at 0
    auto put = [&](int64_t at, const std::vector<int32_t>& v) {
      if (!v.empty()) std::memcpy(p->image.data() + at, v.data(), v.size() * 4);
    };
    put(ws.items, p->items);
    put(ws.nodes, nodes);
    put(ws.pitems, p->pitems);
    put(ws.members, members);
    put(ws.prefix_slot, pslot);
    if (nnz > 0) std::memcpy(p->image.data() + ws.page_ids, kv_indices, nnz * 4);
    if (pre_nnz > 0)
      std::memcpy(p->image.data() + ws.page_ids + nnz * 4, comp->indices, pre_nnz * 4);

    *out_plan = p.release();
    return FI_OK;
  } catch (const std::bad_alloc&) {
    return fail(FI_ERR_NOMEM, "host allocation failed in fi_plan_create");
  } catch (...) {
    return fail(FI_ERR_INVALID_ARG, "unexpected error in fi_plan_create");
  }
}

}  // namespace
}  // namespace fi

extern "C" {

fi_status fi_plan_get_info(const fi_plan* p, fi_plan_info* info) {
  if (!p || !info) return fi::fail(FI_ERR_INVALID_ARG, "NULL plan or info");
  fi_plan_info r{};
  r.num_items = p->num_items();
  r.num_partial_slots = p->num_slots;
  r.num_merge_nodes = p->num_nodes();
  r.workspace_bytes = p->ws.total_bytes;
  r.total_kv_tokens = p->total_tokens;
  r.chunk_pages = p->chunk_pages;
  r.max_chunks_per_request = p->max_chunks;
  r.min_chunks_split_request = p->min_chunks_split;
  r.batch = p->batch;
  r.num_qo_heads = p->num_qo_heads;
  r.num_kv_heads = p->num_kv_heads;
  r.head_dim = p->head_dim;
  r.page_size = p->page_size;
  r.dtype = (int32_t)p->dtype;
  r.shared_pages = p->shared_pages;
  r.num_prefix_items = p->num_pitems();
  r.num_prefix_groups = p->num_groups;
  r.prefix_rows_per_item = p->prefix_rows;
  r.image_bytes = (int64_t)p->image.size();
  r.decode_kernel = p->resolved_kernel;
  r.merge_fan_in = p->merge_fan_in;
  r.prefix_page_size = p->prefix_page_size;
  *info = r;
  return FI_OK;
}

fi_status fi_plan_work_list(const fi_plan* p, const int32_t** items, int64_t* num_items) {
  if (!p || !items || !num_items) return fi::fail(FI_ERR_INVALID_ARG, "NULL argument");
  *items = p->items.data();
  *num_items = p->num_items();
  return FI_OK;
}

fi_status fi_plan_merge_nodes(const fi_plan* p, const int32_t** nodes, int64_t* num_nodes) {
  if (!p || !nodes || !num_nodes) return fi::fail(FI_ERR_INVALID_ARG, "NULL argument");
  *nodes = p->nodes.data();
  *num_nodes = p->num_nodes();
  return FI_OK;
}

fi_status fi_plan_prefix_items(const fi_plan* p, const int32_t** items, int64_t* num_items) {
  if (!p || !items || !num_items) return fi::fail(FI_ERR_INVALID_ARG, "NULL argument");
  *items = p->pitems.data();
  *num_items = p->num_pitems();
  return FI_OK;
}

fi_status fi_plan_prefix_members(const fi_plan* p, const int32_t** members, int64_t* num_members) {
  if (!p || !members || !num_members) return fi::fail(FI_ERR_INVALID_ARG, "NULL argument");
  *members = p->members.data();
  *num_members = (int64_t)p->members.size();
  return FI_OK;
}

}  // extern "C"
