// Host-only driver for the two planners (plan.cpp, prefill_plan.cpp), built
// by tests/test_planner_sanitized.py with AddressSanitizer and
// UndefinedBehaviorSanitizer. It reads planner calls from stdin, makes each
// one through the C ABI with every input array allocated at exactly its
// stated length (so a read past the end is a heap overflow the sanitizer
// reports), reads the plan back through the accessor calls, frees it, and
// prints the status and a hash of what the accessors returned. The test
// compares those lines with the same calls on the regular library.
//
// Input, whitespace separated, one call after another:
//   D|P|C batch num_qo_heads num_kv_heads head_dim page_size num_pool_pages
//       dtype causal
//   n_opts opts...          (0: NULL options; D and C take 7 fields, P 4)
//   n_qo qo_indptr...       (P only)
//   n_indptr kv_indptr...   (-1: NULL pointer, nothing follows)
//   n_indices kv_indices...
//   n_last kv_last_page_len...
//   C only: prefix_page_size num_prefix_pool_pages, then the prefix
//   table's three arrays and prefix_of, as above (num_prefixes is the
//   prefix_indptr array's length - 1, 0 if it is NULL)
// Output per call: "<index> <status> <hash>".
#include <cstdint>
#include <cstdio>
#include <iostream>
#include <memory>
#include <string>
#include <vector>

#include "fi_bsr.h"
#include "plan.h"

namespace {

struct Hash {
  uint64_t h = 1469598103934665603ull;  // FNV-1a over 64-bit words
  void mix(int64_t x) {
    h ^= (uint64_t)x;
    h *= 1099511628211ull;
  }
  void mix_array(const int32_t* p, int64_t n) {
    mix(n);
    for (int64_t i = 0; i < n; ++i) mix(p[i]);
  }
};

// An input array at exactly its stated length, or no array at all.
struct Array {
  std::unique_ptr<int32_t[]> data;
  bool null = false;
  int64_t n = 0;
  const int32_t* ptr() const { return null ? nullptr : data.get(); }
};

bool read_array(Array* a) {
  int64_t n;
  if (!(std::cin >> n)) return false;
  if (n < 0) {
    a->null = true;
    return true;
  }
  a->n = n;
  a->data.reset(new int32_t[n > 0 ? n : 1]);
  for (int64_t i = 0; i < n; ++i)
    if (!(std::cin >> a->data[i])) return false;
  if (n == 0) a->data.reset(new int32_t[0]);
  return true;
}

struct Prefixes {
  int32_t page_size = 0;
  int64_t pool = 0;
  Array ip, ix, lp, of;
};

uint64_t decode_call(const int32_t* hdr, const std::vector<int32_t>& opts, const Array& ip,
                     const Array& ix, const Array& lp, const Prefixes* pre, int* status) {
  fi_plan_opts o{};
  const fi_plan_opts* po = nullptr;
  if (!opts.empty()) {
    o.num_cus = opts[0];
    o.items_per_cu = opts[1];
    o.min_chunk_tokens = opts[2];
    o.max_chunk_tokens = opts[3];
    o.fixed_chunk_tokens = opts[4];
    o.cascade = opts[5];
    o.decode_kernel = opts[6];
    o.rope = opts.size() > 7 ? opts[7] : 0;
    po = &o;
  }
  fi_plan* p = nullptr;
  if (pre) {
    const int32_t num_prefixes = pre->ip.null ? 0 : (int32_t)(pre->ip.n - 1);
    *status = fi_plan_create_composed(ip.ptr(), ix.ptr(), lp.ptr(), hdr[0], pre->ip.ptr(),
                                      pre->ix.ptr(), pre->lp.ptr(), num_prefixes, pre->of.ptr(),
                                      hdr[1], hdr[2], hdr[3], hdr[4], hdr[5], pre->page_size,
                                      pre->pool, (fi_dtype)hdr[6], po, &p);
  } else {
    *status = fi_plan_create(ip.ptr(), ix.ptr(), lp.ptr(), hdr[0], hdr[1], hdr[2], hdr[3],
                             hdr[4], hdr[5], (fi_dtype)hdr[6], po, &p);
  }
  Hash h;
  h.mix(*status);
  if (*status != FI_OK) return h.h;
  fi_plan_info info{};
  fi_plan_get_info(p, &info);
  h.mix(info.num_items);
  h.mix(info.num_partial_slots);
  h.mix(info.workspace_bytes);
  const int32_t* a = nullptr;
  int64_t n = 0;
  fi_plan_work_list(p, &a, &n);
  h.mix_array(a, n * FI_ITEM_STRIDE);
  fi_plan_merge_nodes(p, &a, &n);
  h.mix_array(a, n * FI_NODE_STRIDE);
  fi_plan_prefix_items(p, &a, &n);
  h.mix_array(a, n * FI_PITEM_STRIDE);
  fi_plan_prefix_members(p, &a, &n);
  h.mix_array(a, n);
  fi::plan_free_host(p);
  return h.h;
}

uint64_t prefill_call(const int32_t* hdr, const std::vector<int32_t>& opts, const Array& qo,
                      const Array& ip, const Array& ix, const Array& lp, bool mla, int* status) {
  fi_prefill_opts o{};
  const fi_prefill_opts* po = nullptr;
  if (!opts.empty()) {
    o.num_cus = opts[0];
    o.items_per_cu = opts[1];
    o.fixed_chunk_tokens = opts[2];
    o.num_xcds = opts[3];
    o.rope = opts.size() > 4 ? opts[4] : 0;
    po = &o;
  }
  fi_prefill_plan* p = nullptr;
  // MLA: hdr = batch, heads, latent width, rotary width, page size, pool, -, causal
  *status = mla ? fi_mla_plan_create(qo.ptr(), ip.ptr(), ix.ptr(), lp.ptr(), hdr[0], hdr[1], hdr[2],
                                     hdr[3], hdr[4], hdr[5], hdr[7], po, &p)
                : fi_prefill_plan_create(qo.ptr(), ip.ptr(), ix.ptr(), lp.ptr(), hdr[0], hdr[1],
                                         hdr[2], hdr[3], hdr[4], hdr[5], (fi_dtype)hdr[6], hdr[7],
                                         po, &p);
  Hash h;
  h.mix(*status);
  if (*status != FI_OK) return h.h;
  fi_prefill_info info{};
  fi_prefill_plan_get_info(p, &info);
  h.mix(info.num_items);
  h.mix(info.num_partial_slots);
  h.mix(info.workspace_bytes);
  const int32_t* a = nullptr;
  int64_t n = 0;
  fi_prefill_plan_work_list(p, &a, &n);
  h.mix_array(a, n * FI_QITEM_STRIDE);
  fi_prefill_plan_merges(p, &a, &n);
  h.mix_array(a, n * FI_QMERGE_STRIDE);
  fi::plan_free_host(p);
  return h.h;
}

}  // namespace

int main() {
  std::string kind;
  for (int index = 0; std::cin >> kind; ++index) {
    int32_t hdr[8];
    for (int32_t& x : hdr)
      if (!(std::cin >> x)) return 2;
    int n_opts;
    if (!(std::cin >> n_opts)) return 2;
    std::vector<int32_t> opts(n_opts);
    for (int32_t& x : opts)
      if (!(std::cin >> x)) return 2;
    const bool mla = kind == "M";
    const bool prefill = kind == "P" || mla, composed = kind == "C";
    if ((prefill && n_opts != 0 && n_opts != 4 && n_opts != 5) ||
        (!prefill && n_opts != 0 && n_opts != 7 && n_opts != 8))
      return 2;
    Array qo, ip, ix, lp;
    if (prefill && !read_array(&qo)) return 2;
    if (!read_array(&ip) || !read_array(&ix) || !read_array(&lp)) return 2;
    Prefixes pre;
    if (composed) {
      if (!(std::cin >> pre.page_size >> pre.pool)) return 2;
      if (!read_array(&pre.ip) || !read_array(&pre.ix) || !read_array(&pre.lp) ||
          !read_array(&pre.of))
        return 2;
    }
    int status = 0;
    const uint64_t h = prefill ? prefill_call(hdr, opts, qo, ip, ix, lp, mla, &status)
                               : decode_call(hdr, opts, ip, ix, lp, composed ? &pre : nullptr,
                                             &status);
    std::printf("%d %d %llu\n", index, status, (unsigned long long)h);
  }
  return 0;
}
