// Host-side split-KV planner: data structures shared by the planner (plain
// C++, no HIP headers, so it builds and is tested on a CPU-only host) and the
// HIP launch layer.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "fi_bsr.h"

namespace fi {

// Byte offsets of the sections of the device workspace. Each section starts
// on a 256-byte boundary. The first `image_bytes` are copied from the host
// (work items, merge nodes, their arrival counters (zeros), page ids); the
// rest is written by the kernel (partial outputs and their log-sum-exp).
struct WorkspaceLayout {
  int64_t items = 0;      // int32 [num_items][FI_ITEM_STRIDE]
  int64_t nodes = 0;      // int32 [num_nodes][FI_NODE_STRIDE]
  int64_t counters = 0;   // int32 [num_nodes], 0 between runs
  int64_t page_ids = 0;   // int32 [nnz] (composed: then the prefix cache's block ids)
  int64_t pitems = 0;     // int32 [num_prefix_items][FI_PITEM_STRIDE]
  int64_t members = 0;    // int32 request ids of the prefix groups
  int64_t prefix_slot = 0;  // int32 [batch][num_kv_heads]: first prefix slot or -1
  int64_t part_o = 0;     // float [num_slots][group][head_dim]
  int64_t part_lse = 0;   // float [num_slots][group], log2 units
  int64_t image_bytes = 0;
  int64_t total_bytes = 0;
};

inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Record of the last fatal message for this thread.
void set_error(const std::string& msg);

}  // namespace fi

struct fi_plan {
  int32_t batch = 0, num_qo_heads = 0, num_kv_heads = 0, head_dim = 0, page_size = 0;
  int32_t group = 0;
  fi_dtype dtype = FI_DTYPE_BF16;
  int64_t num_pool_pages = 0;
  int32_t chunk_pages = 0;
  int32_t max_chunks = 0, min_chunks_split = 0;
  int64_t total_tokens = 0;
  int64_t shared_pages = 0;  // distinct physical pages listed more than once
  int64_t num_slots = 0;
  std::vector<int32_t> items;   // num_items * FI_ITEM_STRIDE
  std::vector<int32_t> nodes;   // num_merge_nodes * FI_NODE_STRIDE
  std::vector<int32_t> pitems;  // num_prefix_items * FI_PITEM_STRIDE
  std::vector<int32_t> members; // request ids, grouped
  std::vector<int32_t> prefix_slot;  // [batch * num_kv_heads], empty without groups
  int32_t num_groups = 0, prefix_rows = 0;
  int32_t decode_kernel = FI_DECODE_KERNEL_AUTO;   // as asked for
  int32_t resolved_kernel = FI_DECODE_KERNEL_VECTOR;  // what the runs launch
  int32_t merge_fan_in = FI_MERGE_FAN_IN;             // children per merge node at most
  // composed formats: prefixes in a second cache of prefix_page_size blocks
  bool composed = false;
  int32_t prefix_page_size = 0;
  int64_t num_prefix_pool_pages = 0;
  std::vector<uint8_t> image;   // host copy of the uploaded part of the workspace
  fi::WorkspaceLayout ws;
  // Identity of this plan in the launch layer's upload records (0 until
  // the first upload).
  uint64_t serial = 0;
  int64_t num_items() const { return (int64_t)items.size() / FI_ITEM_STRIDE; }
  int64_t num_nodes() const { return (int64_t)nodes.size() / FI_NODE_STRIDE; }
  int64_t num_pitems() const { return (int64_t)pitems.size() / FI_PITEM_STRIDE; }
};

// Work list of one prefill / append call. Workspace sections (each on a
// 256-byte boundary): items, merges, page ids and one arrival counter per
// merge, all copied from the host (the counters as zeros), then
// the partial states of cut tiles (written by the tile kernel).
struct fi_prefill_plan {
  int32_t batch = 0, num_qo_heads = 0, num_kv_heads = 0, head_dim = 0, page_size = 0;
  int32_t group = 0, causal = 1, tokens_per_tile = 0, chunk_tokens = 0;
  fi_dtype dtype = FI_DTYPE_BF16;  // of the K/V pages (q and out are bf16)
  int32_t rope = 0;                // tiles for fi_prefill_run_rope
  int32_t mla = 0;                 // fi_mla_plan_create: latent attention tiles
  int32_t head_dim_kpe = 0;        // MLA: rotary-key width
  int64_t num_pool_pages = 0, total_qo = 0, total_kv = 0, visible_pairs = 0;
  int64_t num_tiles = 0, num_slots = 0;
  std::vector<int32_t> items;   // num_items * FI_QITEM_STRIDE
  std::vector<int32_t> merges;  // num_merges * FI_QMERGE_STRIDE
  struct {
    int64_t items = 0, merges = 0, page_ids = 0, counters = 0, part_o = 0, part_lse = 0;
    int64_t image_bytes = 0, total_bytes = 0;
  } ws;
  std::vector<uint8_t> image;
  uint64_t serial = 0;  // as for fi_plan
  int64_t num_items() const { return (int64_t)items.size() / FI_QITEM_STRIDE; }
  int64_t num_merges() const { return (int64_t)merges.size() / FI_QMERGE_STRIDE; }
};

namespace fi {
// Frees a plan (host memory only).
void plan_free_host(fi_plan* p);
void plan_free_host(fi_prefill_plan* p);

// Checks a BSR page table (kv_indptr, kv_indices, kv_last_page_len) and
// fills the token count of each request. On failure sets the error message
// and returns the status.
fi_status check_page_table(const int32_t* kv_indptr, const int32_t* kv_indices,
                           const int32_t* kv_last_page_len, int32_t batch, int32_t page_size,
                           int64_t num_pool_pages, std::vector<int64_t>* tokens);
}  // namespace fi
