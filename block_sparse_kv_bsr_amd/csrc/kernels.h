// Launch interface between the C ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fi {

struct DecodeArgs {
  const int32_t* items;     // device, [num_items][FI_ITEM_STRIDE]
  const int32_t* page_ids;  // device, the request page lists
  const void* q;            // [batch, num_qo_heads, head_dim]
  const void* k_pages;      // [pool, num_kv_heads, page_size, head_dim]
  const void* v_pages;
  void* out;                // [batch, num_qo_heads, head_dim]
  float* lse;               // [batch, num_qo_heads] natural log, or null
  float* part_o;            // [slots, group, head_dim]
  float* part_lse;          // [slots, group], log2 units
  const int32_t* nodes;     // merge nodes [num_nodes][FI_NODE_STRIDE]
  int32_t* counters;        // arrivals per merge node
  int64_t num_items;
  int32_t num_qo_heads, num_kv_heads, head_dim, page_size, group;
  int32_t kv_bytes;          // 4 fp32, 2 bf16, 1 fp8 e4m3 (q/out bf16)
  bool stream_kv;           // nontemporal K/V loads (no page listed twice)
  float sm_scale;
  float k_scale, v_scale;   // K/V dequantisation scales (1 unless fp8)
  bool rope;                // K (and q) stored before the rotary embedding
  float rope_theta, rope_scale;
  bool mma;                 // run the matrix-core kernel (decode_mma.hip)
};

struct PrefixArgs {
  const int32_t* pitems;       // device, [num_items][FI_PITEM_STRIDE]
  const int32_t* members;      // device, request ids of the prefix groups
  const int32_t* prefix_slot;  // device, [batch][num_kv_heads] first prefix slot
  const int32_t* page_ids;     // device, the request page lists
  const void* q;
  const void* k_pages;
  const void* v_pages;
  float* part_o;
  float* part_lse;
  int64_t num_items;
  int32_t num_qo_heads, num_kv_heads, head_dim, page_size, group;
  float sm_scale;
};

struct PrefillArgs {
  const int32_t* items;     // device, [num_items][FI_QITEM_STRIDE]
  const int32_t* merges;    // device, [num_merges][FI_QMERGE_STRIDE]
  const int32_t* page_ids;  // device, the request page lists
  const void* q;            // bf16 [N, num_qo_heads, head_dim]
  const void* k_pages;
  const void* v_pages;
  void* out;                // bf16 [N, num_qo_heads, head_dim]
  float* lse;               // [N, num_qo_heads] natural log, or null
  int32_t* counters;        // device, [num_merges] arrival counts, 0 between runs
  float* part_o;            // [slots, FI_PREFILL_ROWS x head_dim] (the kernel's own order)
  float* part_lse;          // [slots, FI_PREFILL_ROWS], log2 units
  int64_t num_items, num_merges;
  int32_t num_qo_heads, num_kv_heads, head_dim, page_size, group, causal;
  int32_t kv_bytes;         // 2 bf16, 1 fp8 e4m3 (q/out bf16)
  float sm_scale;
  float k_scale, v_scale;   // K/V dequantisation scales (1 for bf16)
  bool rope;                // K and q stored before the rotary embedding
  float rope_theta, rope_scale;
};

struct MlaArgs {
  const int32_t* items;     // device, [num_items][FI_QITEM_STRIDE]
  const int32_t* merges;    // device, [num_merges][FI_QMERGE_STRIDE]
  const int32_t* page_ids;  // device, the request page lists
  const void* q_nope;       // bf16 [N, num_heads, 512]
  const void* q_pe;         // bf16 [N, num_heads, 64]
  const void* ckv;          // bf16 [pool, page_size, 512]
  const void* kpe;          // bf16 [pool, page_size, 64]
  void* out;                // bf16 [N, num_heads, 512]
  float* lse;               // [N, num_heads] natural log, or null
  int32_t* counters;        // device, [num_merges] arrival counts, 0 between runs
  float* part_o;            // [slots, FI_MLA_ROWS x 512] (the kernel's own order)
  float* part_lse;          // [slots, FI_MLA_ROWS], log2 units
  int64_t num_items, num_merges;
  int32_t num_heads, page_size, causal;
  float sm_scale;
};

struct MergeTwoArgs {
  const void* v_a;
  const float* s_a;
  const void* v_b;
  const float* s_b;
  void* v_out;
  float* s_out;
  int64_t num_rows;
  int32_t head_dim;
  bool bf16;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// The matrix-core decode kernel: built for head_dim 128, bf16 or fp8 K/V,
// G = 1, 2, 4, 8, page sizes that are multiples of 16, with or without the
// rotary embedding.
bool decode_mma_supported(const DecodeArgs& a);
hipError_t launch_decode_mma(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_merge_two(const MergeTwoArgs& a, hipStream_t stream);
hipError_t launch_prefix(const PrefixArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// Latent attention tiles; cut tiles merge in the same launch (mla_attend.hip).
hipError_t launch_mla(const MlaArgs& a, hipStream_t stream);

}  // namespace fi
