// C ABI entry points that touch the device: plan uploads, the decode and
// prefill runs, state merge and plan destruction. The host-only planners
// live in plan.cpp and prefill_plan.cpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <iterator>
#include <map>
#include <mutex>
#include <string>

#include "fi_bsr.h"
#include "kernels.h"
#include "plan.h"
#include "staging.h"

namespace {

fi_status fail(fi_status st, const std::string& msg) {
  fi::set_error(msg);
  return st;
}

fi_status hip_fail(hipError_t e, const char* what) {
  return fail(FI_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Which plan's image each workspace holds. A run reads the item list, merge
// nodes and page ids of the last plan uploaded to its workspace, so it must
// be that plan: a run of plan A after plan B was uploaded over A's bytes
// would take B's words for A's requests and pages. Records are address
// ranges [start, start + extent), keyed by start and never overlapping; the
// extent is what the plan's runs may touch there (its whole workspace, or
// only its image when the caller gave no more). An upload drops every record
// its range overlaps (decode and prefill plans alike), a run must find its
// own plan's record at exactly its workspace with an extent covering what it
// touches, and destroying a plan drops its records. A plan is identified by
// a serial taken at its first upload, so a new plan that reuses a destroyed
// plan's address is not mistaken for it.
struct UploadRecord {
  uintptr_t end;
  uint64_t serial;
};
std::mutex g_uploads_mu;
std::map<uintptr_t, UploadRecord> g_uploads;
std::atomic<uint64_t> g_next_serial{1};

void record_upload(const void* workspace, int64_t bytes, uint64_t serial) {
  const uintptr_t s = reinterpret_cast<uintptr_t>(workspace);
  const uintptr_t e = s + (uintptr_t)(bytes > 0 ? bytes : 1);
  std::lock_guard<std::mutex> lock(g_uploads_mu);
  auto it = g_uploads.lower_bound(s);
  if (it != g_uploads.begin() && std::prev(it)->second.end > s) it = std::prev(it);
  while (it != g_uploads.end() && it->first < e) it = g_uploads.erase(it);
  g_uploads[s] = UploadRecord{e, serial};
}

// True when the workspace holds this plan's image and its recorded extent
// covers the `bytes` the run will touch.
bool holds_plan(const void* workspace, int64_t bytes, uint64_t serial) {
  if (serial == 0) return false;
  const uintptr_t s = reinterpret_cast<uintptr_t>(workspace);
  std::lock_guard<std::mutex> lock(g_uploads_mu);
  const auto it = g_uploads.find(s);
  return it != g_uploads.end() && it->second.serial == serial &&
         it->second.end >= s + (uintptr_t)(bytes > 0 ? bytes : 1);
}

void forget_plan(uint64_t serial) {
  if (serial == 0) return;
  std::lock_guard<std::mutex> lock(g_uploads_mu);
  for (auto it = g_uploads.begin(); it != g_uploads.end();)
    it = it->second.serial == serial ? g_uploads.erase(it) : std::next(it);
}

// Copies a plan's host image into the workspace, asynchronously on `stream`,
// through a cached pinned staging block. The workspace must hold at least
// the image; the recorded extent is the plan's whole workspace when the
// caller gave that much, else the image alone.
template <class Plan>
fi_status upload(Plan* plan, void* workspace, size_t workspace_bytes, fi_stream_t stream) {
  if (!plan) return fail(FI_ERR_INVALID_ARG, "plan is NULL");
  if (!workspace) return fail(FI_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(FI_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  const int64_t image = (int64_t)plan->image.size();
  if ((int64_t)workspace_bytes < image)
    return fail(FI_ERR_WORKSPACE, "workspace smaller than the plan's image (" +
                                      std::to_string(image) + " bytes)");
  const hipError_t e = fi::staged_upload(workspace, plan->image.data(), plan->image.size(),
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "plan upload");
  if (plan->serial == 0) plan->serial = g_next_serial.fetch_add(1);
  const int64_t extent = std::min<int64_t>((int64_t)workspace_bytes, plan->ws.total_bytes);
  record_upload(workspace, std::max<int64_t>(extent, image), plan->serial);
  return FI_OK;
}

template <class Plan>
void destroy(Plan* plan) {
  if (!plan) return;
  forget_plan(plan->serial);
  fi::plan_free_host(plan);
}

}  // namespace

extern "C" {

fi_status fi_plan_upload(fi_plan* plan, void* workspace, size_t workspace_bytes,
                         fi_stream_t stream) {
  return upload(plan, workspace, workspace_bytes, stream);
}

fi_status fi_prefill_plan_upload(fi_prefill_plan* plan, void* workspace, size_t workspace_bytes,
                                 fi_stream_t stream) {
  return upload(plan, workspace, workspace_bytes, stream);
}

namespace {

// The prefill run shared by the entry points below (checks, then the tile
// kernel, which also merges cut tiles). rope_theta > 0 selects the rotary
// variant.
fi_status prefill_run(const fi_prefill_plan* plan, const void* q, const void* k_pages,
                      const void* v_pages, float k_scale, float v_scale, float rope_theta,
                      float rope_scale, void* out, float* lse, float sm_scale, void* workspace,
                      size_t workspace_bytes, fi_stream_t stream) {
  if (plan->mla) return fail(FI_ERR_INVALID_ARG, "a plan made with fi_mla_plan_create runs with fi_mla_run");
  if (plan->num_items() == 0) return FI_OK;
  if (!q || !out) return fail(FI_ERR_INVALID_ARG, "q or out is NULL");
  if (!k_pages || !v_pages) return fail(FI_ERR_INVALID_ARG, "k_pages or v_pages is NULL");
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(out, 16))
    return fail(FI_ERR_INVALID_ARG, "q, k_pages, v_pages and out must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(FI_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  if (!workspace) return fail(FI_ERR_INVALID_ARG, "workspace is NULL");
  if ((int64_t)workspace_bytes < plan->ws.total_bytes)
    return fail(FI_ERR_WORKSPACE, "workspace smaller than fi_prefill_info.workspace_bytes");
  if (!holds_plan(workspace, plan->ws.total_bytes, plan->serial))
    return fail(FI_ERR_STATE,
                "workspace does not hold this plan: it was not uploaded there, or another plan "
                "was uploaded over it since (call fi_prefill_plan_upload)");
  if (!(sm_scale > 0.f)) sm_scale = 1.0f / std::sqrt((float)plan->head_dim);
  char* ws = static_cast<char*>(workspace);
  fi::PrefillArgs a{};
  a.items = reinterpret_cast<const int32_t*>(ws + plan->ws.items);
  a.merges = reinterpret_cast<const int32_t*>(ws + plan->ws.merges);
  a.page_ids = reinterpret_cast<const int32_t*>(ws + plan->ws.page_ids);
  a.q = q;
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.out = out;
  a.lse = lse;
  a.counters = reinterpret_cast<int32_t*>(ws + plan->ws.counters);
  a.part_o = reinterpret_cast<float*>(ws + plan->ws.part_o);
  a.part_lse = reinterpret_cast<float*>(ws + plan->ws.part_lse);
  a.num_items = plan->num_items();
  a.num_merges = plan->num_merges();
  a.num_qo_heads = plan->num_qo_heads;
  a.num_kv_heads = plan->num_kv_heads;
  a.head_dim = plan->head_dim;
  a.page_size = plan->page_size;
  a.group = plan->group;
  a.causal = plan->causal;
  a.kv_bytes = plan->dtype == FI_DTYPE_FP8_E4M3 ? 1 : 2;
  a.sm_scale = sm_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.rope = rope_theta > 0.f;
  a.rope_theta = rope_theta;
  a.rope_scale = rope_scale;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = fi::launch_prefill(a, s);
  if (e != hipSuccess) return hip_fail(e, "prefill tile kernel launch");
  return FI_OK;
}

}  // namespace

fi_status fi_prefill_run(const fi_prefill_plan* plan, const void* q, const void* k_pages,
                         const void* v_pages, void* out, float* lse, float sm_scale,
                         void* workspace, size_t workspace_bytes, fi_stream_t stream) {
  return fi_prefill_run_scaled(plan, q, k_pages, v_pages, 1.f, 1.f, out, lse, sm_scale, workspace,
                               workspace_bytes, stream);
}

fi_status fi_prefill_run_scaled(const fi_prefill_plan* plan, const void* q, const void* k_pages,
                                const void* v_pages, float k_scale, float v_scale, void* out,
                                float* lse, float sm_scale, void* workspace,
                                size_t workspace_bytes, fi_stream_t stream) {
  if (!plan) return fail(FI_ERR_INVALID_ARG, "plan is NULL");
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || std::isinf(k_scale) || std::isinf(v_scale))
    return fail(FI_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
  if (plan->rope)
    return fail(FI_ERR_INVALID_ARG, "a plan made with fi_prefill_opts.rope runs with "
                                    "fi_prefill_run_rope");
  return prefill_run(plan, q, k_pages, v_pages, k_scale, v_scale, 0.f, 1.f, out, lse, sm_scale,
                     workspace, workspace_bytes, stream);
}

fi_status fi_prefill_run_rope(const fi_prefill_plan* plan, const void* q, const void* k_pages,
                              const void* v_pages, float rope_theta, float rope_scale, void* out,
                              float* lse, float sm_scale, void* workspace,
                              size_t workspace_bytes, fi_stream_t stream) {
  if (!plan) return fail(FI_ERR_INVALID_ARG, "plan is NULL");
  if (!plan->rope)
    return fail(FI_ERR_INVALID_ARG, "fi_prefill_run_rope needs a plan made with "
                                    "fi_prefill_opts.rope");
  if (std::isnan(rope_theta) || std::isinf(rope_theta) || std::isnan(rope_scale) ||
      std::isinf(rope_scale))
    return fail(FI_ERR_INVALID_ARG, "rope_theta and rope_scale must be finite");
  if (!(rope_theta > 0.f)) rope_theta = 10000.f;
  if (!(rope_scale > 0.f)) rope_scale = 1.f;
  if (!(rope_theta > 1.f)) return fail(FI_ERR_INVALID_ARG, "rope_theta must exceed 1");
  return prefill_run(plan, q, k_pages, v_pages, 1.f, 1.f, rope_theta, rope_scale, out, lse,
                     sm_scale, workspace, workspace_bytes, stream);
}

fi_status fi_mla_run(const fi_prefill_plan* plan, const void* q_nope, const void* q_pe,
                     const void* ckv_pages, const void* kpe_pages, void* out, float* lse,
                     float sm_scale, void* workspace, size_t workspace_bytes, fi_stream_t stream) {
  if (!plan) return fail(FI_ERR_INVALID_ARG, "plan is NULL");
  if (!plan->mla) return fail(FI_ERR_INVALID_ARG, "fi_mla_run needs a plan made with fi_mla_plan_create");
  if (!(sm_scale > 0.f) || std::isinf(sm_scale))
    return fail(FI_ERR_INVALID_ARG, "sm_scale must be finite and positive (the model's scale)");
  if (plan->num_items() == 0) return FI_OK;
  if (!q_nope || !q_pe || !out) return fail(FI_ERR_INVALID_ARG, "q_nope, q_pe or out is NULL");
  if (!ckv_pages || !kpe_pages) return fail(FI_ERR_INVALID_ARG, "ckv_pages or kpe_pages is NULL");
  if (!aligned(q_nope, 16) || !aligned(q_pe, 16) || !aligned(ckv_pages, 16) ||
      !aligned(kpe_pages, 16) || !aligned(out, 16))
    return fail(FI_ERR_INVALID_ARG, "q_nope, q_pe, ckv_pages, kpe_pages and out must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(FI_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  if (!workspace) return fail(FI_ERR_INVALID_ARG, "workspace is NULL");
  if ((int64_t)workspace_bytes < plan->ws.total_bytes)
    return fail(FI_ERR_WORKSPACE, "workspace smaller than fi_prefill_info.workspace_bytes");
  if (!holds_plan(workspace, plan->ws.total_bytes, plan->serial))
    return fail(FI_ERR_STATE,
                "workspace does not hold this plan: it was not uploaded there, or another plan "
                "was uploaded over it since (call fi_prefill_plan_upload)");
  char* ws = static_cast<char*>(workspace);
  fi::MlaArgs a{};
  a.items = reinterpret_cast<const int32_t*>(ws + plan->ws.items);
  a.merges = reinterpret_cast<const int32_t*>(ws + plan->ws.merges);
  a.page_ids = reinterpret_cast<const int32_t*>(ws + plan->ws.page_ids);
  a.q_nope = q_nope;
  a.q_pe = q_pe;
  a.ckv = ckv_pages;
  a.kpe = kpe_pages;
  a.out = out;
  a.lse = lse;
  a.counters = reinterpret_cast<int32_t*>(ws + plan->ws.counters);
  a.part_o = reinterpret_cast<float*>(ws + plan->ws.part_o);
  a.part_lse = reinterpret_cast<float*>(ws + plan->ws.part_lse);
  a.num_items = plan->num_items();
  a.num_merges = plan->num_merges();
  a.num_heads = plan->num_qo_heads;
  a.page_size = plan->page_size;
  a.causal = plan->causal;
  a.sm_scale = sm_scale;
  const hipError_t e = fi::launch_mla(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "MLA kernel launch");
  return FI_OK;
}

void fi_prefill_plan_destroy(fi_prefill_plan* plan) { destroy(plan); }

namespace {

// Host-side checks shared by the decode entry points; nothing is launched
// unless they pass.
fi_status check_run(const fi_plan* plan, void* out, float* lse, void* workspace,
                    size_t workspace_bytes) {
  if (!plan) return fail(FI_ERR_INVALID_ARG, "plan is NULL");
  if (plan->batch == 0) return FI_OK;
  if (!out) return fail(FI_ERR_INVALID_ARG, "out is NULL");
  if (!aligned(out, 16)) return fail(FI_ERR_INVALID_ARG, "out must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(FI_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  if (!workspace) return fail(FI_ERR_INVALID_ARG, "workspace is NULL");
  if ((int64_t)workspace_bytes < plan->ws.total_bytes)
    return fail(FI_ERR_WORKSPACE, "workspace smaller than fi_plan_info.workspace_bytes");
  if (!holds_plan(workspace, plan->ws.total_bytes, plan->serial))
    return fail(FI_ERR_STATE,
                "workspace does not hold this plan: it was not uploaded there, another plan "
                "was uploaded over it since, or the upload was given fewer than "
                "fi_plan_info.workspace_bytes (call fi_plan_upload)");
  return FI_OK;
}

fi_status check_inputs(const fi_plan* plan, const void* q, const void* k_pages,
                       const void* v_pages, bool composed_run = false) {
  if (plan->composed != composed_run)
    return fail(FI_ERR_INVALID_ARG, plan->composed
                                        ? "a composed plan runs with fi_decode_run_composed"
                                        : "fi_decode_run_composed needs a plan made by "
                                          "fi_plan_create_composed");
  if (!q) return fail(FI_ERR_INVALID_ARG, "q is NULL");
  if (plan->num_items() > 0 && (!k_pages || !v_pages))
    return fail(FI_ERR_INVALID_ARG, "k_pages or v_pages is NULL");
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16))
    return fail(FI_ERR_INVALID_ARG, "q, k_pages and v_pages must be 16-byte aligned");
  return FI_OK;
}

struct Rope {
  bool on = false;
  float theta = 0.f, scale = 0.f;
};

// Where a run keeps what it writes besides out and lse: the merge nodes'
// arrival counters and the partial states of cut requests.
struct RunScratch {
  int32_t* counters;
  float* part_o;
  float* part_lse;
};

RunScratch workspace_scratch(const fi_plan* plan, void* workspace) {
  char* ws = static_cast<char*>(workspace);
  return RunScratch{reinterpret_cast<int32_t*>(ws + plan->ws.counters),
                    reinterpret_cast<float*>(ws + plan->ws.part_o),
                    reinterpret_cast<float*>(ws + plan->ws.part_lse)};
}

// Launches the run of an uploaded plan: its image (items, nodes, page ids,
// prefix items) is read from `workspace`, its scratch from `sc`.
fi_status launch_run(const fi_plan* plan, const void* q, const void* k_pages,
                     const void* v_pages, float k_scale, float v_scale, void* out, float* lse,
                     float sm_scale, const void* workspace, const RunScratch& sc, hipStream_t s,
                     Rope rope = Rope(), const void* k_prefix = nullptr,
                     const void* v_prefix = nullptr) {
  if (!(sm_scale > 0.f)) sm_scale = 1.0f / std::sqrt((float)plan->head_dim);
  const char* ws = static_cast<const char*>(workspace);
  fi::DecodeArgs d{};
  d.items = reinterpret_cast<const int32_t*>(ws + plan->ws.items);
  d.page_ids = reinterpret_cast<const int32_t*>(ws + plan->ws.page_ids);
  d.q = q;
  d.k_pages = k_pages;
  d.v_pages = v_pages;
  d.out = out;
  d.lse = lse;
  d.part_o = sc.part_o;
  d.part_lse = sc.part_lse;
  d.nodes = reinterpret_cast<const int32_t*>(ws + plan->ws.nodes);
  d.counters = sc.counters;
  d.num_items = plan->num_items();
  d.num_qo_heads = plan->num_qo_heads;
  d.num_kv_heads = plan->num_kv_heads;
  d.head_dim = plan->head_dim;
  d.page_size = plan->page_size;
  d.group = plan->group;
  d.kv_bytes = plan->dtype == FI_DTYPE_F32 ? 4 : plan->dtype == FI_DTYPE_BF16 ? 2 : 1;
  d.k_scale = k_scale;
  d.v_scale = v_scale;
  d.stream_kv = plan->shared_pages == 0;
  d.sm_scale = sm_scale;
  d.rope = rope.on;
  d.rope_theta = rope.theta;
  d.rope_scale = rope.scale;
  // Which decode kernel: the one the plan resolved (by default the
  // matrix-core kernel for fp8 caches and eight query heads per KV head, with
  // or without the rotary embedding: bound by vector work in the other
  // kernel, measured).
  const bool fits = fi::decode_mma_supported(d);
  if (plan->resolved_kernel == FI_DECODE_KERNEL_MATRIX && !fits)
    return fail(FI_ERR_UNSUPPORTED, "the matrix-core decode kernel does not fit this run");
  d.mma = plan->resolved_kernel == FI_DECODE_KERNEL_MATRIX;
  if (plan->num_pitems() > 0) {
    // shared prefixes first: their partials must be in place before the
    // decode kernel's merge trees read them
    fi::PrefixArgs pa{};
    pa.pitems = reinterpret_cast<const int32_t*>(ws + plan->ws.pitems);
    pa.members = reinterpret_cast<const int32_t*>(ws + plan->ws.members);
    pa.prefix_slot = reinterpret_cast<const int32_t*>(ws + plan->ws.prefix_slot);
    pa.page_ids = d.page_ids;
    pa.q = q;
    // a composed plan's prefixes live in the prefix cache, with its block size
    pa.k_pages = plan->composed ? k_prefix : k_pages;
    pa.v_pages = plan->composed ? v_prefix : v_pages;
    pa.part_o = d.part_o;
    pa.part_lse = d.part_lse;
    pa.num_items = plan->num_pitems();
    pa.num_qo_heads = plan->num_qo_heads;
    pa.num_kv_heads = plan->num_kv_heads;
    pa.head_dim = plan->head_dim;
    pa.page_size = plan->composed ? plan->prefix_page_size : plan->page_size;
    pa.group = plan->group;
    pa.sm_scale = sm_scale;
    const hipError_t ep = fi::launch_prefix(pa, s);
    if (ep != hipSuccess) return hip_fail(ep, "shared-prefix kernel launch");
  }
  hipError_t e = fi::launch_decode(d, s);
  if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
  return FI_OK;
}

}  // namespace

fi_status fi_decode_run_composed(const fi_plan* plan, const void* q, const void* k_pages,
                                 const void* v_pages, const void* k_prefix, const void* v_prefix,
                                 void* out, float* lse, float sm_scale, void* workspace,
                                 size_t workspace_bytes, fi_stream_t stream) {
  if (!plan) return fail(FI_ERR_INVALID_ARG, "plan is NULL");
  if (!plan->composed)
    return fail(FI_ERR_INVALID_ARG,
                "fi_decode_run_composed needs a plan made by fi_plan_create_composed");
  if (plan->batch == 0) return FI_OK;
  fi_status st = check_inputs(plan, q, k_pages, v_pages, true);
  if (st != FI_OK) return st;
  if (plan->num_pitems() > 0 && (!k_prefix || !v_prefix))
    return fail(FI_ERR_INVALID_ARG, "k_prefix or v_prefix is NULL");
  if (!aligned(k_prefix, 16) || !aligned(v_prefix, 16))
    return fail(FI_ERR_INVALID_ARG, "k_prefix and v_prefix must be 16-byte aligned");
  st = check_run(plan, out, lse, workspace, workspace_bytes);
  if (st != FI_OK) return st;
  return launch_run(plan, q, k_pages, v_pages, 1.f, 1.f, out, lse, sm_scale, workspace,
                    workspace_scratch(plan, workspace), static_cast<hipStream_t>(stream), Rope(),
                    k_prefix, v_prefix);
}

fi_status fi_decode_run_scaled(const fi_plan* plan, const void* q, const void* k_pages,
                               const void* v_pages, float k_scale, float v_scale, void* out,
                               float* lse, float sm_scale, void* workspace,
                               size_t workspace_bytes, fi_stream_t stream) {
  if (!plan) return fail(FI_ERR_INVALID_ARG, "plan is NULL");
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || std::isinf(k_scale) || std::isinf(v_scale))
    return fail(FI_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
  if (plan->batch == 0) return FI_OK;
  fi_status st = check_inputs(plan, q, k_pages, v_pages);
  if (st != FI_OK) return st;
  st = check_run(plan, out, lse, workspace, workspace_bytes);
  if (st != FI_OK) return st;
  return launch_run(plan, q, k_pages, v_pages, k_scale, v_scale, out, lse, sm_scale, workspace,
                    workspace_scratch(plan, workspace), static_cast<hipStream_t>(stream));
}

fi_status fi_decode_run_rope_scaled(const fi_plan* plan, const void* q, const void* k_pages,
                                    const void* v_pages, float k_scale, float v_scale,
                                    float rope_theta, float rope_scale, void* out, float* lse,
                                    float sm_scale, void* workspace, size_t workspace_bytes,
                                    fi_stream_t stream) {
  if (!plan) return fail(FI_ERR_INVALID_ARG, "plan is NULL");
  const bool built = (plan->dtype == FI_DTYPE_BF16 && (plan->head_dim == 128 || plan->head_dim == 64)) ||
                     (plan->dtype == FI_DTYPE_FP8_E4M3 && plan->head_dim == 128);
  if (!built)
    return fail(FI_ERR_UNSUPPORTED,
                "the rotary embedding is built for bf16 plans with head_dim 128 or 64 and fp8 "
                "plans with head_dim 128");
  if (plan->num_pitems() > 0)
    return fail(FI_ERR_UNSUPPORTED,
                "the rotary embedding does not run with shared-prefix items; plan with cascade = -1");
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || std::isinf(k_scale) || std::isinf(v_scale))
    return fail(FI_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
  if (std::isnan(rope_theta) || std::isinf(rope_theta) || std::isnan(rope_scale) ||
      std::isinf(rope_scale))
    return fail(FI_ERR_INVALID_ARG, "rope_theta and rope_scale must be finite");
  Rope r;
  r.on = true;
  r.theta = rope_theta > 0.f ? rope_theta : 10000.f;
  r.scale = rope_scale > 0.f ? rope_scale : 1.f;
  if (!(r.theta > 1.f)) return fail(FI_ERR_INVALID_ARG, "rope_theta must exceed 1");
  if (plan->batch == 0) return FI_OK;
  fi_status st = check_inputs(plan, q, k_pages, v_pages);
  if (st != FI_OK) return st;
  st = check_run(plan, out, lse, workspace, workspace_bytes);
  if (st != FI_OK) return st;
  return launch_run(plan, q, k_pages, v_pages, k_scale, v_scale, out, lse, sm_scale, workspace,
                    workspace_scratch(plan, workspace), static_cast<hipStream_t>(stream), r);
}

fi_status fi_decode_run_rope(const fi_plan* plan, const void* q, const void* k_pages,
                             const void* v_pages, float rope_theta, float rope_scale, void* out,
                             float* lse, float sm_scale, void* workspace, size_t workspace_bytes,
                             fi_stream_t stream) {
  return fi_decode_run_rope_scaled(plan, q, k_pages, v_pages, 1.f, 1.f, rope_theta, rope_scale,
                                   out, lse, sm_scale, workspace, workspace_bytes, stream);
}

fi_status fi_decode_run(const fi_plan* plan, const void* q, const void* k_pages,
                        const void* v_pages, void* out, float* lse, float sm_scale,
                        void* workspace, size_t workspace_bytes, fi_stream_t stream) {
  return fi_decode_run_scaled(plan, q, k_pages, v_pages, 1.f, 1.f, out, lse, sm_scale, workspace,
                              workspace_bytes, stream);
}

}  // extern "C"

namespace {

// ---- the static scratch of fi_decode_run_noalloc
// One copy of this array per GPU the library runs on, held until the
// process ends. In host code its name is a host-side stand-in, not a device
// address: the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is used.
static __device__ __align__(256) char scratch[FI_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of the scratch array.
fi_status device_scratch(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FI_ERR_UNSUPPORTED, "device ordinal beyond " + std::to_string(kMaxDevices - 1));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the static scratch");
    if (!p) return fail(FI_ERR_HIP, "hipGetSymbolAddress returned NULL for the static scratch");
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return FI_OK;
}

// Bytes of scratch a plan's run writes: arrival counters, partial outputs
// and partial LSE, each section on a 256-byte boundary.
struct ScratchLayout {
  int64_t counters = 0, part_o = 0, part_lse = 0, total = 0;
};

ScratchLayout scratch_layout(const fi_plan* plan) {
  ScratchLayout l;
  l.counters = 0;
  l.part_o = fi::align_up(plan->num_nodes() * 4, 256);
  l.part_lse = l.part_o + fi::align_up(plan->num_slots * plan->group * (int64_t)plan->head_dim * 4, 256);
  l.total = l.part_lse + fi::align_up(plan->num_slots * plan->group * 4, 256);
  return l;
}

__global__ void zero_words_kernel(int32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

extern "C" {

fi_status fi_decode_run_noalloc(const fi_plan* plan, const void* q, const void* k_pages,
                                const void* v_pages, void* out, float* lse, float sm_scale,
                                const void* workspace, size_t workspace_bytes,
                                fi_stream_t stream) {
  if (!plan) return fail(FI_ERR_INVALID_ARG, "plan is NULL");
  if (plan->batch == 0) return FI_OK;
  fi_status st = check_inputs(plan, q, k_pages, v_pages);
  if (st != FI_OK) return st;
  if (!out) return fail(FI_ERR_INVALID_ARG, "out is NULL");
  if (!aligned(out, 16)) return fail(FI_ERR_INVALID_ARG, "out must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(FI_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  if (!workspace) return fail(FI_ERR_INVALID_ARG, "workspace is NULL");
  const int64_t image = (int64_t)plan->image.size();
  if ((int64_t)workspace_bytes < image)
    return fail(FI_ERR_WORKSPACE, "workspace smaller than fi_plan_info.image_bytes");
  if (!holds_plan(workspace, image, plan->serial))
    return fail(FI_ERR_STATE,
                "workspace does not hold this plan: it was not uploaded there, or another plan "
                "was uploaded over it since (call fi_plan_upload)");
  const ScratchLayout l = scratch_layout(plan);
  if (l.total > (int64_t)FI_NOALLOC_SCRATCH_BYTES)
    return fail(FI_ERR_WORKSPACE,
                "the plan's partial states and merge counters need " + std::to_string(l.total) +
                    " bytes; the static scratch holds " +
                    std::to_string((int64_t)FI_NOALLOC_SCRATCH_BYTES) +
                    " (run this plan with fi_decode_run and a workspace)");
  char* base = nullptr;
  st = device_scratch(&base);
  if (st != FI_OK) return st;
  const RunScratch sc{reinterpret_cast<int32_t*>(base + l.counters),
                      reinterpret_cast<float*>(base + l.part_o),
                      reinterpret_cast<float*>(base + l.part_lse)};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t nn = plan->num_nodes();
  if (nn > 0) {
    // the array keeps the previous call's contents: counters start at zero
    hipLaunchKernelGGL(zero_words_kernel, dim3((uint32_t)((nn + 255) / 256)), dim3(256), 0, s,
                       sc.counters, nn);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "scratch counter clear launch");
  }
  return launch_run(plan, q, k_pages, v_pages, 1.f, 1.f, out, lse, sm_scale, workspace, sc, s);
}

fi_status fi_merge_states(fi_dtype dtype, const void* v_a, const float* s_a, const void* v_b,
                          const float* s_b, void* v_out, float* s_out, int64_t num_rows,
                          int32_t head_dim, fi_stream_t stream) {
  if (dtype != FI_DTYPE_F32 && dtype != FI_DTYPE_BF16)
    return fail(FI_ERR_UNSUPPORTED, "dtype must be FI_DTYPE_F32 or FI_DTYPE_BF16");
  if (head_dim != 64 && head_dim != 128) return fail(FI_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (num_rows < 0) return fail(FI_ERR_INVALID_ARG, "num_rows < 0");
  if (num_rows == 0) return FI_OK;
  if (!v_a || !s_a || !v_b || !s_b || !v_out || !s_out)
    return fail(FI_ERR_INVALID_ARG, "NULL state pointer");
  if (!aligned(v_a, 16) || !aligned(v_b, 16) || !aligned(v_out, 16))
    return fail(FI_ERR_INVALID_ARG, "state vectors must be 16-byte aligned");
  if (!aligned(s_a, 4) || !aligned(s_b, 4) || !aligned(s_out, 4))
    return fail(FI_ERR_INVALID_ARG, "LSE arrays must be 4-byte aligned");
  fi::MergeTwoArgs a{v_a, s_a, v_b, s_b, v_out, s_out, num_rows, head_dim, dtype == FI_DTYPE_BF16};
  hipError_t e = fi::launch_merge_two(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge_states kernel launch");
  return FI_OK;
}

void fi_plan_destroy(fi_plan* plan) { destroy(plan); }

}  // extern "C"
