/*
 * fi_bsr.h -- C ABI of a decode-attention library for AMD MI355X (gfx950).
 *
 * Operation. Batched grouped-query decode attention over a KV cache held as
 * a block-sparse-row (BSR) / paged matrix. Sources for what is computed:
 *
 *  - FlashInfer paper explainer, "FlashInfer: Block-Sparse KV 캐시로 어텐션
 *    병목을 해소하다" (visionhong.com):
 *      * section on where the attention bottleneck lies: a decode step attends
 *        one new query token per request over that request's whole KV
 *        history, so the step is bound by reading the KV cache from memory;
 *      * section on the Block-Sparse format: the KV cache is a block-sparse
 *        matrix whose blocks are runs of consecutive tokens; metadata lists
 *        the active blocks; paged, dense and sparse layouts are all BSR;
 *        inactive blocks are skipped;
 *      * benchmark section: a load-balanced scheduler cuts long sequences
 *        into several work units and interleaves them with short ones so no
 *        workgroup idles in a skewed batch.
 *  - FlashInfer 0.6.17 release write-up (llm-wiki.hwlabs.dev), "what is
 *    FlashInfer" and section 5 (JIT warm-up): per-request context lengths
 *    differ; head count, GQA ratio and block size are runtime parameters;
 *    the call takes num_heads, num_kv_heads, head_dim and sm_scale (None =
 *    default scale).
 *
 * For request b with listed pages kv_indices[kv_indptr[b] .. kv_indptr[b+1])
 * and query head h (KV head kvh = h / G, G = num_qo_heads / num_kv_heads):
 *     s_t      = sm_scale * <q[b,h,:], K[page_t, kvh, slot_t, :]>
 *     out[b,h] = sum_t softmax(s)_t * V[page_t, kvh, slot_t, :]
 *     lse[b,h] = ln sum_t exp(s_t)                 (natural log, scaled scores)
 * over the tokens t of the listed pages in listed order: every listed page is
 * full except the last, which holds kv_last_page_len[b] tokens. A request
 * with no pages gets out = 0 and lse = -inf. Pages not listed (inactive
 * blocks, spare pool pages) and slots past the last page's length are never
 * read and may hold anything, NaN included.
 *
 * Memory layout (all contiguous, row-major):
 *     q, out          [batch, num_qo_heads, head_dim]           dtype
 *     lse             [batch, num_qo_heads]                     float32
 *     k_pages,v_pages [num_pool_pages, num_kv_heads, page_size, head_dim] dtype
 * dtype is float32 or bfloat16 for q, K, V and out alike. Arithmetic is
 * float32 throughout; bfloat16 outputs are rounded to nearest even.
 *
 * Ownership. The caller owns every device buffer (q, pages, out, lse and the
 * workspace). The library allocates no device memory. A plan owns host
 * memory only (its work list) and is immutable after fi_plan_create except
 * for the record of which workspace it was last uploaded to. Uploads stage
 * through page-locked host blocks that the library pins on first need and
 * keeps for the life of the process (one per upload in flight, sized to the
 * plan image rounded up to a power of two, 64 KiB at least); a block is
 * reused once the copy it fed has run. No call synchronises a stream or the
 * device.
 *
 * Errors. Every call returns an fi_status; on failure nothing is launched,
 * the outputs are untouched, and fi_last_error() returns a message for the
 * calling thread. No C++ exception crosses this boundary. Metadata are fully
 * validated by fi_plan_create (host only); fi_decode_run checks pointers,
 * alignment, workspace size and that the workspace still holds this plan,
 * then launches without reading device memory on the host. "Still holds"
 * is kept on the host per address range: every upload (decode or prefill
 * plan) records that its plan occupies [workspace, workspace +
 * workspace_bytes of the plan) and drops the record of every earlier upload
 * whose range overlaps it; a run needs its own plan's record at exactly its
 * workspace address, else it returns FI_ERR_STATE without launching; a
 * destroyed plan's records are dropped. The record is keyed by address: a
 * buffer freed and reallocated at the same address by the caller, with no
 * upload in between, is not detected.
 *
 * Thread safety. Distinct plans may be used from distinct threads (the
 * upload records are guarded by a lock). A plan must not be uploaded from
 * two threads at once.
 */
#ifndef FI_BSR_H
#define FI_BSR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FI_OK = 0,
  FI_ERR_INVALID_ARG = -1, /* malformed metadata, null or misaligned pointer */
  FI_ERR_UNSUPPORTED = -2, /* valid but not built: head_dim, group size, dtype */
  FI_ERR_WORKSPACE = -3,   /* workspace too small */
  FI_ERR_HIP = -4,         /* a HIP runtime call failed; message has its text */
  FI_ERR_NOMEM = -5,       /* host allocation failed */
  FI_ERR_STATE = -6        /* workspace does not hold this plan (never uploaded
                              there, or another plan uploaded over it since) */
} fi_status;

/*
 * Element types of a plan. FI_DTYPE_FP8_E4M3 is a quantised KV cache (the
 * quantisation/dequantisation fused into the attention kernel, explainer's
 * JIT section): K and V pages hold OCP FP8 E4M3 bytes (1 sign, 4 exponent
 * bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN) that
 * stand for byte_value * k_scale (resp. v_scale); q and out are bf16;
 * head_dim 128 only. fi_merge_states takes FI_DTYPE_F32 or FI_DTYPE_BF16.
 */
typedef enum { FI_DTYPE_F32 = 0, FI_DTYPE_BF16 = 1, FI_DTYPE_FP8_E4M3 = 2 } fi_dtype;

/* A hipStream_t; NULL is the null stream. */
typedef void* fi_stream_t;

typedef struct fi_plan fi_plan; /* opaque, host-owned */

/* Planner knobs. Zero selects the default for every field. */
typedef struct {
  int32_t num_cus;            /* compute units to balance over (default 256) */
  int32_t items_per_cu;       /* target work items per CU (default 8; for a
                                 plan that runs the matrix-core kernel, 6
                                 without the rotary embedding and 16 with
                                 it, each measured best) */
  int32_t min_chunk_tokens;   /* never cut a request finer than this (default 32) */
  int32_t max_chunk_tokens;   /* cap on chunk length; 0 = no cap */
  int32_t fixed_chunk_tokens; /* >0: use exactly this chunk length (rounded up
                                 to whole pages) instead of the heuristic */
  int32_t cascade;            /* shared-prefix cascade: 0 = when it pays
                                 (see fi_plan_create), 1 = whenever requests
                                 share a prefix, -1 = never */
  int32_t decode_kernel;      /* FI_DECODE_KERNEL_*: which decode kernel the
                                 plan's runs launch */
  int32_t rope;               /* nonzero: the plan's runs apply the rotary
                                 embedding (fi_decode_run_rope*); only sizes
                                 the items (see items_per_cu) -- every run
                                 entry point stays correct with any plan */
} fi_plan_opts;

/* Decode kernels. Both compute the same attention and merge trees, to the
 * same tolerance; they differ in where the products run. VECTOR: per-lane
 * dot products and multiply-adds (every dtype, head_dim and page size).
 * MATRIX: scores and PV on the matrix cores (v_mfma_f32_16x16x32_bf16 /
 * 16x16x16), for head_dim 128, bf16 or fp8 K/V and page sizes that are
 * multiples of 16 (fi_plan_create refuses a MATRIX plan otherwise). AUTO:
 * MATRIX where it was measured faster and fits -- fp8 caches and eight query
 * heads per KV head, with or without the rotary embedding -- else VECTOR. */
enum { FI_DECODE_KERNEL_AUTO = 0, FI_DECODE_KERNEL_VECTOR = 1, FI_DECODE_KERNEL_MATRIX = 2 };

typedef struct {
  int64_t num_items;         /* work items = (request, KV head, chunk) */
  int64_t num_partial_slots; /* partial states, each G rows (one KV-head group) */
  int64_t num_merge_nodes;   /* nodes of the merge trees of cut requests */
  int64_t workspace_bytes;   /* device workspace fi_plan_upload needs */
  int64_t total_kv_tokens;   /* sum of active tokens over the batch */
  int32_t chunk_pages;       /* pages per chunk chosen by the planner */
  int32_t max_chunks_per_request;
  int32_t min_chunks_split_request; /* fewest chunks among split requests; 0 if none */
  int32_t batch, num_qo_heads, num_kv_heads, head_dim, page_size;
  int32_t dtype;
  int64_t shared_pages; /* physical pages the decode items read more than
                           once (a cascade's prefix pages excluded); when 0
                           the kernel streams K/V past the caches
                           (nontemporal loads), else it keeps them cacheable
                           for re-reads */
  int64_t num_prefix_items;  /* shared-prefix work items (0: no cascade) */
  int32_t num_prefix_groups; /* groups of requests sharing a prefix */
  int32_t prefix_rows_per_item; /* query rows one prefix item covers (128) */
  int64_t image_bytes;       /* the uploaded plan (work list, merge nodes, page
                                ids, prefix items): the least workspace
                                fi_plan_upload accepts; workspace_bytes adds
                                the partial states fi_decode_run keeps there */
  int32_t decode_kernel;     /* FI_DECODE_KERNEL_VECTOR or _MATRIX: the kernel
                                the plan's runs launch */
  int32_t merge_fan_in;      /* children per merge node at most: 16, or 8 when
                                G * head_dim = 1024 (see FI_NODE_*) */
  int32_t prefix_page_size;  /* block size of the prefix cache of a composed
                                plan (fi_plan_create_composed); 0 otherwise */
} fi_plan_info;

/* Fields of one work item in the list returned by fi_plan_work_list. */
enum {
  FI_ITEM_REQUEST = 0,    /* request b */
  FI_ITEM_KV_HEAD = 1,    /* KV head; query heads kvh*G .. kvh*G+G-1 */
  FI_ITEM_PAGE_BEGIN = 2, /* first page, as an index into kv_indices */
  FI_ITEM_NUM_TOKENS = 3, /* tokens in this chunk; 0 = a request with no
                             pages (the item writes out = 0, lse = -inf) */
  FI_ITEM_SLOT = 4,       /* -1: writes out/lse directly; else partial slot */
  FI_ITEM_CHUNK = 5,      /* chunk number within the request */
  FI_ITEM_NUM_PAGES = 6,  /* pages in this chunk */
  FI_ITEM_FIRST_PAGE = 7, /* physical id of the chunk's first page (a copy of
                             kv_indices[FI_ITEM_PAGE_BEGIN], so the first
                             loads need no page-table read); 0 if no pages */
  FI_ITEM_MERGE_NODE = 8, /* merge node the partial reports to; -1 if none */
  FI_ITEM_KV_POS = 9,     /* position in the request of the chunk's first token */
  FI_ITEM_Q_POS = 10,     /* position of the request's query: its last token */
  FI_ITEM_STRIDE = 16     /* int32 per item */
};

/*
 * Fields of one merge node in the list returned by fi_plan_merge_nodes.
 * A request cut into k chunks has, per KV head, a tree of merge nodes with
 * at most fi_plan_info.merge_fan_in children each (never more than
 * FI_MERGE_FAN_IN; the planner takes as many as the merging wave loads in
 * one round: 16, or 8 for partials of G * head_dim = 1024 floats): the
 * leaves' children are the chunk
 * partials, an inner node's children are its child nodes' merged states, and
 * the root writes the request's output. The wave that brings a node's last
 * child merges the children in slot order (so the result does not depend on
 * arrival order) and reports to the parent.
 */
enum {
  FI_NODE_COUNT = 0,      /* children */
  FI_NODE_SLOT_BEGIN = 1, /* children's partial slots: [begin, begin + count) */
  FI_NODE_PARENT = 2,     /* parent node; -1 for the root */
  FI_NODE_OUT_SLOT = 3,   /* slot the merged state goes to; -1 for the root */
  FI_NODE_REQUEST = 4,
  FI_NODE_KV_HEAD = 5,
  FI_NODE_LEVEL = 6,      /* 0 for nodes whose children are chunks */
  FI_NODE_ARRIVALS = 7,   /* children that report during the decode kernel:
                             COUNT minus the shared-prefix partials, which
                             are complete before it starts */
  FI_NODE_STRIDE = 8,
  FI_MERGE_FAN_IN = 32
};

/*
 * Fields of one shared-prefix work item (fi_plan_prefix_items). Requests
 * whose page lists start with the same physical pages form a group; the
 * common run of whole pages (never a request's last page) is the group's
 * prefix. A plan made by fi_plan_create_composed has one group per prefix
 * of its prefix cache instead. A prefix item attends the query rows of up to
 * prefix_rows_per_item / G members of one group (row r: member
 * ROW_BEGIN + r / G, query head KV_HEAD * G + r % G) over one chunk of the
 * prefix -- NUM_TOKENS tokens starting TOKEN_BEGIN tokens into page
 * PAGE_BEGIN -- and writes one partial state per member, into the first
 * slots of that member's merge tree.
 */
enum {
  FI_PITEM_GROUP = 0,
  FI_PITEM_KV_HEAD = 1,
  FI_PITEM_MEMBER_BASE = 2, /* index of the group's first member in the member list */
  FI_PITEM_ROW_BEGIN = 3,   /* first member (within the group) of this item */
  FI_PITEM_NUM_ROWS = 4,    /* query rows: members in this item x G */
  FI_PITEM_CHUNK = 5,       /* prefix chunk number = child index in the trees */
  FI_PITEM_PAGE_BEGIN = 6,  /* first page, as an index into kv_indices
                               (composed plans: kv_indices followed by
                               prefix_indices) */
  FI_PITEM_NUM_PAGES = 7,   /* pages the chunk touches, at most FI_PREFIX_MAX_PAGES */
  FI_PITEM_TOKEN_BEGIN = 8, /* first token's slot in page PAGE_BEGIN (0 unless
                               composed) */
  FI_PITEM_NUM_TOKENS = 9,  /* tokens in the chunk */
  FI_PITEM_STRIDE = 12,
  FI_PREFIX_MAX_PAGES = 256 /* a group's prefix is at most (merge_fan_in - 1)
                               chunks of this many pages; shared pages past
                               that stay with the decode items */
};

/*
 * Build the load-balanced split-KV plan for one decode step (the scheduler
 * of the explainer's benchmark section). Host only; touches no device.
 *
 * kv_indptr        host int32 [batch+1], kv_indptr[0] = 0, non-decreasing
 * kv_indices       host int32 [kv_indptr[batch]], each in [0, num_pool_pages)
 * kv_last_page_len host int32 [batch]; in [1, page_size] for requests with
 *                  pages, ignored (any value in [0, page_size]) for empty ones
 * num_qo_heads, num_kv_heads: num_qo_heads % num_kv_heads == 0; the group
 *                  size G = num_qo_heads / num_kv_heads must be 1, 2, 4 or 8
 * head_dim         64 or 128 (128 for FI_DTYPE_FP8_E4M3)
 * page_size        block size in tokens, 1 .. 4096
 * num_pool_pages   pages in the caller's k_pages / v_pages pools
 * dtype            element type of q, K, V, out
 * opts             may be NULL
 * out_plan         receives a plan to free with fi_plan_destroy
 *
 * The planner picks one chunk length C (whole pages) for the batch: the
 * smallest C of at least min_chunk_tokens for which the items
 * sum_b ceil(n_b / C) * num_kv_heads fit in num_cus * items_per_cu (no cut
 * if even the longest request's full length exceeds that budget), capped by
 * max_chunk_tokens. Items are ordered longest first (ties by request, KV
 * head, chunk) so that long chunks start early and short requests fill the
 * gaps, except that every other layer of num_cus items is reversed (a snake
 * order: the dispatcher deals consecutive workgroups to the CUs in turn, so a
 * CU that takes one layer's longest item takes the next layer's shortest).
 * The input arrays are copied; the caller may free them afterwards. Their
 * lengths are not visible across this boundary: kv_indptr must hold batch+1
 * entries, kv_indices at least kv_indptr[batch] and kv_last_page_len batch
 * (the Python binding checks the lengths before calling).
 *
 * Shared prefixes (composable block-sparse formats, explainer's Block-Sparse
 * section; cascade attention): for bf16, requests whose page lists begin with
 * the same physical page are grouped and their common leading run of whole
 * pages (excluding each request's last page) is attended once per KV head
 * for all the group's query rows by a matrix-core kernel; each member's
 * remaining pages go through the decode items, and the two states meet in
 * the member's merge tree. With opts->cascade = 0 a group is formed when the
 * prefix re-reads it saves, (members - 1) x prefix bytes, reach 8 MiB.
 */
fi_status fi_plan_create(const int32_t* kv_indptr, const int32_t* kv_indices,
                         const int32_t* kv_last_page_len, int32_t batch,
                         int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t page_size, int64_t num_pool_pages, fi_dtype dtype,
                         const fi_plan_opts* opts, fi_plan** out_plan);

/*
 * Composed formats (explainer's Block-Sparse section: a prefix that many
 * requests share is stored once, each request's own KV separately, the two
 * with different block sizes). Request b attends the tokens of prefix
 * prefix_of[b], held in a second cache of prefix_page_size-token blocks,
 * followed by its own tokens in the paged cache, exactly as if both sat in
 * one cache. Host only; the run is fi_decode_run_composed.
 *
 * kv_indptr .. num_pool_pages  the requests' own tokens, as fi_plan_create
 * prefix_indptr    host int32 [num_prefixes+1], prefix_indptr[0] = 0,
 *                  non-decreasing
 * prefix_indices   host int32 [prefix_indptr[num_prefixes]], blocks of the
 *                  prefix cache, each in [0, num_prefix_pool_pages)
 * prefix_last_page_len host int32 [num_prefixes]: tokens in a prefix's last
 *                  block, in [1, prefix_page_size] (a prefix with no blocks:
 *                  any value in [0, prefix_page_size], and it holds nothing)
 * num_prefixes     >= 0
 * prefix_of        host int32 [batch]: -1 (no prefix) or a prefix index;
 *                  a request with a non-empty prefix must hold at least one
 *                  token of its own (its newest token, being decoded)
 * prefix_page_size block size of the prefix cache, 1 .. 4096
 * num_prefix_pool_pages blocks in the caller's k_prefix / v_prefix
 * dtype            FI_DTYPE_BF16 (the prefix tile kernel reads bf16)
 *
 * Every prefix with members is one group (see FI_PITEM_*): its tokens are
 * cut into chunks of near-equal token counts, at most merge_fan_in - 1 of
 * them, each touching at most FI_PREFIX_MAX_PAGES blocks (a prefix longer
 * than (merge_fan_in - 1) x (FI_PREFIX_MAX_PAGES - 1) x prefix_page_size
 * tokens is FI_ERR_UNSUPPORTED). opts.cascade is ignored (no shared pages
 * are looked for in the requests' own lists). Other options, the decode
 * items over the requests' own pages and their merge trees as
 * fi_plan_create. Errors: FI_ERR_INVALID_ARG for malformed tables or
 * prefix_of, FI_ERR_UNSUPPORTED as above.
 */
fi_status fi_plan_create_composed(const int32_t* kv_indptr, const int32_t* kv_indices,
                                  const int32_t* kv_last_page_len, int32_t batch,
                                  const int32_t* prefix_indptr, const int32_t* prefix_indices,
                                  const int32_t* prefix_last_page_len, int32_t num_prefixes,
                                  const int32_t* prefix_of, int32_t num_qo_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                  int64_t num_pool_pages, int32_t prefix_page_size,
                                  int64_t num_prefix_pool_pages, fi_dtype dtype,
                                  const fi_plan_opts* opts, fi_plan** out_plan);

/* Sizes and choices of a plan. */
fi_status fi_plan_get_info(const fi_plan* plan, fi_plan_info* info);

/* Host view of the work list (num_items * FI_ITEM_STRIDE int32, in launch
 * order) and of the merge nodes (num_merge_nodes * FI_NODE_STRIDE int32).
 * Valid until fi_plan_destroy. */
fi_status fi_plan_work_list(const fi_plan* plan, const int32_t** items, int64_t* num_items);
fi_status fi_plan_merge_nodes(const fi_plan* plan, const int32_t** nodes, int64_t* num_nodes);
/* Host view of the shared-prefix items (num_prefix_items * FI_PITEM_STRIDE
 * int32) and of the member list (request ids, grouped). */
fi_status fi_plan_prefix_items(const fi_plan* plan, const int32_t** items, int64_t* num_items);
fi_status fi_plan_prefix_members(const fi_plan* plan, const int32_t** members, int64_t* num_members);

/*
 * Copy the work list, merge nodes (with their arrival counters set to 0) and
 * page ids into the caller's device
 * workspace (asynchronous host-to-device copy on `stream` from a cached
 * page-locked staging block; the plan may be destroyed right after).
 * workspace must be 256-byte aligned and at least info.image_bytes long;
 * fi_decode_run needs info.workspace_bytes (it keeps its partial states in
 * the same buffer), fi_decode_run_noalloc only the image.
 * Call once per plan; the uploaded plan may then serve any number of
 * fi_decode_run calls (e.g. every layer of a step). Uploading is not meant
 * for stream capture: capture the runs, not the upload.
 */
fi_status fi_plan_upload(fi_plan* plan, void* workspace, size_t workspace_bytes,
                         fi_stream_t stream);

/*
 * Run decode attention for an uploaded plan on `stream`: one kernel launch.
 * Each work item attends over its chunk; an item of a request cut into
 * several chunks writes a partial (output, log-sum-exp) state and reports to
 * its merge node, and the item that completes a node merges that node's
 * children (see FI_NODE_*), up to the root which writes out/lse. No host
 * synchronisation; safe to capture in a HIP graph once uploaded. Calls that
 * use the same workspace must not overlap (the merge counters live there);
 * the kernel leaves every counter at 0 when it finishes.
 *
 * q        device [batch, num_qo_heads, head_dim], 16-byte aligned; fp32 for
 *          FI_DTYPE_F32, bf16 otherwise
 * k_pages  device [num_pool_pages, num_kv_heads, page_size, head_dim] of the
 *          plan's dtype (bytes for FI_DTYPE_FP8_E4M3)
 * v_pages  same shape and type as k_pages
 * out      device [batch, num_qo_heads, head_dim], same type as q (written)
 * lse      device float32 [batch, num_qo_heads] (written); may be NULL
 * sm_scale score scale; <= 0 selects 1/sqrt(head_dim)
 * workspace the buffer given to fi_plan_upload for this plan
 */
fi_status fi_decode_run(const fi_plan* plan, const void* q, const void* k_pages,
                        const void* v_pages, void* out, float* lse, float sm_scale,
                        void* workspace, size_t workspace_bytes, fi_stream_t stream);

/*
 * The run of a composed plan (fi_plan_create_composed; the other decode
 * runs refuse such a plan with FI_ERR_INVALID_ARG, and this one refuses any
 * other plan): the prefix tile kernel over the prefix cache, then the decode
 * kernel over the requests' own pages, their states merged per request.
 *
 * k_prefix, v_prefix  device bf16 [num_prefix_pool_pages, num_kv_heads,
 *          prefix_page_size, head_dim], 16-byte aligned; may be NULL when no
 *          request has a non-empty prefix
 * Other arguments, ownership, streams and errors as fi_decode_run.
 */
fi_status fi_decode_run_composed(const fi_plan* plan, const void* q, const void* k_pages,
                                 const void* v_pages, const void* k_prefix, const void* v_prefix,
                                 void* out, float* lse, float sm_scale, void* workspace,
                                 size_t workspace_bytes, fi_stream_t stream);

/*
 * For callers that cannot allocate device memory during the run (code under
 * stream capture, tight serving loops, harnesses that forbid hipMalloc):
 * fi_decode_run with its scratch -- the merge nodes' arrival counters and
 * the partial states of cut requests -- in a static device array of
 * FI_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends. The call allocates nothing: it clears the
 * counters with a small kernel and launches the run, both on `stream`,
 * which must belong to the current device.
 *
 * workspace: the buffer the plan was uploaded to (fi_plan_upload); it needs
 *            only info.image_bytes and is only read.
 * Other arguments as for fi_decode_run (unit K/V scales, no rotary
 * embedding).
 * Errors: FI_ERR_WORKSPACE when the plan's counters and partial states need
 * more than FI_NOALLOC_SCRATCH_BYTES (then use fi_decode_run with a
 * workspace), or when workspace_bytes < info.image_bytes; FI_ERR_STATE as
 * for fi_decode_run. Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (two streams, or two threads) race and give wrong
 * results; calls in one stream's order are safe.
 */
#define FI_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
fi_status fi_decode_run_noalloc(const fi_plan* plan, const void* q, const void* k_pages,
                                const void* v_pages, void* out, float* lse, float sm_scale,
                                const void* workspace, size_t workspace_bytes,
                                fi_stream_t stream);

/*
 * fi_decode_run with dequantisation scales: every K element counts as
 * k_scale times its stored value and every V element as v_scale times its
 * stored value (the scores are sm_scale * k_scale * q.k, the output is
 * v_scale times the weighted sum of stored V). Meant for FI_DTYPE_FP8_E4M3
 * plans; valid for every dtype. fi_decode_run is this call with both scales
 * 1. Scales must be finite and positive.
 */
fi_status fi_decode_run_scaled(const fi_plan* plan, const void* q, const void* k_pages,
                               const void* v_pages, float k_scale, float v_scale, void* out,
                               float* lse, float sm_scale, void* workspace,
                               size_t workspace_bytes, fi_stream_t stream);

/*
 * fi_decode_run for a K cache that holds keys before the rotary position
 * embedding, which the kernel applies while it reads them (explainer, JIT
 * section: RoPE is among the operations fused into the attention kernel).
 * Rotate-half convention: dims i and i + head_dim/2 form a pair turned by
 * the angle (pos / rope_scale) * rope_theta^(-2i / head_dim); token t of a
 * request (0-based, listed order) is at position t, the query at position
 * L_b - 1 (it is the request's newest token, whose K is already cached).
 * q is given before the embedding too. bf16 plans with head_dim 128 or 64
 * and FI_DTYPE_FP8_E4M3 plans (head_dim 128), with no shared-prefix items
 * (create the plan with opts.cascade = -1); else FI_ERR_UNSUPPORTED. rope_theta <= 0 selects
 * 10000, rope_scale <= 0 selects 1. Other arguments as fi_decode_run. This
 * is fi_decode_run_rope_scaled with both scales 1.
 */
fi_status fi_decode_run_rope(const fi_plan* plan, const void* q, const void* k_pages,
                             const void* v_pages, float rope_theta, float rope_scale, void* out,
                             float* lse, float sm_scale, void* workspace, size_t workspace_bytes,
                             fi_stream_t stream);

/*
 * fi_decode_run_rope over a quantised cache: K and V elements count as
 * k_scale and v_scale times their stored values, as in fi_decode_run_scaled
 * (the embedding turns the dequantised keys; a scale commutes with the
 * rotation). Scales must be finite and positive. Other arguments and limits
 * as fi_decode_run_rope.
 */
fi_status fi_decode_run_rope_scaled(const fi_plan* plan, const void* q, const void* k_pages,
                                    const void* v_pages, float k_scale, float v_scale,
                                    float rope_theta, float rope_scale, void* out, float* lse,
                                    float sm_scale, void* workspace, size_t workspace_bytes,
                                    fi_stream_t stream);

/*
 * Merge two attention states over disjoint token sets (the closed form of
 * softmax over a union): with M = max(s_a, s_b),
 *     s_out = M + ln(e^(s_a-M) + e^(s_b-M))
 *     v_out = (e^(s_a-M) v_a + e^(s_b-M) v_b) / e^(s_out-M).
 * A state with s = -inf (empty set) has weight 0; two such give v_out = 0,
 * s_out = -inf. The cut-and-merge of the explainer's load-balanced scheduler
 * needs exactly this combination of per-unit results.
 *
 * v_a, v_b, v_out  device [num_rows, head_dim] dtype, 16-byte aligned
 * s_a, s_b, s_out  device float32 [num_rows], natural-log LSE
 * head_dim         64 or 128 (128 for FI_DTYPE_FP8_E4M3); num_rows >= 0 (0 launches nothing)
 * v_out/s_out may alias v_a/s_a or v_b/s_b exactly (elementwise).
 */
fi_status fi_merge_states(fi_dtype dtype, const void* v_a, const float* s_a,
                          const void* v_b, const float* s_b, void* v_out, float* s_out,
                          int64_t num_rows, int32_t head_dim, fi_stream_t stream);

/* Free a plan (NULL is ignored). Host memory only; does not wait for the
 * device (an upload in flight keeps its own staging block). */
void fi_plan_destroy(fi_plan* plan);

/* ======================================================================
 * Prefill / append: several query tokens per request over the same paged /
 * BSR cache (explainer, section on where the attention bottleneck lies:
 * prefill attends all tokens of a prompt at once and is bound by
 * arithmetic, not memory).
 *
 * Request b has n_b = qo_indptr[b+1] - qo_indptr[b] query tokens, rows
 * qo_indptr[b] .. qo_indptr[b+1]-1 of q. They are the request's newest
 * tokens, already written to its pages: with L_b cached tokens, query i
 * (0-based) sits at position L_b - n_b + i and, with the causal mask,
 * attends the first L_b - n_b + i + 1 tokens (itself and everything
 * before); without it, all L_b. n_b = 1 is the decode step. For query row r
 * of request b and query head h (KV head h / G):
 *     out[r,h] = sum_t softmax(s)_t V[page_t, h/G, slot_t, :],
 *     lse[r,h] = ln sum_t exp(s_t),  s_t = sm_scale <q[r,h,:], K[...]>
 * over the attended tokens t; a query that attends no token (only possible
 * without the mask, for a request with no pages) gets out = 0, lse = -inf.
 *
 * Layout: q, out [N, num_qo_heads, head_dim] bf16 (N = qo_indptr[batch]),
 * lse [N, num_qo_heads] float32, K/V pages as for decode, bf16.
 * ====================================================================== */
typedef struct fi_prefill_plan fi_prefill_plan; /* opaque, host-owned */

/* Planner knobs. Zero selects the default for every field. */
typedef struct {
  int32_t num_cus;            /* compute units to balance over (default 256) */
  int32_t items_per_cu;       /* target work items per CU (default 2) */
  int32_t fixed_chunk_tokens; /* >0: cut KV ranges into chunks of exactly this
                                 many tokens (rounded up to whole pages, at
                                 most the chunk cap: FI_PREFILL_MAX_PAGES or
                                 FI_MLA_MAX_PAGES pages) */
  int32_t num_xcds;           /* L2 domains the dispatcher deals workgroups
                                 over in turn (default 8, MI355X's XCDs) */
  int32_t rope;               /* nonzero: a plan for fi_prefill_run_rope --
                                 tiles of FI_PREFILL_ROWS / 2 rows; needs
                                 FI_DTYPE_BF16, head_dim 128, G <= 128 and
                                 every request's queries among its cached
                                 tokens (n_b <= L_b, masked or not) */
} fi_prefill_opts;

typedef struct {
  int64_t num_items;          /* tiles x KV chunks */
  int64_t num_tiles;          /* (request, KV head, block of query tokens) */
  int64_t num_merges;         /* tiles cut into several KV chunks */
  int64_t num_partial_slots;  /* partial states of FI_PREFILL_ROWS rows each */
  int64_t workspace_bytes;    /* device workspace fi_prefill_plan_upload needs */
  int64_t total_qo_tokens;    /* N */
  int64_t total_kv_tokens;    /* sum of L_b */
  int64_t visible_pairs;      /* sum over query tokens of the tokens each attends */
  int32_t tokens_per_tile;    /* query tokens per tile: FI_PREFILL_ROWS / G */
  int32_t chunk_tokens;       /* longest KV chunk of an item */
  int32_t batch, num_qo_heads, num_kv_heads, head_dim, page_size, causal;
  int32_t dtype;              /* fi_dtype of the K/V pages */
  int32_t rope;               /* made with fi_prefill_opts.rope */
  int32_t mla;                /* made with fi_mla_plan_create: num_qo_heads is the
                                 head count, num_kv_heads 1, head_dim the latent
                                 width, head_dim_kpe the rotary-key width, and
                                 partial slots hold FI_MLA_ROWS rows */
  int32_t head_dim_kpe;       /* MLA plans; 0 otherwise */
} fi_prefill_info;

/*
 * Fields of one prefill work item (fi_prefill_plan_work_list). A tile is
 * FI_PREFILL_ROWS query rows (FI_PREFILL_ROWS / 2 in a rope plan) of one
 * request and KV head: row j is query
 * token j / G of the tile and query head KV_HEAD * G + j % G. An item
 * attends a tile over one chunk of the request's tokens; a tile whose
 * attended range exceeds one chunk is cut into several items whose partial
 * states the run merges (in the same launch: the chunk that arrives last
 * merges them all, in chunk order).
 */
enum {
  FI_QITEM_REQUEST = 0,
  FI_QITEM_KV_HEAD = 1,
  FI_QITEM_QO_ROW = 2,     /* row of q / out of the tile's first query token */
  FI_QITEM_NUM_QO = 3,     /* query tokens in the tile (rows = NUM_QO x G) */
  FI_QITEM_KV_BEGIN = 4,   /* first token of the chunk (request order, whole pages) */
  FI_QITEM_NUM_KV = 5,     /* tokens in the chunk; 0 only for a tile that attends nothing */
  FI_QITEM_VISIBLE = 6,    /* tokens the tile's first query attends; with the causal
                              mask query j of the tile attends VISIBLE + j */
  FI_QITEM_PAGE_BEGIN = 7, /* index into kv_indices of the chunk's first page */
  FI_QITEM_SLOT = 8,       /* -1: the item writes out / lse; else its partial slot */
  FI_QITEM_CHUNK = 9,      /* chunk number within the tile */
  FI_QITEM_Q_POS = 10,     /* position of the tile's first query token in its
                              request, L - n + (its index among the request's
                              queries); negative only for an unmasked request
                              with more queries than tokens (rope plans refuse
                              those) */
  FI_QITEM_HEAD_BEGIN = 11, /* MLA plans: first (query token, head) row of the
                              tile, counted token-major from the tile's first
                              query token (0 unless a token's heads span
                              several tiles); 0 in other plans */
  FI_QITEM_MERGE = 12,      /* index of the tile's merge (fi_prefill_plan_merges)
                              when the tile is cut, else -1 */
  FI_QITEM_STRIDE = 16,     /* int32 per item; fields past MERGE are 0 */
  FI_PREFILL_ROWS = 256,      /* query rows per tile */
  FI_MLA_ROWS = 32,           /* (query token, head) rows per MLA tile */
  FI_PREFILL_MAX_PAGES = 512, /* pages per prefill chunk at most, and never
                                 more than 2^20 tokens (256 pages of 4096) */
  FI_MLA_MAX_PAGES = 256      /* pages per MLA chunk at most */
};

/* Fields of one merge of a cut tile (fi_prefill_plan_merges): its chunks'
 * partial states sit in slots SLOT_BEGIN .. SLOT_BEGIN + NUM_CHUNKS - 1. */
enum {
  FI_QMERGE_QO_ROW = 0,
  FI_QMERGE_NUM_QO = 1,
  FI_QMERGE_KV_HEAD = 2,
  FI_QMERGE_SLOT_BEGIN = 3,
  FI_QMERGE_NUM_CHUNKS = 4,
  FI_QMERGE_HEAD_BEGIN = 5, /* MLA plans: as FI_QITEM_HEAD_BEGIN */
  FI_QMERGE_STRIDE = 8
};

/*
 * Build the work list of one prefill / append call. Host only.
 *
 * qo_indptr        host int32 [batch+1], qo_indptr[0] = 0, non-decreasing;
 *                  with causal != 0 every n_b <= L_b
 * kv_indptr, kv_indices, kv_last_page_len: the page table, as for
 *                  fi_plan_create (L_b tokens per request; the same array
 *                  lengths, which this call cannot see, are required)
 * num_qo_heads, num_kv_heads: G = num_qo_heads / num_kv_heads in
 *                  1 .. FI_PREFILL_ROWS (a tile holds FI_PREFILL_ROWS / G query
 *                  tokens; with G not dividing it the last rows are padding)
 * head_dim         64 or 128
 * page_size        1 .. 4096
 * dtype            of the K/V pages: FI_DTYPE_BF16, or FI_DTYPE_FP8_E4M3
 *                  (head_dim 128; run with fi_prefill_run_scaled); q and
 *                  out are bf16 either way
 * causal           nonzero: the causal mask above; 0: every query attends all
 * opts             may be NULL
 *
 * Tiles: each request's query tokens in blocks of FI_PREFILL_ROWS / G, per
 * KV head. A tile attends the tokens its last query sees; that range is cut
 * into chunks of C tokens (whole pages, at most FI_PREFILL_MAX_PAGES
 * pages and 2^20 tokens), C chosen so the items fill num_cus x items_per_cu
 * (never finer than 512 tokens) unless fixed_chunk_tokens is set.
 *
 * Order: every tile of one (request, KV head) reads the same K/V, so the
 * pairs are dealt to num_xcds bins, heaviest pair first into the least
 * loaded bin, and the bins are interleaved item by item: item i runs on L2
 * domain i mod num_xcds (the dispatcher hands workgroups to the XCDs in
 * turn) and the tiles of a pair share that domain's L2. Within a bin pairs
 * keep their dealing order and a pair's items go longest chunk first (ties
 * by query row, chunk).
 */
fi_status fi_prefill_plan_create(const int32_t* qo_indptr, const int32_t* kv_indptr,
                                 const int32_t* kv_indices, const int32_t* kv_last_page_len,
                                 int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t page_size, int64_t num_pool_pages,
                                 fi_dtype dtype, int32_t causal, const fi_prefill_opts* opts,
                                 fi_prefill_plan** out_plan);

fi_status fi_prefill_plan_get_info(const fi_prefill_plan* plan, fi_prefill_info* info);

/* Host views of the items (num_items * FI_QITEM_STRIDE int32, launch order)
 * and of the merges (num_merges * FI_QMERGE_STRIDE int32). */
fi_status fi_prefill_plan_work_list(const fi_prefill_plan* plan, const int32_t** items,
                                    int64_t* num_items);
fi_status fi_prefill_plan_merges(const fi_prefill_plan* plan, const int32_t** merges,
                                 int64_t* num_merges);

/* Copy items, merges and page ids into the caller's device workspace
 * (256-byte aligned, at least info.workspace_bytes), asynchronously on
 * `stream` through a cached page-locked staging block, as fi_plan_upload. */
fi_status fi_prefill_plan_upload(fi_prefill_plan* plan, void* workspace, size_t workspace_bytes,
                                 fi_stream_t stream);

/*
 * Run prefill / append attention for an uploaded plan on `stream`: one
 * launch of the tile kernel (matrix cores). A cut tile's chunks write
 * partial states to the workspace and count their arrival at the tile's
 * merge (a counter in the uploaded workspace image, 0 after the upload); the
 * chunk that arrives last merges them in chunk order, so the result does not
 * depend on which chunk finished last, and sets the counter back to 0. No
 * host synchronisation. Calls that use the same workspace must not overlap.
 *
 * q        device bf16 [N, num_qo_heads, head_dim], 16-byte aligned
 * k_pages, v_pages  device [num_pool_pages, num_kv_heads, page_size, head_dim]
 *          in the plan's dtype (bf16, or one byte per fp8 E4M3 code)
 * out      device bf16 [N, num_qo_heads, head_dim] (written)
 * lse      device float32 [N, num_qo_heads] (written); may be NULL
 * sm_scale score scale; <= 0 selects 1/sqrt(head_dim)
 */
fi_status fi_prefill_run(const fi_prefill_plan* plan, const void* q, const void* k_pages,
                         const void* v_pages, void* out, float* lse, float sm_scale,
                         void* workspace, size_t workspace_bytes, fi_stream_t stream);

/*
 * fi_prefill_run with K/V dequantisation scales, for an fp8 (E4M3) paged
 * cache as the JIT-specialisation section of the FlashInfer blog describes
 * for its decode and append kernels (K/V stored in 8 bits, scores and
 * outputs computed from the widened values): every K element counts as
 * k_scale times its stored value and every V element as v_scale times its
 * stored value, so the scores are sm_scale * k_scale * q.k and the output is
 * v_scale times the softmax-weighted sum of stored V. The codes are widened
 * to bf16 exactly on the way into the matrix cores; the products accumulate
 * in fp32. Valid for every plan dtype (fi_prefill_run is this call with both
 * scales 1). Scales must be finite and positive (else FI_ERR_INVALID_ARG).
 * Other arguments, ownership and errors as fi_prefill_run.
 */
fi_status fi_prefill_run_scaled(const fi_prefill_plan* plan, const void* q, const void* k_pages,
                                const void* v_pages, float k_scale, float v_scale, void* out,
                                float* lse, float sm_scale, void* workspace,
                                size_t workspace_bytes, fi_stream_t stream);

/*
 * Prefill / append over a K cache that holds keys before the rotary
 * position embedding (explainer's JIT section: RoPE fused into the attention
 * kernel), for a plan made with fi_prefill_opts.rope (the other prefill runs
 * refuse such a plan, and this one any other plan, with FI_ERR_INVALID_ARG).
 * Rotate-half pairs (dims i and i + 64) turn by (pos / rope_scale) *
 * rope_theta^(-2i / 128); token t of a request sits at position t and its
 * query i of n at L - n + i (q arrives before the embedding, as K). The
 * kernel turns each K block once per tile in LDS and each query row once,
 * both in fp32 from exact phases, and multiplies them as hi + lo bf16
 * parts (S = Kh.Qh + Kh.Ql + Kl.Qh). rope_theta <= 0 selects 10000,
 * rope_scale <= 0 selects 1. Other arguments, ownership and errors as
 * fi_prefill_run (bf16 q, K, V, out).
 */
fi_status fi_prefill_run_rope(const fi_prefill_plan* plan, const void* q, const void* k_pages,
                              const void* v_pages, float rope_theta, float rope_scale, void* out,
                              float* lse, float sm_scale, void* workspace,
                              size_t workspace_bytes, fi_stream_t stream);

/* ======================================================================
 * Multi-head latent attention (MLA) over a paged latent cache (FlashInfer
 * 0.6.17 release write-up, llm-wiki.hwlabs.dev, section 2 on Blackwell and
 * Kimi K3 MLA support: MLA caches a compressed latent vector per token
 * instead of per-head K and V; restoring K/V by up-projection and writing it
 * to shared memory before attention was the bottleneck, which the kernel
 * removes by packing query-token rows and query-head rows into one tile;
 * head counts that are not powers of two and several (speculative) query
 * tokens per request are supported).
 *
 * Attention runs in the latent space (the up-projections folded into the
 * query and the output by the caller). Token t of a request caches a latent
 * c_t (head_dim_ckv = 512) and a rotary key k_t (head_dim_kpe = 64, stored
 * rotated). Query token i of request b and head h bring q_nope[r,h] (512,
 * the no-rotary query part already multiplied by the head's key
 * up-projection) and q_pe[r,h] (64, rotated), r = qo_indptr[b] + i. Query
 * tokens are the request's newest cached tokens, with the causal mask as for
 * prefill (query i of n over L tokens attends the first L - n + i + 1):
 *     s_t = sm_scale (<q_nope[r,h], c_t> + <q_pe[r,h], k_t>)
 *     out[r,h] = sum_t softmax(s)_t c_t,   lse[r,h] = ln sum_t exp(s_t)
 * Every head reads the same cache rows, so one latent row loaded serves all
 * heads and query tokens of the request.
 *
 * Layout: q_nope [N, num_heads, 512], q_pe [N, num_heads, 64], out [N,
 * num_heads, 512], all bf16 (N = qo_indptr[batch]); lse [N, num_heads]
 * float32; ckv_pages [num_pool_pages, page_size, 512] and kpe_pages
 * [num_pool_pages, page_size, 64] bf16, addressed by one page table.
 * ====================================================================== */

/*
 * Build the work list of one MLA call; the plan is a fi_prefill_plan (get
 * its info, work list and merges, upload it and destroy it with the
 * fi_prefill_plan_* calls; fi_prefill_run* refuse it and fi_mla_run refuses
 * other plans). Host only.
 *
 * qo_indptr, kv_indptr, kv_indices, kv_last_page_len, page_size,
 * num_pool_pages, causal, opts: as for fi_prefill_plan_create (opts.rope
 * must be 0)
 * num_heads        1 .. 4096 query heads (any count)
 * head_dim_ckv     512; head_dim_kpe 64 (else FI_ERR_UNSUPPORTED)
 *
 * Tiles are FI_MLA_ROWS (query token, head) rows of one request, token-major:
 * FI_MLA_ROWS / num_heads whole query tokens when num_heads <= FI_MLA_ROWS,
 * else one query token's heads HEAD_BEGIN .. HEAD_BEGIN + FI_MLA_ROWS - 1.
 * Each tile's range is cut into chunks of C tokens (whole pages, at most
 * FI_MLA_MAX_PAGES pages; C fills num_cus x items_per_cu, default 2, and
 * is never below 1024 tokens) unless fixed_chunk_tokens is set. Every tile of
 * a request reads the same latent rows, so a request's items share an L2
 * domain as a prefill pair's do, and within it the tiles of one chunk are
 * adjacent (they run side by side and the later ones find the rows in L2).
 */
fi_status fi_mla_plan_create(const int32_t* qo_indptr, const int32_t* kv_indptr,
                             const int32_t* kv_indices, const int32_t* kv_last_page_len,
                             int32_t batch, int32_t num_heads, int32_t head_dim_ckv,
                             int32_t head_dim_kpe, int32_t page_size, int64_t num_pool_pages,
                             int32_t causal, const fi_prefill_opts* opts,
                             fi_prefill_plan** out_plan);

/*
 * Run MLA for an uploaded plan on `stream`: one launch of the tile kernel
 * (matrix cores). A cut tile's chunks write partial states to the
 * workspace and count their arrival at the tile's merge (a counter in the
 * uploaded workspace image, 0 after the upload); the chunk that arrives last
 * merges the partials in chunk order, so the result does not depend on
 * which chunk finished last, and sets the counter back to 0. No host
 * synchronisation; calls that use the same workspace must not overlap.
 *
 * q_nope, q_pe, out, lse, ckv_pages, kpe_pages: device buffers in the layout
 *          above, 16-byte aligned; lse may be NULL
 * sm_scale the model's score scale (1 / sqrt of the query/key head width
 *          before absorption, e.g. 1/sqrt(192)); must be finite and
 *          positive (the latent width does not define it)
 * workspace, workspace_bytes, stream: as fi_prefill_run
 *
 * Scores and the weighted latent sum run on the matrix cores in bf16 with
 * fp32 accumulation; the softmax weights are multiplied as hi + lo bf16
 * parts. Errors: FI_ERR_INVALID_ARG (NULL pointer, not an MLA plan, bad
 * scale), FI_ERR_WORKSPACE / FI_ERR_STATE as fi_prefill_run, FI_ERR_HIP.
 */
fi_status fi_mla_run(const fi_prefill_plan* plan, const void* q_nope, const void* q_pe,
                     const void* ckv_pages, const void* kpe_pages, void* out, float* lse,
                     float sm_scale, void* workspace, size_t workspace_bytes, fi_stream_t stream);

/* Free a prefill plan (NULL is ignored); host memory only, no wait. */
void fi_prefill_plan_destroy(fi_prefill_plan* plan);

/* Message of the last failed call on this thread ("" if none). */
const char* fi_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FI_BSR_H */
