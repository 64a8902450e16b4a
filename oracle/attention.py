"""Float64 CPU oracle for batched decode attention over a paged / BSR KV cache.

TEST INFRASTRUCTURE ONLY. Nothing in the library calls this module: only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
import it. It shares no code with the HIP path.

What it computes, and where that comes from:

* FlashInfer paper explainer ("FlashInfer: Block-Sparse KV 캐시로 어텐션 병목을
  해소하다", visionhong.com), section "where the real bottleneck of attention
  is": in decode, each new token attends over the whole KV history of its
  request.
* Same page, section on the Block-Sparse format: the KV cache is a block-sparse
  matrix; a block is a run of consecutive tokens and metadata marks which
  blocks are active; paged, dense and sparse caches are all this format.
  Inactive blocks are skipped. Reading: a request's KV history is exactly the
  tokens of the blocks it lists, in listed order; a block not listed does not
  exist for that request.
* FlashInfer 0.6.17 release write-up (llm-wiki.hwlabs.dev), section 5 on JIT
  warm-up: the attention call is parameterised by num_heads, num_kv_heads (GQA)
  and head_dim, and sm_scale=None means the default scale. Reading: the default
  is 1/sqrt(head_dim); consecutive query heads share a KV head (query head h
  reads KV head floor(h / G), G = num_heads / num_kv_heads).
* Same explainer, benchmark section: the load-balanced scheduler cuts long
  sequences into smaller work units. Cutting one softmax in pieces needs each
  piece's (output, log-sum-exp) state and a merge; the merge below is the
  closed form of softmax over a disjoint union of token sets.

* Same explainer, JIT section: quantisation / dequantisation around attention
  is fused into the attention kernel. Reading: with a quantised KV cache the
  method computes plain attention over the dequantised values, K = k_scale *
  code and V = v_scale * code; ``dequantize_e4m3`` decodes OCP FP8 E4M3 codes
  from the format's definition.

* Same explainer, JIT section: rotary position embedding (RoPE) is one of
  the operations fused into the attention kernel. Reading (the pages name no
  variant): the K cache holds keys before the embedding and the kernel
  rotates q and K at their positions, in the rotate-half convention of the
  Llama models the workloads are shaped after: dims i and i + d/2 form a
  pair turned by the angle (position / rope_scale) * rope_theta^(-2i/d).
  Token t of a request (0-based, listed order) sits at position t; the
  decode query is the newest token, position L - 1.
* Same explainer, Block-Sparse section, on composable formats: when many
  requests share one system prompt, the prefix's KV is stored once and only
  each request's own KV is kept per request, the decomposition being
  expressed with different block sizes. Reading: a request's KV history is
  its prefix's tokens (from a second cache with its own block size) followed
  by its own tokens (from the paged cache); attention runs over that whole
  history exactly as over one cache.
* Same explainer, section on where the attention bottleneck lies: prefill
  attends every token of the prompt at once (and is bound by arithmetic, not
  memory). Reading (the pages give no formula): the query tokens of a
  request are its newest tokens, already in the cache, and each attends
  causally, to itself and every earlier token. A request holding L tokens
  with n query tokens gives query i (0-based) the first L - n + i + 1 tokens;
  n = 1 is the decode step above. Without the causal mask every query sees
  all L tokens. With the rotary embedding the queries keep those
  positions: query i sits at L - n + i (so n <= L is required).
* FlashInfer 0.6.17 release write-up, section 2 on Blackwell / Kimi K3 MLA
  support: multi-head latent attention (MLA, from DeepSeek-V2) caches one
  compressed latent vector per token in place of per-head K and V; attention
  needs the up-projection that turns latents into K and V, and writing the
  restored K/V to shared memory first was the bottleneck the new kernel
  removes by packing query-token rows and query-head rows into one tile; head
  counts need not be powers of two and a request may carry several
  (speculative) query tokens. Reading: the up-projections are folded into
  the query and the output (the absorbed form), so the method attends in the
  latent space. Token t of a request caches a latent c_t (d_c = 512) and a
  rotary key k_t (d_r = 64, stored after its rotation); query token i, head h
  brings q_nope (its no-rotary part already multiplied by that head's key
  up-projection, d_c) and q_pe (its rotary part, already rotated, d_r). The
  score of token t is sm_scale (q_nope . c_t + q_pe . k_t), the output is
  the softmax-weighted sum of the latents c_t (the caller applies the value
  up-projection), and every head reads the same cache: multi-query
  attention with key [c_t, k_t] and value c_t. The query tokens of a request
  are its newest cached tokens with the causal mask, as for prefill. The
  scale is the model's (1 / sqrt(d_nope + d_r) before absorption, not the
  latent width), so the caller passes it.

Everything is float64. The exact result of the method is plain softmax
attention over the listed tokens, so the oracle is that definition, written
out with a library matmul as its only primitive.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

NEG_INF = -math.inf


def kv_head_of(h: int, group_size: int) -> int:
    """Query head h reads KV head floor(h / G): consecutive query heads form
    one GQA group."""
    return h // group_size


def request_tokens(kv_indptr, kv_indices, last_page_len, page_size, b) -> List[Tuple[int, int]]:
    """(physical page, slot) of every token of request b, in logical order.

    The request lists pages kv_indices[kv_indptr[b] : kv_indptr[b+1]]; every
    listed page is full except the last, which holds last_page_len[b] tokens.
    """
    start, end = int(kv_indptr[b]), int(kv_indptr[b + 1])
    toks = []
    for j in range(start, end):
        n = page_size if j < end - 1 else int(last_page_len[b])
        page = int(kv_indices[j])
        for slot in range(n):
            toks.append((page, slot))
    return toks


def attend(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float):
    """Softmax attention of query rows over one token set.

    q_rows [G, d], K [T, d], V [T, d_v] (float64). Returns (O [G, d_v], LSE [G])
    where s_t = sm_scale * q . k_t, O = sum_t softmax(s)_t v_t and
    LSE = ln sum_t exp(s_t) (natural log of the scaled scores).
    An empty token set gives O = 0 and LSE = -inf.
    """
    G = q_rows.shape[0]
    if K.shape[0] == 0:
        return np.zeros((G, V.shape[1])), np.full(G, NEG_INF)
    s = sm_scale * (q_rows @ K.T)              # [G, T]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    den = w.sum(axis=1)
    o = (w @ V) / den[:, None]
    lse = m[:, 0] + np.log(den)
    return o, lse


def gather_kv(k_pool, v_pool, tokens, kv_head):
    """Dense [T, d] K and V of one request for one KV head, in token order."""
    if not tokens:
        d = k_pool.shape[-1]
        return np.zeros((0, d)), np.zeros((0, d))
    pages = np.array([p for p, _ in tokens])
    slots = np.array([s for _, s in tokens])
    K = np.asarray(k_pool[pages, kv_head, slots, :], dtype=np.float64)
    V = np.asarray(v_pool[pages, kv_head, slots, :], dtype=np.float64)
    return K, V


def decode_attention(q, k_pool, v_pool, kv_indptr, kv_indices, last_page_len, sm_scale=None):
    """Batched GQA decode attention over a paged / BSR KV cache.

    q [B, H_q, d]; k_pool, v_pool [num_pages, H_kv, P, d]; page table in BSR
    form (kv_indptr [B+1], kv_indices, last_page_len [B]). Returns float64
    O [B, H_q, d] and LSE [B, H_q]. sm_scale None means 1/sqrt(d).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv, P = k_pool.shape[1], k_pool.shape[2]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    O = np.zeros((B, Hq, d))
    LSE = np.full((B, Hq), NEG_INF)
    for b in range(B):
        toks = request_tokens(kv_indptr, kv_indices, last_page_len, P, b)
        for kvh in range(Hkv):
            heads = [h for h in range(Hq) if kv_head_of(h, G) == kvh]
            K, V = gather_kv(k_pool, v_pool, toks, kvh)
            o, lse = attend(q[b, heads, :], K, V, sm_scale)
            O[b, heads, :] = o
            LSE[b, heads] = lse
    return O, LSE


def decode_attention_composed(q, k_pool, v_pool, kv_indptr, kv_indices, last_page_len,
                              k_prefix, v_prefix, prefix_indptr, prefix_indices,
                              prefix_last_page_len, prefix_of, sm_scale=None):
    """Decode attention over composed formats: request b attends the tokens
    of prefix prefix_of[b] (none if -1), held in k_prefix / v_prefix
    [num_prefix_pages, H_kv, P_prefix, d] with page table (prefix_indptr,
    prefix_indices, prefix_last_page_len), followed by its own tokens in the
    paged cache (k_pool, v_pool, kv_indptr, kv_indices, last_page_len).
    Returns float64 O [B, H_q, d] and LSE [B, H_q]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv, P = k_pool.shape[1], k_pool.shape[2]
    Pp = k_prefix.shape[2]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    O = np.zeros((B, Hq, d))
    LSE = np.full((B, Hq), NEG_INF)
    for b in range(B):
        own = request_tokens(kv_indptr, kv_indices, last_page_len, P, b)
        g = int(prefix_of[b])
        pre = (request_tokens(prefix_indptr, prefix_indices, prefix_last_page_len, Pp, g)
               if g >= 0 else [])
        for kvh in range(Hkv):
            heads = [h for h in range(Hq) if kv_head_of(h, G) == kvh]
            Kp, Vp = gather_kv(k_prefix, v_prefix, pre, kvh)
            Ko, Vo = gather_kv(k_pool, v_pool, own, kvh)
            o, lse = attend(q[b, heads, :], np.concatenate([Kp, Ko]), np.concatenate([Vp, Vo]),
                            sm_scale)
            O[b, heads, :] = o
            LSE[b, heads] = lse
    return O, LSE


def rope_angles(head_dim: int, positions, theta: float = 1e4, scale: float = 1.0):
    """Rotation angle of every dim pair at every position: array
    [len(positions), head_dim / 2], (pos / scale) * theta^(-2i / head_dim)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    pos = np.asarray(positions, dtype=np.float64).reshape(-1, 1)
    return (pos / scale) * inv_freq[None, :]


def apply_rope(x, positions, theta: float = 1e4, scale: float = 1.0):
    """Rotate-half rotary embedding of rows x [n, d] (row j at positions[j]):
    with x = (x1, x2) split at d/2 and angle a, x1' = x1 cos a - x2 sin a and
    x2' = x2 cos a + x1 sin a."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a = rope_angles(d, positions, theta, scale)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[:, :d // 2], x[:, d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=1)


def rope_query_position(kv_len: int) -> int:
    """The decode query is the request's newest token: position L - 1 (0 for
    an empty request, which attends nothing anyway)."""
    return max(kv_len - 1, 0)


def decode_attention_rope(q, k_pool, v_pool, kv_indptr, kv_indices, last_page_len, sm_scale=None,
                          theta: float = 1e4, scale: float = 1.0):
    """decode_attention over a K cache that holds keys before the rotary
    embedding: token t of request b is rotated at position t, the query at
    position L_b - 1, then plain attention. Returns float64 O [B, H_q, d]
    and LSE [B, H_q]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv, P = k_pool.shape[1], k_pool.shape[2]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    O = np.zeros((B, Hq, d))
    LSE = np.full((B, Hq), NEG_INF)
    for b in range(B):
        toks = request_tokens(kv_indptr, kv_indices, last_page_len, P, b)
        L = len(toks)
        for kvh in range(Hkv):
            heads = [h for h in range(Hq) if kv_head_of(h, G) == kvh]
            K, V = gather_kv(k_pool, v_pool, toks, kvh)
            if L:
                K = apply_rope(K, np.arange(L), theta, scale)
            qr = apply_rope(q[b, heads, :], [rope_query_position(L)] * len(heads), theta, scale)
            o, lse = attend(qr, K, V, sm_scale)
            O[b, heads, :] = o
            LSE[b, heads] = lse
    return O, LSE


def visible_tokens(kv_len: int, qo_len: int, i: int, causal: bool) -> int:
    """Tokens of a request holding kv_len tokens that its query token i of
    qo_len (0-based) attends: causally the first kv_len - qo_len + i + 1 (the
    queries are the newest tokens), else all kv_len; never below 0."""
    if not causal:
        return kv_len
    return max(0, kv_len - qo_len + i + 1)


def prefill_attention(q, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices, last_page_len,
                      causal=True, sm_scale=None):
    """Batched GQA attention of several query tokens per request (prefill,
    or a chunk appended to a history) over a paged / BSR KV cache.

    q [N, H_q, d]: request b's query tokens are rows qo_indptr[b] ..
    qo_indptr[b+1]-1, in token order. k_pool, v_pool and the page table are
    as for decode_attention. Query token i of request b attends the first
    visible_tokens(L_b, n_b, i, causal) tokens of the request. Returns float64
    O [N, H_q, d] and LSE [N, H_q] (natural log); a query that sees no token
    gets O = 0 and LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    N, Hq, d = q.shape
    Hkv, P = k_pool.shape[1], k_pool.shape[2]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    O = np.zeros((N, Hq, d))
    LSE = np.full((N, Hq), NEG_INF)
    B = len(qo_indptr) - 1
    for b in range(B):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        n = q1 - q0
        if n == 0:
            continue
        toks = request_tokens(kv_indptr, kv_indices, last_page_len, P, b)
        L = len(toks)
        for kvh in range(Hkv):
            heads = [h for h in range(Hq) if kv_head_of(h, G) == kvh]
            K, V = gather_kv(k_pool, v_pool, toks, kvh)
            for i in range(n):
                c = visible_tokens(L, n, i, causal)
                o, lse = attend(q[q0 + i, heads, :], K[:c], V[:c], sm_scale)
                O[q0 + i, heads, :] = o
                LSE[q0 + i, heads] = lse
    return O, LSE


def prefill_query_position(kv_len: int, qo_len: int, i: int) -> int:
    """Query token i of qo_len is one of the request's newest tokens, all of
    them cached: its position is kv_len - qo_len + i (masked or not)."""
    return kv_len - qo_len + i


def prefill_attention_rope(q, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices, last_page_len,
                           causal=True, sm_scale=None, theta: float = 1e4, scale: float = 1.0):
    """prefill_attention over a K cache that holds keys before the rotary
    embedding: token t of request b is rotated at position t and its query
    token i at prefill_query_position(L_b, n_b, i), then the same masked
    attention. Every request's queries must be cached tokens (n_b <= L_b).
    Returns float64 O [N, H_q, d] and LSE [N, H_q]."""
    q = np.asarray(q, dtype=np.float64)
    N, Hq, d = q.shape
    Hkv, P = k_pool.shape[1], k_pool.shape[2]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    O = np.zeros((N, Hq, d))
    LSE = np.full((N, Hq), NEG_INF)
    for b in range(len(qo_indptr) - 1):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        n = q1 - q0
        if n == 0:
            continue
        toks = request_tokens(kv_indptr, kv_indices, last_page_len, P, b)
        L = len(toks)
        if n > L:
            raise ValueError("the queries of a request must be cached tokens")
        for kvh in range(Hkv):
            heads = [h for h in range(Hq) if kv_head_of(h, G) == kvh]
            K, V = gather_kv(k_pool, v_pool, toks, kvh)
            K = apply_rope(K, np.arange(L), theta, scale)
            for i in range(n):
                c = visible_tokens(L, n, i, causal)
                pos = prefill_query_position(L, n, i)
                qr = apply_rope(q[q0 + i, heads, :], [pos] * len(heads), theta, scale)
                o, lse = attend(qr, K[:c], V[:c], sm_scale)
                O[q0 + i, heads, :] = o
                LSE[q0 + i, heads] = lse
    return O, LSE


def gather_latent(ckv_pool, kpe_pool, tokens):
    """Dense [T, d_c] latents and [T, d_r] rotary keys of one request, in
    token order."""
    if not tokens:
        return np.zeros((0, ckv_pool.shape[-1])), np.zeros((0, kpe_pool.shape[-1]))
    pages = np.array([p for p, _ in tokens])
    slots = np.array([s for _, s in tokens])
    return (np.asarray(ckv_pool[pages, slots, :], dtype=np.float64),
            np.asarray(kpe_pool[pages, slots, :], dtype=np.float64))


def mla_attention(q_nope, q_pe, ckv_pool, kpe_pool, qo_indptr, kv_indptr, kv_indices,
                  last_page_len, sm_scale, causal=True):
    """Multi-head latent attention in the latent space over a paged cache.

    q_nope [N, H, d_c], q_pe [N, H, d_r]: request b's query tokens are rows
    qo_indptr[b] .. qo_indptr[b+1]-1. ckv_pool [pages, P, d_c] and kpe_pool
    [pages, P, d_r] share the page table (kv_indptr, kv_indices,
    last_page_len, as for decode_attention). Query token i of request b
    attends the first visible_tokens(L_b, n_b, i, causal) tokens with score
    sm_scale (q_nope . c_t + q_pe . k_t). Returns float64 O [N, H, d_c] (the
    weighted sum of latents) and LSE [N, H] (natural log); a query that sees
    no token gets O = 0 and LSE = -inf.
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    N, H, dc = q_nope.shape
    P = ckv_pool.shape[1]
    O = np.zeros((N, H, dc))
    LSE = np.full((N, H), NEG_INF)
    for b in range(len(qo_indptr) - 1):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        n = q1 - q0
        if n == 0:
            continue
        toks = request_tokens(kv_indptr, kv_indices, last_page_len, P, b)
        L = len(toks)
        C, R = gather_latent(ckv_pool, kpe_pool, toks)
        K = np.concatenate([C, R], axis=1)  # the key every head reads
        for i in range(n):
            c = visible_tokens(L, n, i, causal)
            rows = np.concatenate([q_nope[q0 + i], q_pe[q0 + i]], axis=1)  # [H, d_c + d_r]
            o, lse = attend(rows, K[:c], C[:c], sm_scale)
            O[q0 + i] = o
            LSE[q0 + i] = lse
    return O, LSE


# ------------------------------------------------------------------ merging
def merge_states(v_a, s_a, v_b, s_b):
    """Merge two attention states over disjoint token sets A and B.

    With e^{s} the softmax denominator of each set, the union has
    s = ln(e^{s_a} + e^{s_b}) and v = (e^{s_a} v_a + e^{s_b} v_b) / e^{s}.
    Evaluated relative to M = max(s_a, s_b). A state with s = -inf (empty set)
    has weight zero; two empty states give v = 0, s = -inf.
    v_* [..., d], s_* [...].
    """
    v_a = np.asarray(v_a, dtype=np.float64)
    v_b = np.asarray(v_b, dtype=np.float64)
    s_a = np.asarray(s_a, dtype=np.float64)
    s_b = np.asarray(s_b, dtype=np.float64)
    M = np.maximum(s_a, s_b)
    both_empty = np.isneginf(M)
    Ms = np.where(both_empty, 0.0, M)
    w_a = np.where(np.isneginf(s_a), 0.0, np.exp(np.where(np.isneginf(s_a), 0.0, s_a - Ms)))
    w_b = np.where(np.isneginf(s_b), 0.0, np.exp(np.where(np.isneginf(s_b), 0.0, s_b - Ms)))
    den = w_a + w_b
    safe = np.where(both_empty, 1.0, den)
    v = (w_a[..., None] * v_a + w_b[..., None] * v_b) / safe[..., None]
    v = np.where(both_empty[..., None], 0.0, v)
    s = np.where(both_empty, NEG_INF, Ms + np.log(safe))
    return v, s


def merge_many(vs: Sequence[np.ndarray], ss: Sequence[np.ndarray]):
    """Merge any number of states (folds merge_states left to right)."""
    if len(vs) == 0:
        raise ValueError("merge_many needs at least one state")
    v, s = np.asarray(vs[0], dtype=np.float64), np.asarray(ss[0], dtype=np.float64)
    for v2, s2 in zip(vs[1:], ss[1:]):
        v, s = merge_states(v, s, v2, s2)
    return v, s


# ------------------------------------------------------- bfloat16 rounding
def _bf16_step(v, up: bool):
    """Adjacent bfloat16 value above (up) or below a bfloat16 value v."""
    bits = np.asarray(v, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.int64)
    neg = (bits >> 31) & 1
    mag = bits & 0x7FFFFFFF
    zero = mag == 0
    # away from zero grows the magnitude: upward for v > 0, downward for v < 0
    away = (neg == 0) == up
    new = np.where(away, bits + 0x10000, bits - 0x10000)
    new = np.where(zero, 0x10000 if up else (0x80000000 | 0x10000), new)
    return new.astype(np.uint32).view(np.float32).astype(np.float64)


def bf16_neighbors(x):
    """The two bfloat16 values that bracket each finite float64 x
    (lo <= x <= hi); lo == hi exactly when x is a bfloat16 value."""
    x = np.asarray(x, dtype=np.float64)
    # float32 rounding is monotone and every bfloat16 value is a float32 value,
    # so x32 stays inside x's bfloat16 bracket (possibly on its upper end).
    x32 = x.astype(np.float32)
    t = (x32.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    lo = np.where(t <= x, t, _bf16_step(t, up=False))
    hi = np.where(lo == x, lo, _bf16_step(lo, up=True))
    return lo, hi


def round_bf16_rne(x):
    """Round float64 to the nearest bfloat16, ties to even mantissa, in one
    step from float64 (no intermediate float32 rounding)."""
    x = np.asarray(x, dtype=np.float64)
    lo, hi = bf16_neighbors(x)
    dlo, dhi = x - lo, hi - x  # exact: both are within one bf16 ulp of x
    lo_even = ((lo.astype(np.float32).view(np.uint32) >> 16) & 1) == 0
    pick_lo = (dlo < dhi) | ((dlo == dhi) & lo_even)
    return np.where(pick_lo, lo, hi)


def dequantize_e4m3(codes, scale: float = 1.0) -> np.ndarray:
    """OCP FP8 E4M3 (E4M3FN) codes (uint8) to float64, times ``scale``.

    The format: bit 7 sign; bits 6..3 exponent e with bias 7; bits 2..0
    mantissa m. e = 0 is subnormal, (m / 8) * 2^-6; otherwise (1 + m / 8) *
    2^(e - 7). There are no infinities; e = 15 with m = 7 is NaN, so the
    largest finite magnitude is 1.75 * 2^8 = 448."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag * scale
    return np.where((e == 15) & (m == 7), np.nan, out)
