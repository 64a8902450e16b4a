"""GPU parity of prefill / append attention: the HIP tile kernel (which also
merges cut tiles) through the C ABI against the float64 oracle.

Small ragged cases cover both head sizes, GQA groups 1..8 and one that is
not a power of two, page sizes 1..64, causal and unmasked, single-chunk
tiles (direct output) and cut tiles (forced chunk lengths, in-kernel merge),
requests with no queries and an unmasked request with no pages, over bf16
and fp8 (E4M3, dequantisation scales) caches. The full-size workloads run
with the plan bench.py times and are checked on every output element.
"""
import time

import numpy as np
import pytest
import torch

import block_sparse_kv_bsr_amd as fb
import oracle.attention as oa
from block_sparse_kv_bsr_amd.workloads import random_prefill_workload, workload
from tests.parity import compare, prefill_request

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fb.lib()


def log(*a):
    print(*a, flush=True)


def make_plan(w, **kw):
    return fb.prefill_plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len,
                           w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                           w.num_pool_pages, causal=w.causal, dtype=w.dtype,
                           rope=bool(w.rope_theta), **kw)


def oracle(w, qh, kh, vh, qo, ip, ix, lp):
    if w.rope_theta:
        return oa.prefill_attention_rope(qh, kh, vh, qo, ip, ix, lp, w.causal, w.sm_scale,
                                         w.rope_theta, w.rope_scale)
    return oa.prefill_attention(qh, kh, vh, qo, ip, ix, lp, w.causal, w.sm_scale)


def host_kv(w, k, v):
    """The cache as the oracle reads it: bf16 widened exactly, fp8 codes
    decoded and multiplied by the dequantisation scales."""
    if w.dtype == "fp8":
        return (oa.dequantize_e4m3(k.view(torch.uint8).cpu().numpy(), w.k_scale),
                oa.dequantize_e4m3(v.view(torch.uint8).cpu().numpy(), w.v_scale))
    return k.double().cpu().numpy(), v.double().cpu().numpy()


def run(w, q, k, v, p, **kw):
    return fb.prefill(q, k, v, p, k_scale=w.k_scale, v_scale=w.v_scale,
                      rope_theta=w.rope_theta or None, rope_scale=w.rope_scale, **kw)


def run_case(w, what, **opts):
    log(f"[case] {what} B={w.batch} N={w.num_qo_tokens} Hq={w.num_qo_heads} "
        f"Hkv={w.num_kv_heads} d={w.head_dim} P={w.page_size} causal={w.causal} "
        f"kv={w.dtype} rope={w.rope_theta} opts={opts}")
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = make_plan(w, **opts)
    out, lse = run(w, q, k, v, p)
    torch.cuda.synchronize()
    t0 = time.time()
    qh = q.double().cpu().numpy()
    kh, vh = host_kv(w, k, v)
    O, LSE = oracle(w, qh, kh, vh, w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len)
    stats = compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True, what)
    log(f"[ok] {what} items={p.info['num_items']} merges={p.info['num_merges']} "
        f"oracle {time.time() - t0:.1f}s {stats}")
    return p, (q, k, v), (out, lse)


CASES = [
    # seed, B, maxL, Hq, Hkv, d, P, causal, max_qo, fixed_chunk
    (1, 4, 300, 8, 2, 64, 16, True, None, 0),
    (2, 3, 200, 4, 4, 64, 4, True, None, 32),
    (3, 5, 150, 16, 2, 128, 16, True, 40, 48),
    (4, 3, 90, 4, 1, 64, 1, False, None, 7),
    (5, 4, 260, 8, 2, 128, 64, True, 1, 0),
    (6, 2, 500, 12, 2, 64, 16, True, None, 16),
    (7, 3, 700, 32, 8, 128, 16, True, None, 0),
    (8, 3, 700, 32, 8, 128, 16, True, None, 128),
    (9, 4, 333, 8, 8, 128, 3, False, 200, 0),
    (10, 2, 1000, 4, 1, 128, 64, True, 300, 192),
    (11, 2, 1500, 8, 2, 128, 1, True, None, 512),  # 512 one-token pages per chunk: the whole id window
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_prefill_small(case):
    seed, B, L, Hq, Hkv, d, P, causal, max_qo, fixed = case
    w = random_prefill_workload(seed, B, L, Hq, Hkv, d, P, causal=causal, max_qo=max_qo)
    p, _, _ = run_case(w, f"prefill seed{seed}", fixed_chunk_tokens=fixed)
    if fixed:
        assert p.info["num_merges"] > 0


# fp8 (E4M3) K/V, head_dim 128: groups 1..8 and 6, page sizes 1..64, causal
# and unmasked, direct output and cut tiles
FP8_CASES = [
    # seed, B, maxL, Hq, Hkv, P, causal, max_qo, fixed_chunk
    (41, 4, 300, 8, 2, 16, True, None, 0),
    (42, 3, 700, 32, 8, 16, True, None, 128),
    (43, 3, 90, 4, 4, 1, False, None, 7),
    (44, 2, 1000, 8, 1, 64, True, 300, 192),
    (45, 3, 333, 12, 2, 3, False, 200, 0),
]


@pytest.mark.parametrize("case", FP8_CASES, ids=lambda c: f"seed{c[0]}")
def test_prefill_fp8_small(case):
    seed, B, L, Hq, Hkv, P, causal, max_qo, fixed = case
    w = random_prefill_workload(seed, B, L, Hq, Hkv, 128, P, causal=causal, max_qo=max_qo,
                                dtype="fp8")
    p, _, _ = run_case(w, f"fp8 prefill seed{seed}", fixed_chunk_tokens=fixed)
    assert p.info["dtype"] == fb.FI_DTYPE_FP8_E4M3
    if fixed:
        assert p.info["num_merges"] > 0


def test_prefill_fp8_whole_prompts_tile_boundaries():
    lens = [1, 31, 32, 33, 63, 64, 65, 129, 257]
    w = random_prefill_workload(46, len(lens), 200, 16, 4, 128, 16, causal=True, lens=lens,
                                qo_lens=lens, dtype="fp8")
    run_case(w, "fp8 whole prompts")


def test_prefill_fp8_scales_are_applied():
    """The same codes under other scales: K's scale acts inside the softmax
    (not a plain factor of the output), V's multiplies the output."""
    import dataclasses
    base = random_prefill_workload(47, 2, 200, 8, 2, 128, 16, causal=True, dtype="fp8")
    w = dataclasses.replace(base, k_scale=base.k_scale * 3.0, v_scale=base.v_scale * 0.25)
    run_case(w, "fp8 prefill, other scales")


def test_prefill_edges_no_queries_and_empty_cache():
    # request 0 asks nothing, request 1 has no pages (unmasked: out 0, lse -inf)
    w = random_prefill_workload(21, 3, 80, 8, 2, 128, 16, causal=False, lens=[40, 0, 77],
                                qo_lens=[0, 6, 77])
    run_case(w, "no queries / empty cache")


def test_prefill_whole_prompts_tile_boundaries():
    # prompts whose length straddles the 64-token tiles of G = 4 and the
    # 32-token sub-blocks and 64-token blocks of the kernel, all of them queries
    lens = [1, 31, 32, 33, 63, 64, 65, 129, 257]
    w = random_prefill_workload(22, len(lens), 200, 16, 4, 128, 16, causal=True, lens=lens,
                                qo_lens=lens)
    run_case(w, "whole prompts")


def test_prefill_is_deterministic():
    w = random_prefill_workload(23, 3, 600, 8, 2, 128, 16, causal=True)
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = make_plan(w, fixed_chunk_tokens=64)
    a = run(w, q, k, v, p)
    b = run(w, q, k, v, p)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("cfg", [8, 14])
def test_full_size_cut_tiles_bitwise_repeatable(cfg):
    """Which chunk of a cut tile arrives last, and so merges the tile,
    depends on timing; the merged result must not. Twenty runs of the
    full-size append batch (bf16, and with the rotary embedding), every
    other one after a cache flush so arrival orders differ, must equal the
    first run bit for bit; the test stops at the first mismatch."""
    w = workload(cfg)
    q, k, v = w.make_values("cuda")
    p = make_plan(w)
    log(f"[case] prefill repeat config {cfg}: {p.info['num_items']} items, "
        f"{p.info['num_merges']} merges")
    assert p.info["num_merges"] > 0
    o0, l0 = run(w, q, k, v, p)
    out, lse = torch.empty_like(o0), torch.empty_like(l0)
    flush = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
    for r in range(1, 21):
        if r % 2:
            flush.zero_()
        run(w, q, k, v, p, out=out, lse=lse)
        torch.cuda.synchronize()
        same = torch.equal(out.view(torch.int16), o0.view(torch.int16)) and torch.equal(lse, l0)
        assert same, f"config {cfg}: run {r} differs from run 0"
    log(f"[ok] prefill repeat config {cfg}: 20 runs bitwise equal")


# rotary embedding (q and K before it), bf16, head_dim 128: groups 1 .. 8 and
# 6, page sizes 1 .. 64, causal and unmasked, direct output and cut tiles,
# positions past 2^15 (theta and scale varied)
ROPE_CASES = [
    # seed, B, maxL, Hq, Hkv, P, causal, max_qo, fixed_chunk, theta, scale
    (61, 4, 300, 8, 2, 16, True, None, 0, 1e4, 1.0),
    (62, 3, 700, 32, 8, 16, True, None, 128, 5e5, 1.0),
    (63, 3, 90, 4, 4, 1, False, None, 7, 1e4, 2.0),
    (64, 2, 1000, 8, 1, 64, True, 300, 192, 5e5, 1.0),
    (65, 3, 333, 12, 2, 3, False, 200, 0, 1e6, 0.5),
]


@pytest.mark.parametrize("case", ROPE_CASES, ids=lambda c: f"seed{c[0]}")
def test_prefill_rope_small(case):
    seed, B, L, Hq, Hkv, P, causal, max_qo, fixed, theta, scale = case
    w = random_prefill_workload(seed, B, L, Hq, Hkv, 128, P, causal=causal, max_qo=max_qo,
                                rope_theta=theta, rope_scale=scale)
    p, _, _ = run_case(w, f"rope prefill seed{seed}", fixed_chunk_tokens=fixed)
    assert p.info["rope"] == 1 and p.info["tokens_per_tile"] == 128 // (Hq // Hkv)
    if fixed:
        assert p.info["num_merges"] > 0


def test_prefill_rope_whole_prompts_and_long_positions():
    """Whole prompts across tile and block edges, and a request of 40,000
    tokens whose last 70 are queries (positions past 2^15, a chunk cut)."""
    lens = [1, 31, 32, 33, 63, 64, 65, 129, 257]
    w = random_prefill_workload(66, len(lens), 200, 16, 4, 128, 16, causal=True, lens=lens,
                                qo_lens=lens, rope_theta=5e5)
    run_case(w, "rope whole prompts")
    w = random_prefill_workload(67, 1, 40000, 8, 2, 128, 16, causal=True, lens=[40000],
                                qo_lens=[70], rope_theta=5e5)
    run_case(w, "rope long positions")


def test_prefill_rope_is_deterministic():
    w = random_prefill_workload(68, 3, 600, 8, 2, 128, 16, causal=True, rope_theta=1e4)
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = make_plan(w, fixed_chunk_tokens=64)
    a = run(w, q, k, v, p)
    b = run(w, q, k, v, p)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("cfg", [7, 8, 12, 14])
def test_prefill_full_size(cfg):
    """Every (query row, head) of the full-size workload, in the launch
    configuration bench.py times, against the oracle evaluated one request
    at a time (memory bounded by the longest request)."""
    w = workload(cfg)
    log(f"[case] full-size prefill config {cfg} {w.name} N={w.num_qo_tokens}")
    q, k, v = w.make_values("cuda")
    p = make_plan(w)
    out, lse = run(w, q, k, v, p)
    torch.cuda.synchronize()
    t0 = time.time()
    if w.dtype == "fp8":
        kh, vh = host_kv(w, k, v)
    else:  # bf16 values are exact in float32; the oracle widens what it gathers
        kh, vh = k.float().cpu().numpy(), v.float().cpu().numpy()
    qh = q.float().cpu().numpy()
    out_h, lse_h = out.double().cpu().numpy(), lse.double().cpu().numpy()
    del k, v
    worst = {"max_abs_vs_rounded": 0.0, "lse_max_abs": 0.0, "faithful_only": 0}
    checked = 0
    for b in range(w.batch):
        q0, q1, qo, ip, ix, lp = prefill_request(w, b)
        if q1 == q0:
            continue
        O, LSE = oracle(w, qh[q0:q1], kh, vh, qo, ip, ix, lp)
        st = compare(out_h[q0:q1], lse_h[q0:q1], O, LSE, True, f"prefill config {cfg} request {b}")
        for key in ("max_abs_vs_rounded", "lse_max_abs"):
            worst[key] = max(worst[key], st.get(key, 0.0))
        worst["faithful_only"] += st["faithful_only"]
        checked += q1 - q0
    assert checked == w.num_qo_tokens
    log(f"[ok] config {cfg} items={p.info['num_items']} merges={p.info['num_merges']} "
        f"rows={checked * w.num_qo_heads} oracle {time.time() - t0:.1f}s {worst}")
