"""The host planner (fi_plan_create) on a CPU-only host: coverage, ordering,
slots, merge tasks and the split-then-merge result in float64."""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import block_sparse_kv_bsr_amd as fb
from block_sparse_kv_bsr_amd.binding import ITEM_STRIDE
from block_sparse_kv_bsr_amd.workloads import random_workload, workload
import oracle.attention as oa

I_REQ, I_KVH, I_PB, I_NTOK, I_SLOT, I_CHUNK, I_NP = range(7)


def make_plan(w, **opts):
    return fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, w.num_qo_heads, w.num_kv_heads,
                   w.head_dim, w.page_size, w.num_pool_pages, w.dtype, **opts)


def check_plan(w, p):
    """Every property a valid plan must have; returns (items, merges)."""
    info = p.info
    items, merges = p.work_list(), p.merge_list()
    P = w.page_size
    assert items.shape[1] == ITEM_STRIDE and info["num_items"] == len(items)
    assert info["total_kv_tokens"] == int(w.kv_lens().sum())
    # longest first, ties by (request, kv head, chunk)
    keys = [(-r[I_NTOK], r[I_REQ], r[I_KVH], r[I_CHUNK]) for r in items]
    assert keys == sorted(keys)
    nchunks = {}
    for b in range(w.batch):
        s, t = int(w.kv_indptr[b]), int(w.kv_indptr[b + 1])
        for h in range(w.num_kv_heads):
            mine = sorted((r for r in items if r[I_REQ] == b and r[I_KVH] == h),
                          key=lambda r: r[I_CHUNK])
            if t == s:
                assert not mine
                continue
            # chunks tile the page list exactly once, in order
            pos = s
            for c, r in enumerate(mine):
                assert r[I_CHUNK] == c and r[I_PB] == pos and r[I_NP] >= 1
                pos += r[I_NP]
                last = pos == t
                want = (r[I_NP] - 1) * P + int(w.last_page_len[b]) if last else r[I_NP] * P
                assert r[I_NTOK] == want
            assert pos == t
            assert sum(r[I_NTOK] for r in mine) == w.kv_len(b)
            nchunks[b] = len(mine)
            if len(mine) == 1:
                assert mine[0][I_SLOT] == -1
    # merge tasks: exactly the requests with 0 or >= 2 chunks, disjoint slot ranges
    seen = set()
    task_of = {int(m[0]): m for m in merges}
    for b in range(w.batch):
        k = nchunks.get(b, 0)
        if k == 1:
            assert b not in task_of
            continue
        m = task_of[b]
        assert m[2] == k
        for c in range(k):
            sl = int(m[1]) + c
            assert sl not in seen
            seen.add(sl)
            its = [r for r in items if r[I_REQ] == b and r[I_CHUNK] == c]
            assert len(its) == w.num_kv_heads and all(r[I_SLOT] == sl for r in its)
    assert len(seen) == info["num_partial_slots"]
    # partial-slot bound: sum_b ceil(n_b / C) <= B + N / C
    C = info["chunk_pages"]
    N = int(w.kv_indptr[-1])
    assert sum(math.ceil(w.num_pages(b) / C) for b in range(w.batch)) <= w.batch + N / C
    # workspace holds every section
    Hq, d = w.num_qo_heads, w.head_dim
    need = len(items) * 32 + len(merges) * 16 + N * 4 + info["num_partial_slots"] * Hq * (d + 1) * 4
    assert info["workspace_bytes"] >= need
    return items, merges


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config_plans(cfg):
    w = workload(cfg)
    p = make_plan(w)
    check_plan(w, p)
    if cfg == 4:
        # each long sequence is cut into at least 64 chunks
        assert p.info["min_chunks_split_request"] >= 64
    if cfg in (2, 3, 4, 5):
        assert p.info["num_items"] <= 256 * 8


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 10_000), batch=st.integers(1, 9), max_len=st.integers(1, 700),
       P=st.sampled_from([1, 3, 8, 16, 64]), hkv=st.sampled_from([1, 2, 4]),
       empty=st.sampled_from([0, 2, 3]), items_per_cu=st.sampled_from([0, 1, 4]),
       num_cus=st.sampled_from([0, 1, 3, 16]), min_chunk=st.sampled_from([0, 1, 40]))
def test_plan_properties(seed, batch, max_len, P, hkv, empty, items_per_cu, num_cus, min_chunk):
    w = random_workload(seed, batch, max_len, 4 * hkv, hkv, 64, P, "bf16", empty_every=empty)
    p = make_plan(w, num_cus=num_cus, items_per_cu=items_per_cu, min_chunk_tokens=min_chunk)
    check_plan(w, p)


@pytest.mark.parametrize("fixed", [1, 16, 48, 100])
def test_fixed_chunk(fixed):
    w = random_workload(5, 5, 300, 8, 2, 64, 16, "bf16", empty_every=3)
    p = make_plan(w, fixed_chunk_tokens=fixed)
    assert p.info["chunk_pages"] == max(1, math.ceil(fixed / 16))
    check_plan(w, p)


def test_cut_and_merge_equals_whole():
    """Running every work item as attention over its own tokens (float64
    oracle) and merging each request's chunk states with the oracle's merge
    gives the whole-request result: the plan covers every token once and the
    merge algebra is right."""
    w = random_workload(77, 6, 260, 8, 2, 64, 4, "f32", empty_every=4)
    p = make_plan(w, fixed_chunk_tokens=24)
    items, _ = check_plan(w, p)
    q, k, v = (t.double().numpy() for t in w.make_values("cpu"))
    O, LSE = oa.decode_attention(q, k, v, w.kv_indptr, w.kv_indices, w.last_page_len, w.sm_scale)
    G = w.group_size
    states = {}
    for r in items:
        b, h, pb, ntok, npg = int(r[I_REQ]), int(r[I_KVH]), int(r[I_PB]), int(r[I_NTOK]), int(r[I_NP])
        last = ntok - (npg - 1) * w.page_size
        toks = oa.request_tokens(np.array([0, npg]), w.kv_indices[pb:pb + npg], np.array([last]),
                                 w.page_size, 0)
        K, V = oa.gather_kv(k, v, toks, h)
        o, lse = oa.attend(q[b, h * G:(h + 1) * G], K, V, w.sm_scale)
        states.setdefault((b, h), []).append((int(r[I_CHUNK]), o, lse))
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            got = sorted(states.get((b, h), []), key=lambda x: x[0])
            if not got:
                assert np.all(np.isneginf(LSE[b, h * G:(h + 1) * G]))
                continue
            vo, so = oa.merge_many([g[1] for g in got], [g[2] for g in got])
            assert np.allclose(vo, O[b, h * G:(h + 1) * G], atol=1e-12, rtol=0)
            assert np.allclose(so, LSE[b, h * G:(h + 1) * G], atol=1e-12, rtol=0)


def test_empty_batch_and_all_empty():
    p = fb.plan(np.array([0]), np.array([], dtype=np.int32), np.array([], dtype=np.int32),
                8, 2, 128, 16, 0, "bf16")
    assert p.info["num_items"] == 0 and p.info["num_merge_tasks"] == 0
    p = fb.plan(np.array([0, 0, 0]), np.array([], dtype=np.int32), np.array([0, 0]), 8, 2, 128, 16, 4, "bf16")
    assert p.info["num_items"] == 0 and p.info["num_merge_tasks"] == 2
    assert p.merge_list()[:, 2].tolist() == [0, 0]
