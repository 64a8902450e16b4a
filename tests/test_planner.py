"""The host planner (fi_plan_create) on a CPU-only host: coverage, ordering,
slots, merge trees and the split-then-merge result in float64."""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import block_sparse_kv_bsr_amd as fb
from block_sparse_kv_bsr_amd.binding import ITEM_STRIDE, MERGE_FAN_IN, NODE_STRIDE
from block_sparse_kv_bsr_amd.workloads import random_workload, workload
import oracle.attention as oa

I_REQ, I_KVH, I_PB, I_NTOK, I_SLOT, I_CHUNK, I_NP, I_FIRST, I_NODE = range(9)
N_COUNT, N_SB, N_PARENT, N_OUT, N_REQ, N_KVH, N_LEVEL = range(7)


def make_plan(w, **opts):
    return fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, w.num_qo_heads, w.num_kv_heads,
                   w.head_dim, w.page_size, w.num_pool_pages, w.dtype, **opts)


def check_plan(w, p):
    """Every property a valid plan must have; returns (items, nodes)."""
    info = p.info
    items, nodes = p.work_list(), p.merge_nodes()
    P = w.page_size
    assert items.shape[1] == ITEM_STRIDE and info["num_items"] == len(items)
    assert nodes.shape[1] == NODE_STRIDE and info["num_merge_nodes"] == len(nodes)
    assert info["total_kv_tokens"] == int(w.kv_lens().sum())
    # longest first, ties by (request, kv head, chunk)
    keys = [(-r[I_NTOK], r[I_REQ], r[I_KVH], r[I_CHUNK]) for r in items]
    assert keys == sorted(keys)
    S = info["num_partial_slots"]
    fed = np.zeros(S, dtype=np.int64)   # producers per partial slot
    roots = {}
    for b in range(w.batch):
        s, t = int(w.kv_indptr[b]), int(w.kv_indptr[b + 1])
        for h in range(w.num_kv_heads):
            mine = sorted((r for r in items if r[I_REQ] == b and r[I_KVH] == h),
                          key=lambda r: r[I_CHUNK])
            if t == s:
                # a request with no pages: one item that writes out = 0, lse = -inf
                assert len(mine) == 1 and mine[0][I_NTOK] == 0
                assert mine[0][I_SLOT] == -1 and mine[0][I_NODE] == -1
                continue
            # chunks tile the page list exactly once, in order
            pos = s
            for c, r in enumerate(mine):
                assert r[I_CHUNK] == c and r[I_PB] == pos and r[I_NP] >= 1
                assert r[I_FIRST] == w.kv_indices[r[I_PB]]  # first physical page, inline
                pos += r[I_NP]
                last = pos == t
                want = (r[I_NP] - 1) * P + int(w.last_page_len[b]) if last else r[I_NP] * P
                assert r[I_NTOK] == want
            assert pos == t
            assert sum(r[I_NTOK] for r in mine) == w.kv_len(b)
            if len(mine) == 1:
                assert mine[0][I_SLOT] == -1 and mine[0][I_NODE] == -1
                continue
            for r in mine:
                n = nodes[r[I_NODE]]
                assert n[N_LEVEL] == 0 and n[N_REQ] == b and n[N_KVH] == h
                assert n[N_SB] <= r[I_SLOT] < n[N_SB] + n[N_COUNT]
                fed[r[I_SLOT]] += 1
    for i, n in enumerate(nodes):
        assert 1 <= n[N_COUNT] <= MERGE_FAN_IN
        assert 0 <= n[N_SB] and n[N_SB] + n[N_COUNT] <= S
        if n[N_PARENT] < 0:
            assert n[N_OUT] == -1
            key = (int(n[N_REQ]), int(n[N_KVH]))
            assert key not in roots
            roots[key] = i
        else:
            par = nodes[n[N_PARENT]]
            assert par[N_LEVEL] == n[N_LEVEL] + 1
            assert (par[N_REQ], par[N_KVH]) == (n[N_REQ], n[N_KVH])
            assert par[N_SB] <= n[N_OUT] < par[N_SB] + par[N_COUNT]
            fed[n[N_OUT]] += 1
    # every slot is one node's child and has exactly one producer
    owner = np.zeros(S, dtype=np.int64)
    for n in nodes:
        owner[n[N_SB]:n[N_SB] + n[N_COUNT]] += 1
    assert np.all(owner == 1) and np.all(fed == 1)
    split = {(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)
             if sum(1 for r in items if r[I_REQ] == b and r[I_KVH] == h and r[I_SLOT] >= 0)}
    assert set(roots) == split
    # partial-slot bound per KV head: sum_b ceil(n_b / C) leaves plus at most
    # ceil(k / 31) inner slots for a request cut into k chunks
    C = info["chunk_pages"]
    N = int(w.kv_indptr[-1])
    assert sum(math.ceil(w.num_pages(b) / C) for b in range(w.batch)) <= w.batch + N / C
    # workspace holds every section
    G, d = w.group_size, w.head_dim
    need = len(items) * ITEM_STRIDE * 4 + len(nodes) * (NODE_STRIDE + 1) * 4 + N * 4 + S * G * (d + 1) * 4
    assert info["workspace_bytes"] >= need
    return items, nodes


def tree_merge(items, nodes, leaf_state):
    """Folds chunk states up each merge tree as the plan prescribes (children
    in slot order, the oracle's float64 merge at every node); returns
    {(b, kv head): (v, lse)} from the roots."""
    slot_state = {int(r[I_SLOT]): leaf_state[i] for i, r in enumerate(items) if r[I_SLOT] >= 0}
    out = {}
    for i in sorted(range(len(nodes)), key=lambda i: nodes[i][N_LEVEL]):
        n = nodes[i]
        kids = [slot_state[s] for s in range(n[N_SB], n[N_SB] + n[N_COUNT])]
        st = oa.merge_many([k[0] for k in kids], [k[1] for k in kids])
        if n[N_PARENT] < 0:
            out[(int(n[N_REQ]), int(n[N_KVH]))] = st
        else:
            slot_state[int(n[N_OUT])] = st
    return out


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


@pytest.mark.parametrize("fixed,lens", [(24, None), (1, [70, 33, 32, 1, 0, 1100])])
def test_cut_and_merge_equals_whole(fixed, lens):
    """Running every work item as attention over its own tokens (float64
    oracle) and folding the chunk states up the plan's merge trees gives the
    whole-request result: the plan covers every token once and its trees
    reach every chunk exactly once (page size 1 with one-token chunks gives
    trees of two and three levels)."""
    if lens is None:
        w = random_workload(77, 6, 260, 8, 2, 64, 4, "f32", empty_every=4)
    else:
        w = random_workload(78, len(lens), 1, 8, 2, 64, 1, "f32", lens=lens)
    p = make_plan(w, fixed_chunk_tokens=fixed)
    items, nodes = check_plan(w, p)
    if lens is not None:
        assert nodes[:, N_LEVEL].max() == 2
    q, k, v = (t.double().numpy() for t in w.make_values("cpu"))
    O, LSE = oa.decode_attention(q, k, v, w.kv_indptr, w.kv_indices, w.last_page_len, w.sm_scale)
    G = w.group_size
    leaf = []
    for r in items:
        b, h, pb, ntok, npg = int(r[I_REQ]), int(r[I_KVH]), int(r[I_PB]), int(r[I_NTOK]), int(r[I_NP])
        if ntok == 0:
            leaf.append(None)
            continue
        last = ntok - (npg - 1) * w.page_size
        toks = oa.request_tokens(np.array([0, npg]), w.kv_indices[pb:pb + npg], np.array([last]),
                                 w.page_size, 0)
        K, V = oa.gather_kv(k, v, toks, h)
        leaf.append(oa.attend(q[b, h * G:(h + 1) * G], K, V, w.sm_scale))
    merged = tree_merge(items, nodes, leaf)
    for i, r in enumerate(items):
        if r[I_SLOT] < 0 and r[I_NTOK] > 0:
            merged[(int(r[I_REQ]), int(r[I_KVH]))] = leaf[i]
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            if w.kv_len(b) == 0:
                assert np.all(np.isneginf(LSE[b, h * G:(h + 1) * G]))
                continue
            vo, so = merged[(b, h)]
            assert np.allclose(vo, O[b, h * G:(h + 1) * G], atol=1e-12, rtol=0)
            assert np.allclose(so, LSE[b, h * G:(h + 1) * G], atol=1e-12, rtol=0)


def test_empty_batch_and_all_empty():
    p = fb.plan(np.array([0]), np.array([], dtype=np.int32), np.array([], dtype=np.int32),
                8, 2, 128, 16, 0, "bf16")
    assert p.info["num_items"] == 0 and p.info["num_merge_nodes"] == 0
    p = fb.plan(np.array([0, 0, 0]), np.array([], dtype=np.int32), np.array([0, 0]), 8, 2, 128, 16, 4, "bf16")
    items = p.work_list()
    assert p.info["num_items"] == 4 and p.info["num_merge_nodes"] == 0
    assert items[:, I_NTOK].tolist() == [0] * 4 and items[:, I_SLOT].tolist() == [-1] * 4
