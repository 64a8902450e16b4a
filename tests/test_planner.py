"""The host planner (fi_plan_create) on a CPU-only host: coverage, ordering,
slots, merge trees and the split-then-merge result in float64."""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import block_sparse_kv_bsr_amd as fb
from block_sparse_kv_bsr_amd.binding import ITEM_STRIDE, MERGE_FAN_IN, NODE_STRIDE
from block_sparse_kv_bsr_amd.workloads import prefix_workload, random_workload, workload
import oracle.attention as oa

I_REQ, I_KVH, I_PB, I_NTOK, I_SLOT, I_CHUNK, I_NP, I_FIRST, I_NODE = range(9)
N_COUNT, N_SB, N_PARENT, N_OUT, N_REQ, N_KVH, N_LEVEL, N_ARR = range(8)
P_GROUP, P_KVH, P_MBASE, P_ROW0, P_NROWS, P_CHUNK, P_PB, P_NP, P_TOFF, P_NTOK = range(10)


def make_plan(w, **opts):
    return fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, w.num_qo_heads, w.num_kv_heads,
                   w.head_dim, w.page_size, w.num_pool_pages, w.dtype, **opts)


def prefix_layout(w, p):
    """(prefix pages per request, prefix chunks per request, {(b, h): first
    tree slot}) of a plan, derived from its prefix items and merge nodes."""
    pitems, members = p.prefix_items(), p.prefix_members()
    G = w.group_size
    pre = np.zeros(w.batch, dtype=np.int64)
    cpre = np.zeros(w.batch, dtype=np.int64)
    for r in pitems:
        ms = members[r[P_MBASE] + r[P_ROW0]: r[P_MBASE] + r[P_ROW0] + r[P_NROWS] // G]
        for b in ms:
            if r[P_KVH] == 0:
                pre[b] += r[P_NP]
                cpre[b] = max(cpre[b], r[P_CHUNK] + 1)
    base = {}
    for n in p.merge_nodes():
        if n[N_LEVEL] == 0:
            key = (int(n[N_REQ]), int(n[N_KVH]))
            base[key] = min(base.get(key, 1 << 40), int(n[N_SB]))
    return pre, cpre, base


def check_plan(w, p, num_cus=256):
    """Every property a valid plan must have; returns (items, nodes)."""
    info = p.info
    items, nodes = p.work_list(), p.merge_nodes()
    pitems, members = p.prefix_items(), p.prefix_members()
    P, G = w.page_size, w.group_size
    assert items.shape[1] == ITEM_STRIDE and info["num_items"] == len(items)
    assert nodes.shape[1] == NODE_STRIDE and info["num_merge_nodes"] == len(nodes)
    assert info["num_prefix_items"] == len(pitems)
    assert info["total_kv_tokens"] == int(w.kv_lens().sum())
    # longest first, ties by (request, kv head, chunk), every other layer of
    # num_cus items reversed (snake)
    keys = [(-r[I_NTOK], r[I_REQ], r[I_KVH], r[I_CHUNK]) for r in items]
    ref = sorted(keys)
    layer = max(1, num_cus)
    for k, b0 in enumerate(range(0, len(keys), layer)):
        want = ref[b0:b0 + layer]
        assert keys[b0:b0 + layer] == (want if k % 2 == 0 else want[::-1]), k
    S = info["num_partial_slots"]
    fed = np.zeros(S, dtype=np.int64)   # producers per partial slot
    dyn = np.zeros(S, dtype=np.int64)   # producers that report during the decode kernel
    pre, cpre, base = prefix_layout(w, p)
    # shared prefixes: members share the first pre[b] pages, never their last
    assert len(set(members.tolist())) == len(members)
    for r in pitems:
        ms = members[r[P_MBASE] + r[P_ROW0]: r[P_MBASE] + r[P_ROW0] + r[P_NROWS] // G]
        assert r[P_NROWS] % G == 0 and 0 < r[P_NROWS] <= info["prefix_rows_per_item"]
        assert r[P_NP] >= 1
        for b in ms:
            s0 = int(w.kv_indptr[b])
            assert pre[b] <= w.num_pages(b) - 1
            # the item's pages are b's pages at the same positions
            off = r[P_PB] - int(w.kv_indptr[members[r[P_MBASE]]])
            assert np.array_equal(w.kv_indices[s0 + off: s0 + off + r[P_NP]],
                                  w.kv_indices[r[P_PB]: r[P_PB] + r[P_NP]])
            slot = base[(int(b), int(r[P_KVH]))] + r[P_CHUNK]
            fed[slot] += 1
    assert len(pitems) == 0 or w.dtype == "bf16"
    for b in range(w.batch):
        s, t = int(w.kv_indptr[b]) + int(pre[b]), int(w.kv_indptr[b + 1])
        for h in range(w.num_kv_heads):
            mine = sorted((r for r in items if r[I_REQ] == b and r[I_KVH] == h),
                          key=lambda r: r[I_CHUNK])
            if t == s:
                # a request with no pages: one item that writes out = 0, lse = -inf
                assert len(mine) == 1 and mine[0][I_NTOK] == 0
                assert mine[0][I_SLOT] == -1 and mine[0][I_NODE] == -1
                continue
            # decode chunks tile the pages after the prefix exactly once, in order
            pos = s
            for c, r in enumerate(mine):
                assert r[I_CHUNK] == c and r[I_PB] == pos and r[I_NP] >= 1
                assert r[I_FIRST] == w.kv_indices[r[I_PB]]  # first physical page, inline
                pos += r[I_NP]
                last = pos == t
                want = (r[I_NP] - 1) * P + int(w.last_page_len[b]) if last else r[I_NP] * P
                assert r[I_NTOK] == want
            assert pos == t
            assert sum(r[I_NTOK] for r in mine) + pre[b] * P == w.kv_len(b)
            if len(mine) == 1 and cpre[b] == 0:
                assert mine[0][I_SLOT] == -1 and mine[0][I_NODE] == -1
                continue
            for c, r in enumerate(mine):
                n = nodes[r[I_NODE]]
                assert n[N_LEVEL] == 0 and n[N_REQ] == b and n[N_KVH] == h
                assert n[N_SB] <= r[I_SLOT] < n[N_SB] + n[N_COUNT]
                assert r[I_SLOT] == base[(b, h)] + cpre[b] + c
                fed[r[I_SLOT]] += 1
                dyn[r[I_SLOT]] += 1
    roots = {}
    for i, n in enumerate(nodes):
        assert 1 <= n[N_COUNT] <= info["merge_fan_in"] <= MERGE_FAN_IN
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
            dyn[n[N_OUT]] += 1
    # every slot is one node's child and has exactly one producer; a node
    # waits for exactly the children that report during the decode kernel,
    # and at least one does (so nodes complete there)
    owner = np.zeros(S, dtype=np.int64)
    for n in nodes:
        owner[n[N_SB]:n[N_SB] + n[N_COUNT]] += 1
        assert n[N_ARR] == dyn[n[N_SB]:n[N_SB] + n[N_COUNT]].sum() >= 1
    assert np.all(owner == 1) and np.all(fed == 1)
    split = {(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)
             if sum(1 for r in items if r[I_REQ] == b and r[I_KVH] == h and r[I_SLOT] >= 0)}
    assert set(roots) == split
    # partial-slot bound: sum_b ceil(n_b / C) <= B + N / C over the decode pages
    C = info["chunk_pages"]
    N = int(w.kv_indptr[-1]) - int(pre.sum())
    assert sum(math.ceil((w.num_pages(b) - pre[b]) / C) for b in range(w.batch)) <= w.batch + N / C
    # workspace holds every section
    d = w.head_dim
    need = (len(items) * ITEM_STRIDE * 4 + len(nodes) * (NODE_STRIDE + 1) * 4 + int(w.kv_indptr[-1]) * 4
            + S * G * (d + 1) * 4)
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
    check_plan(w, p, num_cus=num_cus or 256)


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


def run_plan_f64(w, p):
    """Execute a plan on the CPU in float64 with the oracle's own routines:
    every decode item and every prefix item row attends over its tokens, and
    the states are folded up the plan's merge trees. Returns (out, lse)."""
    items, nodes = p.work_list(), p.merge_nodes()
    pitems, members = p.prefix_items(), p.prefix_members()
    pre, cpre, base = prefix_layout(w, p)
    q, k, v = (t.double().numpy() for t in w.make_values("cpu"))
    G, P = w.group_size, w.page_size
    slot_state = {}
    out = np.zeros((w.batch, w.num_qo_heads, w.head_dim))
    lse = np.full((w.batch, w.num_qo_heads), -np.inf)

    def span(pb, npg, last):
        return oa.request_tokens(np.array([0, npg]), w.kv_indices[pb:pb + npg], np.array([last]), P, 0)

    for r in items:
        b, h, ntok, npg = int(r[I_REQ]), int(r[I_KVH]), int(r[I_NTOK]), int(r[I_NP])
        if ntok == 0:
            continue
        K, V = oa.gather_kv(k, v, span(int(r[I_PB]), npg, ntok - (npg - 1) * P), h)
        st = oa.attend(q[b, h * G:(h + 1) * G], K, V, w.sm_scale)
        if r[I_SLOT] < 0:
            out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G] = st
        else:
            slot_state[int(r[I_SLOT])] = st
    for r in pitems:
        h = int(r[P_KVH])
        assert r[P_TOFF] == 0 and r[P_NTOK] == r[P_NP] * P  # whole shared pages
        K, V = oa.gather_kv(k, v, span(int(r[P_PB]), int(r[P_NP]), P), h)
        ms = members[r[P_MBASE] + r[P_ROW0]: r[P_MBASE] + r[P_ROW0] + r[P_NROWS] // G]
        for b in ms:
            slot_state[base[(int(b), h)] + int(r[P_CHUNK])] = oa.attend(
                q[b, h * G:(h + 1) * G], K, V, w.sm_scale)
    for i in sorted(range(len(nodes)), key=lambda i: nodes[i][N_LEVEL]):
        n = nodes[i]
        kids = [slot_state[s] for s in range(n[N_SB], n[N_SB] + n[N_COUNT])]
        st = oa.merge_many([c[0] for c in kids], [c[1] for c in kids])
        if n[N_PARENT] < 0:
            b, h = int(n[N_REQ]), int(n[N_KVH])
            out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G] = st
        else:
            slot_state[int(n[N_OUT])] = st
    return out, lse


PREFIX_CASES = [
    # seed, groups [(members, prefix pages)], singles, suffix_max, Hq, Hkv, d, P
    (1, [(5, 3)], 2, 40, 8, 2, 64, 4),
    (2, [(3, 1), (4, 6)], 3, 70, 16, 4, 128, 8),
    (3, [(40, 2)], 0, 20, 16, 4, 64, 4),     # 40 members x G 4 = 160 rows: two row blocks
    (4, [(2, 9)], 1, 9, 4, 4, 64, 3),        # prefix of many chunks, G 1
    (5, [(3, 4)], 0, 5, 32, 4, 64, 16),      # G 8
]


@pytest.mark.parametrize("case", PREFIX_CASES, ids=lambda c: f"prefix{c[0]}")
def test_cascade_plan_equals_oracle(case):
    """A cascade plan (forced on) covers every token once, groups exactly the
    requests that share leading pages, and -- executed in float64 with the
    oracle's own attention and merge -- gives the oracle's result."""
    seed, groups, singles, smax, hq, hkv, d, P = case
    w = prefix_workload(seed, groups, singles, smax, hq, hkv, d, P, "bf16")
    p = make_plan(w, cascade=1, fixed_chunk_tokens=2 * P)
    check_plan(w, p)
    assert p.info["num_prefix_groups"] == len(groups)
    pre, cpre, _ = prefix_layout(w, p)
    for gsize, pages in groups:
        # the first two members also share the next page; with two members
        # that page belongs to the common run
        want = pages + 1 if gsize == 2 else pages
        assert sum(1 for b in range(w.batch) if pre[b] == want) >= gsize
    out, lse = run_plan_f64(w, p)
    q, k, v = (t.double().numpy() for t in w.make_values("cpu"))
    O, LSE = oa.decode_attention(q, k, v, w.kv_indptr, w.kv_indices, w.last_page_len, w.sm_scale)
    assert np.allclose(out, O, atol=1e-12, rtol=0) and np.allclose(lse, LSE, atol=1e-12, rtol=0)


def test_cascade_off_and_auto():
    w = workload(5)
    assert make_plan(w).info["num_prefix_groups"] == 1          # auto: 31 x 8 MiB saved
    assert make_plan(w, cascade=-1).info["num_prefix_items"] == 0
    assert make_plan(w, cascade=-1).info["shared_pages"] == 128
    assert make_plan(w).info["shared_pages"] == 0                # prefix left to the prefix items
    small = prefix_workload(9, [(3, 2)], 1, 30, 8, 2, 64, 4, "bf16")
    assert make_plan(small).info["num_prefix_items"] == 0       # auto: saves far below 8 MiB
    assert make_plan(small, cascade=1).info["num_prefix_items"] > 0
    f32 = prefix_workload(9, [(3, 2)], 1, 30, 8, 2, 64, 4, "f32")
    assert make_plan(f32, cascade=1).info["num_prefix_items"] == 0   # matrix-core path is bf16


@settings(max_examples=25, deadline=None)
@given(seed=st.integers(0, 10_000), members=st.integers(2, 12), pages=st.integers(1, 12),
       singles=st.integers(0, 4), P=st.sampled_from([1, 4, 16]), hkv=st.sampled_from([1, 2]),
       fixed=st.sampled_from([0, 1, 32]))
def test_cascade_plan_properties(seed, members, pages, singles, P, hkv, fixed):
    w = prefix_workload(seed, [(members, pages)], singles, 50, 4 * hkv, hkv, 64, P, "bf16")
    p = make_plan(w, cascade=1, fixed_chunk_tokens=fixed)
    check_plan(w, p)


@pytest.mark.parametrize("hq,hkv,d,want", [(32, 8, 128, 16), (64, 8, 128, 8), (8, 8, 128, 16),
                                          (32, 4, 64, 16), (8, 1, 64, 16), (16, 2, 128, 8)])
def test_merge_fan_in_is_what_one_merge_round_loads(hq, hkv, d, want):
    """A merge node has as many children as the merging wave loads in its first
    round: 64 / (float pairs per lane of a G x head_dim partial), at most 16."""
    w = random_workload(77, 3, 3000, hq, hkv, d, 16, "bf16")
    p = make_plan(w, fixed_chunk_tokens=16)
    assert p.info["merge_fan_in"] == want
    nodes = p.merge_nodes()
    assert nodes[:, N_COUNT].max() == want


def test_items_per_cu_default_follows_the_kernel():
    """Plans that run the matrix-core kernel default to 6 items per CU
    without the rotary embedding and 16 with it, plans for the vector kernel
    to 8 (measured best for each); an explicit items_per_cu overrides them."""
    for cfg, want_mma in ((3, False), (6, True), (11, True)):
        w = workload(cfg)
        p = make_plan(w)
        assert (p.info["decode_kernel"] == fb.binding.DECODE_KERNEL_MATRIX) == want_mma
        budget = (6 if want_mma else 8) * 256
        assert p.info["num_items"] <= budget
        pr = make_plan(w, rope=True)
        assert pr.info["num_items"] <= (16 if want_mma else 8) * 256
        if want_mma:
            # the skewed batch fills its budget: the default changes the cut
            assert p.info["num_items"] > 5 * 256
            assert pr.info["num_items"] > 12 * 256
        assert make_plan(w, items_per_cu=4).info["num_items"] <= 4 * 256
