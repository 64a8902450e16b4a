"""The prefill / append planner on a CPU-only host: structure of the work
list, a float64 execution of the plan (each item attends its chunk, cut
tiles merge their chunks) against the oracle, and the checks that reject
malformed calls."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import block_sparse_kv_bsr_amd as fb
from block_sparse_kv_bsr_amd import binding
from block_sparse_kv_bsr_amd.workloads import random_prefill_workload, workload
import oracle.attention as oa

REQ, KVH, QROW, NQO, KV0, NKV, VIS, PG0, SLOT, CHUNK = range(10)
MERGE = 12
M_QROW, M_NQO, M_KVH, M_SLOT0, M_NCH = range(5)


def make_plan(w, **kw):
    return fb.prefill_plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len,
                           w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                           w.num_pool_pages, causal=w.causal, **kw)


def check_prefill_plan(w, p):
    """Every (query token, KV head) lies in exactly one tile; the tile's
    chunks tile [0, range) with whole pages; VISIBLE matches the causal rule;
    slots and merges are consistent; a pair's items go longest chunk first."""
    items, merges = p.work_list(), p.merges()
    info = p.info
    G = w.num_qo_heads // w.num_kv_heads
    T = binding.PREFILL_ROWS // G
    assert info["tokens_per_tile"] == T
    P = w.page_size
    L = w.kv_lens()
    qo = w.qo_indptr
    # within each (request, KV head) pair: longest chunk first
    for key in {(int(x[REQ]), int(x[KVH])) for x in items}:
        sel = items[(items[:, REQ] == key[0]) & (items[:, KVH] == key[1])]
        assert np.all(np.diff(sel[:, NKV]) <= 0), key
    tiles = {}
    for it in items:
        b = int(it[REQ])
        key = (b, int(it[KVH]), int(it[QROW]))
        tiles.setdefault(key, []).append(it)
        n, Lb = int(qo[b + 1] - qo[b]), int(L[b])
        t0 = int(it[QROW]) - int(qo[b])
        assert 0 <= t0 < max(n, 1) and t0 % T == 0
        assert int(it[NQO]) == min(T, n - t0)
        want_vis = Lb - n + t0 + 1 if w.causal else Lb
        assert int(it[VIS]) == want_vis
        assert int(it[KV0]) % P == 0
        assert int(it[PG0]) == int(w.kv_indptr[b]) + int(it[KV0]) // P
        # the chunk cap: the kernel's page-id window and 2^20 tokens
        assert int(it[NKV]) <= min(binding.PREFILL_MAX_PAGES, (1 << 20) // P) * P
        assert int(it[NKV]) > 0 or Lb == 0
    # every (request, head, query token) covered by exactly one tile
    cover = {}
    for (b, h, r0), its in tiles.items():
        nq = int(its[0][NQO])
        for r in range(r0, r0 + nq):
            cover[(h, r)] = cover.get((h, r), 0) + 1
        its = sorted(its, key=lambda x: int(x[CHUNK]))
        assert [int(x[CHUNK]) for x in its] == list(range(len(its)))
        # chunks tile [0, range of the tile's last query)
        pos = 0
        for x in its:
            assert int(x[KV0]) == pos
            pos += int(x[NKV])
        last_vis = int(its[0][VIS]) + (nq - 1 if w.causal else 0)
        assert pos == (last_vis if w.causal else int(L[b]))
        if len(its) == 1:
            assert int(its[0][SLOT]) == -1
        else:
            slots = [int(x[SLOT]) for x in its]
            assert slots == list(range(slots[0], slots[0] + len(its)))
    assert len(cover) == w.num_kv_heads * w.num_qo_tokens and set(cover.values()) <= {1}
    # merges: exactly the cut tiles
    cut = {k: its for k, its in tiles.items() if len(its) > 1}
    assert len(merges) == len(cut) == info["num_merges"]
    for mi, m in enumerate(merges):
        b = int(np.searchsorted(qo, m[M_QROW], side="right")) - 1
        its = cut[(b, int(m[M_KVH]), int(m[M_QROW]))]
        assert int(m[M_NCH]) == len(its) and int(m[M_NQO]) == int(its[0][NQO])
        assert int(m[M_SLOT0]) == min(int(x[SLOT]) for x in its)
        # each chunk of a cut tile names the tile's merge (its arrival counter)
        assert all(int(x[MERGE]) == mi for x in its)
    for its in tiles.values():
        if len(its) == 1:
            assert int(its[0][MERGE]) == -1
    assert np.all(items[:, MERGE + 1:] == 0)
    used = sorted(int(x) for x in items[:, SLOT] if x >= 0)
    assert used == list(range(info["num_partial_slots"]))
    assert info["visible_pairs"] == w.visible_pairs()


def run_prefill_plan_f64(w, p, q, k, v):
    """Execute the plan in float64: each item attends its chunk (tokens
    KV_BEGIN .. +NUM_KV, cut at each row's visible count), cut tiles fold
    their chunks' states in chunk order."""
    items = p.work_list()
    Hq, d = w.num_qo_heads, w.head_dim
    G = Hq // w.num_kv_heads
    O = np.full((w.num_qo_tokens, Hq, d), np.nan)
    LSE = np.full((w.num_qo_tokens, Hq), np.nan)
    parts = {}
    for it in items:
        b, h = int(it[REQ]), int(it[KVH])
        toks = oa.request_tokens(w.kv_indptr, w.kv_indices, w.last_page_len, w.page_size, b)
        K, V = oa.gather_kv(k, v, toks, h)
        k0, nk = int(it[KV0]), int(it[NKV])
        for j in range(int(it[NQO])):
            r = int(it[QROW]) + j
            lim = int(it[VIS]) + (j if w.causal else 0)
            hi = min(k0 + nk, lim)
            lo = min(k0, hi)
            heads = list(range(h * G, h * G + G))
            o, lse = oa.attend(q[r, heads], K[lo:hi], V[lo:hi], w.sm_scale)
            parts.setdefault((r, h), []).append((int(it[CHUNK]), o, lse))
    for (r, h), chunks in parts.items():
        chunks.sort(key=lambda x: x[0])
        o, lse = oa.merge_many([c[1] for c in chunks], [c[2] for c in chunks])
        O[r, h * G:(h + 1) * G] = o
        LSE[r, h * G:(h + 1) * G] = lse
    return O, LSE


CASES = [
    # seed, batch, max_len, Hq, Hkv, d, P, causal, max_qo, fixed_chunk
    (1, 4, 300, 8, 2, 64, 16, True, None, 0),
    (2, 3, 200, 4, 4, 64, 4, True, None, 32),     # G = 1: 128 tokens per tile, cut chunks
    (3, 5, 150, 16, 2, 128, 16, True, 40, 48),    # G = 8, chunks of 3 pages
    (4, 3, 90, 4, 1, 64, 1, False, None, 7),      # page size 1, no mask
    (5, 4, 260, 8, 2, 128, 64, True, 1, 0),       # one query per request (decode shape)
    (6, 2, 500, 12, 2, 64, 16, True, None, 16),   # G = 6 (not a power of two)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_prefill_plan_structure_and_f64_execution(case):
    seed, B, L, Hq, Hkv, d, P, causal, max_qo, fixed = case
    w = random_prefill_workload(seed, B, L, Hq, Hkv, d, P, causal=causal, max_qo=max_qo)
    p = make_plan(w, fixed_chunk_tokens=fixed)
    check_prefill_plan(w, p)
    if fixed:
        assert p.info["num_merges"] > 0
    q, k, v = (t.double().numpy() for t in w.make_values("cpu"))
    O, LSE = run_prefill_plan_f64(w, p, q, k, v)
    Oo, LSEo = oa.prefill_attention(q, k, v, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                    w.last_page_len, causal, w.sm_scale)
    assert np.max(np.abs(O - Oo)) <= 1e-12
    assert np.max(np.abs(LSE - LSEo)) <= 1e-12


def test_empty_requests_and_no_mask_on_an_empty_cache():
    # a request with no queries gets no tile; without the mask a request with
    # no pages still gets a tile that attends nothing
    w = random_prefill_workload(9, 3, 50, 4, 2, 64, 16, causal=False, lens=[20, 0, 33],
                                qo_lens=[0, 5, 7])
    p = make_plan(w)
    check_prefill_plan(w, p)
    items = p.work_list()
    assert not np.any(items[:, REQ] == 0)
    empty = items[items[:, REQ] == 1]
    assert len(empty) == 2 and np.all(empty[:, NKV] == 0) and np.all(empty[:, SLOT] == -1)


def test_full_size_workloads_plan():
    for cfg in (7, 8):
        w = workload(cfg)
        p = make_plan(w)
        info = p.info
        assert info["total_qo_tokens"] == w.num_qo_tokens
        assert info["visible_pairs"] == w.visible_pairs()
        items = p.work_list()
        assert items[:, NKV].max() <= binding.PREFILL_MAX_PAGES * w.page_size
    # the prompt batch is not cut; the skewed append batch is
    assert make_plan(workload(7)).info["num_merges"] == 0
    assert make_plan(workload(8)).info["num_merges"] > 0


def _pair_positions(items):
    pos = {}
    for i, x in enumerate(items):
        pos.setdefault((int(x[REQ]), int(x[KVH])), []).append(i)
    return pos


@pytest.mark.parametrize("P", [16, 1000, 3000, 4096])
def test_chunk_cap_is_the_window_and_2_20_tokens(P):
    """A prefill chunk holds at most FI_PREFILL_MAX_PAGES pages (the tile
    kernel's page-id window) and at most 2^20 tokens (the range over which
    its reciprocal division by the page size is exact), whatever chunk
    length is asked for."""
    cap = min(binding.PREFILL_MAX_PAGES, (1 << 20) // P) * P
    L = 3 * cap + P // 2
    w = random_prefill_workload(31, 1, L, 4, 1, 128, P, causal=True, lens=[L], qo_lens=[3])
    p = make_plan(w, fixed_chunk_tokens=1 << 30)
    items = p.work_list()
    assert items[:, NKV].max() == cap and len(items) == 4
    assert items[:, NKV].max() <= 1 << 20
    check_prefill_plan(w, p)


def test_order_one_bin_is_pairs_heaviest_first():
    w = random_prefill_workload(31, 6, 900, 8, 2, 128, 16, causal=True)
    items = make_plan(w, num_xcds=1, fixed_chunk_tokens=128).work_list()
    pos = _pair_positions(items)
    work = {}
    for key, ps in pos.items():
        assert ps == list(range(ps[0], ps[0] + len(ps))), key  # contiguous
        work[ps[0]] = sum((int(items[i, NKV]) + 63) // 64 + 1 for i in ps)
    starts = sorted(work)
    assert all(work[a] >= work[b] for a, b in zip(starts, starts[1:]))


def test_order_keeps_each_pair_on_one_xcd():
    # the prompt batch: 128 equal pairs over 8 bins, so every item of a pair
    # sits at positions of one residue mod 8
    items = make_plan(workload(7)).work_list()
    for key, ps in _pair_positions(items).items():
        assert len({i % 8 for i in ps}) == 1, key
    # and the XCDs get equal work
    per = np.zeros(8)
    for i, x in enumerate(items):
        per[i % 8] += int(x[NKV])
    assert per.max() == per.min()


def _status(qo, ip, ix, lp, Hq=8, Hkv=2, d=128, P=16, pool=100, dtype=1, causal=1):
    import ctypes
    L = fb.lib()
    arrs = [np.asarray(a, dtype=np.int32) for a in (qo, ip, ix, lp)]
    p32 = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    h = ctypes.c_void_p()
    st = L.fi_prefill_plan_create(p32(arrs[0]), p32(arrs[1]), p32(arrs[2]), p32(arrs[3]),
                                  len(arrs[1]) - 1, Hq, Hkv, d, P, pool, dtype, causal, None,
                                  ctypes.byref(h))
    if st == 0:
        L.fi_prefill_plan_destroy(h)
    return st, L.fi_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(qo=[1, 2, 3]), -1, "qo_indptr[0]"),
    (dict(qo=[0, 3, 2]), -1, "non-decreasing"),
    (dict(qo=[0, 40, 41]), -1, "more query tokens"),
    (dict(dtype=0), -2, "BF16"),
    (dict(dtype=7), -2, "BF16"),
    (dict(dtype=2, d=64), -2, "fp8 prefill is built for head_dim 128"),
    (dict(d=96), -2, "head_dim"),
    (dict(Hq=8, Hkv=3), -1, "multiple"),
    (dict(Hq=512, Hkv=1), -2, "group size"),
    (dict(ix=[5, 6, 700]), -1, "num_pool_pages"),
])
def test_prefill_plan_rejects(kw, code, needle):
    args = dict(qo=[0, 2, 3], ip=[0, 2, 3], ix=[5, 6, 7], lp=[16, 3])
    args.update(kw)
    st, msg = _status(args.pop("qo"), args.pop("ip"), args.pop("ix"), args.pop("lp"), **args)
    assert st == code and needle in msg, (st, msg)


def test_rope_plan_has_half_height_tiles_and_query_positions():
    """A rope plan cuts each request's queries into tiles of 128 / G tokens
    and records the position of each tile's first query, L - n + index."""
    from block_sparse_kv_bsr_amd.workloads import random_prefill_workload
    w = random_prefill_workload(5, 4, 700, 16, 4, 128, 16, causal=True)
    a = fb.prefill_plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, 16, 4, 128, 16,
                        w.num_pool_pages)
    b = fb.prefill_plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, 16, 4, 128, 16,
                        w.num_pool_pages, rope=True)
    assert a.info["rope"] == 0 and b.info["rope"] == 1
    assert a.info["tokens_per_tile"] == 64 and b.info["tokens_per_tile"] == 32
    L, n = w.kv_lens(), np.diff(w.qo_indptr)
    for p in (a, b):
        T = p.info["tokens_per_tile"]
        for r in p.work_list():
            req = int(r[0])
            first = int(r[2]) - int(w.qo_indptr[req])   # tile's first query index
            assert first % T == 0 and r[3] <= T
            assert r[10] == L[req] - n[req] + first


@pytest.mark.parametrize("kw,code,needle", [
    (dict(dtype=2), -2, "rotary"),
    (dict(d=64), -2, "rotary"),
    (dict(Hq=256, Hkv=1), -2, "G <="),
])
def test_rope_plan_rejects(kw, code, needle):
    import ctypes
    L = fb.lib()
    a = dict(Hq=8, Hkv=2, d=128, dtype=1)
    a.update(kw)
    arrs = [np.asarray(x, dtype=np.int32) for x in ([0, 2, 3], [0, 2, 3], [5, 6, 7], [16, 3])]
    p32 = lambda x: x.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    opts = binding.PrefillOpts(0, 0, 0, 0, 1)
    h = ctypes.c_void_p()
    st = L.fi_prefill_plan_create(p32(arrs[0]), p32(arrs[1]), p32(arrs[2]), p32(arrs[3]), 2,
                                  a["Hq"], a["Hkv"], a["d"], 16, 100, a["dtype"], 1,
                                  ctypes.byref(opts), ctypes.byref(h))
    assert st == code and needle in L.fi_last_error().decode(), (st, L.fi_last_error())


def test_rope_plan_needs_cached_queries_also_unmasked():
    """Rotated queries are cached tokens: an unmasked request with more
    queries than tokens is refused for a rope plan (allowed without)."""
    ip, ix, lp = np.array([0, 1]), np.array([3]), np.array([5])
    qo = np.array([0, 7])
    fb.prefill_plan(qo, ip, ix, lp, 8, 2, 128, 16, 10, causal=False)
    with pytest.raises(fb.FiError, match="more query tokens"):
        fb.prefill_plan(qo, ip, ix, lp, 8, 2, 128, 16, 10, causal=False, rope=True)


def test_fp8_plan_is_the_bf16_plan_with_its_dtype():
    """The cache's element type changes no scheduling: same items and merges,
    and get_info reports the dtype."""
    qo, ip, ix, lp = [0, 2, 3], [0, 2, 3], [5, 6, 7], [16, 3]
    a = fb.prefill_plan(np.array(qo), np.array(ip), np.array(ix), np.array(lp), 8, 2, 128, 16, 100)
    b = fb.prefill_plan(np.array(qo), np.array(ip), np.array(ix), np.array(lp), 8, 2, 128, 16, 100,
                        dtype="fp8")
    assert a.info["dtype"] == fb.FI_DTYPE_BF16 and b.info["dtype"] == fb.FI_DTYPE_FP8_E4M3
    ia, ib = dict(a.info), dict(b.info)
    ia.pop("dtype"), ib.pop("dtype")
    assert ia == ib
    assert np.array_equal(a.work_list(), b.work_list()) and np.array_equal(a.merges(), b.merges())


def test_group_size_limit_is_the_tile_height():
    # G = FI_PREFILL_ROWS is the largest group: one query token per tile
    assert _status([0, 2, 3], [0, 2, 3], [5, 6, 7], [16, 3], Hq=256, Hkv=1)[0] == 0
    assert _status([0, 2, 3], [0, 2, 3], [5, 6, 7], [16, 3], Hq=257, Hkv=1)[0] == -2


def test_more_queries_than_tokens_is_fine_without_the_mask():
    assert _status([0, 40, 41], [0, 2, 3], [5, 6, 7], [16, 3], causal=0)[0] == 0


@settings(max_examples=25, deadline=None)
@given(seed=st.integers(0, 10_000), B=st.integers(1, 6), L=st.integers(1, 700),
       G=st.sampled_from([1, 2, 3, 4, 8, 16]), P=st.sampled_from([1, 4, 16, 64]),
       causal=st.booleans(), fixed=st.sampled_from([0, 1, 50, 300]),
       cus=st.sampled_from([0, 4, 64]))
def test_prefill_plan_properties(seed, B, L, G, P, causal, fixed, cus):
    w = random_prefill_workload(seed, B, L, 2 * G, 2, 64, P, causal=causal)
    p = make_plan(w, fixed_chunk_tokens=fixed, num_cus=cus)
    check_prefill_plan(w, p)
