"""Composed formats on the host (fi_plan_create_composed): the plan covers
every prefix token and every own token exactly once, keeps within its
limits, refuses malformed input, and -- executed in float64 with the
oracle's own routines -- gives the composed oracle's result."""
import ctypes

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import block_sparse_kv_bsr_amd as fb
import oracle.attention as oa
from block_sparse_kv_bsr_amd.binding import PITEM_STRIDE
from block_sparse_kv_bsr_amd.workloads import random_composed_workload, workload

I_REQ, I_KVH, I_PB, I_NTOK, I_SLOT, I_CHUNK, I_NP, I_FIRST, I_NODE, I_KVPOS, I_QPOS = range(11)
N_COUNT, N_SB, N_PARENT, N_OUT, N_REQ, N_KVH, N_LEVEL, N_ARR = range(8)
P_GROUP, P_KVH, P_MBASE, P_ROW0, P_NROWS, P_CHUNK, P_PB, P_NP, P_TOFF, P_NTOK = range(10)
MAX_PAGES = 256


def make(w, **opts):
    return fb.plan_composed(w.kv_indptr, w.kv_indices, w.last_page_len, w.prefix_indptr,
                            w.prefix_indices, w.prefix_last_page_len, w.prefix_of,
                            w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                            w.num_pool_pages, w.prefix_page_size, w.num_prefix_pool_pages, **opts)


def run_composed_f64(w, p):
    """Every decode item and every prefix-item row attends over its tokens
    in float64 (oracle routines), and the states are folded up the plan's
    merge trees. Returns (out, lse)."""
    items, nodes = p.work_list(), p.merge_nodes()
    pitems, members = p.prefix_items(), p.prefix_members()
    q, k, v, kp, vp = (t.double().numpy() for t in w.make_values("cpu"))
    G, P, Pp = w.group_size, w.page_size, w.prefix_page_size
    ids = np.concatenate([w.kv_indices, w.prefix_indices]).astype(np.int64)
    nnz = len(w.kv_indices)
    # first tree slot of each (request, kv head): the smallest level-0 slot
    base = {}
    for n in nodes:
        if n[N_LEVEL] == 0:
            key = (int(n[N_REQ]), int(n[N_KVH]))
            base[key] = min(base.get(key, 1 << 40), int(n[N_SB]))
    slot_state = {}
    out = np.zeros((w.batch, w.num_qo_heads, w.head_dim))
    lse = np.full((w.batch, w.num_qo_heads), -np.inf)
    for r in items:
        b, h, ntok, npg = int(r[I_REQ]), int(r[I_KVH]), int(r[I_NTOK]), int(r[I_NP])
        if ntok == 0:
            continue
        assert r[I_PB] + npg <= nnz  # decode items read the requests' own pages
        toks = oa.request_tokens(np.array([0, npg]), ids[r[I_PB]:r[I_PB] + npg],
                                 np.array([ntok - (npg - 1) * P]), P, 0)
        K, V = oa.gather_kv(k, v, toks, h)
        st_ = oa.attend(q[b, h * G:(h + 1) * G], K, V, w.sm_scale)
        if r[I_SLOT] < 0:
            out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G] = st_
        else:
            slot_state[int(r[I_SLOT])] = st_
    for r in pitems:
        h, pb, npg, off, nt = (int(r[i]) for i in (P_KVH, P_PB, P_NP, P_TOFF, P_NTOK))
        assert pb >= nnz and 0 <= off < Pp and npg == -(-(off + nt) // Pp) and npg <= MAX_PAGES
        toks = [(int(ids[pb + j]), s) for j in range(npg) for s in range(Pp)][off:off + nt]
        K, V = oa.gather_kv(kp, vp, toks, h)
        ms = members[r[P_MBASE] + r[P_ROW0]: r[P_MBASE] + r[P_ROW0] + r[P_NROWS] // G]
        for b in ms:
            slot_state[base[(int(b), h)] + int(r[P_CHUNK])] = oa.attend(
                q[b, h * G:(h + 1) * G], K, V, w.sm_scale)
    for i in sorted(range(len(nodes)), key=lambda i: nodes[i][N_LEVEL]):
        n = nodes[i]
        kids = [slot_state[s] for s in range(n[N_SB], n[N_SB] + n[N_COUNT])]
        st_ = oa.merge_many([c[0] for c in kids], [c[1] for c in kids])
        if n[N_PARENT] < 0:
            b, h = int(n[N_REQ]), int(n[N_KVH])
            out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G] = st_
        else:
            slot_state[int(n[N_OUT])] = st_
    return out, lse


def check_composed(w, p):
    """Structure: each group's members are the requests of one prefix; per
    (group, KV head, row block) the chunks tile the prefix's tokens in order;
    positions of the decode items count the prefix first."""
    info = p.info
    pitems, members = p.prefix_items(), p.prefix_members()
    assert pitems.shape[1] == PITEM_STRIDE
    assert info["prefix_page_size"] == w.prefix_page_size
    assert info["total_kv_tokens"] == int(w.total_kv_lens().sum())
    fan = info["merge_fan_in"]
    G = w.group_size
    seen = {}
    for r in pitems:
        key = (int(r[P_GROUP]), int(r[P_KVH]), int(r[P_ROW0]))
        seen.setdefault(key, []).append((int(r[P_CHUNK]), int(r[P_PB]), int(r[P_TOFF]),
                                         int(r[P_NTOK]), int(r[P_MBASE]), int(r[P_NROWS])))
    nnz = len(w.kv_indices)
    groups_seen = set()
    for (g, h, row0), chunks in seen.items():
        chunks.sort()
        assert [c[0] for c in chunks] == list(range(len(chunks))) and len(chunks) <= fan - 1
        mbase, nrows = chunks[0][4], chunks[0][5]
        ms = members[mbase + row0: mbase + row0 + nrows // G]
        pg = {int(w.prefix_of[b]) for b in ms}
        assert len(pg) == 1 and -1 not in pg
        pref = pg.pop()
        groups_seen.add(pref)
        # the chunks cover tokens 0 .. prefix_len - 1 in order
        t = 0
        for c, pb, off, nt, _, _ in chunks:
            start = (pb - nnz - int(w.prefix_indptr[pref])) * w.prefix_page_size + off
            assert start == t and nt >= 1
            t += nt
        assert t == w.prefix_len(pref)
    want = {int(g) for b, g in enumerate(w.prefix_of) if g >= 0 and w.prefix_len(int(g)) > 0}
    assert groups_seen == want
    for b in range(w.batch):
        g = int(w.prefix_of[b])
        lead = w.prefix_len(g) if g >= 0 else 0
        for r in p.work_list():
            if r[I_REQ] == b and r[I_NTOK] > 0:
                assert r[I_QPOS] == lead + w.kv_len(b) - 1
                assert r[I_KVPOS] >= lead


CASES = [
    # seed, prefix_lens, members, singles, own_max, Hq, Hkv, d, P, Pp, fixed chunk
    (1, [40, 0, 17], [2, 1, 2], 1, 30, 8, 2, 64, 4, 16, 0),
    (2, [300], [3], 0, 20, 4, 1, 64, 1, 64, 8),
    (3, [33, 64], [1, 2], 2, 9, 16, 2, 128, 16, 32, 0),
    (4, [5, 129], [2, 2], 1, 40, 8, 8, 64, 16, 1, 16),
    (5, [4096 + 77], [40], 0, 5, 16, 4, 64, 16, 4096, 0),   # two row blocks, a partial block
    (6, [1000], [5], 3, 300, 32, 4, 128, 16, 100, 64),      # G 8, a non-power-of-two block
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"composed{c[0]}")
def test_composed_plan_equals_oracle(case):
    seed, plens, mem, singles, own_max, hq, hkv, d, P, Pp, fixed = case
    w = random_composed_workload(seed, plens, mem, singles, own_max, hq, hkv, d, P, Pp)
    p = make(w, fixed_chunk_tokens=fixed)
    check_composed(w, p)
    out, lse = run_composed_f64(w, p)
    q, k, v, kp, vp = (t.double().numpy() for t in w.make_values("cpu"))
    O, LSE = oa.decode_attention_composed(q, k, v, w.kv_indptr, w.kv_indices, w.last_page_len,
                                          kp, vp, w.prefix_indptr, w.prefix_indices,
                                          w.prefix_last_page_len, w.prefix_of, w.sm_scale)
    assert np.allclose(out, O, atol=1e-12, rtol=0) and np.allclose(lse, LSE, atol=1e-12, rtol=0)


@settings(max_examples=30, deadline=None)
@given(seed=st.integers(0, 10_000), plen=st.integers(0, 3000), members=st.integers(1, 40),
       singles=st.integers(0, 3), Pp=st.sampled_from([1, 7, 16, 64, 4096]),
       hkv=st.sampled_from([1, 2, 8]), num_cus=st.sampled_from([0, 3, 1000]))
def test_composed_plan_properties(seed, plen, members, singles, Pp, hkv, num_cus):
    if Pp == 1:
        plen = min(plen, 3000)
    w = random_composed_workload(seed, [plen], [members], singles, 40, 4 * hkv, hkv, 64, 16, Pp)
    p = make(w, num_cus=num_cus)
    check_composed(w, p)


def test_config13_plan():
    w = workload(13)
    p = make(w)
    check_composed(w, p)
    info = p.info
    assert info["num_prefix_groups"] == 1 and info["num_prefix_items"] == 15 * 8
    assert info["total_kv_tokens"] == int(workload(5).kv_lens().sum())


def _status(w, **kw):
    L = fb.lib()
    a = dict(ip=w.kv_indptr, ix=w.kv_indices, lp=w.last_page_len, pip=w.prefix_indptr,
             pix=w.prefix_indices, plp=w.prefix_last_page_len, of=w.prefix_of, Hq=w.num_qo_heads,
             Hkv=w.num_kv_heads, d=w.head_dim, P=w.page_size, pool=w.num_pool_pages,
             Pp=w.prefix_page_size, ppool=w.num_prefix_pool_pages, dtype=1)
    a.update(kw)
    arr = {k: np.ascontiguousarray(np.asarray(a[k], dtype=np.int32))
           for k in ("ip", "ix", "lp", "pip", "pix", "plp", "of")}
    p32 = lambda x: x.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    h = ctypes.c_void_p()
    st_ = L.fi_plan_create_composed(p32(arr["ip"]), p32(arr["ix"]), p32(arr["lp"]),
                                    len(arr["ip"]) - 1, p32(arr["pip"]), p32(arr["pix"]),
                                    p32(arr["plp"]), len(arr["pip"]) - 1, p32(arr["of"]), a["Hq"],
                                    a["Hkv"], a["d"], a["P"], a["pool"], a["Pp"], a["ppool"],
                                    a["dtype"], None, ctypes.byref(h))
    if st_ == 0:
        L.fi_plan_destroy(h)
    return st_, L.fi_last_error().decode()


def test_composed_rejects():
    w = random_composed_workload(7, [50, 20], [2, 1], 1, 30, 8, 2, 64, 16, 16)
    assert _status(w) == (0, "") or _status(w)[0] == 0
    of = w.prefix_of.copy()
    of[0] = 2
    st_, msg = _status(w, of=of)
    assert st_ == -1 and "prefix_of[0]" in msg
    of[0] = -2
    assert _status(w, of=of)[0] == -1
    assert _status(w, dtype=2)[0] == -2          # fp8: the prefix kernel reads bf16
    bad = w.prefix_indices.copy()
    bad[0] = w.num_prefix_pool_pages
    st_, msg = _status(w, pix=bad)
    assert st_ == -1 and msg.startswith("prefix table:")
    plp = w.prefix_last_page_len.copy()
    plp[0] = w.prefix_page_size + 1
    assert _status(w, plp=plp)[0] == -1
    # a request with a prefix needs one token of its own
    b = int(np.nonzero(w.prefix_of >= 0)[0][0])
    lens = [w.kv_len(i) for i in range(w.batch)]
    lists = [list(w.kv_indices[w.kv_indptr[i]:w.kv_indptr[i + 1]]) for i in range(w.batch)]
    lists[b], lens[b] = [], 0
    ip = np.cumsum([0] + [len(x) for x in lists])
    ix = np.array([x for l in lists for x in l], dtype=np.int32)
    lp = np.array([(L - 16 * (len(l) - 1)) if l else 0 for L, l in zip(lens, lists)])
    st_, msg = _status(w, ip=ip, ix=ix, lp=lp)
    assert st_ == -1 and "no token of its own" in msg
    # too long a prefix: more than (fan_in - 1) x 255 blocks
    long = random_composed_workload(8, [15 * 255 + 1], [1], 0, 5, 8, 2, 64, 16, 1)
    st_, msg = _status(long)
    assert st_ == -2 and "chunks" in msg


def test_runs_refuse_the_other_kind_of_plan():
    """Host checks, no launch: a composed plan is refused by fi_decode_run,
    and a plain plan by fi_decode_run_composed."""
    L = fb.lib()
    w = random_composed_workload(9, [40], [2], 1, 20, 8, 2, 128, 16, 16)
    pc = make(w)
    pp = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, 8, 2, 128, 16, w.num_pool_pages)
    fake = ctypes.c_void_p(0x100000)
    ws = pc.info["workspace_bytes"]
    assert L.fi_decode_run(pc.handle, fake, fake, fake, fake, None, 0.0, fake, ws, None) == -1
    assert "fi_decode_run_composed" in L.fi_last_error().decode()
    assert L.fi_decode_run_composed(pp.handle, fake, fake, fake, fake, fake, fake, None, 0.0, fake,
                                    ws, None) == -1
    assert "fi_plan_create_composed" in L.fi_last_error().decode()
    # NULL prefix caches with prefix items to run
    assert L.fi_decode_run_composed(pc.handle, fake, fake, fake, None, fake, fake, None, 0.0, fake,
                                    ws, None) == -1
    # not uploaded: FI_ERR_STATE after the argument checks
    assert L.fi_decode_run_composed(pc.handle, fake, fake, fake, fake, fake, fake, None, 0.0, fake,
                                    ws, None) == -6
