"""The MLA planner (fi_mla_plan_create) on a CPU-only host: tile structure
(FI_MLA_ROWS (query token, head) rows: whole tokens for few heads, head
blocks of one token for many), chunks of whole pages, merges of cut tiles,
chunk-major order within a request, a float64 execution of the plan against
the latent-attention oracle, and the checks that reject malformed calls."""
import numpy as np
import pytest

import block_sparse_kv_bsr_amd as fb
from block_sparse_kv_bsr_amd import binding
from block_sparse_kv_bsr_amd.workloads import mla_workload, random_mla_workload
import oracle.attention as oa

REQ, KVH, QROW, NQO, KV0, NKV, VIS, PG0, SLOT, CHUNK, QPOS, HB, MERGE = range(13)
M_QROW, M_NQO, M_KVH, M_SLOT0, M_NCH, M_HB = range(6)
R = binding.MLA_ROWS
ERR_INVALID, ERR_UNSUPPORTED = -1, -2


def make(w, **kw):
    return fb.mla_plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, w.num_heads,
                       w.page_size, w.num_pool_pages, causal=w.causal, **kw)


def tile_rows(it, H):
    """(query row, head) pairs of an item's tile."""
    f0, n = int(it[HB]), int(it[NQO]) * H
    return [(int(it[QROW]) + f // H, f % H) for f in range(f0, min(f0 + R, n))]


def check_plan(w, p):
    items, merges, info = p.work_list(), p.merges(), p.info
    H, P = w.num_heads, w.page_size
    assert info["mla"] == 1 and info["num_kv_heads"] == 1 and info["num_qo_heads"] == H
    assert info["head_dim"] == 512 and info["head_dim_kpe"] == 64
    T = max(1, R // H)
    assert info["tokens_per_tile"] == T
    L, qo = w.kv_lens(), w.qo_indptr
    tiles = {}
    for it in items:
        b = int(it[REQ])
        n = int(qo[b + 1] - qo[b])
        t0 = int(it[QROW]) - int(qo[b])
        assert int(it[KVH]) == 0 and 0 <= t0 < n
        if H <= R:
            assert t0 % T == 0 and int(it[HB]) == 0 and int(it[NQO]) == min(T, n - t0)
        else:
            assert int(it[NQO]) == 1 and int(it[HB]) % R == 0 and int(it[HB]) < H
        assert int(it[VIS]) == (int(L[b]) - n + t0 + 1 if w.causal else int(L[b]))
        assert int(it[KV0]) % P == 0
        assert int(it[PG0]) == int(w.kv_indptr[b]) + int(it[KV0]) // P
        assert int(it[NKV]) <= binding.MLA_MAX_PAGES * P
        tiles.setdefault((int(it[QROW]), int(it[HB])), []).append(it)
    # every (query token, head) row in exactly one tile
    cover = {}
    for its in tiles.values():
        for rh in tile_rows(its[0], H):
            cover[rh] = cover.get(rh, 0) + 1
    assert len(cover) == w.num_qo_tokens * H and set(cover.values()) <= {1}
    for (r0, hb), its in tiles.items():
        its = sorted(its, key=lambda x: int(x[CHUNK]))
        pos = 0
        for x in its:
            assert int(x[KV0]) == pos
            pos += int(x[NKV])
        b = int(its[0][REQ])
        last_vis = int(its[0][VIS]) + (int(its[0][NQO]) - 1 if w.causal else 0)
        assert pos == last_vis
        slots = [int(x[SLOT]) for x in its]
        assert slots == ([-1] if len(its) == 1 else list(range(slots[0], slots[0] + len(its))))
    cut = {k: v for k, v in tiles.items() if len(v) > 1}
    assert len(merges) == len(cut) == info["num_merges"]
    for mi, m in enumerate(merges):
        its = cut[(int(m[M_QROW]), int(m[M_HB]))]
        assert int(m[M_NCH]) == len(its) and int(m[M_NQO]) == int(its[0][NQO])
        assert int(m[M_SLOT0]) == min(int(x[SLOT]) for x in its)
        # each chunk of a cut tile names the tile's merge (its arrival counter)
        assert all(int(x[MERGE]) == mi for x in its)
    for its in tiles.values():
        if len(its) == 1:
            assert int(its[0][MERGE]) == -1
    assert np.all(items[:, MERGE + 1:] == 0)
    # within a request, chunk-major: the tiles that read one chunk are adjacent
    for b in set(int(x) for x in items[:, REQ]):
        kv0 = items[items[:, REQ] == b][:, KV0]
        assert np.all(np.diff(kv0) >= 0), b
    assert info["visible_pairs"] == w.visible_pairs()


def run_plan_f64(w, p, qn, qp, ckv, kpe):
    """Each item attends its chunk (cut at each row's visible count) with
    the oracle's attention; cut tiles merge their chunks in chunk order."""
    items, H = p.work_list(), w.num_heads
    parts = {}
    for it in items:
        b = int(it[REQ])
        toks = oa.request_tokens(w.kv_indptr, w.kv_indices, w.last_page_len, w.page_size, b)
        C, Rk = oa.gather_latent(ckv, kpe, toks)
        K = np.concatenate([C, Rk], axis=1)
        k0, nk = int(it[KV0]), int(it[NKV])
        for (r, h) in tile_rows(it, H):
            j = r - int(it[QROW])
            lim = int(it[VIS]) + (j if w.causal else 0)
            hi = min(k0 + nk, lim)
            lo = min(k0, hi)
            q = np.concatenate([qn[r, h], qp[r, h]])[None]
            o, lse = oa.attend(q, K[lo:hi], C[lo:hi], w.sm_scale)
            parts.setdefault((r, h), []).append((int(it[CHUNK]), o[0], lse[0]))
    O = np.full((w.num_qo_tokens, H, 512), np.nan)
    LSE = np.full((w.num_qo_tokens, H), np.nan)
    for (r, h), ch in parts.items():
        ch.sort(key=lambda x: x[0])
        o, lse = oa.merge_many([c[1][None] for c in ch], [np.array([c[2]]) for c in ch])
        O[r, h], LSE[r, h] = o[0], lse[0]
    return O, LSE


CASES = [
    # seed, batch, max_len, heads, page size, max query tokens, causal, fixed chunk
    (1, 3, 300, 96, 16, 1, True, 64),     # three head blocks, cut tiles
    (2, 4, 200, 12, 4, 3, True, 32),      # two tokens per tile, speculative queries
    (3, 3, 150, 40, 1, 2, True, 17),      # a tile across token boundaries, page size 1
    (6, 3, 150, 200, 16, 2, True, 48),    # six blocks of 32 heads and one of 8
    (4, 2, 90, 5, 64, 4, False, 0),       # six tokens per tile, no mask
    (5, 3, 400, 128, 16, 1, True, 0),     # planner's own chunk length
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_mla_plan_structure_and_f64_execution(case):
    seed, B, L, H, P, mq, causal, fixed = case
    w = random_mla_workload(seed, B, L, H, P, max_qo=mq, causal=causal)
    p = make(w, fixed_chunk_tokens=fixed)
    check_plan(w, p)
    rng = np.random.default_rng([seed, 9])
    qn = rng.standard_normal((w.num_qo_tokens, H, 512))
    qp = rng.standard_normal((w.num_qo_tokens, H, 64))
    ckv = rng.standard_normal((w.num_pool_pages, P, 512))
    kpe = rng.standard_normal((w.num_pool_pages, P, 64))
    O, LSE = run_plan_f64(w, p, qn, qp, ckv, kpe)
    Oo, LSEo = oa.mla_attention(qn, qp, ckv, kpe, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                w.last_page_len, w.sm_scale, w.causal)
    assert np.allclose(O, Oo, atol=1e-12, rtol=0) and np.allclose(LSE, LSEo, atol=1e-12, rtol=0)


def test_full_size_mla_workload_plans():
    w = mla_workload(15)
    p = make(w)
    check_plan(w, p)
    info = p.info
    # 96 heads: three tiles of 32 heads per request; long requests cut into
    # chunks of at least 1024 tokens
    assert info["num_tiles"] == 3 * w.batch
    assert info["chunk_tokens"] >= 1024 and info["num_items"] >= 2 * 256
    # the workspace's partial states: FI_MLA_ROWS rows x 512 floats per slot
    assert info["workspace_bytes"] >= info["num_partial_slots"] * R * 512 * 4


def test_mla_plan_rejects():
    w = random_mla_workload(7, 2, 50, 8, 16)
    L = binding.lib()
    import ctypes
    h = ctypes.c_void_p()

    def call(H=8, dc=512, dr=64, rope=0):
        o = binding.PrefillOpts(0, 0, 0, 0, rope)
        qp_, ip, ix, lp = (binding._i32(a) for a in (w.qo_indptr, w.kv_indptr, w.kv_indices,
                                                       w.last_page_len))
        return L.fi_mla_plan_create(binding._ptr32(qp_), binding._ptr32(ip), binding._ptr32(ix),
                                    binding._ptr32(lp), w.batch, H, dc, dr, w.page_size,
                                    w.num_pool_pages, 1, ctypes.byref(o), ctypes.byref(h))
    assert call() == binding.FI_OK
    L.fi_prefill_plan_destroy(h)
    assert call(dc=576) == ERR_UNSUPPORTED
    assert b"512-wide latent" in L.fi_last_error()
    assert call(dr=128) == ERR_UNSUPPORTED
    assert call(H=0) == ERR_INVALID
    assert call(rope=1) == ERR_UNSUPPORTED
    # more queries than cached tokens under the causal mask
    with pytest.raises(binding.FiError, match="more query tokens"):
        fb.mla_plan([0, 3], [0, 1], [0], [2], 8, 16, 4)


def test_prefill_runs_refuse_an_mla_plan_and_mla_refuses_others():
    import ctypes
    w = random_mla_workload(8, 2, 40, 8, 16)
    p = make(w)
    L = binding.lib()
    null = ctypes.c_void_p(16)
    st = L.fi_prefill_run(p.handle, null, null, null, null, None, 0.0, null, 1 << 20, None)
    assert st == ERR_INVALID and b"fi_mla_run" in L.fi_last_error()
    st = L.fi_mla_run(p.handle, null, null, null, null, null, None, 0.0, null, 1 << 20, None)
    assert st == ERR_INVALID and b"sm_scale" in L.fi_last_error()
    pw = fb.prefill_plan([0, 1], [0, 1], [0], [5], 8, 2, 128, 16, 4)
    st = L.fi_mla_run(pw.handle, null, null, null, null, null, None, 0.1, null, 1 << 20, None)
    assert st == ERR_INVALID and b"fi_mla_plan_create" in L.fi_last_error()
