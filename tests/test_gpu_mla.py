"""GPU parity of multi-head latent attention (fi_mla_run) through the C ABI
against the float64 latent-attention oracle, element by element.

Small ragged cases cover head counts 1 .. 128 (powers of two and not: 5, 12,
40, 96), one to six (speculative) query tokens per request, page sizes 1 ..
64, the causal mask and none, tiles cut into several chunks and not, and
chunks that end inside a 32-token block; NaN fills every unlisted page and
every slot past a request's last token. The full 96-head workload runs with
the plan bench.py times and is checked on every output element, and twenty
runs of it must agree bit for bit (cut tiles merge in whichever chunk
arrives last).
"""
import time

import numpy as np
import pytest
import torch

import block_sparse_kv_bsr_amd as fb
import oracle.attention as oa
from block_sparse_kv_bsr_amd.workloads import mla_workload, random_mla_workload
from tests.parity import compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fb.lib()


def log(*a):
    print(*a, flush=True)


def make(w, **opts):
    return fb.mla_plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, w.num_heads,
                       w.page_size, w.num_pool_pages, causal=w.causal, **opts)


def oracle(w, qn, qp, ckv, kpe):
    h = [t.double().cpu().numpy() for t in (qn, qp, ckv, kpe)]
    return oa.mla_attention(h[0], h[1], h[2], h[3], w.qo_indptr, w.kv_indptr, w.kv_indices,
                            w.last_page_len, w.sm_scale, w.causal)


def run_case(w, what, **opts):
    log(f"[case] {what} B={w.batch} N={w.num_qo_tokens} H={w.num_heads} P={w.page_size} "
        f"causal={w.causal} lens={list(w.kv_lens())[:8]} opts={opts}")
    qn, qp, ckv, kpe = (t.cuda() for t in w.make_values("cpu"))
    p = make(w, **opts)
    out, lse = fb.mla(qn, qp, ckv, kpe, p, w.sm_scale)
    torch.cuda.synchronize()
    t0 = time.time()
    O, LSE = oracle(w, qn, qp, ckv, kpe)
    stats = compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True, what)
    log(f"[ok] {what} items={p.info['num_items']} merges={p.info['num_merges']} "
        f"oracle {time.time() - t0:.1f}s {stats}")
    return p, (qn, qp, ckv, kpe), (out, lse)


CASES = [
    # seed, batch, max_len, heads, page size, max query tokens, causal, fixed chunk
    (1, 4, 300, 96, 16, 1, True, 0),
    (2, 4, 300, 96, 16, 1, True, 64),      # three head blocks, cut tiles
    (3, 5, 200, 12, 4, 3, True, 32),       # speculative tokens, two per tile
    (4, 3, 150, 40, 1, 2, True, 17),       # 32 + 8 head split, page size 1
    (5, 3, 90, 5, 64, 6, False, 0),        # six tokens per tile, no mask
    (6, 4, 700, 128, 16, 1, True, 0),
    (7, 6, 500, 16, 64, 4, True, 96),
    (8, 3, 260, 1, 16, 5, True, 48),       # one head
    (9, 4, 333, 32, 3, 1, True, 0),        # page size 3
    (10, 2, 40, 64, 16, 2, True, 0),       # short histories (a row attends one block)
    (11, 3, 150, 200, 16, 1, True, 48),    # six blocks of 32 heads and one of 8
    (12, 4, 120, 24, 16, 3, True, 0),      # a tile of one whole token (24 rows of 32)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_mla_small(case):
    seed, B, L, H, P, mq, causal, fixed = case
    w = random_mla_workload(seed, B, L, H, P, max_qo=mq, causal=causal)
    p, _, _ = run_case(w, f"mla seed{seed}", fixed_chunk_tokens=fixed)
    if fixed:
        assert p.info["num_merges"] > 0


def test_mla_one_token_histories_and_queries_equal_to_history():
    """Histories of 1 .. 3 tokens (every row attends few tokens: the hi + lo
    split of the weights is what keeps these within the bar), and requests
    whose every token is a query."""
    w = random_mla_workload(21, 5, 3, 24, 16, lens=[1, 2, 3, 1, 3], qo_lens=[1, 2, 3, 1, 1])
    run_case(w, "mla few tokens")


def test_mla_unmasked_empty_history():
    """No mask and a request without pages: its rows attend nothing (out 0,
    lse -inf); the other requests are unaffected."""
    w = random_mla_workload(22, 3, 80, 16, 16, lens=[40, 0, 77], qo_lens=[2, 1, 3], causal=False)
    run_case(w, "mla empty history")


def test_mla_is_deterministic():
    w = random_mla_workload(23, 4, 900, 96, 16)
    qn, qp, ckv, kpe = (t.cuda() for t in w.make_values("cpu"))
    p = make(w, fixed_chunk_tokens=128)
    a = [t.clone() for t in fb.mla(qn, qp, ckv, kpe, p, w.sm_scale)]
    b = fb.mla(qn, qp, ckv, kpe, p, w.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_mla_full_size_bitwise_repeatable():
    """Which chunk of a cut tile arrives last, and so merges the tile,
    depends on timing; the merged result must not. Twenty runs of the
    full-size 96-head batch (96 merged tiles), every other one after a cache
    flush so arrival orders differ, must equal the first run bit for bit;
    the test stops at the first mismatch and names the run."""
    w = mla_workload(15)
    qn, qp, ckv, kpe = (t.cuda() for t in w.make_values("cuda"))
    p = make(w)
    log(f"[case] mla repeat: {p.info['num_items']} items, {p.info['num_merges']} merges")
    assert p.info["num_merges"] > 0
    o0, l0 = fb.mla(qn, qp, ckv, kpe, p, w.sm_scale)
    out, lse = torch.empty_like(o0), torch.empty_like(l0)
    flush = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
    for run in range(1, 21):
        if run % 2:
            flush.zero_()
        fb.mla(qn, qp, ckv, kpe, p, w.sm_scale, out=out, lse=lse)
        torch.cuda.synchronize()
        same = torch.equal(out.view(torch.int16), o0.view(torch.int16)) and torch.equal(lse, l0)
        assert same, f"run {run} differs from run 0"
    log("[ok] mla repeat: 20 runs bitwise equal")


def test_mla_full_size():
    """The 96-head workload with the plan bench.py times, every output
    element against the oracle (one request at a time on the host)."""
    w = mla_workload(15)
    log(f"[case] mla full size {w.name}")
    qn, qp, ckv, kpe = (t.cuda() for t in w.make_values("cuda"))
    p = make(w)
    out, lse = fb.mla(qn, qp, ckv, kpe, p, w.sm_scale)
    torch.cuda.synchronize()
    t0 = time.time()
    hq = [t.double().cpu().numpy() for t in (qn, qp)]
    ckv_h, kpe_h = ckv.float().cpu().numpy(), kpe.float().cpu().numpy()
    out_h, lse_h = out.double().cpu().numpy(), lse.double().cpu().numpy()
    worst = {}
    for b in range(w.batch):
        q0, q1 = int(w.qo_indptr[b]), int(w.qo_indptr[b + 1])
        ip = np.array([0, w.kv_indptr[b + 1] - w.kv_indptr[b]], dtype=np.int64)
        ix = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
        O, LSE = oa.mla_attention(hq[0][q0:q1], hq[1][q0:q1], ckv_h, kpe_h, np.array([0, q1 - q0]),
                                  ip, ix, w.last_page_len[b:b + 1], w.sm_scale, w.causal)
        st = compare(out_h[q0:q1], lse_h[q0:q1], O, LSE, True, f"mla full size request {b}")
        for k, v in st.items():
            worst[k] = max(worst.get(k, 0), v)
    log(f"[ok] mla full size items={p.info['num_items']} merges={p.info['num_merges']} "
        f"oracle {time.time() - t0:.1f}s {worst}")
