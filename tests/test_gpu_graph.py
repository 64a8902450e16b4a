"""The run entry points inside a captured HIP graph: no host synchronisation,
no allocation and no memset in the captured work (the merge counters reset
themselves), so a graph replays correctly. Each replay is checked bit for bit
against an eager run on the same inputs, with eager work and a change of
inputs between replays."""
import pytest
import torch

import block_sparse_kv_bsr_amd as fb
from block_sparse_kv_bsr_amd.workloads import (prefix_workload, random_composed_workload,
                                               random_prefill_workload, random_workload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fb.lib()


def log(*a):
    print(*a, flush=True)


def _replays(run, inputs, outputs, fresh_inputs, what):
    """Capture run() into a graph, then replay it three times: twice on the
    captured inputs and once after overwriting them with fresh_inputs; every
    replay must equal an eager run on the inputs it saw."""
    log(f"[case] graph {what}")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    originals = [t.clone() for t in inputs]
    for rep in range(3):
        if rep == 2:
            for t, f in zip(inputs, fresh_inputs):
                t.copy_(f)
        for o in outputs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outputs]
        # eager work between replays, then the eager reference
        run()
        torch.cuda.synchronize()
        for a, b in zip(got, outputs):
            assert torch.equal(a, b), f"{what}: replay {rep} differs from the eager run"
        torch.ones(1 << 20, device="cuda").sum().item()
    for t, o in zip(inputs, originals):
        t.copy_(o)
    log(f"[ok] graph {what}")


def test_graph_decode_with_split_requests():
    w = random_workload(101, 6, 3000, 32, 8, 128, 16, "bf16")
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, 32, 8, 128, 16, w.num_pool_pages, "bf16",
                fixed_chunk_tokens=256)
    assert p.info["num_merge_nodes"] > 0
    ws = torch.empty(p.info["workspace_bytes"], dtype=torch.uint8, device="cuda")
    p.upload(ws)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    _replays(lambda: fb.decode(q, k, v, p, out=out, lse=lse, workspace=ws), [q], [out, lse],
             [torch.randn_like(q)], "decode")


def test_graph_decode_rope_over_fp8_cache():
    """The rotary-embedding variant over an fp8 cache with dequantisation
    scales, requests cut into chunks at nonzero positions."""
    w = random_workload(104, 5, 2000, 32, 8, 128, 16, "fp8")
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, 32, 8, 128, 16, w.num_pool_pages, "fp8",
                fixed_chunk_tokens=192, cascade=-1)
    assert p.info["num_merge_nodes"] > 0
    ws = torch.empty(p.info["workspace_bytes"], dtype=torch.uint8, device="cuda")
    p.upload(ws)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    _replays(lambda: fb.decode(q, k, v, p, out=out, lse=lse, workspace=ws, k_scale=w.k_scale,
                               v_scale=w.v_scale, rope_theta=5e5), [q], [out, lse],
             [torch.randn_like(q)], "decode rope fp8")


def test_graph_decode_cascade():
    w = prefix_workload(102, [(6, 6)], 3, 300, 32, 8, 128, 16, "bf16")
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, 32, 8, 128, 16, w.num_pool_pages, "bf16",
                cascade=1)
    assert p.info["num_prefix_items"] > 0
    ws = torch.empty(p.info["workspace_bytes"], dtype=torch.uint8, device="cuda")
    p.upload(ws)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    _replays(lambda: fb.decode(q, k, v, p, out=out, lse=lse, workspace=ws), [q], [out, lse],
             [torch.randn_like(q)], "cascade")


def test_graph_prefill_with_cut_tiles():
    w = random_prefill_workload(103, 3, 900, 8, 2, 128, 16, causal=True)
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = fb.prefill_plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, 8, 2, 128, 16,
                        w.num_pool_pages, causal=True, fixed_chunk_tokens=128)
    assert p.info["num_merges"] > 0
    ws = torch.empty(p.info["workspace_bytes"], dtype=torch.uint8, device="cuda")
    p.upload(ws)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    _replays(lambda: fb.prefill(q, k, v, p, out=out, lse=lse, workspace=ws), [q], [out, lse],
             [torch.randn_like(q)], "prefill")


def test_graph_decode_composed():
    """Composed formats: the prefix cache's blocks (256 tokens) and the
    requests' own pages in one captured run, requests cut into chunks."""
    w = random_composed_workload(105, [3000], [9], 2, 400, 32, 8, 128, 16, 256)
    q, k, v, kp, vp = (t.cuda() for t in w.make_values("cpu"))
    p = fb.plan_composed(w.kv_indptr, w.kv_indices, w.last_page_len, w.prefix_indptr,
                         w.prefix_indices, w.prefix_last_page_len, w.prefix_of, w.num_qo_heads,
                         w.num_kv_heads, w.head_dim, w.page_size, w.num_pool_pages,
                         w.prefix_page_size, w.num_prefix_pool_pages)
    assert p.info["num_prefix_items"] > 0 and p.info["num_merge_nodes"] > 0
    ws = torch.empty(p.info["workspace_bytes"], dtype=torch.uint8, device="cuda")
    p.upload(ws)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    _replays(lambda: fb.decode_composed(q, k, v, kp, vp, p, out=out, lse=lse, workspace=ws), [q],
             [out, lse], [torch.randn_like(q)], "decode composed")


def _prefill_graph(w, what):
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = fb.prefill_plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, w.num_qo_heads,
                        w.num_kv_heads, w.head_dim, w.page_size, w.num_pool_pages,
                        causal=w.causal, dtype=w.dtype, rope=bool(w.rope_theta),
                        fixed_chunk_tokens=128)
    assert p.info["num_merges"] > 0
    ws = torch.empty(p.info["workspace_bytes"], dtype=torch.uint8, device="cuda")
    p.upload(ws)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    _replays(lambda: fb.prefill(q, k, v, p, out=out, lse=lse, workspace=ws, k_scale=w.k_scale,
                                v_scale=w.v_scale, rope_theta=w.rope_theta or None,
                                rope_scale=w.rope_scale), [q], [out, lse],
             [torch.randn_like(q)], what)


def test_graph_prefill_fp8_cache():
    _prefill_graph(random_prefill_workload(106, 3, 900, 8, 2, 128, 16, causal=True, dtype="fp8"),
                   "prefill fp8")


def test_graph_prefill_rope():
    _prefill_graph(random_prefill_workload(107, 3, 900, 8, 2, 128, 16, causal=True,
                                           rope_theta=5e5), "prefill rope")


def test_graph_mla():
    """MLA decode (tile kernel + merge of cut tiles) captured and replayed."""
    from block_sparse_kv_bsr_amd.workloads import random_mla_workload
    w = random_mla_workload(108, 4, 900, 96, 16, max_qo=2)
    qn, qp, ckv, kpe = (t.cuda() for t in w.make_values("cpu"))
    p = fb.mla_plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, w.num_heads,
                    w.page_size, w.num_pool_pages, fixed_chunk_tokens=128)
    assert p.info["num_merges"] > 0
    ws = torch.empty(p.info["workspace_bytes"], dtype=torch.uint8, device="cuda")
    p.upload(ws)
    out = torch.empty((w.num_qo_tokens, w.num_heads, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.num_qo_tokens, w.num_heads), dtype=torch.float32, device="cuda")
    _replays(lambda: fb.mla(qn, qp, ckv, kpe, p, w.sm_scale, out=out, lse=lse, workspace=ws),
             [qn], [out, lse], [torch.randn_like(qn)], "mla")
