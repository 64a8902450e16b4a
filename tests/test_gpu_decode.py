"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Small ragged cases cover every built variant (dtype x head_dim x GQA group),
page sizes that do and do not divide the 8-token step, empty requests, forced
splits and NaN in every slot that must not be read; the five workloads run at
full size with the same default plan bench.py times.
"""
import time

import numpy as np
import pytest
import torch

import block_sparse_kv_bsr_amd as fb
import oracle.attention as oa
from block_sparse_kv_bsr_amd.workloads import (prefix_workload, random_prefill_workload,
                                               random_workload, workload)
from tests.parity import compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fb.lib()


def log(*a):
    print(*a, flush=True)


def host_values(w, q, k, v):
    """q, K, V for the oracle in float64 (an fp8 cache dequantised by the
    oracle's own E4M3 decoder and scales)."""
    qh = q.double().cpu().numpy()
    if w.dtype == "fp8":
        return (qh, oa.dequantize_e4m3(k.view(torch.uint8).cpu().numpy(), w.k_scale),
                oa.dequantize_e4m3(v.view(torch.uint8).cpu().numpy(), w.v_scale))
    return qh, k.double().cpu().numpy(), v.double().cpu().numpy()


def run_case(w, device_values=False, what="", **opts):
    log(f"[case] {what} B={w.batch} Hq={w.num_qo_heads} Hkv={w.num_kv_heads} d={w.head_dim} "
        f"P={w.page_size} {w.dtype} opts={opts}")
    if device_values:
        q, k, v = w.make_values("cuda")
    else:
        q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, w.num_qo_heads, w.num_kv_heads,
                w.head_dim, w.page_size, w.num_pool_pages, w.dtype, **opts)
    out, lse = fb.decode(q, k, v, p, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    t0 = time.time()
    qh, kh, vh = host_values(w, q, k, v)
    O, LSE = oa.decode_attention(qh, kh, vh, w.kv_indptr, w.kv_indices, w.last_page_len, w.sm_scale)
    stats = compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE,
                    w.dtype != "f32", what)
    log(f"[ok] {what} plan={p.info['num_items']} items chunk={p.info['chunk_pages']}p "
        f"oracle {time.time() - t0:.1f}s {stats}")
    return p, (q, k, v), (out, lse)


SMALL = [
    # seed, B, maxL, Hq, Hkv, d, P, dtype, empty_every
    (1, 4, 300, 4, 1, 64, 16, "f32", 0),
    (2, 5, 257, 8, 2, 128, 16, "bf16", 0),
    (3, 6, 200, 8, 8, 128, 16, "bf16", 3),
    (4, 3, 500, 16, 8, 128, 16, "bf16", 0),
    (5, 4, 333, 32, 4, 128, 16, "bf16", 0),
    (6, 4, 180, 8, 2, 64, 16, "bf16", 2),
    (7, 3, 99, 4, 4, 64, 8, "f32", 0),
    (8, 3, 140, 8, 2, 128, 16, "f32", 0),
    (9, 3, 90, 16, 2, 64, 4, "f32", 0),
    (10, 2, 130, 16, 2, 128, 16, "f32", 0),
    (11, 4, 70, 8, 2, 128, 1, "bf16", 0),
    (12, 4, 90, 8, 2, 128, 3, "bf16", 0),
    (13, 4, 220, 8, 2, 128, 12, "bf16", 0),
    (14, 3, 700, 8, 2, 128, 64, "bf16", 0),
    (15, 3, 300, 8, 1, 128, 32, "bf16", 0),
    (16, 2, 50, 4, 4, 64, 5, "f32", 0),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"s{c[0]}_{c[7]}_d{c[5]}_G{c[3] // c[4]}_P{c[6]}")
def test_small_default_plan(case):
    seed, B, L, Hq, Hkv, d, P, dt, ee = case
    w = random_workload(seed, B, L, Hq, Hkv, d, P, dt, empty_every=ee)
    run_case(w, what=f"small{seed}")


@pytest.mark.parametrize("case", SMALL[:8] + SMALL[10:14], ids=lambda c: f"s{c[0]}_split")
def test_small_forced_split(case):
    """A tiny chunk length forces many chunks per request, partial states and
    the in-kernel merge, including chunks that end inside the 8-token step."""
    seed, B, L, Hq, Hkv, d, P, dt, ee = case
    w = random_workload(seed, B, L, Hq, Hkv, d, P, dt, empty_every=ee)
    run_case(w, what=f"split{seed}", fixed_chunk_tokens=max(P, 20))


def test_single_token_and_exact_step_lengths():
    lens = [1, 7, 8, 9, 15, 16, 17, 64, 0]
    w = random_workload(31, len(lens), 0, 8, 2, 128, 16, "bf16", lens=lens)
    run_case(w, what="edge-lengths")
    run_case(w, what="edge-lengths-split", fixed_chunk_tokens=16)


def test_all_requests_empty():
    w = random_workload(32, 3, 0, 8, 2, 128, 16, "bf16", lens=[0, 0, 0])
    run_case(w, what="all-empty")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 11])
def test_config_full_size(cfg):
    w = workload(cfg)
    p, _, _ = run_case(w, device_values=cfg > 1, what=f"config{cfg}")
    if cfg == 4:
        assert p.info["min_chunks_split_request"] >= 64


@pytest.mark.parametrize("dtype,d,hq,hkv", [("bf16", 128, 8, 2), ("bf16", 64, 4, 4),
                                           ("f32", 64, 16, 2), ("f32", 128, 8, 8)])
def test_merge_tree_levels(dtype, d, hq, hkv):
    """One-token chunks on page size 1 cut requests into up to 1100 chunks:
    in-kernel merge trees of one to four levels, leaf nodes with a single
    child, every per-lane merge width, and repeated runs
    on one workspace. The runs alternate between two query sets, so a merge
    that read a partial state left in some cache by the previous run, or a
    counter not returned to zero, would give a wrong result."""
    lens = [70, 33, 32, 1, 0, 1100, 2]
    w = random_workload(41, len(lens), 0, hq, hkv, d, 1, dtype, lens=lens)
    p, (q, k, v), (o0, l0) = run_case(w, what=f"tree-{dtype}-d{d}-G{hq // hkv}",
                                      fixed_chunk_tokens=1)
    # levels of the tree over the longest request's 1100 chunks
    f, n, levels = p.info["merge_fan_in"], 1100, 0
    while n > 1:
        n, levels = -(-n // f), levels + 1
    assert p.merge_nodes()[:, 6].max() == levels - 1 >= 2
    q2 = torch.flip(q, dims=[0]).contiguous()
    o2, l2 = fb.decode(q2, k, v, p)
    torch.cuda.synchronize()
    O2, LSE2 = oa.decode_attention(q2.float().cpu().numpy(), k.float().cpu().numpy(),
                                   v.float().cpu().numpy(), w.kv_indptr, w.kv_indices,
                                   w.last_page_len, w.sm_scale)
    compare(o2.double().cpu().numpy(), l2.double().cpu().numpy(), O2, LSE2, dtype == "bf16",
            "tree-q2")
    for i in range(4):
        qi, oi, li = (q, o0, l0) if i % 2 == 0 else (q2, o2, l2)
        o1, l1 = fb.decode(qi, k, v, p)
        torch.cuda.synchronize()
        assert torch.equal(o1, oi) and torch.equal(l1, li), f"run {i}"


CASCADE = [
    # seed, groups [(members, prefix pages)], singles, suffix_max, Hq, Hkv, d, P, fixed chunk
    (1, [(5, 3)], 2, 40, 8, 2, 64, 4, 0),
    (2, [(3, 1), (4, 6)], 3, 70, 16, 4, 128, 8, 16),
    (3, [(40, 2)], 0, 20, 16, 4, 64, 4, 0),          # two row blocks of members
    (4, [(2, 9)], 1, 9, 4, 4, 64, 3, 3),             # G 1, page size 3 (prefix 30 tokens)
    (5, [(3, 4)], 0, 5, 32, 4, 128, 16, 0),          # G 8
    (6, [(33, 40), (2, 3)], 4, 300, 32, 8, 128, 16, 64),  # 40-page prefix, fan-in - 1 chunks
    (7, [(6, 5)], 2, 700, 32, 8, 128, 64, 0),        # page size 64
]


@pytest.mark.parametrize("case", CASCADE, ids=lambda c: f"cascade{c[0]}")
def test_cascade(case):
    """Shared prefixes through the matrix-core prefix kernel (forced on), then
    the decode kernel and its merge trees; repeated runs on one workspace give
    identical results."""
    seed, groups, singles, smax, hq, hkv, d, P, fixed = case
    w = prefix_workload(seed, groups, singles, smax, hq, hkv, d, P, "bf16")
    p, (q, k, v), (o0, l0) = run_case(w, what=f"cascade{seed}", cascade=1, fixed_chunk_tokens=fixed)
    assert p.info["num_prefix_items"] > 0
    for _ in range(2):
        o1, l1 = fb.decode(q, k, v, p)
        torch.cuda.synchronize()
        assert torch.equal(o1, o0) and torch.equal(l1, l0)


def test_cascade_matches_plain_decode_on_shared_prefix_workload():
    """The sparse shared-prefix workload with and without the cascade: both
    within tolerance of the oracle (run_case), and of each other."""
    w = workload(5)
    p1, vals, (o1, l1) = run_case(w, device_values=True, what="config5-cascade")
    assert p1.info["num_prefix_items"] > 0
    p0, _, (o0, l0) = run_case(w, device_values=True, what="config5-plain", cascade=-1)
    assert p0.info["num_prefix_items"] == 0
    assert (o1.float() - o0.float()).abs().max().item() <= 2 * 2 ** -7
    assert (l1 - l0).abs().max().item() <= 1e-4


FP8 = [
    # seed, B, maxL, Hq, Hkv, P, empty_every, fixed chunk
    (51, 4, 300, 8, 2, 16, 0, 0),
    (52, 5, 257, 8, 8, 16, 3, 0),     # G 1
    (53, 3, 500, 16, 8, 16, 0, 48),   # G 2, forced split
    (54, 4, 333, 32, 4, 16, 0, 32),   # G 8, forced split
    (55, 4, 90, 8, 2, 3, 2, 0),       # page size 3 (per-lane addressing)
    (56, 3, 700, 8, 2, 64, 0, 64),
    (57, 4, 70, 8, 2, 1, 0, 20),
]


@pytest.mark.parametrize("case", FP8, ids=lambda c: f"fp8_s{c[0]}_G{c[3] // c[4]}_P{c[5]}")
def test_fp8_kv(case):
    """fp8 e4m3 K/V with bf16 q/out, dequantised inside the kernel, against the
    oracle over the dequantised cache; NaN codes in every slot that must not
    be read."""
    seed, B, L, hq, hkv, P, ee, fixed = case
    w = random_workload(seed, B, L, hq, hkv, 128, P, "fp8", empty_every=ee)
    run_case(w, what=f"fp8-{seed}", fixed_chunk_tokens=fixed)


def test_fp8_skewed_batch_full_size():
    w = workload(6)
    p, (q, k, v), (o0, l0) = run_case(w, device_values=True, what="config6-fp8")
    o1, l1 = fb.decode(q, k, v, p, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o0) and torch.equal(l1, l0)


def test_kv_scales_on_bf16_cache():
    """fi_decode_run_scaled on a bf16 cache: scaling K by a and V by c equals
    the oracle with K and V multiplied by a and c."""
    w = random_workload(58, 4, 200, 8, 2, 128, 16, "bf16")
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, w.num_qo_heads, w.num_kv_heads,
                w.head_dim, w.page_size, w.num_pool_pages, w.dtype)
    out, lse = fb.decode(q, k, v, p, k_scale=0.5, v_scale=3.0)
    torch.cuda.synchronize()
    qh, kh, vh = host_values(w, q, k, v)
    O, LSE = oa.decode_attention(qh, 0.5 * kh, 3.0 * vh, w.kv_indptr, w.kv_indices, w.last_page_len,
                                 w.sm_scale)
    compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True, "kv-scales")


def test_deterministic_for_fixed_plan():
    w = workload(3)
    q, k, v = w.make_values("cuda")
    p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, w.num_qo_heads, w.num_kv_heads,
                w.head_dim, w.page_size, w.num_pool_pages, w.dtype)
    o1, l1 = fb.decode(q, k, v, p)
    o2, l2 = fb.decode(q, k, v, p)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_page_order_permutation():
    """Permuting a request's full pages (the partial page stays last) gives the
    same result within tolerance."""
    w = random_workload(40, 5, 600, 16, 4, 128, 16, "bf16")
    p0, (q, k, v), (o0, l0) = run_case(w, what="perm-base")
    rng = np.random.default_rng(1)
    ix = w.kv_indices.copy()
    for b in range(w.batch):
        s, t = w.kv_indptr[b], w.kv_indptr[b + 1]
        if t - s > 2:
            ix[s:t - 1] = ix[s:t - 1][rng.permutation(t - 1 - s)]
    p1 = fb.plan(w.kv_indptr, ix, w.last_page_len, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                 w.page_size, w.num_pool_pages, w.dtype)
    o1, l1 = fb.decode(q, k, v, p1)
    torch.cuda.synchronize()
    assert (o1.float() - o0.float()).abs().max().item() <= 2 * 2 ** -7
    assert (l1 - l0).abs().max().item() <= 1e-4


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_merge_states(dtype, d):
    g = torch.Generator().manual_seed(5)
    n = 1000
    va = torch.randn(n, d, generator=g)
    vb = torch.randn(n, d, generator=g)
    sa = torch.randn(n, generator=g) * 4
    sb = torch.randn(n, generator=g) * 4
    sa[::7] = -float("inf")
    sb[::11] = -float("inf")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    va, vb = va.to(tdt), vb.to(tdt)
    log(f"[case] merge_states {dtype} d={d}")
    vo, so = fb.merge_states(va.cuda(), sa.cuda(), vb.cuda(), sb.cuda())
    torch.cuda.synchronize()
    V, S = oa.merge_states(va.double().numpy(), sa.double().numpy(), vb.double().numpy(),
                           sb.double().numpy())
    compare(vo.double().cpu().numpy(), so.double().cpu().numpy(), V, S, dtype == "bf16",
            f"merge_states {dtype} d={d}")
    # in place on a (output aliases the first state)
    va2, sa2 = va.cuda(), sa.cuda()
    fb.merge_states(va2, sa2, vb.cuda(), sb.cuda(), v_out=va2, s_out=sa2)
    torch.cuda.synchronize()
    assert torch.equal(va2.cpu().view(torch.int16 if dtype == "bf16" else torch.int32),
                       vo.cpu().view(torch.int16 if dtype == "bf16" else torch.int32))


def test_binding_refuses_bad_buffers():
    """The C ABI cannot see buffer sizes, so the binding refuses outputs of the
    wrong shape or dtype, a pool smaller than the plan's, tensors on another
    device kind, and mismatched merge inputs, before any kernel runs."""
    w = random_workload(59, 3, 100, 8, 2, 128, 16, "bf16")
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, 8, 2, 128, 16, w.num_pool_pages, "bf16")
    B = w.batch
    with pytest.raises(ValueError, match="out must be"):
        fb.decode(q, k, v, p, out=torch.empty((B, 8, 64), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError, match="lse must be"):
        fb.decode(q, k, v, p, lse=torch.empty((B, 8), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError, match="pages"):
        fb.decode(q, k[:-4].contiguous(), v[:-4].contiguous(), p)
    with pytest.raises(RuntimeError, match="GPU tensor"):
        fb.decode(q.cpu(), k, v, p)
    a = torch.randn(5, 64, device="cuda")
    s = torch.randn(5, device="cuda")
    with pytest.raises(ValueError, match="one dtype"):
        fb.merge_states(a, s, a.bfloat16(), s)
    with pytest.raises(ValueError, match="v_out must be"):
        fb.merge_states(a, s, a, s, v_out=torch.empty(4, 64, device="cuda"))
    wp = random_prefill_workload(60, 2, 80, 8, 2, 128, 16)
    qp, kp, vp = (t.cuda() for t in wp.make_values("cpu"))
    pp = fb.prefill_plan(wp.qo_indptr, wp.kv_indptr, wp.kv_indices, wp.last_page_len, 8, 2, 128,
                         16, wp.num_pool_pages)
    with pytest.raises(ValueError, match="out must be"):
        fb.prefill(qp, kp, vp, pp, out=torch.empty((1, 8, 128), dtype=torch.bfloat16, device="cuda"))
    # the same calls with good buffers still run
    fb.decode(q, k, v, p)
    fb.prefill(qp, kp, vp, pp)
    torch.cuda.synchronize()


def test_fp8_tails_of_five_to_eight_steps():
    """The fp8 variant keeps 8 steps in flight; a chunk whose last ragged
    stretch spans 5..8 steps reads ring stages 4..7 in the tail pass, each
    only after its own loads have landed (lengths 37 .. 127 tokens, one item
    per request, and the same cut into 40-token chunks)."""
    lens = [37, 45, 53, 61, 63, 100, 109, 127]
    for fixed in (0, 40):
        w = random_workload(61, len(lens), 0, 8, 2, 128, 16, "fp8", lens=lens)
        run_case(w, what=f"fp8-tails fixed={fixed}", fixed_chunk_tokens=fixed)


def test_back_to_back_uploads_through_the_staging_cache():
    """Plan uploads stage through page-locked blocks the library caches for the
    process and reuses once their copies have run. Plans whose images fall in
    different size classes (64 KiB to 512 KiB) are uploaded back to back on
    one stream with no wait, each followed by a plan that is uploaded and
    destroyed at once; every surviving plan's decode must then match the
    oracle, and uploading the same plans again (now through reclaimed
    blocks) must give bit-identical results."""
    shapes = [(3, 200, 16), (4, 20000, 1), (2, 60000, 1), (5, 900, 4)]
    cases = []
    for i, (B, L, P) in enumerate(shapes):
        w = random_workload(300 + i, B, L, 8, 2, 128, P, "bf16")
        q, k, v = (t.cuda() for t in w.make_values("cpu"))
        p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, 8, 2, 128, P,
                    w.num_pool_pages, "bf16")
        cases.append((w, (q, k, v), p))
    log("[case] staging: workspace bytes", [p.info["workspace_bytes"] for _, _, p in cases])
    results = []
    for rnd in range(2):
        torch.cuda.synchronize()
        for w, _, p in cases:
            p.upload(torch.empty(max(256, p.info["workspace_bytes"]), dtype=torch.uint8,
                                 device="cuda"))
            other = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, 8, 2, 128, w.page_size,
                            w.num_pool_pages, "bf16", fixed_chunk_tokens=64)
            other.upload(torch.empty(max(256, other.info["workspace_bytes"]),
                                     dtype=torch.uint8, device="cuda"))
            del other
        outs = [fb.decode(q, k, v, p) for _, (q, k, v), p in cases]
        torch.cuda.synchronize()
        results.append(outs)
    for (w, (q, k, v), p), (o1, l1), (o2, l2) in zip(cases, results[0], results[1]):
        qh, kh, vh = host_values(w, q, k, v)
        O, LSE = oa.decode_attention(qh, kh, vh, w.kv_indptr, w.kv_indices, w.last_page_len,
                                     w.sm_scale)
        compare(o1.double().cpu().numpy(), l1.double().cpu().numpy(), O, LSE, True, "staging")
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    log("[ok] staging")


def test_workspace_holds_only_the_last_uploaded_plan():
    """A run reads the item list of the plan last uploaded to its workspace,
    so it must be that plan: uploading plan B (or a prefill plan) over plan
    A's workspace makes A's runs fail with FI_ERR_STATE, on the host, with
    nothing launched, until A is uploaded again; a plan never uploaded fails
    the same way."""
    w = random_workload(41, 4, 300, 8, 2, 128, 16, "bf16")
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    mk = lambda **o: fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, 8, 2, 128, 16,
                             w.num_pool_pages, "bf16", **o)
    pa, pb = mk(), mk(fixed_chunk_tokens=16)
    assert pb.info["num_items"] != pa.info["num_items"]
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    pa.upload(ws)
    oa1, la1 = fb.decode(q, k, v, pa, workspace=ws)
    pb.upload(ws)
    with pytest.raises(fb.FiError) as e:
        fb.decode(q, k, v, pa, workspace=ws)
    assert e.value.status == -6
    ob, lb = fb.decode(q, k, v, pb, workspace=ws)
    torch.cuda.synchronize()
    qh, kh, vh = host_values(w, q, k, v)
    O, LSE = oa.decode_attention(qh, kh, vh, w.kv_indptr, w.kv_indices, w.last_page_len, w.sm_scale)
    compare(ob.double().cpu().numpy(), lb.double().cpu().numpy(), O, LSE, True, "second plan")
    # a prefill plan uploaded over part of the same bytes drops pb's record
    wp = random_prefill_workload(42, 2, 100, 8, 2, 128, 16)
    pf = fb.prefill_plan(wp.qo_indptr, wp.kv_indptr, wp.kv_indices, wp.last_page_len, 8, 2, 128,
                         16, wp.num_pool_pages)
    pf.upload(ws[256:])
    with pytest.raises(fb.FiError) as e:
        fb.decode(q, k, v, pb, workspace=ws)
    assert e.value.status == -6
    # uploading A again makes it valid again, with the same result
    pa.upload(ws)
    oa2, la2 = fb.decode(q, k, v, pa, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(oa1.view(torch.int16), oa2.view(torch.int16)) and torch.equal(la1, la2)
    compare(oa2.double().cpu().numpy(), la2.double().cpu().numpy(), O, LSE, True, "first plan again")
    # a plan that was never uploaded, whatever address it lives at
    pc = mk(fixed_chunk_tokens=32)
    with pytest.raises(fb.FiError) as e:
        fb.decode(q, k, v, pc, workspace=ws)
    assert e.value.status == -6
    log("[ok] upload records")


@pytest.mark.parametrize("cfg", [3, 4])
def test_full_size_bitwise_repeatable(cfg):
    """Which wave completes a merge node depends on timing; the merged result
    must not. Twenty runs of the full-size skewed batch (one-level trees) and
    the long batch (two-level trees), every other one after a cache flush so
    arrival orders differ, must equal the first run bit for bit; the test
    stops at the first mismatch and names the run."""
    w = workload(cfg)
    q, k, v = w.make_values("cuda")
    p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, w.num_qo_heads, w.num_kv_heads,
                w.head_dim, w.page_size, w.num_pool_pages, w.dtype)
    nodes = p.merge_nodes()
    levels = int(nodes[:, 6].max()) + 1 if len(nodes) else 0
    log(f"[case] repeat config {cfg}: {p.info['num_items']} items, {len(nodes)} merge nodes, "
        f"{levels} level(s)")
    if cfg == 4:
        assert levels >= 2
    o0, l0 = fb.decode(q, k, v, p)
    out, lse = torch.empty_like(o0), torch.empty_like(l0)
    flush = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
    for run in range(1, 21):
        if run % 2:
            flush.zero_()
        fb.decode(q, k, v, p, out=out, lse=lse)
        torch.cuda.synchronize()
        same = torch.equal(out.view(torch.int16), o0.view(torch.int16)) and torch.equal(lse, l0)
        assert same, f"config {cfg}: run {run} differs from run 0"
    log(f"[ok] repeat config {cfg}: 20 runs bitwise equal")
