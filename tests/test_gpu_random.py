"""Seeded random configurations across the built space, each checked element
by element against the float64 oracle, in the style of the fixed cases but
drawn independently:

* decode: dtype (f32, bf16, fp8 E4M3 cache) x head_dim (64, 128) x GQA group
  (1, 2, 4, 8) x page size (1 .. 64, dividing the 8-token step or not), with
  empty requests, forced chunk lengths (merge trees), and the fused rotary
  embedding on some bf16 d = 128 cases;
* cascade: random groups of requests sharing a prefix, forced on;
* prefill / append: any GQA group the tile holds (not only powers of two),
  causal or not, forced chunk lengths (cut tiles merged in the kernel);
* in-kernel merges of prefill and latent-attention tiles cut into many short
  chunks, repeated for bit-identical results and checked against the oracle.

Every case prints its parameters before it runs.
"""
import numpy as np
import pytest
import torch

import block_sparse_kv_bsr_amd as fb
import oracle.attention as oa
from block_sparse_kv_bsr_amd.workloads import (prefix_workload, random_mla_workload,
                                               random_prefill_workload, random_workload)
from tests.parity import compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fb.lib()


def log(*a):
    print(*a, flush=True)


def _decode_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = str(rng.choice(["f32", "bf16", "bf16", "fp8"]))
        d = 128 if dtype == "fp8" else int(rng.choice([64, 128]))
        G = int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.choice([1, 2, 4, 8]))
        P = int(rng.choice([1, 3, 5, 8, 16, 32, 64]))
        B = int(rng.integers(1, 9))
        L = int(rng.integers(1, 1500))
        empty = int(rng.choice([0, 0, 3]))
        fixed = int(rng.choice([0, 0, 16, 48, 200]))
        rope = bool(dtype == "bf16" and d == 128 and rng.random() < 0.75)
        theta = float(rng.choice([1e4, 5e5]))
        out.append((7000 + i, dtype, d, G, hkv, P, B, L, empty, fixed, rope, theta))
    return out


DECODE = _decode_cases(28, 20261202)


@pytest.mark.parametrize("case", DECODE, ids=lambda c: f"dec{c[0]}_{c[1]}_d{c[2]}_G{c[3]}_P{c[5]}")
def test_random_decode(case):
    seed, dtype, d, G, hkv, P, B, L, empty, fixed, rope, theta = case
    hq = G * hkv
    what = f"decode seed{seed} {dtype} d={d} G={G} Hkv={hkv} P={P} B={B} L<={L} " \
           f"empty_every={empty} fixed={fixed} rope={rope}"
    log(f"[case] {what}")
    w = random_workload(seed, B, L, hq, hkv, d, P, dtype, empty_every=empty)
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    opts = {"fixed_chunk_tokens": fixed}
    if rope:
        opts["cascade"] = -1
    p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, hq, hkv, d, P, w.num_pool_pages,
                dtype, **opts)
    qh = q.double().cpu().numpy()
    if dtype == "fp8":
        kh = oa.dequantize_e4m3(k.view(torch.uint8).cpu().numpy(), w.k_scale)
        vh = oa.dequantize_e4m3(v.view(torch.uint8).cpu().numpy(), w.v_scale)
    else:
        kh, vh = k.double().cpu().numpy(), v.double().cpu().numpy()
    if rope:
        out, lse = fb.decode(q, k, v, p, rope_theta=theta, rope_scale=1.0)
        O, LSE = oa.decode_attention_rope(qh, kh, vh, w.kv_indptr, w.kv_indices,
                                          w.last_page_len, w.sm_scale, theta, 1.0)
    else:
        out, lse = fb.decode(q, k, v, p, k_scale=w.k_scale, v_scale=w.v_scale)
        O, LSE = oa.decode_attention(qh, kh, vh, w.kv_indptr, w.kv_indices, w.last_page_len,
                                     w.sm_scale)
    torch.cuda.synchronize()
    stats = compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE,
                    dtype != "f32", what)
    log(f"[ok] items={p.info['num_items']} {stats}")


def _cascade_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        ngroups = int(rng.integers(1, 3))
        groups = [(int(rng.integers(2, 9)), int(rng.integers(1, 7))) for _ in range(ngroups)]
        G = int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        P = int(rng.choice([3, 4, 8, 16]))
        out.append((7100 + i, groups, int(rng.integers(0, 4)), int(rng.integers(5, 200)),
                    G * hkv, hkv, d, P, int(rng.choice([0, 0, 8, 32]))))
    return out


CASCADE = _cascade_cases(8, 20261203)


@pytest.mark.parametrize("case", CASCADE, ids=lambda c: f"cas{c[0]}")
def test_random_cascade(case):
    seed, groups, singles, smax, hq, hkv, d, P, fixed = case
    what = f"cascade seed{seed} groups={groups} singles={singles} suffix<={smax} Hq={hq} " \
           f"Hkv={hkv} d={d} P={P} fixed={fixed}"
    log(f"[case] {what}")
    w = prefix_workload(seed, groups, singles, smax, hq, hkv, d, P, "bf16")
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, hq, hkv, d, P, w.num_pool_pages,
                "bf16", cascade=1, fixed_chunk_tokens=fixed)
    assert p.info["num_prefix_items"] > 0
    out, lse = fb.decode(q, k, v, p)
    torch.cuda.synchronize()
    qh, kh, vh = (t.double().cpu().numpy() for t in (q, k, v))
    O, LSE = oa.decode_attention(qh, kh, vh, w.kv_indptr, w.kv_indices, w.last_page_len,
                                 w.sm_scale)
    stats = compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True, what)
    log(f"[ok] prefix items={p.info['num_prefix_items']} items={p.info['num_items']} {stats}")


def _prefill_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
        hkv = int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        P = int(rng.choice([1, 4, 7, 16, 64]))
        causal = bool(rng.random() < 0.7)
        B = int(rng.integers(1, 6))
        L = int(rng.integers(1, 700))
        max_qo = None if rng.random() < 0.5 else int(rng.integers(1, 130))
        fixed = int(rng.choice([0, 0, 16, 64, 200]))
        out.append((7200 + i, B, L, G * hkv, hkv, d, P, causal, max_qo, fixed))
    return out


PREFILL = _prefill_cases(16, 20261204)


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: f"pf{c[0]}_G{c[3] // c[4]}_d{c[5]}_P{c[6]}")
def test_random_prefill(case):
    seed, B, L, hq, hkv, d, P, causal, max_qo, fixed = case
    what = f"prefill seed{seed} B={B} L<={L} Hq={hq} Hkv={hkv} d={d} P={P} causal={causal} " \
           f"max_qo={max_qo} fixed={fixed}"
    log(f"[case] {what}")
    w = random_prefill_workload(seed, B, L, hq, hkv, d, P, causal=causal, max_qo=max_qo)
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = fb.prefill_plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, hq, hkv, d, P,
                        w.num_pool_pages, causal=causal, fixed_chunk_tokens=fixed)
    out, lse = fb.prefill(q, k, v, p)
    torch.cuda.synchronize()
    qh, kh, vh = (t.double().cpu().numpy() for t in (q, k, v))
    O, LSE = oa.prefill_attention(qh, kh, vh, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                  w.last_page_len, causal, w.sm_scale)
    stats = compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True, what)
    log(f"[ok] items={p.info['num_items']} merges={p.info['num_merges']} {stats}")


LARGE_PAGES = [
    # seed, page size, dtype, head_dim, fixed chunk tokens (0: planner's choice)
    (7300, 100, "bf16", 128, 0),
    (7301, 256, "bf16", 128, 300),
    (7302, 1024, "f32", 64, 0),
    (7303, 4096, "bf16", 128, 0),
    (7304, 4096, "fp8", 128, 1000),
]


@pytest.mark.parametrize("case", LARGE_PAGES, ids=lambda c: f"P{c[1]}_{c[2]}")
def test_large_page_sizes_decode(case):
    """Pages of 100 .. 4096 tokens (the largest the planner takes): requests
    that end inside their first page, span several, and are cut mid-page."""
    seed, P, dtype, d, fixed = case
    lens = [1, P - 1, P, P + 1, 3 * P // 2, 2 * P + 7]
    what = f"large pages P={P} {dtype} d={d} fixed={fixed} lens={lens}"
    log(f"[case] {what}")
    w = random_workload(seed, len(lens), 0, 8, 2, d, P, dtype, lens=lens)
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, 8, 2, d, P, w.num_pool_pages, dtype,
                fixed_chunk_tokens=fixed)
    out, lse = fb.decode(q, k, v, p, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    qh = q.double().cpu().numpy()
    if dtype == "fp8":
        kh = oa.dequantize_e4m3(k.view(torch.uint8).cpu().numpy(), w.k_scale)
        vh = oa.dequantize_e4m3(v.view(torch.uint8).cpu().numpy(), w.v_scale)
    else:
        kh, vh = k.double().cpu().numpy(), v.double().cpu().numpy()
    O, LSE = oa.decode_attention(qh, kh, vh, w.kv_indptr, w.kv_indices, w.last_page_len,
                                 w.sm_scale)
    stats = compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE,
                    dtype != "f32", what)
    log(f"[ok] items={p.info['num_items']} {stats}")


@pytest.mark.parametrize("P", [100, 256, 1024, 4096])
def test_large_page_sizes_prefill(P):
    lens = [P - 1, P + 1, 2 * P + 7]
    what = f"prefill large pages P={P} lens={lens}"
    log(f"[case] {what}")
    w = random_prefill_workload(7310 + P, len(lens), 0, 8, 2, 128, P, causal=True, lens=lens,
                                qo_lens=[min(L, 70) for L in lens])
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = fb.prefill_plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, 8, 2, 128, P,
                        w.num_pool_pages, causal=True, fixed_chunk_tokens=P if P <= 256 else 0)
    out, lse = fb.prefill(q, k, v, p)
    torch.cuda.synchronize()
    qh, kh, vh = (t.double().cpu().numpy() for t in (q, k, v))
    O, LSE = oa.prefill_attention(qh, kh, vh, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                  w.last_page_len, True, w.sm_scale)
    stats = compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True, what)
    log(f"[ok] items={p.info['num_items']} merges={p.info['num_merges']} {stats}")


def _merge_cases(n, seed):
    """Random plans with many chunks per cut tile (short forced chunks), for
    the in-kernel merges of the prefill and latent-attention tile kernels."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = "mla" if i % 2 else "prefill"
        P = int(rng.choice([1, 4, 16]))
        B = int(rng.integers(1, 5))
        L = int(rng.integers(100, 1500))
        fixed = int(rng.choice([16, 32, 48, 96]))
        heads = int(rng.choice([8, 16, 40, 96])) if kind == "mla" else int(rng.choice([4, 8, 16]))
        out.append((7400 + i, kind, B, L, P, fixed, heads))
    return out


MERGE_CASES = _merge_cases(12, 20261205)


@pytest.mark.parametrize("case", MERGE_CASES, ids=lambda c: f"mg{c[0]}_{c[1]}_P{c[4]}_c{c[5]}")
def test_random_in_kernel_merges(case):
    """Cut tiles merged by whichever chunk arrives last: each case is run five
    times, every other run after a cache flush so arrival orders differ, and
    every run must equal the first bit for bit; the first is also compared
    with the float64 oracle. Chunks of 16-96 tokens give up to ~90 chunks
    per tile (many groups in the merging loop)."""
    seed, kind, B, L, P, fixed, heads = case
    log(f"[case] merges seed{seed} {kind} B={B} L<={L} P={P} chunk={fixed} heads={heads}")
    if kind == "mla":
        w = random_mla_workload(seed, B, L, heads, P, max_qo=2)
        qn, qp, ckv, kpe = (t.cuda() for t in w.make_values("cpu"))
        p = fb.mla_plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, heads, P,
                        w.num_pool_pages, causal=w.causal, fixed_chunk_tokens=fixed)
        run = lambda out=None, lse=None: fb.mla(qn, qp, ckv, kpe, p, w.sm_scale, out=out, lse=lse)
    else:
        w = random_prefill_workload(seed, B, L, heads, 2, 128, P, causal=True, max_qo=60)
        q, k, v = (t.cuda() for t in w.make_values("cpu"))
        p = fb.prefill_plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, heads, 2, 128,
                            P, w.num_pool_pages, causal=True, fixed_chunk_tokens=fixed)
        run = lambda out=None, lse=None: fb.prefill(q, k, v, p, out=out, lse=lse)
    assert p.info["num_merges"] > 0
    o0, l0 = run()
    out, lse = torch.empty_like(o0), torch.empty_like(l0)
    flush = torch.empty(1 << 26, dtype=torch.uint8, device="cuda")
    for r in range(1, 5):
        if r % 2:
            flush.zero_()
        run(out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), o0.view(torch.int16)) and torch.equal(lse, l0), r
    if kind == "mla":
        h = [t.double().cpu().numpy() for t in (qn, qp, ckv, kpe)]
        O, LSE = oa.mla_attention(h[0], h[1], h[2], h[3], w.qo_indptr, w.kv_indptr, w.kv_indices,
                                  w.last_page_len, w.sm_scale, w.causal)
    else:
        qh, kh, vh = (t.double().cpu().numpy() for t in (q, k, v))
        O, LSE = oa.prefill_attention(qh, kh, vh, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                      w.last_page_len, True, w.sm_scale)
    stats = compare(o0.double().cpu().numpy(), l0.double().cpu().numpy(), O, LSE, True, kind)
    log(f"[ok] items={p.info['num_items']} merges={p.info['num_merges']} {stats}")
