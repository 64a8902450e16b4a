"""GPU parity of decode with the rotary embedding fused into the K gather
(fi_decode_run_rope / fi_decode_run_rope_scaled), over bf16 caches at
head_dim 128 and 64 and fp8 caches at 128, against the float64 oracle's
decode_attention_rope.

The kernel carries each lane's rotation from step to step and recomputes it
exactly every 32 steps (256 tokens), so the cases run past several
recomputations, cut requests into chunks that start at nonzero positions,
and cover every GQA group, page sizes that do and do not divide the 8-token
step, and both rotary bases.
"""
import time

import numpy as np
import pytest
import torch

import block_sparse_kv_bsr_amd as fb
import oracle.attention as oa
from block_sparse_kv_bsr_amd.workloads import random_workload, workload
from tests.parity import compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fb.lib()


def log(*a):
    print(*a, flush=True)


def host_values(w, q, k, v):
    """q, K, V in float64 for the oracle; an fp8 cache is dequantised by the
    oracle's own E4M3 decoder and the workload's scales."""
    qh = q.double().cpu().numpy()
    if w.dtype == "fp8":
        return (qh, oa.dequantize_e4m3(k.view(torch.uint8).cpu().numpy(), w.k_scale),
                oa.dequantize_e4m3(v.view(torch.uint8).cpu().numpy(), w.v_scale))
    return qh, k.double().cpu().numpy(), v.double().cpu().numpy()


def run_rope(w, theta, scale, what, device_values=False, **opts):
    log(f"[case] {what} B={w.batch} Hq={w.num_qo_heads} Hkv={w.num_kv_heads} P={w.page_size} "
        f"{w.dtype} theta={theta} scale={scale} opts={opts}")
    if device_values:
        q, k, v = w.make_values("cuda")
    else:
        q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, w.num_qo_heads, w.num_kv_heads,
                w.head_dim, w.page_size, w.num_pool_pages, w.dtype, cascade=-1, **opts)
    out, lse = fb.decode(q, k, v, p, rope_theta=theta, rope_scale=scale, k_scale=w.k_scale,
                         v_scale=w.v_scale)
    torch.cuda.synchronize()
    t0 = time.time()
    qh, kh, vh = host_values(w, q, k, v)
    O, LSE = oa.decode_attention_rope(qh, kh, vh, w.kv_indptr, w.kv_indices, w.last_page_len,
                                      w.sm_scale, theta, scale)
    stats = compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True, what)
    log(f"[ok] {what} items={p.info['num_items']} chunk={p.info['chunk_pages']}p "
        f"oracle {time.time() - t0:.1f}s {stats}")
    return p


CASES = [
    # seed, B, maxL, Hq, Hkv, P, theta, scale, fixed_chunk_tokens
    (81, 4, 3000, 32, 8, 16, 1e4, 1.0, 0),
    (82, 3, 5000, 8, 8, 16, 5e5, 1.0, 512),
    (83, 4, 2500, 16, 8, 64, 1e4, 4.0, 0),
    (84, 5, 700, 16, 2, 12, 5e5, 1.0, 96),
    (85, 3, 1200, 8, 1, 1, 1e4, 1.0, 0),
    (86, 4, 900, 64, 8, 16, 1e4, 1.0, 160),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_rope_small(case):
    seed, B, L, Hq, Hkv, P, theta, scale, fixed = case
    w = random_workload(seed, B, L, Hq, Hkv, 128, P, "bf16")
    p = run_rope(w, theta, scale, f"rope{seed}", fixed_chunk_tokens=fixed)
    if fixed:
        assert p.info["max_chunks_per_request"] > 1


def test_rope_empty_and_one_token_requests():
    w = random_workload(87, 5, 50, 32, 8, 128, 16, "bf16", lens=[0, 1, 9, 0, 300])
    run_rope(w, 1e4, 1.0, "rope empty/one-token")


def test_rope_skewed_batch_full_size():
    w = workload(9)
    run_rope(w, w.rope_theta, w.rope_scale, "config9-rope", device_values=True)


FP8_CASES = [
    # seed, B, maxL, Hq, Hkv, P, theta, scale, fixed_chunk_tokens
    (91, 4, 3000, 32, 8, 16, 1e4, 1.0, 0),      # G 4, several exact recomputations
    (92, 3, 2000, 8, 8, 16, 5e5, 1.0, 512),     # G 1, chunks at nonzero positions
    (93, 4, 1500, 16, 8, 64, 1e4, 4.0, 0),      # G 2, large pages, position scaling
    (94, 5, 700, 16, 2, 12, 5e5, 1.0, 96),      # G 8, page size not dividing the step
    (95, 3, 900, 8, 1, 1, 1e4, 1.0, 0),         # G 8, one token per page
    (96, 8, 127, 8, 2, 16, 1e4, 1.0, 40),       # ragged tails of 5 .. 8 ring stages
]


@pytest.mark.parametrize("case", FP8_CASES, ids=lambda c: f"fp8_seed{c[0]}")
def test_rope_fp8_cache(case):
    """The rotary embedding over an OCP E4M3 cache with dequantisation
    scales: each K row is read back from LDS as two 8-byte halves so a lane
    holds rotate-half pairs; the oracle turns the dequantised keys."""
    seed, B, L, Hq, Hkv, P, theta, scale, fixed = case
    w = random_workload(seed, B, L, Hq, Hkv, 128, P, "fp8")
    assert w.k_scale != 1.0 and w.v_scale != 1.0
    p = run_rope(w, theta, scale, f"rope-fp8-{seed}", fixed_chunk_tokens=fixed)
    if fixed:
        assert p.info["max_chunks_per_request"] > 1


def test_rope_fp8_skewed_batch_full_size():
    w = workload(10)
    run_rope(w, w.rope_theta, w.rope_scale, "config10-rope-fp8", device_values=True)


D64_CASES = [
    # seed, B, maxL, Hq, Hkv, P, theta, scale, fixed_chunk_tokens
    (71, 4, 3000, 32, 8, 16, 1e4, 1.0, 0),      # G 4, several exact recomputations
    (72, 3, 2000, 8, 8, 16, 5e5, 1.0, 512),     # G 1, chunks at nonzero positions
    (73, 4, 1500, 16, 2, 64, 1e4, 2.0, 0),      # G 8, large pages, position scaling
    (74, 5, 700, 16, 8, 12, 5e5, 1.0, 96),      # G 2, page size not dividing the step
    (75, 3, 400, 8, 1, 1, 1e4, 1.0, 0),         # G 8, one token per page
]


@pytest.mark.parametrize("case", D64_CASES, ids=lambda c: f"d64_seed{c[0]}")
def test_rope_head_dim_64(case):
    """bf16 at head_dim 64: a K row is one 128-byte line, read back from LDS
    as two 8-byte halves (4 rotate-half pairs per lane)."""
    seed, B, L, Hq, Hkv, P, theta, scale, fixed = case
    w = random_workload(seed, B, L, Hq, Hkv, 64, P, "bf16")
    p = run_rope(w, theta, scale, f"rope-d64-{seed}", fixed_chunk_tokens=fixed)
    if fixed:
        assert p.info["max_chunks_per_request"] > 1


def test_rope_rejects_what_is_not_built():
    w = random_workload(88, 2, 40, 8, 2, 64, 16, "f32")
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, 8, 2, 64, 16, w.num_pool_pages, "f32")
    with pytest.raises(fb.FiError, match="rotary"):
        fb.decode(q, k, v, p, rope_theta=1e4)
