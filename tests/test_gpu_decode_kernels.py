"""GPU parity of both decode kernels, each forced through the plan's
decode_kernel option: the vector-ALU kernel and the matrix-core kernel
(scores and PV on v_mfma_f32_16x16x32 / 16x16x16, bf16 and fp8 caches,
page sizes that are multiples of 16). Every case runs through each kernel
it fits, against the float64 oracle: ragged lengths around the 16- and
32-token blocks, empty requests, forced splits (merge trees), every group
size, pages of 16 to 4096 tokens, an item longer than the page-id window,
the rotary embedding, the five full-size skewed workloads, and repeat runs
for bit equality."""
import numpy as np
import pytest
import torch

import block_sparse_kv_bsr_amd as fb
import oracle.attention as oa
from block_sparse_kv_bsr_amd import binding
from block_sparse_kv_bsr_amd.workloads import random_workload, workload
from tests.parity import compare

pytestmark = pytest.mark.gpu

VECTOR, MATRIX = binding.DECODE_KERNEL_VECTOR, binding.DECODE_KERNEL_MATRIX


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fb.lib()


def log(*a):
    print(*a, flush=True)


def oracle_of(w, q, k, v):
    # bf16 values are exact in float32; the oracle widens what it gathers
    qh = q.float().cpu().numpy()
    if w.dtype == "fp8":
        kh = oa.dequantize_e4m3(k.view(torch.uint8).cpu().numpy(), w.k_scale)
        vh = oa.dequantize_e4m3(v.view(torch.uint8).cpu().numpy(), w.v_scale)
    else:
        kh, vh = k.float().cpu().numpy(), v.float().cpu().numpy()
    return oa.decode_attention(qh, kh, vh, w.kv_indptr, w.kv_indices, w.last_page_len, w.sm_scale)


def run(w, kernel, device_values=False, **opts):
    if device_values:
        q, k, v = w.make_values("cuda")
    else:
        q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, w.num_qo_heads, w.num_kv_heads,
                w.head_dim, w.page_size, w.num_pool_pages, w.dtype, decode_kernel=kernel, **opts)
    out, lse = fb.decode(q, k, v, p, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    return p, (q, k, v), (out, lse)


CASES = [
    # seed, B, maxL, Hq, Hkv, P, dtype, empty_every, fixed chunk tokens
    (201, 5, 700, 8, 2, 16, "bf16", 0, 0),
    (202, 4, 900, 16, 2, 16, "bf16", 2, 0),
    (203, 3, 500, 8, 8, 32, "bf16", 0, 48),
    (204, 4, 600, 16, 8, 64, "bf16", 0, 64),
    (205, 5, 700, 8, 2, 16, "fp8", 0, 0),
    (206, 4, 900, 16, 2, 16, "fp8", 3, 0),
    (207, 3, 500, 8, 8, 48, "fp8", 0, 96),
    (208, 4, 1200, 32, 8, 64, "fp8", 0, 128),
    (209, 3, 300, 8, 2, 4096, "bf16", 0, 0),
    (210, 3, 300, 32, 4, 4096, "fp8", 0, 0),
]


@pytest.mark.parametrize("kernel", [VECTOR, MATRIX], ids=["vector", "matrix"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}_{c[6]}_G{c[3] // c[4]}_P{c[5]}")
def test_small(case, kernel):
    seed, B, L, hq, hkv, P, dt, ee, fixed = case
    w = random_workload(seed, B, L, hq, hkv, 128, P, dt, empty_every=ee)
    log(f"[case] kernel={kernel} seed={seed} {dt} G={hq // hkv} P={P} fixed={fixed}")
    p, qkv, (out, lse) = run(w, kernel, fixed_chunk_tokens=fixed)
    O, LSE = oracle_of(w, *qkv)
    st = compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True, f"s{seed}")
    log(f"[ok] kernel={kernel} seed={seed} items={p.info['num_items']} {st}")


@pytest.mark.parametrize("kernel", [VECTOR, MATRIX], ids=["vector", "matrix"])
@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_lengths_around_the_blocks(dt, kernel):
    """Requests ending on and around 16- and 32-token block edges and page
    edges, unsplit and cut into 16-token chunks (every chunk one page)."""
    lens = [1, 2, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 95, 96, 97, 0]
    w = random_workload(220 if dt == "bf16" else 221, len(lens), 0, 16, 4, 128, 16, dt, lens=lens)
    for fixed in (0, 16):
        p, qkv, (out, lse) = run(w, kernel, fixed_chunk_tokens=fixed)
        O, LSE = oracle_of(w, *qkv)
        compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True,
                f"lengths {dt} fixed={fixed}")


@pytest.mark.parametrize("kernel", [VECTOR, MATRIX], ids=["vector", "matrix"])
@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_item_longer_than_the_page_id_window(dt, kernel):
    """One chunk of 330 pages: the kernel slides its 256-entry window of
    page ids part-way through the item."""
    w = random_workload(230, 2, 0, 8, 2, 128, 16, dt, lens=[330 * 16 - 5, 70])
    p, qkv, (out, lse) = run(w, kernel, fixed_chunk_tokens=330 * 16)
    assert p.info["chunk_pages"] >= 330 and p.info["num_items"] == 4
    O, LSE = oracle_of(w, *qkv)
    compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True, f"window {dt}")


@pytest.mark.parametrize("cfg", [3, 6, 11])
def test_full_size_skewed(cfg):
    """Both kernels on the full-size workload, against one oracle evaluation."""
    w = workload(cfg)
    q, k, v = w.make_values("cuda")
    O, LSE = oracle_of(w, q, k, v)
    for kernel in (VECTOR, MATRIX):
        log(f"[case] full size config {cfg} kernel={kernel}")
        p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, w.num_qo_heads, w.num_kv_heads,
                    w.head_dim, w.page_size, w.num_pool_pages, w.dtype, decode_kernel=kernel)
        out, lse = fb.decode(q, k, v, p, k_scale=w.k_scale, v_scale=w.v_scale)
        torch.cuda.synchronize()
        st = compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True, w.name)
        log(f"[ok] config {cfg} kernel={kernel} {st}")


@pytest.mark.parametrize("cfg", [6, 11])
def test_matrix_kernel_bitwise_repeatable(cfg):
    w = workload(cfg)
    q, k, v = w.make_values("cuda")
    p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, w.num_qo_heads, w.num_kv_heads,
                w.head_dim, w.page_size, w.num_pool_pages, w.dtype, decode_kernel=MATRIX)
    o0, l0 = fb.decode(q, k, v, p, k_scale=w.k_scale, v_scale=w.v_scale)
    out, lse = torch.empty_like(o0), torch.empty_like(l0)
    flush = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
    for run_i in range(1, 11):
        if run_i % 2:
            flush.zero_()
        fb.decode(q, k, v, p, out=out, lse=lse, k_scale=w.k_scale, v_scale=w.v_scale)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), o0.view(torch.int16)) and torch.equal(lse, l0), \
            f"config {cfg}: run {run_i} differs"


def test_matrix_kernel_refusals():
    w = random_workload(240, 2, 100, 8, 2, 128, 8, "bf16")
    with pytest.raises(fb.FiError) as e:  # page size not a multiple of 16
        fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, 8, 2, 128, 8, w.num_pool_pages, "bf16",
                decode_kernel=MATRIX)
    assert e.value.status == -2
    w = random_workload(241, 2, 100, 8, 2, 64, 16, "bf16")
    with pytest.raises(fb.FiError) as e:  # head_dim 64
        fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, 8, 2, 64, 16, w.num_pool_pages, "bf16",
                decode_kernel=MATRIX)
    assert e.value.status == -2
    w = random_workload(242, 2, 100, 8, 2, 128, 16, "f32")
    with pytest.raises(fb.FiError) as e:  # an fp32 cache
        fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, 8, 2, 128, 16, w.num_pool_pages, "f32",
                decode_kernel=MATRIX)
    assert e.value.status == -2


def rope_oracle(w, q, k, v, theta, scale):
    qh = q.float().cpu().numpy()
    if w.dtype == "fp8":
        kh = oa.dequantize_e4m3(k.view(torch.uint8).cpu().numpy(), w.k_scale)
        vh = oa.dequantize_e4m3(v.view(torch.uint8).cpu().numpy(), w.v_scale)
    else:
        kh, vh = k.float().cpu().numpy(), v.float().cpu().numpy()
    return oa.decode_attention_rope(qh, kh, vh, w.kv_indptr, w.kv_indices, w.last_page_len,
                                    w.sm_scale, theta, scale)


ROPE_CASES = [
    # seed, B, maxL, Hq, Hkv, P, dtype, fixed chunk tokens, theta, position scale
    (251, 4, 1500, 8, 2, 16, "bf16", 0, 1e4, 1.0),
    (252, 3, 2000, 32, 4, 64, "bf16", 192, 5e5, 1.0),
    (253, 4, 1500, 8, 2, 16, "fp8", 64, 1e4, 2.0),
    (254, 3, 2500, 16, 2, 32, "fp8", 0, 5e5, 1.0),
    (255, 5, 700, 8, 8, 48, "bf16", 48, 1e4, 1.0),
    (256, 4, 1200, 64, 8, 16, "fp8", 320, 5e5, 1.0),
]


@pytest.mark.parametrize("kernel", [VECTOR, MATRIX], ids=["vector", "matrix"])
@pytest.mark.parametrize("case", ROPE_CASES, ids=lambda c: f"rope{c[0]}_{c[6]}_G{c[3] // c[4]}_P{c[5]}")
def test_rope(case, kernel):
    """The rotary embedding in both kernels: items longer than 32 score tiles
    (the matrix kernel's exact recomputation interval), chunks that start at
    nonzero positions, both bases, a position scale, every group size."""
    seed, B, L, hq, hkv, P, dt, fixed, theta, scale = case
    w = random_workload(seed, B, L, hq, hkv, 128, P, dt)
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, hq, hkv, 128, P, w.num_pool_pages, dt,
                cascade=-1, decode_kernel=kernel, fixed_chunk_tokens=fixed)
    out, lse = fb.decode(q, k, v, p, rope_theta=theta, rope_scale=scale, k_scale=w.k_scale,
                         v_scale=w.v_scale)
    torch.cuda.synchronize()
    O, LSE = rope_oracle(w, q, k, v, theta, scale)
    st = compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True, f"rope{seed}")
    log(f"[ok] rope{seed} kernel={kernel} {st}")


@pytest.mark.parametrize("cfg", [9, 10])
def test_rope_full_size_skewed(cfg):
    """Both kernels on the full-size skewed batch with the rotary embedding
    (bf16 and fp8 caches, theta 5e5), against one oracle evaluation."""
    w = workload(cfg)
    q, k, v = w.make_values("cuda")
    O, LSE = rope_oracle(w, q, k, v, w.rope_theta, w.rope_scale)
    for kernel in (VECTOR, MATRIX):
        p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, w.num_qo_heads, w.num_kv_heads,
                    w.head_dim, w.page_size, w.num_pool_pages, w.dtype, decode_kernel=kernel)
        out, lse = fb.decode(q, k, v, p, rope_theta=w.rope_theta, rope_scale=w.rope_scale,
                             k_scale=w.k_scale, v_scale=w.v_scale)
        torch.cuda.synchronize()
        st = compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True, w.name)
        log(f"[ok] config {cfg} kernel={kernel} {st}")
