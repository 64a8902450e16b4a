"""Page pools larger than 4 GiB: K/V byte offsets need 64-bit arithmetic in
every kernel. The pool is left uninitialised except for the pages the
requests list, which sit above the 4 GiB mark (and one below it); the oracle
runs on a compact copy of those pages with the page ids remapped."""
import numpy as np
import pytest
import torch

import block_sparse_kv_bsr_amd as fb
import oracle.attention as oa
from block_sparse_kv_bsr_amd.workloads import random_prefill_workload, random_workload
from tests.parity import compare

pytestmark = pytest.mark.gpu

PAGE_BYTES = 8 * 16 * 128 * 2           # H_kv x P x d x bf16
POOL = (5 << 30) // PAGE_BYTES + 7       # just over 5 GiB per pool


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fb.lib()


def _big_pools(w, k, v):
    """Pools of POOL pages holding the compact pages k, v at high ids; returns
    (k_big, v_big, kv_indices with the new ids)."""
    used = np.unique(w.kv_indices)
    rng = np.random.default_rng(7)
    high = (4 << 30) // PAGE_BYTES + 1 + rng.choice(POOL - (4 << 30) // PAGE_BYTES - 1, len(used) - 1,
                                                   replace=False)
    new_ids = np.concatenate([[3], high]).astype(np.int64)  # one page below 4 GiB
    remap = {int(o): int(n) for o, n in zip(used, new_ids)}
    k_big = torch.empty((POOL,) + tuple(k.shape[1:]), dtype=k.dtype, device="cuda")
    v_big = torch.empty_like(k_big)
    idx = torch.as_tensor(new_ids, device="cuda")
    k_big.index_copy_(0, idx, k[torch.as_tensor(used, device="cuda")])
    v_big.index_copy_(0, idx, v[torch.as_tensor(used, device="cuda")])
    ix = np.array([remap[int(x)] for x in w.kv_indices], dtype=np.int32)
    return k_big, v_big, ix


def test_decode_pool_beyond_4gib():
    w = random_workload(111, 4, 900, 32, 8, 128, 16, "bf16")
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    k_big, v_big, ix = _big_pools(w, k, v)
    p = fb.plan(w.kv_indptr, ix, w.last_page_len, 32, 8, 128, 16, POOL, "bf16", fixed_chunk_tokens=128)
    out, lse = fb.decode(q, k_big, v_big, p)
    torch.cuda.synchronize()
    O, LSE = oa.decode_attention(q.double().cpu().numpy(), k.double().cpu().numpy(), v.double().cpu().numpy(),
                                 w.kv_indptr, w.kv_indices, w.last_page_len, w.sm_scale)
    compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True, "decode >4 GiB")
    out2, lse2 = fb.decode(q, k_big, v_big, p, rope_theta=1e4)  # the RoPE variant addresses alike
    torch.cuda.synchronize()
    O2, LSE2 = oa.decode_attention_rope(q.double().cpu().numpy(), k.double().cpu().numpy(),
                                        v.double().cpu().numpy(), w.kv_indptr, w.kv_indices,
                                        w.last_page_len, w.sm_scale, 1e4, 1.0)
    compare(out2.double().cpu().numpy(), lse2.double().cpu().numpy(), O2, LSE2, True, "rope >4 GiB")
    del k_big, v_big
    torch.cuda.empty_cache()


def test_prefill_pool_beyond_4gib():
    w = random_prefill_workload(112, 3, 700, 32, 8, 128, 16, causal=True)
    q, k, v = (t.cuda() for t in w.make_values("cpu"))
    k_big, v_big, ix = _big_pools(w, k, v)
    p = fb.prefill_plan(w.qo_indptr, w.kv_indptr, ix, w.last_page_len, 32, 8, 128, 16, POOL, causal=True,
                        fixed_chunk_tokens=256)
    out, lse = fb.prefill(q, k_big, v_big, p)
    torch.cuda.synchronize()
    O, LSE = oa.prefill_attention(q.double().cpu().numpy(), k.double().cpu().numpy(), v.double().cpu().numpy(),
                                  w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, True, w.sm_scale)
    compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True, "prefill >4 GiB")
    del k_big, v_big
    torch.cuda.empty_cache()


def test_mla_pool_beyond_4gib():
    """The latent pool (1 KiB per token) past 4 GiB: every listed page but
    one sits above the 4 GiB mark of the latent pool."""
    from block_sparse_kv_bsr_amd.workloads import random_mla_workload
    P = 16
    page = P * 512 * 2
    pool = (5 << 30) // page + 7
    w = random_mla_workload(113, 4, 700, 40, P, max_qo=2)
    qn, qp, ckv, kpe = (t.cuda() for t in w.make_values("cpu"))
    used = np.unique(w.kv_indices)
    rng = np.random.default_rng(8)
    low = (4 << 30) // page + 1
    new_ids = np.concatenate([[5], low + rng.choice(pool - low, len(used) - 1, replace=False)])
    remap = {int(o): int(n) for o, n in zip(used, new_ids)}
    idx = torch.as_tensor(new_ids.astype(np.int64), device="cuda")
    src = torch.as_tensor(used.astype(np.int64), device="cuda")
    ckv_big = torch.empty((pool, P, 512), dtype=torch.bfloat16, device="cuda")
    kpe_big = torch.empty((pool, P, 64), dtype=torch.bfloat16, device="cuda")
    ckv_big.index_copy_(0, idx, ckv[src])
    kpe_big.index_copy_(0, idx, kpe[src])
    ix = np.array([remap[int(x)] for x in w.kv_indices], dtype=np.int32)
    p = fb.mla_plan(w.qo_indptr, w.kv_indptr, ix, w.last_page_len, w.num_heads, P, pool,
                    fixed_chunk_tokens=128)
    out, lse = fb.mla(qn, qp, ckv_big, kpe_big, p, w.sm_scale)
    torch.cuda.synchronize()
    O, LSE = oa.mla_attention(*(t.double().cpu().numpy() for t in (qn, qp, ckv, kpe)), w.qo_indptr,
                              w.kv_indptr, w.kv_indices, w.last_page_len, w.sm_scale, True)
    compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True, "mla >4 GiB")
    del ckv_big, kpe_big
    torch.cuda.empty_cache()
