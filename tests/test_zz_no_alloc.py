"""fi_decode_run_noalloc through the C ABI: the run's partial states and
merge counters in the library's static device scratch instead of a
workspace. Its output must equal fi_decode_run's on the same uploaded plan,
bit for bit, on two calls in a row (a large plan, then a smaller one, so
the second runs over what the first left in the scratch), and match the
oracle; a plan whose scratch would not fit is refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_kv_bsr_amd as fb
import oracle.attention as oa
from block_sparse_kv_bsr_amd import binding
from block_sparse_kv_bsr_amd.workloads import random_workload, workload
from tests.parity import compare

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)


def _plan(w, **o):
    return fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, w.num_qo_heads, w.num_kv_heads,
                   w.head_dim, w.page_size, w.num_pool_pages, w.dtype, **o)


def _host(w, q, k, v):
    return q.double().cpu().numpy(), k.double().cpu().numpy(), v.double().cpu().numpy()


def test_noalloc_matches_the_workspace_run_on_two_calls_in_a_row():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cases = [("skewed batch (config 3)", workload(3), {}),
             ("small forced split", random_workload(77, 5, 900, 8, 2, 128, 16, "bf16"),
              {"fixed_chunk_tokens": 48})]
    results = []
    for what, w, opts in cases:
        log(f"[case] noalloc {what}")
        q, k, v = w.make_values("cuda")
        p = _plan(w, **opts)
        info = p.info
        assert info["image_bytes"] < info["workspace_bytes"]
        # the regular run with its own workspace
        full = torch.empty(info["workspace_bytes"], dtype=torch.uint8, device="cuda")
        p.upload(full)
        o_ref, l_ref = fb.decode(q, k, v, p, workspace=full)
        # the no-allocation run: a buffer holding only the uploaded image
        img = torch.empty(max(256, info["image_bytes"]), dtype=torch.uint8, device="cuda")
        p.upload(img)
        with pytest.raises(fb.FiError) as e:  # too small for the workspace run
            fb.decode(q, k, v, p, workspace=img)
        assert e.value.status in (-3, -6)
        o, l = fb.decode_noalloc(q, k, v, p, img)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), what
        assert torch.equal(l, l_ref), what
        results.append((w, (q, k, v), (o, l)))
        log(f"[ok] noalloc {what}: equal to fi_decode_run, {info['num_merge_nodes']} merge nodes, "
            f"{info['num_partial_slots']} partial slots")
    # the second (smaller) call ran over the first call's leftovers: check it,
    # and the first, against the oracle
    for w, (q, k, v), (o, l) in results:
        qh, kh, vh = _host(w, q, k, v)
        O, LSE = oa.decode_attention(qh, kh, vh, w.kv_indptr, w.kv_indices, w.last_page_len,
                                     w.sm_scale)
        compare(o.double().cpu().numpy(), l.double().cpu().numpy(), O, LSE, True, w.name)


def test_noalloc_refuses_a_plan_whose_scratch_does_not_fit():
    """Chunks of one page over the skewed batch give ~124k partial slots
    (~250 MB): refused on the host with FI_ERR_WORKSPACE, nothing launched."""
    w = workload(3)
    p = _plan(w, fixed_chunk_tokens=16)
    info = p.info
    need = info["num_partial_slots"] * 4 * 128 * 4
    assert need > binding.NOALLOC_SCRATCH_BYTES
    img = torch.empty(max(256, info["image_bytes"]), dtype=torch.uint8, device="cuda")
    p.upload(img)
    q = torch.zeros((w.batch, w.num_qo_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((w.num_pool_pages, w.num_kv_heads, w.page_size, w.head_dim),
                     dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fb.FiError) as e:
        fb.decode_noalloc(q, kv, kv, p, img)
    assert e.value.status == -3 and "static scratch" in str(e.value)
    L = fb.lib()
    fake = ctypes.c_void_p(0x100000)
    # a workspace the plan was never uploaded to
    st = L.fi_decode_run_noalloc(p.handle, fake, fake, fake, fake, None, 0.0, fake,
                                 info["image_bytes"], None)
    assert st == -6
    log("[ok] noalloc refusals")
