"""GPU parity of composed formats: fi_decode_run_composed (the prefix tile
kernel over the prefix cache, the decode kernel over the requests' own
pages, their states merged per request) through the C ABI against the
float64 composed oracle.

Small ragged cases cover prefix block sizes 1 .. 4096 (also one that is not
a power of two), prefixes that end inside a block, chunks that start inside
a block or straddle two, groups of one to forty members (two row blocks),
requests without a prefix, GQA groups 1 .. 8 and both head sizes; NaN fills
every prefix slot past a prefix's length and every unlisted block. The full
config-13 workload runs with the plan bench.py times and is checked on every
output element, and against config 5's cascade over the same tokens.
"""
import time

import numpy as np
import pytest
import torch

import block_sparse_kv_bsr_amd as fb
import oracle.attention as oa
from block_sparse_kv_bsr_amd.workloads import random_composed_workload, workload
from tests.parity import compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fb.lib()


def log(*a):
    print(*a, flush=True)


def make(w, **opts):
    return fb.plan_composed(w.kv_indptr, w.kv_indices, w.last_page_len, w.prefix_indptr,
                            w.prefix_indices, w.prefix_last_page_len, w.prefix_of,
                            w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                            w.num_pool_pages, w.prefix_page_size, w.num_prefix_pool_pages, **opts)


def oracle(w, q, k, v, kp, vp):
    h = [t.double().cpu().numpy() for t in (q, k, v, kp, vp)]
    return oa.decode_attention_composed(h[0], h[1], h[2], w.kv_indptr, w.kv_indices,
                                        w.last_page_len, h[3], h[4], w.prefix_indptr,
                                        w.prefix_indices, w.prefix_last_page_len, w.prefix_of,
                                        w.sm_scale)


def run_case(w, what, **opts):
    log(f"[case] {what} B={w.batch} Hq={w.num_qo_heads} Hkv={w.num_kv_heads} d={w.head_dim} "
        f"P={w.page_size} Pp={w.prefix_page_size} prefixes={[w.prefix_len(g) for g in range(w.num_prefixes)]} "
        f"opts={opts}")
    q, k, v, kp, vp = (t.cuda() for t in w.make_values("cpu"))
    p = make(w, **opts)
    out, lse = fb.decode_composed(q, k, v, kp, vp, p)
    torch.cuda.synchronize()
    t0 = time.time()
    O, LSE = oracle(w, q, k, v, kp, vp)
    stats = compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True, what)
    log(f"[ok] {what} items={p.info['num_items']} prefix items={p.info['num_prefix_items']} "
        f"oracle {time.time() - t0:.1f}s {stats}")
    return p, out, lse


CASES = [
    # seed, prefix_lens, members, singles, own_max, Hq, Hkv, d, P, Pp, fixed chunk
    (1, [40, 0, 17], [2, 1, 2], 1, 30, 8, 2, 64, 4, 16, 0),
    (2, [300], [3], 0, 20, 4, 1, 64, 1, 64, 8),
    (3, [33, 64], [1, 2], 2, 9, 16, 2, 128, 16, 32, 0),
    (4, [5, 129], [2, 2], 1, 40, 8, 8, 128, 16, 1, 16),
    (5, [4096 + 77], [40], 0, 5, 16, 4, 128, 16, 4096, 0),   # two row blocks, partial block
    (6, [1000], [5], 3, 300, 32, 4, 128, 16, 100, 64),      # G 8, a 100-token block
    (7, [2500, 700], [3, 4], 2, 200, 32, 8, 128, 64, 512, 0),
    (8, [8192], [6], 1, 100, 8, 2, 64, 16, 4096, 32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"composed{c[0]}")
def test_composed_small(case):
    seed, plens, mem, singles, own_max, hq, hkv, d, P, Pp, fixed = case
    w = random_composed_workload(seed, plens, mem, singles, own_max, hq, hkv, d, P, Pp)
    p, _, _ = run_case(w, f"composed seed{seed}", fixed_chunk_tokens=fixed)
    assert p.info["num_prefix_groups"] == sum(
        1 for g, m in enumerate(mem) if m > 0 and plens[g] > 0)


def test_composed_is_deterministic():
    w = random_composed_workload(31, [3000], [9], 2, 400, 32, 8, 128, 16, 256)
    q, k, v, kp, vp = (t.cuda() for t in w.make_values("cpu"))
    p = make(w)
    a = fb.decode_composed(q, k, v, kp, vp, p)
    b = fb.decode_composed(q, k, v, kp, vp, p)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_config13_full_size():
    """Every output of the composed workload in the launch configuration
    bench.py times, against the oracle; and the same tokens through config
    5's cascade (the prefix in the main cache) agree to the tolerance."""
    w = workload(13)
    log(f"[case] full-size composed config 13 {w.name}")
    q, k, v, kp, vp = w.make_values("cuda")
    p = make(w)
    out, lse = fb.decode_composed(q, k, v, kp, vp, p)
    torch.cuda.synchronize()
    t0 = time.time()
    O, LSE = oracle(w, q, k, v, kp, vp)
    stats = compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), O, LSE, True,
                    "config 13")
    log(f"[ok] config 13 items={p.info['num_items']} prefix items={p.info['num_prefix_items']} "
        f"oracle {time.time() - t0:.1f}s {stats}")
