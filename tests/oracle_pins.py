"""Checks that pin the float64 oracle to things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
an independent source: the pure-Python brute force, torch's CPU float64
scaled_dot_product_attention (a library definition of GQA attention), closed
forms of softmax attention, invariants of the definition, and the algebra of
merging softmax states. They read the oracle through the module object they
are given, so ``test_oracle_mutations`` can plant a mistake in the oracle and
show that some pin catches it.
"""
import dataclasses
import math

import numpy as np
import torch

from block_sparse_kv_bsr_amd.workloads import (random_composed_workload, random_mla_workload,
                                               random_prefill_workload, random_workload)
from tests.bruteforce import bruteforce_decode, bruteforce_mla, bruteforce_prefill, rope_rows_loops


def f64_inputs(w):
    q, k, v = w.make_values("cpu")
    return q.double().numpy(), k.double().numpy(), v.double().numpy()


def _oracle(mod, w, q, k, v, sm_scale=None, indptr=None, indices=None, last=None):
    return mod.decode_attention(q, k, v,
                                w.kv_indptr if indptr is None else indptr,
                                w.kv_indices if indices is None else indices,
                                w.last_page_len if last is None else last,
                                w.sm_scale if sm_scale is None else sm_scale)


TINY_CASES = [
    # seed, batch, max_len, Hq, Hkv, d, P, empty_every
    (1, 3, 40, 4, 1, 8, 16, 0),
    (2, 3, 37, 4, 2, 4, 4, 0),
    (3, 2, 25, 2, 2, 8, 1, 0),
    (4, 3, 40, 4, 4, 4, 16, 2),
    (5, 2, 33, 8, 2, 8, 4, 0),
]


def pin_bruteforce(mod, cases=TINY_CASES, tol=1e-12):
    for (seed, B, L, Hq, Hkv, d, P, ee) in cases:
        w = random_workload(seed, B, L, Hq, Hkv, d, P, "f32", empty_every=ee)
        q, k, v = f64_inputs(w)
        O, LSE = _oracle(mod, w, q, k, v)
        Ob, LSEb = bruteforce_decode(q, k, v, w.kv_indptr, w.kv_indices, w.last_page_len, w.sm_scale)
        Ob, LSEb = np.array(Ob), np.array(LSEb)
        assert np.array_equal(np.isneginf(LSE), np.isneginf(LSEb)), (seed, "empty-set pattern")
        fin = ~np.isneginf(LSEb)
        assert np.max(np.abs(O - Ob)) <= tol, (seed, np.max(np.abs(O - Ob)))
        assert np.max(np.abs(LSE[fin] - LSEb[fin]), initial=0.0) <= tol, seed


def _dense(w, k, v, b):
    """Dense [H_kv, T, d] K and V of request b, built straight from the page
    table (independent of the oracle's helpers)."""
    P = w.page_size
    rows_k, rows_v = [], []
    pages = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
    for j, p in enumerate(pages):
        n = P if j + 1 < len(pages) else int(w.last_page_len[b])
        rows_k.append(k[p, :, :n, :])
        rows_v.append(v[p, :, :n, :])
    return np.concatenate(rows_k, axis=1), np.concatenate(rows_v, axis=1)


def pin_sdpa(mod, seeds=(11, 12, 13), default_scale=True):
    """torch SDPA in float64 with enable_gqa=True: query head h reads KV head
    h // (H_q / H_kv) by torch's own definition. LSE from torch.logsumexp."""
    F = torch.nn.functional
    for seed in seeds:
        w = random_workload(seed, 3, 90, 8, 2, 16, 16, "f32")
        q, k, v = f64_inputs(w)
        sm = None if default_scale else w.sm_scale
        O, LSE = mod.decode_attention(q, k, v, w.kv_indptr, w.kv_indices, w.last_page_len, sm)
        for b in range(w.batch):
            K, V = _dense(w, k, v, b)
            qt = torch.from_numpy(q[b][:, None, :])              # [Hq, 1, d]
            Kt, Vt = torch.from_numpy(K), torch.from_numpy(V)    # [Hkv, T, d]
            ref = F.scaled_dot_product_attention(qt[None], Kt[None], Vt[None], enable_gqa=True)[0]
            assert torch.allclose(torch.from_numpy(O[b]), ref[:, 0, :], atol=1e-12, rtol=0), seed
            G = w.num_qo_heads // w.num_kv_heads
            Kr = Kt.repeat_interleave(G, dim=0)
            s = (qt @ Kr.transpose(1, 2))[:, 0, :] / math.sqrt(w.head_dim)
            lse = torch.logsumexp(s, dim=-1)
            assert torch.allclose(torch.from_numpy(LSE[b]), lse, atol=1e-12, rtol=0), seed


def pin_closed_forms(mod):
    rng = np.random.default_rng(5)
    d, P = 8, 4
    # constant V: every output row equals that V row
    w = random_workload(21, 3, 30, 4, 2, d, P, "f32")
    q, k, v = f64_inputs(w)
    vc = np.empty_like(v)
    const = rng.standard_normal((w.num_kv_heads, d))
    vc[:] = const[None, :, None, :]
    O, _ = _oracle(mod, w, q, k, vc)
    for b in range(w.batch):
        for h in range(w.num_qo_heads):
            assert np.allclose(O[b, h], const[h // 2], atol=1e-13, rtol=0)
    # one-token context: O = v, LSE = sm_scale * q . k
    w1 = random_workload(22, 4, 1, 4, 2, d, P, "f32", lens=[1, 1, 1, 1])
    q, k, v = f64_inputs(w1)
    O, LSE = _oracle(mod, w1, q, k, v)
    for b in range(4):
        p = int(w1.kv_indices[w1.kv_indptr[b]])
        for h in range(4):
            assert np.allclose(O[b, h], v[p, h // 2, 0], atol=1e-13, rtol=0)
            assert abs(LSE[b, h] - (q[b, h] @ k[p, h // 2, 0]) / math.sqrt(d)) <= 1e-13
    # K = 0: uniform weights, O = mean of V rows, LSE = ln L
    w0 = random_workload(23, 3, 29, 4, 1, d, P, "f32")
    q, k, v = f64_inputs(w0)
    O, LSE = _oracle(mod, w0, q, np.zeros_like(k), v)
    for b in range(3):
        K, V = _dense(w0, np.zeros_like(k), v, b)
        L = V.shape[1]
        for h in range(4):
            assert np.allclose(O[b, h], V[0].mean(axis=0), atol=1e-13, rtol=0)
            assert abs(LSE[b, h] - math.log(L)) <= 1e-13
    # every full page listed twice: same O, LSE + ln 2
    w2 = random_workload(24, 3, 32, 4, 2, d, P, "f32", lens=[8, 16, 12])
    q, k, v = f64_inputs(w2)
    O, LSE = _oracle(mod, w2, q, k, v)
    ip2, ix2 = [0], []
    for b in range(3):
        pages = list(w2.kv_indices[w2.kv_indptr[b]:w2.kv_indptr[b + 1]])
        ix2 += pages + pages
        ip2.append(len(ix2))
    O2, LSE2 = _oracle(mod, w2, q, k, v, indptr=np.array(ip2), indices=np.array(ix2))
    assert np.allclose(O2, O, atol=1e-13, rtol=0)
    assert np.allclose(LSE2, LSE + math.log(2.0), atol=1e-13, rtol=0)


def pin_invariants(mod):
    d, P = 8, 4
    w = random_workload(31, 4, 45, 4, 2, d, P, "f32", lens=[45, 30, 21, 9])
    q, k, v = f64_inputs(w)
    O, LSE = _oracle(mod, w, q, k, v)
    # permuting the full pages (the partial page stays last) changes nothing
    rng = np.random.default_rng(3)
    ix = w.kv_indices.copy()
    for b in range(w.batch):
        s, t = w.kv_indptr[b], w.kv_indptr[b + 1]
        if t - s > 2:
            ix[s:t - 1] = ix[s:t - 1][rng.permutation(t - 1 - s)]
    Op, LSEp = _oracle(mod, w, q, k, v, indices=ix)
    assert np.allclose(Op, O, atol=1e-13, rtol=0) and np.allclose(LSEp, LSE, atol=1e-13, rtol=0)
    # dropping a listed block = dense attention with that block's scores at -inf
    b, drop = 1, 0
    s, t = w.kv_indptr[b], w.kv_indptr[b + 1]
    assert t - s >= 2
    ip2 = w.kv_indptr.copy()
    ip2[b + 1:] -= 1
    ix2 = np.delete(w.kv_indices, s + drop)
    O2, LSE2 = _oracle(mod, w, q, k, v, indptr=ip2, indices=ix2)
    K, V = _dense(w, k, v, b)
    G = w.num_qo_heads // w.num_kv_heads
    for h in range(w.num_qo_heads):
        sc = (K[h // G] @ q[b, h]) * w.sm_scale
        sc[drop * P:(drop + 1) * P] = -np.inf
        m = sc.max()
        e = np.exp(sc - m)
        assert np.allclose(O2[b, h], e @ V[h // G] / e.sum(), atol=1e-13, rtol=0)
        assert abs(LSE2[b, h] - (m + math.log(e.sum()))) <= 1e-13
    # identical query rows inside a GQA group give identical outputs
    qg = q.copy()
    qg[:, 1, :] = qg[:, 0, :]
    Og, LSEg = _oracle(mod, w, qg, k, v)
    assert np.array_equal(Og[:, 1], Og[:, 0]) and np.array_equal(LSEg[:, 1], LSEg[:, 0])


def pin_merge(mod):
    """Splitting a request's token list in two, attending over each half and
    merging the two states gives the whole-list result."""
    d, P = 8, 4
    w = random_workload(41, 3, 60, 4, 2, d, P, "f32", lens=[60, 17, 33])
    q, k, v = f64_inputs(w)
    O, LSE = _oracle(mod, w, q, k, v)
    for b in range(3):
        s, t = int(w.kv_indptr[b]), int(w.kv_indptr[b + 1])
        cut = (t - s) // 2
        # first half: full pages only; second half keeps the partial last page
        ipa = np.array([0, cut])
        ipb = np.array([0, t - s - cut])
        ixa, ixb = w.kv_indices[s:s + cut], w.kv_indices[s + cut:t]
        lasta, lastb = np.array([P]), np.array([w.last_page_len[b]])
        qa = q[b:b + 1]
        Oa, La = mod.decode_attention(qa, k, v, ipa, ixa, lasta, w.sm_scale)
        Ob, Lb = mod.decode_attention(qa, k, v, ipb, ixb, lastb, w.sm_scale)
        Om, Lm = mod.merge_states(Oa, La, Ob, Lb)
        assert np.allclose(Om[0], O[b], atol=1e-13, rtol=0), b
        assert np.allclose(Lm[0], LSE[b], atol=1e-13, rtol=0), b
        # order of the two states does not matter
        Om2, Lm2 = mod.merge_states(Ob, Lb, Oa, La)
        assert np.allclose(Om2, Om, atol=1e-14, rtol=0) and np.allclose(Lm2, Lm, atol=1e-14, rtol=0)
    # an empty state is the identity; two empty states give (0, -inf)
    va = np.random.default_rng(1).standard_normal((5, d))
    sa = np.random.default_rng(2).standard_normal(5)
    vz, sz = np.full((5, d), 7.0), np.full(5, -np.inf)
    vm, sm = mod.merge_states(va, sa, vz, sz)
    assert np.array_equal(vm, va) and np.array_equal(sm, sa)
    vm, sm = mod.merge_states(vz, sz, vz, sz)
    assert np.all(vm == 0) and np.all(np.isneginf(sm))


def pin_bf16(mod):
    """Round-to-nearest-even into bfloat16 checked against exact rational
    arithmetic over the candidate bfloat16 values."""
    from fractions import Fraction
    rng = np.random.default_rng(9)
    xs = np.concatenate([rng.standard_normal(400) * 3, rng.standard_normal(100) * 1e-3,
                         [1 + 2 ** -8, 1 + 2 ** -8 + 2 ** -40, 1 + 2 ** -8 - 2 ** -40,
                          -(1 + 2 ** -8 + 2 ** -40), 0.619140640, 0.0, 2.0 ** -7 * 3]])
    got = mod.round_bf16_rne(xs)
    lo, hi = mod.bf16_neighbors(xs)
    for x, g, a, c in zip(xs, got, lo, hi):
        fx = Fraction(float(x))
        if x == 0:
            assert g == 0
            continue
        e = math.frexp(abs(x))[1]
        step = Fraction(2) ** (e - 1 - 7)
        below = (fx // step) * step
        above = below if below == fx else below + step
        assert Fraction(float(a)) == below and Fraction(float(c)) == above, x
        if below == above:
            want = below
        else:
            db, da = fx - below, above - fx
            if db != da:
                want = below if db < da else above
            else:
                mant = int(abs(below) / step)
                want = below if mant % 2 == 0 else above
        assert Fraction(float(g)) == want, (x, g, want)


ALL_PINS = [pin_bruteforce, pin_sdpa, pin_closed_forms, pin_invariants, pin_merge]


# ------------------------------------------------------------------ prefill
def _prefill(mod, w, q, k, v, causal=None, qo_indptr=None):
    return mod.prefill_attention(q, k, v, w.qo_indptr if qo_indptr is None else qo_indptr,
                                 w.kv_indptr, w.kv_indices, w.last_page_len,
                                 w.causal if causal is None else causal, w.sm_scale)


PREFILL_TINY = [
    # seed, batch, max_len, Hq, Hkv, d, P, causal
    (51, 3, 23, 4, 1, 4, 4, True),
    (52, 3, 19, 4, 2, 8, 16, True),
    (53, 2, 17, 2, 2, 4, 1, False),
    (54, 3, 21, 8, 2, 4, 4, True),
]


def pin_prefill_bruteforce(mod, tol=1e-12):
    for (seed, B, L, Hq, Hkv, d, P, causal) in PREFILL_TINY:
        w = random_prefill_workload(seed, B, L, Hq, Hkv, d, P, causal=causal)
        q, k, v = f64_inputs(w)
        O, LSE = _prefill(mod, w, q, k, v)
        Ob, LSEb = bruteforce_prefill(q, k, v, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                      w.last_page_len, w.sm_scale, causal)
        assert np.max(np.abs(O - np.array(Ob))) <= tol, seed
        assert np.max(np.abs(LSE - np.array(LSEb))) <= tol, seed


def pin_prefill_is_decode_per_row(mod):
    """One query token per request (causal) is the decode step; without the
    mask every query token is a decode step over the whole request."""
    w = random_prefill_workload(61, 4, 40, 4, 2, 8, 4, causal=True, qo_lens=[1, 1, 1, 1])
    q, k, v = f64_inputs(w)
    O, LSE = _prefill(mod, w, q, k, v)
    Od, LSEd = mod.decode_attention(q, k, v, w.kv_indptr, w.kv_indices, w.last_page_len, w.sm_scale)
    assert np.allclose(O, Od, atol=1e-13, rtol=0) and np.allclose(LSE, LSEd, atol=1e-13, rtol=0)
    w = random_prefill_workload(62, 3, 30, 4, 2, 8, 4, causal=False)
    q, k, v = f64_inputs(w)
    O, LSE = _prefill(mod, w, q, k, v)
    for b in range(w.batch):
        for r in range(int(w.qo_indptr[b]), int(w.qo_indptr[b + 1])):
            qb = q[r][None]
            ip = np.array([0, w.kv_indptr[b + 1] - w.kv_indptr[b]])
            ix = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
            Od, LSEd = mod.decode_attention(qb, k, v, ip, ix, w.last_page_len[b:b + 1], w.sm_scale)
            assert np.allclose(O[r], Od[0], atol=1e-13, rtol=0), (b, r)
            assert np.allclose(LSE[r], LSEd[0], atol=1e-13, rtol=0), (b, r)


def pin_prefill_causal_prefix(mod):
    """Causal query i of a request with n queries over L tokens is a decode
    step over the request cut after token L - n + i (its own position): the
    page table is truncated by hand, pages and last-page length included."""
    w = random_prefill_workload(63, 3, 45, 4, 2, 8, 4, causal=True, lens=[45, 13, 8],
                                qo_lens=[9, 13, 3])
    q, k, v = f64_inputs(w)
    O, LSE = _prefill(mod, w, q, k, v)
    P = w.page_size
    for b in range(w.batch):
        L = int(w.kv_lens()[b])
        n = int(w.qo_indptr[b + 1] - w.qo_indptr[b])
        pages = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
        for i in range(n):
            keep = L - n + i + 1
            npg = (keep + P - 1) // P
            ip, ix = np.array([0, npg]), pages[:npg]
            last = np.array([keep - P * (npg - 1)])
            r = int(w.qo_indptr[b]) + i
            Od, LSEd = mod.decode_attention(q[r][None], k, v, ip, ix, last, w.sm_scale)
            assert np.allclose(O[r], Od[0], atol=1e-13, rtol=0), (b, i)
            assert np.allclose(LSE[r], LSEd[0], atol=1e-13, rtol=0), (b, i)


def pin_prefill_sdpa(mod):
    """A whole prompt as queries (n = L): torch's causal scaled dot-product
    attention in float64 (its mask aligns query i with key i, which is the
    same as the newest-token alignment when n = L), GQA by enable_gqa."""
    F = torch.nn.functional
    w = random_prefill_workload(64, 3, 50, 8, 2, 16, 16, causal=True, lens=[50, 31, 7],
                                qo_lens=[50, 31, 7])
    q, k, v = f64_inputs(w)
    O, LSE = _prefill(mod, w, q, k, v)
    for b in range(w.batch):
        K, V = _dense(w, k, v, b)                              # [Hkv, L, d]
        r0, r1 = int(w.qo_indptr[b]), int(w.qo_indptr[b + 1])
        qt = torch.from_numpy(q[r0:r1]).transpose(0, 1)[None]  # [1, Hq, n, d]
        ref = F.scaled_dot_product_attention(qt, torch.from_numpy(K)[None],
                                             torch.from_numpy(V)[None], is_causal=True,
                                             enable_gqa=True)[0]
        assert torch.allclose(torch.from_numpy(O[r0:r1]).transpose(0, 1), ref, atol=1e-12, rtol=0), b


PREFILL_PINS = [pin_prefill_bruteforce, pin_prefill_is_decode_per_row, pin_prefill_causal_prefix,
                pin_prefill_sdpa]


# --------------------------------------------------------------------- rope
def pin_rope_closed_forms(mod):
    """d = 2 is a plane rotation by pos / scale radians (theta^0 = 1); for
    d = 4 the second pair turns by pos / (scale * sqrt(theta)); position 0
    is the identity; the embedding keeps every row's norm."""
    rng = np.random.default_rng(71)
    x = rng.standard_normal((6, 2))
    pos = np.array([0, 1, 3, 17, 1000, 32767])
    for scale in (1.0, 4.0):
        y = mod.apply_rope(x, pos, 1e4, scale)
        a = pos / scale
        want = np.stack([x[:, 0] * np.cos(a) - x[:, 1] * np.sin(a),
                         x[:, 1] * np.cos(a) + x[:, 0] * np.sin(a)], axis=1)
        assert np.allclose(y, want, atol=1e-12, rtol=0)
    x4 = rng.standard_normal((3, 4))
    p4 = np.array([5, 250, 9000])
    y4 = mod.apply_rope(x4, p4, 1e4, 1.0)
    a1 = p4 / 100.0  # 1e4 ** (-2 * 1 / 4) = 1 / 100
    assert np.allclose(y4[:, 1], x4[:, 1] * np.cos(a1) - x4[:, 3] * np.sin(a1), atol=1e-12, rtol=0)
    assert np.allclose(y4[:, 3], x4[:, 3] * np.cos(a1) + x4[:, 1] * np.sin(a1), atol=1e-12, rtol=0)
    x8 = rng.standard_normal((4, 128))
    assert np.array_equal(mod.apply_rope(x8, [0, 0, 0, 0], 1e4, 1.0), x8)
    y8 = mod.apply_rope(x8, [1, 77, 4096, 131071], 5e5, 1.0)
    assert np.allclose(np.linalg.norm(y8, axis=1), np.linalg.norm(x8, axis=1), atol=1e-12, rtol=0)


def pin_rope_relative(mod):
    """The score of a rotated query and key depends on the positions only
    through their difference."""
    rng = np.random.default_rng(72)
    q = rng.standard_normal((1, 64))
    k = rng.standard_normal((1, 64))
    for m, n, c in ((10, 3, 100), (0, 500, 7), (2047, 2047, 30000)):
        s1 = (mod.apply_rope(q, [m]) @ mod.apply_rope(k, [n]).T)[0, 0]
        s2 = (mod.apply_rope(q, [m + c]) @ mod.apply_rope(k, [n + c]).T)[0, 0]
        assert abs(s1 - s2) <= 1e-10, (m, n, c)
    # and it does change with the difference
    s3 = (mod.apply_rope(q, [10]) @ mod.apply_rope(k, [4]).T)[0, 0]
    s4 = (mod.apply_rope(q, [10]) @ mod.apply_rope(k, [3]).T)[0, 0]
    assert abs(s3 - s4) > 1e-3


def pin_rope_decode(mod):
    """decode_attention_rope equals the brute-force decode over a cache whose
    rows were rotated beforehand, by plain loops, at their token index, and a
    query rotated at position L - 1."""
    for seed, theta, scale in ((73, 1e4, 1.0), (74, 5e5, 2.0)):
        w = random_workload(seed, 3, 40, 4, 2, 8, 4, "f32", lens=[37, 1, 20])
        q, k, v = f64_inputs(w)
        O, LSE = mod.decode_attention_rope(q, k, v, w.kv_indptr, w.kv_indices, w.last_page_len,
                                           w.sm_scale, theta, scale)
        kr, qr = k.copy(), q.copy()
        P = w.page_size
        for b in range(w.batch):
            pages = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
            L = int(w.kv_lens()[b])
            for t in range(L):
                pg, sl = int(pages[t // P]), t % P
                kr[pg, :, sl, :] = np.array(rope_rows_loops(k[pg, :, sl, :], [t] * w.num_kv_heads,
                                                            theta, scale))
            qr[b] = np.array(rope_rows_loops(q[b], [L - 1] * w.num_qo_heads, theta, scale))
        Ob, LSEb = bruteforce_decode(qr, kr, v, w.kv_indptr, w.kv_indices, w.last_page_len,
                                     w.sm_scale)
        assert np.max(np.abs(O - np.array(Ob))) <= 1e-12, seed
        assert np.max(np.abs(LSE - np.array(LSEb))) <= 1e-12, seed


def _prefill_rope(mod, w, q, k, v, theta, scale, causal=None):
    return mod.prefill_attention_rope(q, k, v, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                      w.last_page_len, w.causal if causal is None else causal,
                                      w.sm_scale, theta, scale)


def pin_prefill_rope_bruteforce(mod):
    """prefill_attention_rope equals the pure-Python prefill brute force over
    a cache rotated beforehand by plain loops (token t at position t) and
    query rows rotated at L - n + i, causal and unmasked."""
    for seed, causal, theta, scale in ((81, True, 1e4, 1.0), (82, False, 5e5, 2.0)):
        w = random_prefill_workload(seed, 3, 30, 4, 2, 8, 4, causal=causal,
                                    lens=[29, 1, 12], qo_lens=[5, 1, 12])
        q, k, v = f64_inputs(w)
        O, LSE = _prefill_rope(mod, w, q, k, v, theta, scale)
        kr, qr = k.copy(), q.copy()
        P = w.page_size
        for b in range(w.batch):
            pages = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
            L = int(w.kv_lens()[b])
            n = int(w.qo_indptr[b + 1] - w.qo_indptr[b])
            for t in range(L):
                pg, sl = int(pages[t // P]), t % P
                kr[pg, :, sl, :] = np.array(rope_rows_loops(k[pg, :, sl, :], [t] * w.num_kv_heads,
                                                            theta, scale))
            for i in range(n):
                row = int(w.qo_indptr[b]) + i
                qr[row] = np.array(rope_rows_loops(q[row], [L - n + i] * w.num_qo_heads, theta,
                                                   scale))
        Ob, LSEb = bruteforce_prefill(qr, kr, v, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                      w.last_page_len, w.sm_scale, causal)
        assert np.max(np.abs(O - np.array(Ob))) <= 1e-12, seed
        fin = ~np.isneginf(np.array(LSEb))
        assert np.max(np.abs(LSE[fin] - np.array(LSEb)[fin])) <= 1e-12, seed


def pin_prefill_rope_is_decode_rope(mod):
    """Causal query i of a request is a decode step over the request cut
    after its own position (decode puts its query at the last position):
    each row equals decode_attention_rope over that cut page table."""
    w = random_prefill_workload(83, 2, 70, 8, 2, 16, 8, causal=True, lens=[70, 33],
                                qo_lens=[9, 33])
    q, k, v = f64_inputs(w)
    theta, scale = 1e4, 1.0
    O, LSE = _prefill_rope(mod, w, q, k, v, theta, scale)
    P = w.page_size
    for b in range(w.batch):
        L = int(w.kv_lens()[b])
        n = int(w.qo_indptr[b + 1] - w.qo_indptr[b])
        pages = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
        for i in range(n):
            c = L - n + i + 1
            npg = (c + P - 1) // P
            row = int(w.qo_indptr[b]) + i
            Od, LSEd = mod.decode_attention_rope(q[row:row + 1], k, v, np.array([0, npg]),
                                                 pages[:npg], np.array([c - (npg - 1) * P]),
                                                 w.sm_scale, theta, scale)
            assert np.max(np.abs(O[row] - Od[0])) <= 1e-12, (b, i)
            assert np.max(np.abs(LSE[row] - LSEd[0])) <= 1e-12, (b, i)


ROPE_PINS = [pin_rope_closed_forms, pin_rope_relative, pin_rope_decode]
PREFILL_ROPE_PINS = [pin_prefill_rope_bruteforce, pin_prefill_rope_is_decode_rope]


# ---- composed formats: a prefix cache with its own block size + own pages
COMPOSED_CASES = [
    # seed, prefix_lens, members, singles, own_max, Hq, Hkv, d, P, P_prefix
    (1, [40, 0, 17], [2, 1, 2], 1, 30, 4, 2, 8, 4, 16),
    (2, [100], [3], 0, 20, 4, 1, 8, 1, 64),
    (3, [33, 64], [1, 2], 2, 9, 8, 2, 4, 16, 32),
    (4, [5, 129], [2, 2], 1, 40, 2, 2, 8, 16, 1),
]


def _one_cache(w, k, v, kp, vp):
    """The composed cache rewritten as one cache of 1-token pages: request
    b's prefix tokens (block by block, slot by slot, the last block up to its
    length), then its own tokens, each copied to a page of its own. Returns
    (k1, v1, indptr, indices, last) for the plain decode definition."""
    Hkv, d = k.shape[1], k.shape[3]
    rows_k, rows_v, indptr, indices = [], [], [0], []
    for b in range(w.batch):
        toks = []
        g = int(w.prefix_of[b])
        if g >= 0:
            first, stop = int(w.prefix_indptr[g]), int(w.prefix_indptr[g + 1])
            for j in range(first, stop):
                n = w.prefix_page_size if j + 1 < stop else int(w.prefix_last_page_len[g])
                toks += [(kp, vp, int(w.prefix_indices[j]), s) for s in range(n)]
        first, stop = int(w.kv_indptr[b]), int(w.kv_indptr[b + 1])
        for j in range(first, stop):
            n = w.page_size if j + 1 < stop else int(w.last_page_len[b])
            toks += [(k, v, int(w.kv_indices[j]), s) for s in range(n)]
        for (kk, vv, pg, s) in toks:
            indices.append(len(rows_k))
            rows_k.append(kk[pg, :, s, :])
            rows_v.append(vv[pg, :, s, :])
        indptr.append(len(indices))
    k1 = np.stack(rows_k)[:, :, None, :] if rows_k else np.zeros((0, Hkv, 1, d))
    v1 = np.stack(rows_v)[:, :, None, :] if rows_v else np.zeros((0, Hkv, 1, d))
    last = np.array([1 if indptr[b + 1] > indptr[b] else 0 for b in range(w.batch)])
    return k1, v1, np.array(indptr), np.array(indices, dtype=np.int64), last


def _composed(mod, w, q, k, v, kp, vp):
    return mod.decode_attention_composed(q, k, v, w.kv_indptr, w.kv_indices, w.last_page_len,
                                         kp, vp, w.prefix_indptr, w.prefix_indices,
                                         w.prefix_last_page_len, w.prefix_of, w.sm_scale)


def _composed_inputs(case):
    seed, plens, members, singles, own_max, Hq, Hkv, d, P, Pp = case
    w = random_composed_workload(seed, plens, members, singles, own_max, Hq, Hkv, d, P, Pp)
    return w, [t.double().numpy() for t in w.make_values("cpu")]


def pin_composed_is_one_cache(mod):
    """Composed formats are a storage layout: the result equals the plain
    decode definition over the same token sequence held in one cache."""
    for case in COMPOSED_CASES:
        w, (q, k, v, kp, vp) = _composed_inputs(case)
        O, LSE = _composed(mod, w, q, k, v, kp, vp)
        k1, v1, ip, ix, lp = _one_cache(w, k, v, kp, vp)
        O1, LSE1 = mod.decode_attention(q, k1, v1, ip, ix, lp, w.sm_scale)
        assert np.max(np.abs(O - O1)) <= 1e-12, case[0]
        assert np.array_equal(np.isneginf(LSE), np.isneginf(LSE1)), case[0]
        assert np.max(np.abs(LSE - LSE1)) <= 1e-12, case[0]


def pin_composed_bruteforce(mod):
    """The same one-cache layout through the pure-Python brute force."""
    for case in COMPOSED_CASES[:2]:
        w, (q, k, v, kp, vp) = _composed_inputs(case)
        O, LSE = _composed(mod, w, q, k, v, kp, vp)
        k1, v1, ip, ix, lp = _one_cache(w, k, v, kp, vp)
        Ob, LSEb = bruteforce_decode(q, k1, v1, ip, ix, lp, w.sm_scale)
        assert np.max(np.abs(O - np.array(Ob))) <= 1e-12, case[0]
        assert np.max(np.abs(LSE - np.array(LSEb))) <= 1e-12, case[0]


def pin_composed_prefix_counts(mod):
    """A request that shares a prefix with others gets what it gets alone
    (each request's result depends only on its own tokens), and a constant
    V over prefix and own tokens returns that constant."""
    w, (q, k, v, kp, vp) = _composed_inputs(COMPOSED_CASES[0])
    O, _ = _composed(mod, w, q, k, v, kp, vp)
    for b in range(w.batch):
        sub = dataclasses.replace(
            w, batch=1, kv_indptr=np.array([0, w.kv_indptr[b + 1] - w.kv_indptr[b]]),
            kv_indices=w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]],
            last_page_len=w.last_page_len[b:b + 1], prefix_of=w.prefix_of[b:b + 1])
        Ob, _ = _composed(mod, sub, q[b:b + 1], k, v, kp, vp)
        assert np.max(np.abs(Ob[0] - O[b])) <= 1e-13, b
    c = 0.375
    O, _ = _composed(mod, w, q, k, np.full_like(v, c), kp, np.full_like(vp, c))
    assert np.max(np.abs(O - c)) <= 1e-13


COMPOSED_PINS = [pin_composed_is_one_cache, pin_composed_bruteforce, pin_composed_prefix_counts]



# ------------------------------------------------------ latent attention (MLA)
MLA_TINY = [
    # seed, batch, max_len, heads, page size, max query tokens, d_c, d_r, causal
    (71, 3, 23, 3, 4, 3, 8, 4, True),
    (72, 4, 19, 2, 16, 1, 6, 2, True),
    (73, 2, 17, 5, 1, 4, 4, 4, False),
    (74, 3, 30, 1, 8, 5, 8, 2, True),
]


def _mla_values(w, dc, dr, seed):
    """float64 q_nope, q_pe, latent pool, rotary-key pool of small widths
    for the structure of ``w`` (unlisted slots hold NaN)."""
    rng = np.random.default_rng([seed, 5])
    N, H, P = w.num_qo_tokens, w.num_heads, w.page_size
    qn, qp = rng.standard_normal((N, H, dc)), rng.standard_normal((N, H, dr))
    ckv = np.full((w.num_pool_pages, P, dc), np.nan)
    kpe = np.full((w.num_pool_pages, P, dr), np.nan)
    for b in range(w.batch):
        first, stop = int(w.kv_indptr[b]), int(w.kv_indptr[b + 1])
        for j in range(first, stop):
            n = P if j + 1 < stop else int(w.last_page_len[b])
            pg = int(w.kv_indices[j])
            ckv[pg, :n] = rng.standard_normal((n, dc))
            kpe[pg, :n] = rng.standard_normal((n, dr))
    return qn, qp, ckv, kpe


def _mla(mod, w, qn, qp, ckv, kpe, sm_scale=0.3, qo_indptr=None, causal=None):
    return mod.mla_attention(qn, qp, ckv, kpe, w.qo_indptr if qo_indptr is None else qo_indptr,
                             w.kv_indptr, w.kv_indices, w.last_page_len, sm_scale,
                             w.causal if causal is None else causal)


def _mla_dense(w, ckv, kpe, b):
    """Dense [L, d_c] latents and [L, d_r] rotary keys of request b, straight
    from the page table."""
    P = w.page_size
    first, stop = int(w.kv_indptr[b]), int(w.kv_indptr[b + 1])
    rows = [(int(w.kv_indices[j]), s) for j in range(first, stop)
            for s in range(P if j + 1 < stop else int(w.last_page_len[b]))]
    if not rows:
        return np.zeros((0, ckv.shape[-1])), np.zeros((0, kpe.shape[-1]))
    return (np.stack([ckv[p, s] for p, s in rows]), np.stack([kpe[p, s] for p, s in rows]))


def pin_mla_bruteforce(mod, tol=1e-12):
    for (seed, B, L, H, P, mq, dc, dr, causal) in MLA_TINY + [(70, 3, 9, 2, 4, 2, 6, 4, False)]:
        # seed 70: no mask and a request without tokens (its rows: O = 0 of
        # the latent width, LSE = -inf)
        lens = [9, 0, 5] if seed == 70 else None
        w = random_mla_workload(seed, B, L, H, P, max_qo=mq, causal=causal, lens=lens,
                                qo_lens=[2, 1, 1] if lens else None)
        qn, qp, ckv, kpe = _mla_values(w, dc, dr, seed)
        O, LSE = _mla(mod, w, qn, qp, ckv, kpe)
        Ob, LSEb = bruteforce_mla(qn, qp, ckv, kpe, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                  w.last_page_len, 0.3, causal)
        Ob, LSEb = np.array(Ob), np.array(LSEb)
        assert O.shape == Ob.shape, seed
        assert np.max(np.abs(O - Ob)) <= tol, seed
        assert np.array_equal(np.isneginf(LSE), np.isneginf(LSEb)), seed
        fin = ~np.isneginf(LSEb)
        assert np.max(np.abs(LSE[fin] - LSEb[fin]), initial=0.0) <= tol, seed


def pin_mla_explicit_heads(mod):
    """The latent form against per-head attention over up-projected K and V
    (torch's float64 scaled_dot_product_attention): head h has key
    up-projection W_k[h] [d_c, d_n] and value up-projection W_v[h] [d_c, d_v];
    its key of token t is [c_t W_k[h], k_t], its value c_t W_v[h], its query
    [q_n, q_pe]. The latent form takes q_nope = W_k[h] q_n, and its output
    times W_v[h] must equal the per-head output."""
    F = torch.nn.functional
    dc, dr, dn, dv, H = 12, 4, 6, 5, 3
    w = random_mla_workload(75, 3, 29, H, 4, max_qo=4, lens=[29, 11, 6], qo_lens=[4, 2, 6])
    rng = np.random.default_rng([75, 6])
    _, qp, ckv, kpe = _mla_values(w, dc, dr, 75)
    Wk, Wv = rng.standard_normal((H, dc, dn)), rng.standard_normal((H, dc, dv))
    qn_heads = rng.standard_normal((w.num_qo_tokens, H, dn))
    qn = np.einsum("hcn,thn->thc", Wk, qn_heads)
    scale = 1.0 / math.sqrt(dn + dr)
    O, _ = _mla(mod, w, qn, qp, ckv, kpe, sm_scale=scale)
    for b in range(w.batch):
        C, R = _mla_dense(w, ckv, kpe, b)
        L, r0, r1 = C.shape[0], int(w.qo_indptr[b]), int(w.qo_indptr[b + 1])
        n = r1 - r0
        mask = torch.tensor([[t <= L - n + i for t in range(L)] for i in range(n)])
        for h in range(H):
            K = torch.from_numpy(np.concatenate([C @ Wk[h], R], axis=1))[None]   # [1, L, dn+dr]
            V = torch.from_numpy(C @ Wv[h])[None]                               # [1, L, dv]
            Q = torch.from_numpy(np.concatenate([qn_heads[r0:r1, h], qp[r0:r1, h]], axis=1))[None]
            ref = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)[0]
            got = torch.from_numpy(O[r0:r1, h] @ Wv[h])
            assert torch.allclose(got, ref, atol=1e-11, rtol=0), (b, h)


def pin_mla_without_rotary_is_mqa(mod):
    """With q_pe = 0 the rotary keys drop out: latent attention is the
    (pinned) prefill / decode oracle with one KV head whose K and V are both
    the latents and every head in its group."""
    for causal, mq in ((True, 4), (True, 1), (False, 3)):
        w = random_mla_workload(76, 4, 26, 4, 4, max_qo=mq, causal=causal)
        qn, qp, ckv, kpe = _mla_values(w, 8, 4, 76)
        O, LSE = _mla(mod, w, qn, np.zeros_like(qp), ckv, kpe)
        pool = ckv[:, None]  # [pages, 1 KV head, P, d_c]
        Oref, LSEref = mod.prefill_attention(qn, pool, pool, w.qo_indptr, w.kv_indptr,
                                             w.kv_indices, w.last_page_len, causal, 0.3)
        assert np.allclose(O, Oref, atol=1e-13, rtol=0) and np.allclose(LSE, LSEref, atol=1e-13,
                                                                         rtol=0), (causal, mq)


def pin_mla_rotary_shift(mod):
    """Adding one vector u to every cached rotary key moves each score of a
    (query token, head) by sm_scale q_pe . u, the same for all its tokens:
    outputs stay, LSE moves by exactly that amount."""
    w = random_mla_workload(77, 3, 31, 3, 8, max_qo=3)
    qn, qp, ckv, kpe = _mla_values(w, 8, 4, 77)
    u = np.array([0.5, -1.25, 2.0, 0.75])
    O, LSE = _mla(mod, w, qn, qp, ckv, kpe)
    O2, LSE2 = _mla(mod, w, qn, qp, ckv, kpe + u)
    assert np.allclose(O, O2, atol=1e-12, rtol=0)
    assert np.allclose(LSE2 - LSE, 0.3 * (qp @ u), atol=1e-12, rtol=0)


def pin_mla_single_and_constant(mod):
    """A one-token history returns its latent with LSE = the scaled score; a
    history whose latents are all one vector returns that vector."""
    w = random_mla_workload(78, 3, 1, 2, 4, lens=[1, 1, 1], qo_lens=[1, 1, 1])
    qn, qp, ckv, kpe = _mla_values(w, 6, 2, 78)
    O, LSE = _mla(mod, w, qn, qp, ckv, kpe)
    for b in range(3):
        pg = int(w.kv_indices[w.kv_indptr[b]])
        assert np.allclose(O[b], ckv[pg, 0][None], atol=1e-14, rtol=0)
        assert np.allclose(LSE[b], 0.3 * (qn[b] @ ckv[pg, 0] + qp[b] @ kpe[pg, 0]), atol=1e-12)
    w = random_mla_workload(79, 3, 40, 2, 4, max_qo=3)
    qn, qp, ckv, kpe = _mla_values(w, 6, 2, 79)
    c = np.array([1.5, -2.0, 0.25, 3.0, -0.5, 1.0])
    ckv = np.where(np.isnan(ckv), np.nan, c[None, None, :])
    O, _ = _mla(mod, w, qn, qp, ckv, kpe)
    assert np.allclose(O, np.broadcast_to(c, O.shape), atol=1e-13, rtol=0)


MLA_PINS = [pin_mla_bruteforce, pin_mla_explicit_heads, pin_mla_without_rotary_is_mqa,
            pin_mla_rotary_shift, pin_mla_single_and_constant]
