"""The host planners under AddressSanitizer and UndefinedBehaviorSanitizer.

plan.cpp and prefill_plan.cpp parse caller-supplied page tables. They are
compiled here with g++ and both sanitizers into a small driver
(tests/planner_driver.cpp) that makes each planner call with its input
arrays allocated at exactly their stated lengths, reads the plan back
through the accessor calls and frees it. The calls are the malformed ones
the ABI tests reject, seeded random valid ones of the kind the property
tests draw (ragged and empty requests, every page size class, GQA groups,
dtypes, planner options, shared prefixes, causal and unmasked prefill), and
the full-size workloads. The driver must exit cleanly with no sanitizer
report, and every call's status and plan must equal what the regular
library returns for the same call.
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

import block_sparse_kv_bsr_amd as fb
from block_sparse_kv_bsr_amd import binding
from block_sparse_kv_bsr_amd.workloads import mla_workload, prefill_workload, workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_kv_bsr_amd", "csrc")
MASK = (1 << 64) - 1


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ is not installed")
    exe = str(tmp_path_factory.mktemp("sanitized") / "planner_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "prefill_plan.cpp"),
           os.path.join(ROOT, "tests", "planner_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


# ------------------------------------------------------------------ cases
class Call:
    """One planner call: kind 'D' (fi_plan_create), 'P' (prefill), 'C'
    (composed) or 'M' (MLA: hq = heads, hkv = latent width, d = rotary
    width)."""

    def __init__(self, kind, batch, hq, hkv, d, P, pool, dtype, ip, ix, lp, opts=None, qo=None,
                 causal=1, prefixes=None):
        self.kind, self.hdr = kind, [batch, hq, hkv, d, P, pool, dtype, causal]
        self.ip, self.ix, self.lp, self.qo, self.opts = ip, ix, lp, qo, opts
        # kind 'C': (prefix_page_size, pool, prefix_indptr, prefix_indices,
        # prefix_last_page_len, prefix_of)
        self.prefixes = prefixes

    def text(self):
        def arr(a):
            if a is None:
                return "-1"
            a = [int(x) for x in a]
            return " ".join(map(str, [len(a)] + a))
        parts = [self.kind, " ".join(map(str, self.hdr))]
        parts.append(arr(self.opts) if self.opts is not None else "0")
        if self.kind in ("P", "M"):
            parts.append(arr(self.qo))
        parts += [arr(self.ip), arr(self.ix), arr(self.lp)]
        if self.kind == "C":
            Pp, ppool, pip, pix, plp, of = self.prefixes
            parts += [f"{Pp} {ppool}", arr(pip), arr(pix), arr(plp), arr(of)]
        return "\n".join(parts)


def malformed_calls():
    good = ([0, 2, 3], [5, 6, 7], [16, 3])
    out = []
    dec = [
        (([1, 2, 3], [5, 6, 7], [16, 3]), {}),
        (([0, 3, 2], [5, 6, 7], [16, 3]), {}),
        (([0, 2, 3], [5, 6, 700], [16, 3]), {}),
        (([0, 2, 3], [5, -1, 7], [16, 3]), {}),
        (([0, 2, 3], [5, 6, 7], [0, 3]), {}),
        (([0, 2, 3], [5, 6, 7], [16, 17]), {}),
        (good, {"hq": 6, "hkv": 4}), (good, {"hq": 24, "hkv": 2}), (good, {"d": 96}),
        (good, {"dtype": 7}), (good, {"P": 0}), (good, {"P": 5000}), (good, {"hq": 0}),
        (good, {"pool": -1}), (good, {"dtype": 2, "d": 64}),
        (good, {"opts": [-1, 0, 0, 0, 0, 0, 0]}), (good, {"opts": [0, 0, 0, 0, -5, 0, 0]}),
        (good, {"opts": [0, 0, 0, 0, 0, 0, 3]}), (good, {"opts": [0, 0, 0, 0, 0, 0, 2], "d": 64}),
        (good, {"opts": [0, 0, 0, 0, 0, 0, 2], "P": 8}),
        ((None, [5, 6, 7], [16, 3]), {}), (([0, 2, 3], None, [16, 3]), {}),
        (([0, 2, 3], [5, 6, 7], None), {}),
    ]
    for (ip, ix, lp), kw in dec:
        a = dict(hq=8, hkv=2, d=128, P=16, pool=100, dtype=1, opts=None)
        a.update(kw)
        batch = len(ip) - 1 if ip is not None else 2
        out.append(Call("D", batch, a["hq"], a["hkv"], a["d"], a["P"], a["pool"], a["dtype"],
                        ip, ix, lp, a["opts"]))
    out.append(Call("D", -1, 8, 2, 128, 16, 100, 1, [0], [], []))
    pre = [dict(opts=[0, 0, 0, 0, 1], dtype=2), dict(opts=[0, 0, 0, 0, 1], d=64),
           dict(opts=[0, 0, 0, 0, 1], causal=0, qo=[0, 2, 40]),
           dict(qo=[1, 2, 3]), dict(qo=[0, 3, 2]), dict(qo=[0, 40, 41]), dict(dtype=0),
           dict(d=96), dict(hq=8, hkv=3), dict(hq=512, hkv=1), dict(ix=[5, 6, 700]),
           dict(hq=257, hkv=1), dict(qo=None), dict(lp=[16, 0]),
           dict(opts=[-1, 0, 0, 0]), dict(opts=[0, 0, -3, 0])]
    for kw in pre:
        a = dict(qo=[0, 2, 3], ip=[0, 2, 3], ix=[5, 6, 7], lp=[16, 3], hq=8, hkv=2, d=128, P=16,
                 pool=100, dtype=1, causal=1, opts=None)
        a.update(kw)
        out.append(Call("P", 2, a["hq"], a["hkv"], a["d"], a["P"], a["pool"], a["dtype"], a["ip"],
                        a["ix"], a["lp"], a["opts"], a["qo"], a["causal"]))
    mla = [dict(hkv=576), dict(d=128), dict(hq=0), dict(hq=5000), dict(opts=[0, 0, 0, 0, 1]),
           dict(qo=[0, 40, 41]), dict(ix=[5, 6, 700]), dict(qo=None), dict(opts=[0, -2, 0, 0])]
    for kw in mla:
        a = dict(qo=[0, 2, 3], ip=[0, 2, 3], ix=[5, 6, 7], lp=[16, 3], hq=96, hkv=512, d=64, P=16,
                 pool=100, causal=1, opts=None)
        a.update(kw)
        out.append(Call("M", 2, a["hq"], a["hkv"], a["d"], a["P"], a["pool"], 1, a["ip"], a["ix"],
                        a["lp"], a["opts"], a["qo"], a["causal"]))
    comp = [dict(of=[0, 2]), dict(of=[-2, 0]), dict(of=None), dict(pix=[4, 1, 10]),
            dict(plp=[70, 5]), dict(plp=[0, 5]), dict(Pp=0), dict(Pp=5000), dict(dtype=2),
            dict(pip=None), dict(pip=[1, 2, 3]), dict(pip=[0, 2, 1]), dict(ppool=-1),
            dict(ip=[0, 0, 1], ix=[7], lp=[0, 3]),                 # a prefix, no own token
            dict(Pp=1, pip=[0, 4000, 4001], pix=list(range(4001)), plp=[1, 1], ppool=4001)]
    for kw in comp:
        a = dict(ip=[0, 2, 3], ix=[5, 6, 7], lp=[16, 3], Pp=64, ppool=10, pip=[0, 2, 3],
                 pix=[4, 1, 8], plp=[64, 5], of=[0, 1], dtype=1)
        a.update(kw)
        out.append(Call("C", 2, 8, 2, 128, 16, 100, a["dtype"], a["ip"], a["ix"], a["lp"],
                        prefixes=(a["Pp"], a["ppool"], a["pip"], a["pix"], a["plp"], a["of"])))
    return out


def _page_table(rng, lens, P, spare, share=None):
    """Page lists for the given token counts in a permuted pool; with
    share = (members, pages), the first `members` requests list the same
    `pages` leading physical pages."""
    npg = [(L + P - 1) // P for L in lens]
    shared = share[1] if share else 0
    pool = sum(npg) - (share[0] - 1) * shared if share else sum(npg)
    pool += spare
    perm = rng.permutation(pool)
    ip, ix, lp, used = [0], [], [], 0
    common = [int(x) for x in perm[:shared]]
    used = shared
    for b, (L, n) in enumerate(zip(lens, npg)):
        if share and b < share[0] and n >= shared:
            pages = common + [int(x) for x in perm[used:used + n - shared]]
            used += n - shared
        else:
            pages = [int(x) for x in perm[used:used + n]]
            used += n
        ix += pages
        ip.append(ip[-1] + n)
        lp.append(L - (n - 1) * P if n else 0)
    return ip, ix, lp, pool


def random_calls(seed=7, n_decode=160, n_prefill=100):
    rng = np.random.default_rng(seed)
    out = []
    sizes = [1, 3, 5, 8, 12, 16, 32, 64]
    for i in range(n_decode):
        B = int(rng.integers(1, 10))
        P = int(rng.choice(sizes))
        lens = [int(x) for x in rng.integers(0, 900, size=B)]
        if rng.random() < 0.3:
            lens[int(rng.integers(B))] = 0
        G = int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.choice([1, 2, 8]))
        d = int(rng.choice([64, 128]))
        dtype = int(rng.choice([0, 1, 2])) if d == 128 else int(rng.choice([0, 1]))
        share = None
        if B >= 2 and rng.random() < 0.4:
            m = int(rng.integers(2, B + 1))
            pages = int(rng.integers(1, 6))
            for b in range(m):
                lens[b] = max(lens[b], (pages + 1) * P)
            share = (m, pages)
        ip, ix, lp, pool = _page_table(rng, lens, P, int(rng.integers(0, 4)), share)
        opts = None
        if rng.random() < 0.7:
            opts = [int(rng.choice([0, 8, 64, 256])), int(rng.choice([0, 1, 4, 8])),
                    int(rng.choice([0, 1, 16, 300])), int(rng.choice([0, 64, 4096])),
                    int(rng.choice([0, 0, 1, 20, 100])), int(rng.choice([-1, 0, 1])),
                    int(rng.choice([0, 1, 2])) if (d == 128 and dtype and P % 16 == 0) else 0]
        out.append(Call("D", B, G * hkv, hkv, d, P, pool, dtype, ip, ix, lp, opts))
    for i in range(n_prefill):
        B = int(rng.integers(1, 7))
        P = int(rng.choice(sizes))
        lens = [int(x) for x in rng.integers(0, 800, size=B)]
        causal = int(rng.random() < 0.7)
        qo = [int(rng.integers(0, L + 1)) if causal else int(rng.integers(0, 300)) for L in lens]
        G = int(rng.choice([1, 2, 3, 4, 8, 16]))
        hkv = int(rng.choice([1, 2, 8]))
        ip, ix, lp, pool = _page_table(rng, lens, P, int(rng.integers(0, 4)))
        opts = None
        if rng.random() < 0.7:
            opts = [int(rng.choice([0, 8, 256])), int(rng.choice([0, 1, 4])),
                    int(rng.choice([0, 0, 16, 64, 512])), int(rng.choice([0, 1, 3, 8]))]
        qoi = np.concatenate([[0], np.cumsum(qo)]).tolist()
        d = int(rng.choice([64, 128]))
        # rope plans: bf16, d 128, every request's queries cached
        if d == 128 and all(n <= L for n, L in zip(qo, lens)) and rng.random() < 0.4:
            opts = (opts or [0, 0, 0, 0]) + [1]
        out.append(Call("P", B, G * hkv, hkv, d, P, pool, 1, ip, ix, lp, opts, qoi, causal))
    for i in range(60):
        B = int(rng.integers(1, 10))
        P = int(rng.choice(sizes))
        lens = [int(x) for x in rng.integers(1, 500, size=B)]
        nprefix = int(rng.integers(0, 4))
        Pp = int(rng.choice([1, 7, 16, 64, 512, 4096]))
        plens = [int(x) for x in rng.integers(0, 3000 if Pp > 1 else 900, size=nprefix)]
        of = [int(rng.integers(-1, nprefix)) for _ in range(B)]
        G = int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.choice([1, 2, 8]))
        ip, ix, lp, pool = _page_table(rng, lens, P, int(rng.integers(0, 4)))
        pip, pix, plp, ppool = _page_table(rng, plens, Pp, int(rng.integers(0, 3)))
        opts = None
        if rng.random() < 0.5:
            opts = [int(rng.choice([0, 8, 256])), int(rng.choice([0, 1, 8])),
                    int(rng.choice([0, 16, 300])), 0, int(rng.choice([0, 1, 100])), 0, 0]
        out.append(Call("C", B, G * hkv, hkv, int(rng.choice([64, 128])), P, pool, 1, ip, ix, lp,
                        opts, prefixes=(Pp, ppool, pip, pix, plp, of)))
    for i in range(60):
        B = int(rng.integers(1, 7))
        P = int(rng.choice(sizes))
        lens = [int(x) for x in rng.integers(0, 900, size=B)]
        causal = int(rng.random() < 0.8)
        qo = [int(rng.integers(0, min(L, 6) + 1)) if causal else int(rng.integers(0, 5)) for L in lens]
        H = int(rng.choice([1, 5, 12, 16, 32, 40, 96, 128, 200]))
        ip, ix, lp, pool = _page_table(rng, lens, P, int(rng.integers(0, 4)))
        opts = None
        if rng.random() < 0.7:
            opts = [int(rng.choice([0, 8, 256])), int(rng.choice([0, 1, 4])),
                    int(rng.choice([0, 0, 16, 64, 1000])), int(rng.choice([0, 1, 8]))]
        qoi = np.concatenate([[0], np.cumsum(qo)]).tolist()
        out.append(Call("M", B, H, 512, 64, P, pool, 1, ip, ix, lp, opts, qoi, causal))
    return out


def full_size_calls():
    out = []
    for cfg in (2, 3, 4, 5):
        w = workload(cfg)
        dt = {"f32": 0, "bf16": 1, "fp8": 2}[w.dtype]
        out.append(Call("D", w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                        w.num_pool_pages, dt, w.kv_indptr, w.kv_indices, w.last_page_len))
    w = workload(13)
    out.append(Call("C", w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                    w.num_pool_pages, 1, w.kv_indptr, w.kv_indices, w.last_page_len,
                    prefixes=(w.prefix_page_size, w.num_prefix_pool_pages, w.prefix_indptr,
                              w.prefix_indices, w.prefix_last_page_len, w.prefix_of)))
    w = mla_workload(15)
    out.append(Call("M", w.batch, w.num_heads, 512, 64, w.page_size, w.num_pool_pages, 1,
                    w.kv_indptr, w.kv_indices, w.last_page_len, None, w.qo_indptr, int(w.causal)))
    for cfg in (7, 8):
        w = prefill_workload(cfg)
        out.append(Call("P", w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                        w.num_pool_pages, 1, w.kv_indptr, w.kv_indices, w.last_page_len,
                        None, w.qo_indptr, int(w.causal)))
    return out


# ------------------------------------------------- the regular library
def _fnv(h, x):
    return ((h ^ (int(x) & MASK)) * 1099511628211) & MASK


def _mix_array(h, a):
    a = np.asarray(a).reshape(-1)
    h = _fnv(h, a.size)
    for x in a.tolist():
        h = _fnv(h, x)
    return h


def regular_line(call: Call):
    L = fb.lib()
    extra = call.prefixes[2:] if call.kind == "C" else ()
    keep = [np.ascontiguousarray(a, dtype=np.int32) if a is not None else None
            for a in (call.qo, call.ip, call.ix, call.lp, *extra)]
    ptrs = [None if a is None else (a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
                                    if a.size else ctypes.cast(ctypes.c_void_p(16),
                                                               ctypes.POINTER(ctypes.c_int32)))
            for a in keep]
    h = ctypes.c_void_p()
    b, hq, hkv, d, P, pool, dtype, causal = call.hdr
    if call.kind == "C":
        opts = ctypes.byref(binding.PlanOpts(*call.opts)) if call.opts is not None else None
        nprefix = len(keep[4]) - 1 if keep[4] is not None else 0
        st = L.fi_plan_create_composed(ptrs[1], ptrs[2], ptrs[3], b, ptrs[4], ptrs[5], ptrs[6],
                                       nprefix, ptrs[7], hq, hkv, d, P, pool, call.prefixes[0],
                                       call.prefixes[1], dtype, opts, ctypes.byref(h))
    elif call.kind == "D":
        opts = ctypes.byref(binding.PlanOpts(*call.opts)) if call.opts is not None else None
        st = L.fi_plan_create(ptrs[1], ptrs[2], ptrs[3], b, hq, hkv, d, P, pool, dtype, opts,
                              ctypes.byref(h))
    elif call.kind == "M":
        opts = ctypes.byref(binding.PrefillOpts(*call.opts)) if call.opts is not None else None
        st = L.fi_mla_plan_create(ptrs[0], ptrs[1], ptrs[2], ptrs[3], b, hq, hkv, d, P, pool,
                                  causal, opts, ctypes.byref(h))
    else:
        opts = ctypes.byref(binding.PrefillOpts(*call.opts)) if call.opts is not None else None
        st = L.fi_prefill_plan_create(ptrs[0], ptrs[1], ptrs[2], ptrs[3], b, hq, hkv, d, P, pool,
                                      dtype, causal, opts, ctypes.byref(h))
    hs = _fnv(1469598103934665603, st)
    if st != 0:
        return st, hs
    if call.kind in ("D", "C"):
        p = binding.Plan(h.value)
        for k in ("num_items", "num_partial_slots", "workspace_bytes"):
            hs = _fnv(hs, p.info[k])
        for a in (p.work_list(), p.merge_nodes(), p.prefix_items(), p.prefix_members()):
            hs = _mix_array(hs, a)
    else:
        p = binding.PrefillPlan(h.value)
        for k in ("num_items", "num_partial_slots", "workspace_bytes"):
            hs = _fnv(hs, p.info[k])
        for a in (p.work_list(), p.merges()):
            hs = _mix_array(hs, a)
    del p
    return st, hs


def run_driver(exe, calls):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], input="\n".join(c.text() for c in calls) + "\n",
                       capture_output=True, text=True, env=env, timeout=600)
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.returncode, r.stderr[-4000:])
    lines = r.stdout.split("\n")
    got = {}
    for ln in lines:
        if ln.strip():
            i, st, hv = ln.split()
            got[int(i)] = (int(st), int(hv))
    assert sorted(got) == list(range(len(calls)))
    return got


@pytest.mark.parametrize("which", ["malformed", "random", "full_size"])
def test_planners_clean_under_sanitizers(driver, which):
    calls = {"malformed": malformed_calls, "random": random_calls,
             "full_size": full_size_calls}[which]()
    got = run_driver(driver, calls)
    statuses = set()
    for i, c in enumerate(calls):
        want = regular_line(c)
        assert got[i] == want, (i, c.text()[:400], got[i], want)
        statuses.add(want[0])
    if which == "malformed":
        assert statuses <= {-1, -2} and statuses == {-1, -2}
    else:
        assert statuses == {0}


def test_the_driver_reports_a_read_past_an_input_array(driver):
    """The instrumentation is live: a call that breaks the documented length
    contract (kv_indices shorter than kv_indptr[batch] says) makes the
    planner read past the array, and AddressSanitizer stops the driver."""
    bad = Call("D", 1, 8, 2, 128, 16, 100, 1, [0, 3], [5, 6], [16])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([driver], input=bad.text() + "\n", capture_output=True, text=True,
                       env=env, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
