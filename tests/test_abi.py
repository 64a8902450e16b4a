"""The C-ABI library on a CPU-only host: it loads, exports every function the
header declares, and rejects malformed calls with a status and a message
before touching any device."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_kv_bsr_amd as fb
from block_sparse_kv_bsr_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions(header="fi_bsr.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fi_[a-z_]+)\s*\(", text)))


def test_header_matches_binding_list():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = fb.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_bench_helper_library_loads_and_exports_its_symbol():
    # the benchmark's streaming-read helper lives in its own library
    path = os.path.join(ROOT, "block_sparse_kv_bsr_amd", "libfi_bench.so")
    L = ctypes.CDLL(path)
    names = declared_functions("fi_bench.h")
    assert names == ["fi_bench_stream_read"]
    for name in names:
        assert hasattr(L, name), name
    # malformed calls are refused before any launch (hipErrorInvalidValue)
    L.fi_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert L.fi_bench_stream_read(None, 16, None, None) != 0
    assert L.fi_bench_stream_read(ctypes.c_void_p(16), 15, ctypes.c_void_p(16), None) != 0


def _plan_status(indptr, indices, last, Hq=8, Hkv=2, d=128, P=16, pool=100, dtype=1, opts=None):
    L = fb.lib()
    ip = np.asarray(indptr, dtype=np.int32)
    ix = np.asarray(indices, dtype=np.int32)
    lp = np.asarray(last, dtype=np.int32)
    h = ctypes.c_void_p()
    p32 = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    st = L.fi_plan_create(p32(ip), p32(ix) if ix.size else None, p32(lp), len(ip) - 1, Hq, Hkv, d, P,
                          pool, dtype, ctypes.byref(opts) if opts else None, ctypes.byref(h))
    if st == 0:
        L.fi_plan_destroy(h)
    return st, L.fi_last_error().decode()


GOOD = ([0, 2, 3], [5, 6, 7], [16, 3])


def test_good_plan_is_ok():
    assert _plan_status(*GOOD)[0] == 0


@pytest.mark.parametrize("args,kw,code,needle", [
    (([1, 2, 3], [5, 6, 7], [16, 3]), {}, -1, "kv_indptr[0]"),
    (([0, 3, 2], [5, 6, 7], [16, 3]), {}, -1, "non-decreasing"),
    (([0, 2, 3], [5, 6, 700], [16, 3]), {}, -1, "num_pool_pages"),
    (([0, 2, 3], [5, -1, 7], [16, 3]), {}, -1, "num_pool_pages"),
    (([0, 2, 3], [5, 6, 7], [0, 3]), {}, -1, "kv_last_page_len[0]"),
    (([0, 2, 3], [5, 6, 7], [16, 17]), {}, -1, "kv_last_page_len[1]"),
    (GOOD, {"Hq": 6, "Hkv": 4}, -1, "multiple"),
    (GOOD, {"Hq": 24, "Hkv": 2}, -2, "group size"),
    (GOOD, {"d": 96}, -2, "head_dim"),
    (GOOD, {"dtype": 7}, -2, "dtype"),
    (GOOD, {"P": 0}, -1, "page_size"),
    (GOOD, {"Hq": 0}, -1, "positive"),
])
def test_plan_rejects(args, kw, code, needle):
    st, msg = _plan_status(*args, **kw)
    assert st == code and needle in msg, (st, msg)


def test_negative_option_rejected():
    o = binding.PlanOpts(-1, 0, 0, 0, 0)
    st, msg = _plan_status(*GOOD, opts=o)
    assert st == -1 and "option" in msg


def test_run_without_upload_is_state_error():
    """fi_decode_run refuses a workspace the plan was not uploaded to; the
    check happens on the host before any launch."""
    p = fb.plan(*[np.asarray(a) for a in GOOD], 8, 2, 128, 16, 100, "bf16")
    L = fb.lib()
    fake = ctypes.c_void_p(0x100000)
    ws = p.info["workspace_bytes"]
    st = L.fi_decode_run(p.handle, fake, fake, fake, fake, None, 0.0, fake, ws, None)
    assert st == -6 and "upload" in L.fi_last_error().decode()
    st = L.fi_decode_run(p.handle, fake, fake, fake, fake, None, 0.0, fake, ws - 1, None)
    assert st == -3
    st = L.fi_decode_run(p.handle, ctypes.c_void_p(0x100001), fake, fake, fake, None, 0.0, fake, ws, None)
    assert st == -1 and "aligned" in L.fi_last_error().decode()
    st = L.fi_decode_run(None, fake, fake, fake, fake, None, 0.0, fake, ws, None)
    assert st == -1


def test_upload_rejects_small_or_misaligned_workspace():
    # cut requests: the image (what an upload needs) is smaller than the
    # whole workspace (image + partial states, what fi_decode_run needs)
    p = fb.plan([0, 40, 41], list(range(41)), [16, 3], 8, 2, 128, 16, 100, "bf16",
                fixed_chunk_tokens=64)
    L = fb.lib()
    img, ws = p.info["image_bytes"], p.info["workspace_bytes"]
    assert 0 < img < ws
    assert L.fi_plan_upload(p.handle, ctypes.c_void_p(0x100000), img - 1, None) == -3
    assert "image" in L.fi_last_error().decode()
    assert L.fi_plan_upload(p.handle, ctypes.c_void_p(0x100010), ws, None) == -1
    assert L.fi_plan_upload(p.handle, None, ws, None) == -1


def test_merge_states_rejects():
    L = fb.lib()
    fake = ctypes.c_void_p(0x100000)
    assert L.fi_merge_states(3, fake, fake, fake, fake, fake, fake, 4, 128, None) == -2
    assert L.fi_merge_states(1, fake, fake, fake, fake, fake, fake, 4, 96, None) == -2
    assert L.fi_merge_states(1, fake, fake, fake, fake, fake, fake, -1, 128, None) == -1
    assert L.fi_merge_states(1, None, fake, fake, fake, fake, fake, 4, 128, None) == -1
    assert L.fi_merge_states(1, fake, fake, fake, fake, fake, fake, 0, 128, None) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    p = fb.plan(*[np.asarray(a) for a in GOOD], 8, 2, 128, 16, 100, "bf16")
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    k = torch.zeros(100, 2, 16, 128, dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="GPU"):
        fb.decode(q, k, k, p)


def test_rope_run_rejects_what_is_not_built():
    """fi_decode_run_rope(_scaled) checks the plan before touching any
    device: only bf16 plans (head_dim 128 or 64) and fp8 plans (128) with no
    shared-prefix items, finite parameters, finite positive scales."""
    L = fb.lib()
    fake = ctypes.c_void_p(0x100000)
    ip, ix, lp = [np.asarray(a) for a in GOOD]
    for dtype, d in (("f32", 128), ("f32", 64)):
        p = fb.plan(ip, ix, lp, 8, 2, d, 16, 100, dtype)
        st = L.fi_decode_run_rope(p.handle, fake, fake, fake, 1e4, 1.0, fake, None, 0.0, fake,
                                  p.info["workspace_bytes"], None)
        assert st == -2 and "rotary" in L.fi_last_error().decode(), (dtype, d)
    p = fb.plan(ip, ix, lp, 8, 2, 128, 16, 100, "bf16")
    st = L.fi_decode_run_rope(p.handle, fake, fake, fake, float("nan"), 1.0, fake, None, 0.0, fake,
                              p.info["workspace_bytes"], None)
    assert st == -1
    st = L.fi_decode_run_rope(p.handle, fake, fake, fake, 0.5, 1.0, fake, None, 0.0, fake,
                              p.info["workspace_bytes"], None)
    assert st == -1 and "exceed 1" in L.fi_last_error().decode()
    # accepted parameters, but the plan was not uploaded to this workspace
    st = L.fi_decode_run_rope(p.handle, fake, fake, fake, 0.0, 0.0, fake, None, 0.0, fake,
                              p.info["workspace_bytes"], None)
    assert st == -6
    p8 = fb.plan(ip, ix, lp, 8, 2, 128, 16, 100, "fp8")
    for ks, vs in ((0.0, 1.0), (1.0, -1.0), (float("inf"), 1.0), (1.0, float("nan"))):
        st = L.fi_decode_run_rope_scaled(p8.handle, fake, fake, fake, ks, vs, 1e4, 1.0, fake, None,
                                         0.0, fake, p8.info["workspace_bytes"], None)
        assert st == -1 and "scale" in L.fi_last_error().decode(), (ks, vs)
    st = L.fi_decode_run_rope_scaled(p8.handle, fake, fake, fake, 0.5, 2.0, 1e4, 1.0, fake, None,
                                     0.0, fake, p8.info["workspace_bytes"], None)
    assert st == -6
    p64 = fb.plan(ip, ix, lp, 8, 2, 64, 16, 100, "bf16")
    st = L.fi_decode_run_rope(p64.handle, fake, fake, fake, 1e4, 1.0, fake, None, 0.0, fake,
                              p64.info["workspace_bytes"], None)
    assert st == -6


def test_prefill_run_checks_on_the_host():
    L = fb.lib()
    fake = ctypes.c_void_p(0x100000)
    ip, ix, lp = [np.asarray(a) for a in GOOD]
    p = fb.prefill_plan(np.array([0, 2, 3]), ip, ix, lp, 8, 2, 128, 16, 100)
    ws = p.info["workspace_bytes"]
    assert L.fi_prefill_run(None, fake, fake, fake, fake, None, 0.0, fake, ws, None) == -1
    assert L.fi_prefill_run(p.handle, fake, fake, fake, fake, None, 0.0, fake, ws, None) == -6
    assert L.fi_prefill_run(p.handle, fake, fake, fake, fake, None, 0.0, fake, ws - 1, None) == -3
    assert L.fi_prefill_run(p.handle, None, fake, fake, fake, None, 0.0, fake, ws, None) == -1
    assert L.fi_prefill_run(p.handle, ctypes.c_void_p(0x100008), fake, fake, fake, None, 0.0, fake, ws,
                            None) == -1
    assert L.fi_prefill_plan_upload(p.handle, ctypes.c_void_p(0x100010), ws, None) == -1
    assert L.fi_prefill_plan_upload(p.handle, fake, ws - 1, None) == -3
    # the scaled run checks its scales first, then the same as fi_prefill_run
    for ks, vs in ((0.0, 1.0), (1.0, -1.0), (float("inf"), 1.0), (1.0, float("nan"))):
        st = L.fi_prefill_run_scaled(p.handle, fake, fake, fake, ks, vs, fake, None, 0.0, fake, ws,
                                     None)
        assert st == -1 and "scale" in L.fi_last_error().decode(), (ks, vs)
    assert L.fi_prefill_run_scaled(p.handle, fake, fake, fake, 0.5, 2.0, fake, None, 0.0, fake, ws,
                                   None) == -6
    # rope runs and plans go together
    assert L.fi_prefill_run_rope(p.handle, fake, fake, fake, 1e4, 1.0, fake, None, 0.0, fake, ws,
                                 None) == -1
    assert "fi_prefill_opts.rope" in L.fi_last_error().decode()
    pr = fb.prefill_plan(np.array([0, 2, 3]), ip, ix, lp, 8, 2, 128, 16, 100, rope=True)
    wr = pr.info["workspace_bytes"]
    assert L.fi_prefill_run(pr.handle, fake, fake, fake, fake, None, 0.0, fake, wr, None) == -1
    assert "fi_prefill_run_rope" in L.fi_last_error().decode()
    for th, sc in ((0.5, 1.0), (float("inf"), 1.0), (1e4, float("nan"))):
        assert L.fi_prefill_run_rope(pr.handle, fake, fake, fake, th, sc, fake, None, 0.0, fake, wr,
                                     None) == -1, (th, sc)
    assert L.fi_prefill_run_rope(pr.handle, fake, fake, fake, 0.0, 0.0, fake, None, 0.0, fake, wr,
                                 None) == -6   # defaults accepted; not uploaded


def test_binding_refuses_arrays_shorter_than_the_page_table():
    """The C ABI reads kv_indices up to kv_indptr[batch] and cannot see the
    array's length: the binding refuses a short array before the call."""
    with pytest.raises(ValueError, match="kv_indices holds 2 entries"):
        fb.plan([0, 40], [1, 2], [16], 8, 2, 128, 16, 100, "bf16")
    with pytest.raises(ValueError, match="kv_indices holds 3 entries"):
        fb.plan([0, 5, 3], [1, 2, 3], [16, 16], 8, 2, 128, 16, 100, "bf16")
    with pytest.raises(ValueError, match="one entry per request"):
        fb.plan([0, 2, 3], [5, 6, 7], [16], 8, 2, 128, 16, 100, "bf16")
    with pytest.raises(ValueError, match="kv_indices holds 2 entries"):
        fb.prefill_plan([0, 1], [0, 40], [1, 2], [16], 8, 2, 128, 16, 100)
    with pytest.raises(ValueError, match="disagree"):
        fb.prefill_plan([0, 1, 2], [0, 2], [1, 2], [16], 8, 2, 128, 16, 100)
    # the same arrays at their full lengths are accepted
    fb.plan([0, 2, 3], [5, 6, 7], [16, 3], 8, 2, 128, 16, 100, "bf16")
    fb.prefill_plan([0, 1], [0, 2], [1, 2], [16], 8, 2, 128, 16, 100)
