"""Thin ctypes binding over ``libfi_bsr.so`` (the C ABI in include/fi_bsr.h).

Only argument marshalling lives here: torch supplies device memory and the
current stream; every step of decode attention runs in the library's HIP
kernels. There is no fallback: if the library is missing or a tensor is not on
a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfi_bsr.so")

FI_OK = 0
FI_DTYPE_F32 = 0
FI_DTYPE_BF16 = 1
FI_DTYPE_FP8_E4M3 = 2
ITEM_STRIDE = 16
NODE_STRIDE = 8
PITEM_STRIDE = 12
MERGE_FAN_IN = 32
DECODE_KERNEL_AUTO, DECODE_KERNEL_VECTOR, DECODE_KERNEL_MATRIX = 0, 1, 2

STATUS_NAMES = {0: "FI_OK", -1: "FI_ERR_INVALID_ARG", -2: "FI_ERR_UNSUPPORTED",
                -3: "FI_ERR_WORKSPACE", -4: "FI_ERR_HIP", -5: "FI_ERR_NOMEM", -6: "FI_ERR_STATE"}

# Every symbol include/fi_bsr.h declares.
EXPORTED = ["fi_plan_create", "fi_plan_get_info", "fi_plan_work_list", "fi_plan_merge_nodes",
            "fi_plan_prefix_items", "fi_plan_prefix_members", "fi_plan_upload", "fi_decode_run",
            "fi_decode_run_scaled", "fi_merge_states", "fi_plan_destroy", "fi_last_error",
            "fi_prefill_plan_create", "fi_prefill_plan_get_info", "fi_prefill_plan_work_list",
            "fi_prefill_plan_merges", "fi_prefill_plan_upload", "fi_prefill_run",
            "fi_prefill_plan_destroy", "fi_decode_run_rope", "fi_decode_run_rope_scaled",
            "fi_decode_run_noalloc", "fi_prefill_run_scaled", "fi_plan_create_composed",
            "fi_decode_run_composed", "fi_prefill_run_rope", "fi_mla_plan_create", "fi_mla_run"]
NOALLOC_SCRATCH_BYTES = 64 << 20
QITEM_STRIDE = 16
QMERGE_STRIDE = 8
PREFILL_ROWS = 256
PREFILL_MAX_PAGES = 512
MLA_MAX_PAGES = 256
MLA_ROWS = 32
MLA_DC = 512
MLA_DR = 64


class FiError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class PlanOpts(ctypes.Structure):
    _fields_ = [("num_cus", ctypes.c_int32), ("items_per_cu", ctypes.c_int32),
                ("min_chunk_tokens", ctypes.c_int32), ("max_chunk_tokens", ctypes.c_int32),
                ("fixed_chunk_tokens", ctypes.c_int32), ("cascade", ctypes.c_int32),
                ("decode_kernel", ctypes.c_int32), ("rope", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("num_items", ctypes.c_int64), ("num_partial_slots", ctypes.c_int64),
                ("num_merge_nodes", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("total_kv_tokens", ctypes.c_int64), ("chunk_pages", ctypes.c_int32),
                ("max_chunks_per_request", ctypes.c_int32),
                ("min_chunks_split_request", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("num_qo_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("shared_pages", ctypes.c_int64), ("num_prefix_items", ctypes.c_int64),
                ("num_prefix_groups", ctypes.c_int32), ("prefix_rows_per_item", ctypes.c_int32),
                ("image_bytes", ctypes.c_int64), ("decode_kernel", ctypes.c_int32),
                ("merge_fan_in", ctypes.c_int32), ("prefix_page_size", ctypes.c_int32)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class PrefillOpts(ctypes.Structure):
    _fields_ = [("num_cus", ctypes.c_int32), ("items_per_cu", ctypes.c_int32),
                ("fixed_chunk_tokens", ctypes.c_int32), ("num_xcds", ctypes.c_int32),
                ("rope", ctypes.c_int32)]


class PrefillInfo(ctypes.Structure):
    _fields_ = [("num_items", ctypes.c_int64), ("num_tiles", ctypes.c_int64),
                ("num_merges", ctypes.c_int64), ("num_partial_slots", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64), ("total_qo_tokens", ctypes.c_int64),
                ("total_kv_tokens", ctypes.c_int64), ("visible_pairs", ctypes.c_int64),
                ("tokens_per_tile", ctypes.c_int32), ("chunk_tokens", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("num_qo_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("rope", ctypes.c_int32), ("mla", ctypes.c_int32),
                ("head_dim_kpe", ctypes.c_int32)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                           "`python -m block_sparse_kv_bsr_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    pi32 = ctypes.POINTER(ctypes.c_int32)
    L.fi_plan_create.argtypes = [pi32, pi32, pi32, i32, i32, i32, i32, i32, i64, i32,
                                 ctypes.POINTER(PlanOpts), ctypes.POINTER(vp)]
    L.fi_plan_create.restype = i32
    L.fi_plan_create_composed.argtypes = [pi32, pi32, pi32, i32, pi32, pi32, pi32, i32, pi32, i32,
                                          i32, i32, i32, i64, i32, i64, i32,
                                          ctypes.POINTER(PlanOpts), ctypes.POINTER(vp)]
    L.fi_plan_create_composed.restype = i32
    L.fi_plan_get_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    L.fi_plan_get_info.restype = i32
    L.fi_plan_work_list.argtypes = [vp, ctypes.POINTER(pi32), ctypes.POINTER(i64)]
    L.fi_plan_work_list.restype = i32
    for name in ("fi_plan_merge_nodes", "fi_plan_prefix_items", "fi_plan_prefix_members"):
        getattr(L, name).argtypes = [vp, ctypes.POINTER(pi32), ctypes.POINTER(i64)]
        getattr(L, name).restype = i32
    L.fi_plan_upload.argtypes = [vp, vp, sz, vp]
    L.fi_plan_upload.restype = i32
    L.fi_decode_run.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, sz, vp]
    L.fi_decode_run.restype = i32
    f32 = ctypes.c_float
    L.fi_decode_run_scaled.argtypes = [vp, vp, vp, vp, f32, f32, vp, vp, f32, vp, sz, vp]
    L.fi_decode_run_scaled.restype = i32
    L.fi_decode_run_composed.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, sz, vp]
    L.fi_decode_run_composed.restype = i32
    L.fi_decode_run_rope.argtypes = [vp, vp, vp, vp, f32, f32, vp, vp, f32, vp, sz, vp]
    L.fi_decode_run_rope.restype = i32
    L.fi_decode_run_rope_scaled.argtypes = [vp, vp, vp, vp, f32, f32, f32, f32, vp, vp, f32, vp,
                                            sz, vp]
    L.fi_decode_run_rope_scaled.restype = i32
    L.fi_decode_run_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, f32, vp, sz, vp]
    L.fi_decode_run_noalloc.restype = i32
    L.fi_merge_states.argtypes = [i32, vp, vp, vp, vp, vp, vp, i64, i32, vp]
    L.fi_merge_states.restype = i32
    L.fi_plan_destroy.argtypes = [vp]
    L.fi_plan_destroy.restype = None
    L.fi_prefill_plan_create.argtypes = [pi32, pi32, pi32, pi32, i32, i32, i32, i32, i32, i64,
                                         i32, i32, ctypes.POINTER(PrefillOpts),
                                         ctypes.POINTER(vp)]
    L.fi_prefill_plan_create.restype = i32
    L.fi_prefill_plan_get_info.argtypes = [vp, ctypes.POINTER(PrefillInfo)]
    L.fi_prefill_plan_get_info.restype = i32
    for name in ("fi_prefill_plan_work_list", "fi_prefill_plan_merges"):
        getattr(L, name).argtypes = [vp, ctypes.POINTER(pi32), ctypes.POINTER(i64)]
        getattr(L, name).restype = i32
    L.fi_prefill_plan_upload.argtypes = [vp, vp, sz, vp]
    L.fi_prefill_plan_upload.restype = i32
    L.fi_prefill_run.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, sz, vp]
    L.fi_prefill_run.restype = i32
    L.fi_prefill_run_scaled.argtypes = [vp, vp, vp, vp, f32, f32, vp, vp, f32, vp, sz, vp]
    L.fi_prefill_run_scaled.restype = i32
    L.fi_prefill_run_rope.argtypes = [vp, vp, vp, vp, f32, f32, vp, vp, f32, vp, sz, vp]
    L.fi_prefill_run_rope.restype = i32
    L.fi_prefill_plan_destroy.argtypes = [vp]
    L.fi_prefill_plan_destroy.restype = None
    L.fi_mla_plan_create.argtypes = [pi32, pi32, pi32, pi32, i32, i32, i32, i32, i32, i64, i32,
                                     ctypes.POINTER(PrefillOpts), ctypes.POINTER(vp)]
    L.fi_mla_plan_create.restype = i32
    L.fi_mla_run.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, vp, sz, vp]
    L.fi_mla_run.restype = i32
    L.fi_last_error.argtypes = []
    L.fi_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int):
    if status != FI_OK:
        raise FiError(status, lib().fi_last_error().decode())


def _i32(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr32(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _dtype_code(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    name = str(dtype)
    if name in ("bf16", "torch.bfloat16", "bfloat16"):
        return FI_DTYPE_BF16
    if name in ("f32", "torch.float32", "float32"):
        return FI_DTYPE_F32
    if name in ("fp8", "fp8_e4m3", "torch.float8_e4m3fn", "float8_e4m3fn"):
        return FI_DTYPE_FP8_E4M3
    raise ValueError(f"unsupported dtype {dtype}")


class Plan:
    """A split-KV work plan (host memory, owned by the library)."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)
        info = PlanInfo()
        _check(lib().fi_plan_get_info(self._h, ctypes.byref(info)))
        self.info = info.as_dict()
        self._workspace = None

    @property
    def handle(self):
        return self._h

    def work_list(self) -> np.ndarray:
        p = ctypes.POINTER(ctypes.c_int32)()
        n = ctypes.c_int64()
        _check(lib().fi_plan_work_list(self._h, ctypes.byref(p), ctypes.byref(n)))
        if n.value == 0:
            return np.zeros((0, ITEM_STRIDE), dtype=np.int32)
        return np.ctypeslib.as_array(p, shape=(n.value * ITEM_STRIDE,)).reshape(-1, ITEM_STRIDE).copy()

    def _view(self, fn, stride) -> np.ndarray:
        p = ctypes.POINTER(ctypes.c_int32)()
        n = ctypes.c_int64()
        _check(fn(self._h, ctypes.byref(p), ctypes.byref(n)))
        if n.value == 0:
            return np.zeros((0, stride), dtype=np.int32)
        return np.ctypeslib.as_array(p, shape=(n.value * stride,)).reshape(-1, stride).copy()

    def merge_nodes(self) -> np.ndarray:
        return self._view(lib().fi_plan_merge_nodes, NODE_STRIDE)

    def prefix_items(self) -> np.ndarray:
        return self._view(lib().fi_plan_prefix_items, PITEM_STRIDE)

    def prefix_members(self) -> np.ndarray:
        return self._view(lib().fi_plan_prefix_members, 1).reshape(-1)

    def upload(self, workspace, stream=None):
        """Copy the plan into ``workspace`` (a torch uint8 CUDA tensor)."""
        _require_gpu(workspace, "workspace")
        _check(lib().fi_plan_upload(self._h, ctypes.c_void_p(workspace.data_ptr()),
                                    workspace.numel() * workspace.element_size(),
                                    ctypes.c_void_p(_stream(stream))))
        self._workspace = workspace

    def ensure_uploaded(self, device, stream=None):
        """Allocate a workspace on ``device`` and upload once."""
        import torch
        if self._workspace is None or self._workspace.device != torch.device(device):
            ws = torch.empty(max(256, self.info["workspace_bytes"]), dtype=torch.uint8, device=device)
            self.upload(ws, stream)
        return self._workspace

    @property
    def workspace(self):
        return self._workspace

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.fi_plan_destroy(h)
            self._h = None


def _check_lengths(ip: np.ndarray, ix: np.ndarray, lp: np.ndarray) -> int:
    """The C ABI cannot see array lengths and reads kv_indices up to
    kv_indptr[batch]: refuse arrays shorter than the page table says, before
    any pointer crosses. Returns the batch size."""
    if ip.ndim != 1 or len(ip) < 1:
        raise ValueError("kv_indptr must be a 1-d array of batch + 1 entries")
    batch = len(ip) - 1
    if lp.ndim != 1 or len(lp) != batch:
        raise ValueError("kv_last_page_len must have one entry per request")
    if ix.ndim != 1:
        raise ValueError("kv_indices must be a 1-d array")
    if int(ip.max()) > len(ix):
        raise ValueError(f"kv_indices holds {len(ix)} entries; kv_indptr refers to "
                         f"{int(ip.max())}")
    return batch


def plan(kv_indptr, kv_indices, kv_last_page_len, num_qo_heads: int, num_kv_heads: int,
         head_dim: int, page_size: int, num_pool_pages: int, dtype="bf16",
         num_cus: int = 0, items_per_cu: int = 0, min_chunk_tokens: int = 0,
         max_chunk_tokens: int = 0, fixed_chunk_tokens: int = 0, cascade: int = 0,
         decode_kernel: int = 0, rope: bool = False) -> Plan:
    """fi_plan_create over host page-table arrays (numpy or CPU tensors).
    decode_kernel: DECODE_KERNEL_AUTO (0), _VECTOR (1) or _MATRIX (2); rope:
    the plan's runs apply the rotary embedding (sizes the items only)."""
    ip, ix, lp = _i32(kv_indptr), _i32(kv_indices), _i32(kv_last_page_len)
    batch = _check_lengths(ip, ix, lp)
    opts = PlanOpts(num_cus, items_per_cu, min_chunk_tokens, max_chunk_tokens, fixed_chunk_tokens,
                    cascade, decode_kernel, int(bool(rope)))
    h = ctypes.c_void_p()
    ix_ptr = _ptr32(ix) if ix.size else ctypes.POINTER(ctypes.c_int32)()
    _check(lib().fi_plan_create(_ptr32(ip), ix_ptr, _ptr32(lp), batch, num_qo_heads,
                                num_kv_heads, head_dim, page_size, int(num_pool_pages),
                                _dtype_code(dtype), ctypes.byref(opts), ctypes.byref(h)))
    p = Plan(h.value)
    p.num_pool_pages = int(num_pool_pages)
    return p


def plan_composed(kv_indptr, kv_indices, kv_last_page_len, prefix_indptr, prefix_indices,
                  prefix_last_page_len, prefix_of, num_qo_heads: int, num_kv_heads: int,
                  head_dim: int, page_size: int, num_pool_pages: int, prefix_page_size: int,
                  num_prefix_pool_pages: int, dtype="bf16", num_cus: int = 0,
                  items_per_cu: int = 0, min_chunk_tokens: int = 0, max_chunk_tokens: int = 0,
                  fixed_chunk_tokens: int = 0, decode_kernel: int = 0) -> Plan:
    """fi_plan_create_composed: the requests' own pages (kv_*), the prefix
    cache's table (prefix_*) and prefix_of [batch] (-1: no prefix)."""
    ip, ix, lp = _i32(kv_indptr), _i32(kv_indices), _i32(kv_last_page_len)
    batch = _check_lengths(ip, ix, lp)
    pip, pix, plp = _i32(prefix_indptr), _i32(prefix_indices), _i32(prefix_last_page_len)
    num_prefixes = _check_lengths(pip, pix, plp)
    of = _i32(prefix_of)
    if of.ndim != 1 or len(of) != batch:
        raise ValueError("prefix_of must have one entry per request")
    opts = PlanOpts(num_cus, items_per_cu, min_chunk_tokens, max_chunk_tokens, fixed_chunk_tokens,
                    0, decode_kernel)
    h = ctypes.c_void_p()
    null = ctypes.POINTER(ctypes.c_int32)()
    _check(lib().fi_plan_create_composed(
        _ptr32(ip), _ptr32(ix) if ix.size else null, _ptr32(lp), batch, _ptr32(pip),
        _ptr32(pix) if pix.size else null, _ptr32(plp) if plp.size else null, num_prefixes,
        _ptr32(of) if of.size else null, num_qo_heads, num_kv_heads, head_dim, page_size,
        int(num_pool_pages), prefix_page_size, int(num_prefix_pool_pages), _dtype_code(dtype),
        ctypes.byref(opts), ctypes.byref(h)))
    p = Plan(h.value)
    p.num_pool_pages = int(num_pool_pages)
    p.num_prefix_pool_pages = int(num_prefix_pool_pages)
    return p


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _require_gpu(t, name):
    if not getattr(t, "is_cuda", False):
        raise RuntimeError(f"{name} must be a GPU tensor; this library has no CPU path")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _require_like(t, name, shape, dtype, device):
    """A caller-supplied output: the kernels write every element of `shape`,
    so a smaller or differently typed buffer is refused here, before the
    pointer crosses the C ABI (which cannot see sizes)."""
    _require_gpu(t, name)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, q on {device}")


def _require_pool(k_pages, v_pages, q, plan_):
    """K/V pools on q's device holding at least the plan's pool pages (the
    planner checked every listed page id against that count)."""
    for t, n in ((k_pages, "k_pages"), (v_pages, "v_pages")):
        if t.device != q.device:
            raise ValueError(f"{n} is on {t.device}, q on {q.device}")
        if t.shape[0] < plan_.num_pool_pages:
            raise ValueError(f"{n} holds {t.shape[0]} pages; the plan was made for "
                             f"{plan_.num_pool_pages}")


def _decode_args(q, k_pages, v_pages, plan_: Plan, out, lse, workspace, stream):
    import torch
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages")):
        _require_gpu(t, n)
    info = plan_.info
    B, Hq, d = info["batch"], info["num_qo_heads"], info["head_dim"]
    want = torch.float32 if info["dtype"] == FI_DTYPE_F32 else torch.bfloat16
    want_kv = {FI_DTYPE_F32: (torch.float32,), FI_DTYPE_BF16: (torch.bfloat16,),
               FI_DTYPE_FP8_E4M3: (torch.float8_e4m3fn, torch.uint8)}[info["dtype"]]
    if q.dtype != want or k_pages.dtype not in want_kv or v_pages.dtype not in want_kv:
        raise ValueError(f"q must be {want} and k_pages, v_pages one of {want_kv}")
    if tuple(q.shape) != (B, Hq, d):
        raise ValueError(f"q must have shape {(B, Hq, d)}, got {tuple(q.shape)}")
    kshape = (k_pages.shape[0], info["num_kv_heads"], info["page_size"], d)
    if tuple(k_pages.shape) != kshape or tuple(v_pages.shape) != kshape:
        raise ValueError(f"k_pages/v_pages must have shape [pool, {kshape[1]}, {kshape[2]}, {d}]")
    _require_pool(k_pages, v_pages, q, plan_)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=want, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _require_like(out, "out", (B, Hq, d), want, q.device)
    _require_like(lse, "lse", (B, Hq), torch.float32, q.device)
    if workspace is None:
        workspace = plan_.ensure_uploaded(q.device, stream)
    elif workspace.device != q.device:
        raise ValueError(f"workspace is on {workspace.device}, q on {q.device}")
    return out, lse, workspace


def decode(q, k_pages, v_pages, plan_: Plan, out=None, lse=None, sm_scale: Optional[float] = None,
           workspace=None, stream=None, k_scale: float = 1.0, v_scale: float = 1.0,
           rope_theta: Optional[float] = None, rope_scale: float = 1.0):
    """fi_decode_run_scaled: returns (out [B, H_q, d] in q's dtype, lse [B, H_q]
    float32). k_scale / v_scale dequantise an fp8 KV cache. With rope_theta
    set, K (and q) hold values before the rotary embedding and the kernel
    applies it (fi_decode_run_rope_scaled)."""
    out, lse, workspace = _decode_args(q, k_pages, v_pages, plan_, out, lse, workspace, stream)
    s = ctypes.c_void_p(_stream(stream))
    ws = ctypes.c_void_p(workspace.data_ptr())
    nbytes = workspace.numel() * workspace.element_size()
    o, l = ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr())
    scale = float(sm_scale) if sm_scale else 0.0
    if rope_theta:
        _check(lib().fi_decode_run_rope_scaled(plan_.handle, ctypes.c_void_p(q.data_ptr()),
                                               ctypes.c_void_p(k_pages.data_ptr()),
                                               ctypes.c_void_p(v_pages.data_ptr()), float(k_scale),
                                               float(v_scale), float(rope_theta),
                                               float(rope_scale), o, l, scale, ws, nbytes, s))
        return out, lse
    _check(lib().fi_decode_run_scaled(plan_.handle, ctypes.c_void_p(q.data_ptr()),
                                      ctypes.c_void_p(k_pages.data_ptr()),
                                      ctypes.c_void_p(v_pages.data_ptr()), float(k_scale),
                                      float(v_scale), o, l, scale, ws, nbytes, s))
    return out, lse


def decode_composed(q, k_pages, v_pages, k_prefix, v_prefix, plan_: Plan, out=None, lse=None,
                    sm_scale: Optional[float] = None, workspace=None, stream=None):
    """fi_decode_run_composed: the requests' own pages in k_pages / v_pages,
    the prefixes in k_prefix / v_prefix [prefix pool, H_kv, prefix_page_size,
    d]. Returns (out, lse)."""
    import torch
    info = plan_.info
    for t, n in ((k_prefix, "k_prefix"), (v_prefix, "v_prefix")):
        _require_gpu(t, n)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{n} must be bf16")
        want = (info["num_kv_heads"], info["prefix_page_size"], info["head_dim"])
        if tuple(t.shape[1:]) != want or t.shape[0] < plan_.num_prefix_pool_pages:
            raise ValueError(f"{n} must have shape [>= {plan_.num_prefix_pool_pages}, "
                             f"{want[0]}, {want[1]}, {want[2]}]")
        if t.device != q.device:
            raise ValueError(f"{n} is on {t.device}, q on {q.device}")
    out, lse, workspace = _decode_args(q, k_pages, v_pages, plan_, out, lse, workspace, stream)
    scale = float(sm_scale) if sm_scale else 0.0
    _check(lib().fi_decode_run_composed(
        plan_.handle, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_pages.data_ptr()),
        ctypes.c_void_p(v_pages.data_ptr()), ctypes.c_void_p(k_prefix.data_ptr()),
        ctypes.c_void_p(v_prefix.data_ptr()), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(lse.data_ptr()), scale, ctypes.c_void_p(workspace.data_ptr()),
        workspace.numel() * workspace.element_size(), ctypes.c_void_p(_stream(stream))))
    return out, lse


def decode_noalloc(q, k_pages, v_pages, plan_: Plan, workspace, out=None, lse=None,
                   sm_scale: Optional[float] = None, stream=None):
    """fi_decode_run_noalloc: the run's partial states and merge counters in
    the library's static device scratch; ``workspace`` is the buffer the plan
    was uploaded to (at least info["image_bytes"]). Returns (out, lse)."""
    if workspace is None:
        raise ValueError("decode_noalloc needs the workspace the plan was uploaded to")
    out, lse, workspace = _decode_args(q, k_pages, v_pages, plan_, out, lse, workspace, stream)
    _check(lib().fi_decode_run_noalloc(plan_.handle, ctypes.c_void_p(q.data_ptr()),
                                       ctypes.c_void_p(k_pages.data_ptr()),
                                       ctypes.c_void_p(v_pages.data_ptr()),
                                       ctypes.c_void_p(out.data_ptr()),
                                       ctypes.c_void_p(lse.data_ptr()),
                                       float(sm_scale) if sm_scale else 0.0,
                                       ctypes.c_void_p(workspace.data_ptr()),
                                       workspace.numel() * workspace.element_size(),
                                       ctypes.c_void_p(_stream(stream))))
    return out, lse


def merge_states(v_a, s_a, v_b, s_b, v_out=None, s_out=None, stream=None):
    """fi_merge_states over [rows, head_dim] states with float32 natural-log LSE."""
    import torch
    for t, n in ((v_a, "v_a"), (s_a, "s_a"), (v_b, "v_b"), (s_b, "s_b")):
        _require_gpu(t, n)
    if v_a.shape != v_b.shape or v_a.dim() != 2 or v_a.dtype != v_b.dtype:
        raise ValueError("v_a and v_b must both be [rows, head_dim] of one dtype")
    rows, d = v_a.shape
    if s_a.shape != (rows,) or s_b.shape != (rows,) or s_a.dtype != torch.float32 or s_b.dtype != torch.float32:
        raise ValueError("s_a and s_b must be float32 [rows]")
    for t, n in ((s_a, "s_a"), (v_b, "v_b"), (s_b, "s_b")):
        if t.device != v_a.device:
            raise ValueError(f"{n} is on {t.device}, v_a on {v_a.device}")
    if v_out is None:
        v_out = torch.empty_like(v_a)
    if s_out is None:
        s_out = torch.empty_like(s_a)
    _require_like(v_out, "v_out", (rows, d), v_a.dtype, v_a.device)
    _require_like(s_out, "s_out", (rows,), torch.float32, v_a.device)
    _check(lib().fi_merge_states(_dtype_code(v_a.dtype), ctypes.c_void_p(v_a.data_ptr()),
                                 ctypes.c_void_p(s_a.data_ptr()), ctypes.c_void_p(v_b.data_ptr()),
                                 ctypes.c_void_p(s_b.data_ptr()), ctypes.c_void_p(v_out.data_ptr()),
                                 ctypes.c_void_p(s_out.data_ptr()), rows, d,
                                 ctypes.c_void_p(_stream(stream))))
    return v_out, s_out


# ------------------------------------------------------------------ prefill
class PrefillPlan:
    """A prefill / append work list (host memory, owned by the library)."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)
        info = PrefillInfo()
        _check(lib().fi_prefill_plan_get_info(self._h, ctypes.byref(info)))
        self.info = info.as_dict()
        self._workspace = None

    @property
    def handle(self):
        return self._h

    def _view(self, fn, stride) -> np.ndarray:
        p = ctypes.POINTER(ctypes.c_int32)()
        n = ctypes.c_int64()
        _check(fn(self._h, ctypes.byref(p), ctypes.byref(n)))
        if n.value == 0:
            return np.zeros((0, stride), dtype=np.int32)
        return np.ctypeslib.as_array(p, shape=(n.value * stride,)).reshape(-1, stride).copy()

    def work_list(self) -> np.ndarray:
        return self._view(lib().fi_prefill_plan_work_list, QITEM_STRIDE)

    def merges(self) -> np.ndarray:
        return self._view(lib().fi_prefill_plan_merges, QMERGE_STRIDE)

    def upload(self, workspace, stream=None):
        _require_gpu(workspace, "workspace")
        _check(lib().fi_prefill_plan_upload(self._h, ctypes.c_void_p(workspace.data_ptr()),
                                            workspace.numel() * workspace.element_size(),
                                            ctypes.c_void_p(_stream(stream))))
        self._workspace = workspace

    def ensure_uploaded(self, device, stream=None):
        import torch
        if self._workspace is None or self._workspace.device != torch.device(device):
            ws = torch.empty(max(256, self.info["workspace_bytes"]), dtype=torch.uint8, device=device)
            self.upload(ws, stream)
        return self._workspace

    @property
    def workspace(self):
        return self._workspace

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.fi_prefill_plan_destroy(h)
            self._h = None


def prefill_plan(qo_indptr, kv_indptr, kv_indices, kv_last_page_len, num_qo_heads: int,
                 num_kv_heads: int, head_dim: int, page_size: int, num_pool_pages: int,
                 causal: bool = True, dtype="bf16", num_cus: int = 0, items_per_cu: int = 0,
                 fixed_chunk_tokens: int = 0, num_xcds: int = 0, rope: bool = False) -> PrefillPlan:
    """fi_prefill_plan_create over host arrays (numpy or CPU tensors). With
    ``rope`` the plan is for runs over a K cache of keys before the rotary
    embedding (fi_prefill_run_rope)."""
    qp, ip, ix, lp = _i32(qo_indptr), _i32(kv_indptr), _i32(kv_indices), _i32(kv_last_page_len)
    batch = _check_lengths(ip, ix, lp)
    if qp.ndim != 1 or len(qp) != batch + 1:
        raise ValueError("qo_indptr, kv_indptr and kv_last_page_len disagree on the batch size")
    opts = PrefillOpts(num_cus, items_per_cu, fixed_chunk_tokens, num_xcds, int(bool(rope)))
    h = ctypes.c_void_p()
    ix_ptr = _ptr32(ix) if ix.size else ctypes.POINTER(ctypes.c_int32)()
    _check(lib().fi_prefill_plan_create(_ptr32(qp), _ptr32(ip), ix_ptr, _ptr32(lp), batch,
                                        num_qo_heads, num_kv_heads, head_dim, page_size,
                                        int(num_pool_pages), _dtype_code(dtype), int(bool(causal)),
                                        ctypes.byref(opts), ctypes.byref(h)))
    p = PrefillPlan(h.value)
    p.num_pool_pages = int(num_pool_pages)
    return p


def prefill(q, k_pages, v_pages, plan_: PrefillPlan, out=None, lse=None,
            sm_scale: Optional[float] = None, workspace=None, stream=None,
            k_scale: float = 1.0, v_scale: float = 1.0, rope_theta: Optional[float] = None,
            rope_scale: float = 1.0):
    """fi_prefill_run_scaled: returns (out [N, H_q, d] bf16, lse [N, H_q]
    float32). k_scale / v_scale dequantise an fp8 KV cache. A plan made with
    ``rope=True`` runs fi_prefill_run_rope (q and K before the embedding;
    rope_theta None or <= 0 selects 10000)."""
    import torch
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages")):
        _require_gpu(t, n)
    info = plan_.info
    N, Hq, d = info["total_qo_tokens"], info["num_qo_heads"], info["head_dim"]
    want_kv = {FI_DTYPE_BF16: (torch.bfloat16,),
               FI_DTYPE_FP8_E4M3: (torch.float8_e4m3fn, torch.uint8)}[info["dtype"]]
    if q.dtype != torch.bfloat16 or k_pages.dtype not in want_kv or v_pages.dtype not in want_kv:
        raise ValueError(f"prefill takes bf16 q and k_pages, v_pages one of {want_kv}")
    if tuple(q.shape) != (N, Hq, d):
        raise ValueError(f"q must have shape {(N, Hq, d)}, got {tuple(q.shape)}")
    kshape = (k_pages.shape[0], info["num_kv_heads"], info["page_size"], d)
    if tuple(k_pages.shape) != kshape or tuple(v_pages.shape) != kshape:
        raise ValueError(f"k_pages/v_pages must have shape [pool, {kshape[1]}, {kshape[2]}, {d}]")
    _require_pool(k_pages, v_pages, q, plan_)
    if out is None:
        out = torch.empty((N, Hq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((N, Hq), dtype=torch.float32, device=q.device)
    _require_like(out, "out", (N, Hq, d), torch.bfloat16, q.device)
    _require_like(lse, "lse", (N, Hq), torch.float32, q.device)
    if workspace is None:
        workspace = plan_.ensure_uploaded(q.device, stream)
    elif workspace.device != q.device:
        raise ValueError(f"workspace is on {workspace.device}, q on {q.device}")
    scale = float(sm_scale) if sm_scale else 0.0
    if info["rope"]:
        if k_scale != 1.0 or v_scale != 1.0:
            raise ValueError("a rope prefill plan runs over bf16 caches (no scales)")
        _check(lib().fi_prefill_run_rope(plan_.handle, ctypes.c_void_p(q.data_ptr()),
                                         ctypes.c_void_p(k_pages.data_ptr()),
                                         ctypes.c_void_p(v_pages.data_ptr()),
                                         float(rope_theta or 0.0), float(rope_scale),
                                         ctypes.c_void_p(out.data_ptr()),
                                         ctypes.c_void_p(lse.data_ptr()), scale,
                                         ctypes.c_void_p(workspace.data_ptr()),
                                         workspace.numel() * workspace.element_size(),
                                         ctypes.c_void_p(_stream(stream))))
        return out, lse
    if rope_theta:
        raise ValueError("rope_theta given for a plan made without rope=True")
    _check(lib().fi_prefill_run_scaled(plan_.handle, ctypes.c_void_p(q.data_ptr()),
                                       ctypes.c_void_p(k_pages.data_ptr()),
                                       ctypes.c_void_p(v_pages.data_ptr()), float(k_scale),
                                       float(v_scale), ctypes.c_void_p(out.data_ptr()),
                                       ctypes.c_void_p(lse.data_ptr()), scale,
                                       ctypes.c_void_p(workspace.data_ptr()),
                                       workspace.numel() * workspace.element_size(),
                                       ctypes.c_void_p(_stream(stream))))
    return out, lse


def mla_plan(qo_indptr, kv_indptr, kv_indices, kv_last_page_len, num_heads: int, page_size: int,
             num_pool_pages: int, causal: bool = True, num_cus: int = 0, items_per_cu: int = 0,
             fixed_chunk_tokens: int = 0, num_xcds: int = 0) -> PrefillPlan:
    """fi_mla_plan_create (latent width 512, rotary-key width 64) over host
    arrays; the plan is a PrefillPlan run by ``mla``."""
    qp, ip, ix, lp = _i32(qo_indptr), _i32(kv_indptr), _i32(kv_indices), _i32(kv_last_page_len)
    batch = _check_lengths(ip, ix, lp)
    if qp.ndim != 1 or len(qp) != batch + 1:
        raise ValueError("qo_indptr, kv_indptr and kv_last_page_len disagree on the batch size")
    opts = PrefillOpts(num_cus, items_per_cu, fixed_chunk_tokens, num_xcds, 0)
    h = ctypes.c_void_p()
    ix_ptr = _ptr32(ix) if ix.size else ctypes.POINTER(ctypes.c_int32)()
    _check(lib().fi_mla_plan_create(_ptr32(qp), _ptr32(ip), ix_ptr, _ptr32(lp), batch, num_heads,
                                    MLA_DC, MLA_DR, page_size, int(num_pool_pages),
                                    int(bool(causal)), ctypes.byref(opts), ctypes.byref(h)))
    p = PrefillPlan(h.value)
    p.num_pool_pages = int(num_pool_pages)
    return p


def mla(q_nope, q_pe, ckv_pages, kpe_pages, plan_: PrefillPlan, sm_scale: float, out=None,
        lse=None, workspace=None, stream=None):
    """fi_mla_run: returns (out [N, H, 512] bf16, lse [N, H] float32).
    q_nope [N, H, 512], q_pe [N, H, 64], ckv_pages [pool, P, 512], kpe_pages
    [pool, P, 64], all bf16; sm_scale is required (the model's)."""
    import torch
    for t, n in ((q_nope, "q_nope"), (q_pe, "q_pe"), (ckv_pages, "ckv_pages"),
                 (kpe_pages, "kpe_pages")):
        _require_gpu(t, n)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{n} must be bf16")
        if t.device != q_nope.device:
            raise ValueError(f"{n} is on {t.device}, q_nope on {q_nope.device}")
    info = plan_.info
    if not info["mla"]:
        raise ValueError("mla() runs plans made by mla_plan()")
    N, H, P = info["total_qo_tokens"], info["num_qo_heads"], info["page_size"]
    if tuple(q_nope.shape) != (N, H, MLA_DC) or tuple(q_pe.shape) != (N, H, MLA_DR):
        raise ValueError(f"q_nope / q_pe must have shapes {(N, H, MLA_DC)} / {(N, H, MLA_DR)}")
    for t, n, d in ((ckv_pages, "ckv_pages", MLA_DC), (kpe_pages, "kpe_pages", MLA_DR)):
        if t.dim() != 3 or tuple(t.shape[1:]) != (P, d):
            raise ValueError(f"{n} must have shape [pool, {P}, {d}]")
        if t.shape[0] < plan_.num_pool_pages:
            raise ValueError(f"{n} holds {t.shape[0]} pages; the plan was made for "
                             f"{plan_.num_pool_pages}")
    if out is None:
        out = torch.empty((N, H, MLA_DC), dtype=torch.bfloat16, device=q_nope.device)
    if lse is None:
        lse = torch.empty((N, H), dtype=torch.float32, device=q_nope.device)
    _require_like(out, "out", (N, H, MLA_DC), torch.bfloat16, q_nope.device)
    _require_like(lse, "lse", (N, H), torch.float32, q_nope.device)
    if workspace is None:
        workspace = plan_.ensure_uploaded(q_nope.device, stream)
    elif workspace.device != q_nope.device:
        raise ValueError(f"workspace is on {workspace.device}, q_nope on {q_nope.device}")
    _check(lib().fi_mla_run(plan_.handle, ctypes.c_void_p(q_nope.data_ptr()),
                            ctypes.c_void_p(q_pe.data_ptr()), ctypes.c_void_p(ckv_pages.data_ptr()),
                            ctypes.c_void_p(kpe_pages.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                            ctypes.c_void_p(lse.data_ptr()), float(sm_scale),
                            ctypes.c_void_p(workspace.data_ptr()),
                            workspace.numel() * workspace.element_size(),
                            ctypes.c_void_p(_stream(stream))))
    return out, lse
