"""Seeded synthetic inputs for paged / block-sparse-row (BSR) decode attention.

This module only builds inputs: page tables, lengths and random values. It
holds none of the attention arithmetic, so the oracle and the HIP path can both
be fed from it without sharing any of the method.

Layout of what is produced (the same for every consumer):

* ``kv_indptr``  int32 [B+1]  -- request b lists pages kv_indices[kv_indptr[b]:kv_indptr[b+1]]
* ``kv_indices`` int32 [nnz]  -- physical page ids, in logical (token) order
* ``last_page_len`` int32 [B] -- valid tokens in the last listed page (1..P; 0 if no page)
* ``q``  [B, H_q, d]
* ``k_pool``, ``v_pool`` [num_pool_pages, H_kv, P, d]   (page-major, head, token, dim)

The block-sparse view (FlashInfer paper explainer, "FlashInfer: Block-Sparse
KV 캐시로 어텐션 병목을 해소하다", section on the Block-Sparse format): the KV
cache is a block-sparse matrix whose blocks are runs of consecutive tokens; a
request lists only its active blocks. A page table is that matrix in BSR form
with block size = page size. Blocks that are not listed are inactive.

Structure (lengths, permutations, masks) comes from
``numpy.random.default_rng([config_id, 0])``; values come from a torch
generator seeded with ``1_000_003 * config_id + 1`` on the device the caller
asks for, drawn as q, then K, then V, each N(0, 1) in float32 and then cast to
the config dtype (torch's cast, round-to-nearest-even). Every pool page that no
request lists and every slot past ``last_page_len`` in a last page is set to
NaN, so a kernel that touches them poisons its output.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

# Five workloads. Sizes follow the decode-attention study cases: a tiny fp32
# case, a uniform Llama-3-8B-shaped batch (32 query heads, 8 KV heads,
# head_dim 128), a skewed batch, a long-context batch, and a block-sparse
# batch with a shared prefix.
CONFIG_NAMES = {
    1: "tiny_paged_f32",
    2: "uniform_b64_l2048",
    3: "skewed_b64_loguniform_32_32768",
    4: "long_b2_l131072_65536",
    5: "sparse_prefix_b32_p64",
    6: "skewed_b64_loguniform_32_32768_fp8kv",
    # prefill / append (several query tokens per request, causal)
    7: "prefill_b16_l2048_causal",
    8: "append_b64_q128_skewed",
    # the skewed batch over a K cache that holds keys before the rotary embedding
    9: "skewed_b64_loguniform_32_32768_rope",
    # the same over an fp8 KV cache
    10: "skewed_b64_loguniform_32_32768_fp8kv_rope",
    # the skewed batch at 64 query heads per 8 KV heads (group 8)
    11: "skewed_b64_loguniform_32_32768_g8",
    # the append batch over an fp8 KV cache
    12: "append_b64_q128_skewed_fp8kv",
    # config 5 with the shared prefix held once in a second cache of
    # 4096-token blocks (composed formats)
    13: "sparse_prefix_b32_p64_composed_b4096",
    # the append batch over a K cache that holds keys before the rotary embedding
    14: "append_b64_q128_skewed_rope",
    # multi-head latent attention decode: the skewed batch's histories as a
    # paged latent cache (512 + 64 per token, 64-token pages), 96 heads
    15: "mla_skewed_b64_loguniform_32_32768_h96",
}

# Rotary embedding base of the rope workload (the Llama-3 value).
ROPE_THETA = 500000.0

# fp8 KV caches hold x / FP8_SCALE rounded to OCP E4M3 (torch's cast, round
# to nearest even; |x / scale| <= 448 for |x| <= 7); the kernel multiplies by
# the scale again.
FP8_SCALE = 1.0 / 64.0


@dataclasses.dataclass
class Workload:
    name: str
    config_id: int
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str  # "f32", "bf16" or "fp8" (K/V fp8 e4m3 with q/out bf16)
    num_pool_pages: int
    kv_indptr: np.ndarray
    kv_indices: np.ndarray
    last_page_len: np.ndarray
    # pool pages no request lists (filled with NaN)
    unused_pages: np.ndarray
    value_seed: int
    # physical pages listed by more than one request (config 5 prefix)
    shared_pages: int = 0
    # dequantisation scales of an fp8 KV cache (1 otherwise)
    k_scale: float = 1.0
    v_scale: float = 1.0
    # rotary embedding applied in the kernel (0: K is stored as used)
    rope_theta: float = 0.0
    rope_scale: float = 1.0

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def group_size(self) -> int:
        return self.num_qo_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        """Bytes per q / out element."""
        return 4 if self.dtype == "f32" else 2

    @property
    def kv_elem_bytes(self) -> int:
        """Bytes per K / V element in the cache."""
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.dtype]

    def num_pages(self, b: int) -> int:
        return int(self.kv_indptr[b + 1] - self.kv_indptr[b])

    def kv_len(self, b: int) -> int:
        n = self.num_pages(b)
        if n == 0:
            return 0
        return (n - 1) * self.page_size + int(self.last_page_len[b])

    def kv_lens(self) -> np.ndarray:
        return np.array([self.kv_len(b) for b in range(self.batch)], dtype=np.int64)

    def algorithmic_bytes(self, unique: bool = True) -> int:
        """Bytes the method must move: each active K and V row once per KV
        head, plus reading q and writing the output. With ``unique`` a
        physical page listed by several requests counts once (shared prefix)."""
        if unique:
            tok = self._unique_tokens()
        else:
            tok = int(self.kv_lens().sum())
        kv = 2 * self.num_kv_heads * self.head_dim * tok * self.kv_elem_bytes
        qo = 2 * self.batch * self.num_qo_heads * self.head_dim * self.elem_bytes
        return kv + qo

    def _unique_tokens(self) -> int:
        # token slots per physical page that some request reads
        used = {}
        P = self.page_size
        for b in range(self.batch):
            s, t = int(self.kv_indptr[b]), int(self.kv_indptr[b + 1])
            for j in range(s, t):
                n = P if j < t - 1 else int(self.last_page_len[b])
                pg = int(self.kv_indices[j])
                used[pg] = max(used.get(pg, 0), n)
        return int(sum(used.values()))

    # ------------------------------------------------------------------ values
    def make_values(self, device="cpu"):
        """Return (q, k_pool, v_pool) as torch tensors on ``device``. For an
        fp8 cache the pools are float8_e4m3fn holding x / k_scale (resp.
        v_scale) of the same float32 draws."""
        import torch

        tdt = torch.float32 if self.dtype == "f32" else torch.bfloat16
        g = torch.Generator(device=device)
        g.manual_seed(self.value_seed)
        B, Hq, Hkv, d, P = (self.batch, self.num_qo_heads, self.num_kv_heads,
                            self.head_dim, self.page_size)
        N = self.num_pool_pages

        def draw(shape):
            x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
            return x.to(tdt)

        q = draw((B, Hq, d))
        if self.dtype == "fp8":
            def draw_fp8(shape, scale):
                x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
                self._poison(x, device)  # NaN stays NaN through the cast
                return (x / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
            return q, draw_fp8((N, Hkv, P, d), self.k_scale), draw_fp8((N, Hkv, P, d), self.v_scale)
        k = draw((N, Hkv, P, d))
        v = draw((N, Hkv, P, d))
        self._poison(k, device)
        self._poison(v, device)
        return q, k, v

    def _poison(self, pool, device):
        import torch

        nan = float("nan")
        if len(self.unused_pages):
            idx = torch.as_tensor(self.unused_pages.astype(np.int64), device=device)
            pool.index_fill_(0, idx, nan)
        P = self.page_size
        for b in range(self.batch):
            n = self.num_pages(b)
            if n == 0:
                continue
            ell = int(self.last_page_len[b])
            if ell < P:
                last = int(self.kv_indices[self.kv_indptr[b + 1] - 1])
                pool[last, :, ell:, :] = nan


# ---------------------------------------------------------------- structure
def _pack(page_lists: List[List[int]], lens: List[int], page_size: int):
    indptr = np.zeros(len(page_lists) + 1, dtype=np.int32)
    for b, pl in enumerate(page_lists):
        indptr[b + 1] = indptr[b] + len(pl)
    indices = (np.concatenate([np.asarray(p, dtype=np.int32) for p in page_lists])
               if indptr[-1] > 0 else np.zeros(0, dtype=np.int32))
    last = np.zeros(len(page_lists), dtype=np.int32)
    for b, L in enumerate(lens):
        if len(page_lists[b]):
            last[b] = L - page_size * (len(page_lists[b]) - 1)
    return indptr, indices, last


def paged_structure(lens, page_size, pool_pages, rng):
    """Dense-in-logical-order paging: request b holds ceil(L_b/P) pages, taken
    in order from one seeded permutation of the pool."""
    npg = [(int(L) + page_size - 1) // page_size for L in lens]
    total = sum(npg)
    assert pool_pages >= total
    perm = rng.permutation(pool_pages).astype(np.int32)
    lists, off = [], 0
    for n in npg:
        lists.append(list(perm[off:off + n]))
        off += n
    indptr, indices, last = _pack(lists, [int(L) for L in lens], page_size)
    unused = np.sort(perm[total:]).astype(np.int32)
    return indptr, indices, last, unused


@dataclasses.dataclass
class PrefillWorkload(Workload):
    """Several query tokens per request: request b's n_b query tokens are
    rows qo_indptr[b] .. qo_indptr[b+1]-1 of q [N, H_q, d]; they are the
    request's newest cached tokens (n_b <= L_b when causal)."""
    qo_indptr: np.ndarray = None
    causal: bool = True

    @property
    def num_qo_tokens(self) -> int:
        return int(self.qo_indptr[-1])

    def qo_lens(self) -> np.ndarray:
        return np.diff(self.qo_indptr).astype(np.int64)

    def visible_pairs(self) -> int:
        """Sum over query tokens of the KV tokens each attends."""
        tot = 0
        for L, n in zip(self.kv_lens(), self.qo_lens()):
            L, n = int(L), int(n)
            if self.causal:
                # query i sees max(0, L - n + i + 1) tokens
                lo = max(0, n - L)
                tot += sum(L - n + i + 1 for i in range(lo, n))
            else:
                tot += L * n
        return tot

    def flops(self) -> int:
        """QK^T and PV: 2 * d multiply-adds each per (query head, visible token)."""
        return 4 * self.head_dim * self.num_qo_heads * self.visible_pairs()

    def algorithmic_bytes(self, unique: bool = True) -> int:
        tok = self._unique_tokens() if unique else int(self.kv_lens().sum())
        kv = 2 * self.num_kv_heads * self.head_dim * tok * self.kv_elem_bytes
        qo = 2 * self.num_qo_tokens * self.num_qo_heads * self.head_dim * self.elem_bytes
        return kv + qo

    def make_values(self, device="cpu"):
        """(q [N, H_q, d], k_pool, v_pool) drawn like the decode workloads:
        q, then K, then V, N(0, 1) float32 cast to bf16; an fp8 cache holds
        x / k_scale (resp. v_scale) of the same draws as float8_e4m3fn."""
        import torch

        if self.dtype not in ("bf16", "fp8"):
            raise ValueError("prefill workloads are bf16 or fp8 (K/V)")
        g = torch.Generator(device=device)
        g.manual_seed(self.value_seed)
        Hq, Hkv, d, P = self.num_qo_heads, self.num_kv_heads, self.head_dim, self.page_size
        N = self.num_pool_pages

        def draw(shape, scale=None):
            x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
            if scale is None:
                return x.to(torch.bfloat16)
            self._poison(x, device)  # NaN stays NaN through the cast
            return (x / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)

        q = draw((self.num_qo_tokens, Hq, d))
        if self.dtype == "fp8":
            return q, draw((N, Hkv, P, d), self.k_scale), draw((N, Hkv, P, d), self.v_scale)
        k = draw((N, Hkv, P, d))
        v = draw((N, Hkv, P, d))
        self._poison(k, device)
        self._poison(v, device)
        return q, k, v


def _qo_indptr(qo_lens) -> np.ndarray:
    ip = np.zeros(len(qo_lens) + 1, dtype=np.int32)
    ip[1:] = np.cumsum(np.asarray(qo_lens, dtype=np.int64))
    return ip


def prefill_workload(config_id: int) -> PrefillWorkload:
    """7: 16 prompts of 2048 tokens each, all of them queries (pure causal
    prefill), page size 16, pool with 20% spare pages. 8: the skewed batch's
    64 histories (log-uniform lengths in [32, 32768]) with their newest
    min(128, L_b) tokens as queries (a chunk appended to each request).
    32 query / 8 KV heads, head_dim 128, bf16. 12: config 8 over an fp8
    (E4M3) KV cache with scales 1/64. 14: config 8 with q and K before the
    rotary embedding (theta 5e5)."""
    rng = np.random.default_rng([config_id, 0])
    seed = 1_000_003 * config_id + 1
    if config_id == 7:
        lens = [2048] * 16
        ip, ix, lp, un = paged_structure(lens, 16, 2560, rng)
        return PrefillWorkload(CONFIG_NAMES[7], 7, 16, 32, 8, 128, 16, "bf16", 2560, ip, ix, lp,
                               un, seed, qo_indptr=_qo_indptr(lens), causal=True)
    if config_id == 8:
        base = workload(3)
        qo = [min(128, int(L)) for L in base.kv_lens()]
        return PrefillWorkload(CONFIG_NAMES[8], 8, base.batch, 32, 8, 128, 16, "bf16",
                               base.num_pool_pages, base.kv_indptr, base.kv_indices,
                               base.last_page_len, base.unused_pages, seed,
                               qo_indptr=_qo_indptr(qo), causal=True)
    if config_id == 12:
        return dataclasses.replace(prefill_workload(8), name=CONFIG_NAMES[12], config_id=12,
                                   dtype="fp8", value_seed=seed, k_scale=FP8_SCALE,
                                   v_scale=FP8_SCALE)
    if config_id == 14:
        return dataclasses.replace(prefill_workload(8), name=CONFIG_NAMES[14], config_id=14,
                                   value_seed=seed, rope_theta=ROPE_THETA)
    raise ValueError(f"unknown prefill config {config_id}")


def random_prefill_workload(seed: int, batch: int, max_len: int, num_qo_heads: int,
                            num_kv_heads: int, head_dim: int, page_size: int,
                            causal: bool = True, max_qo: Optional[int] = None,
                            lens: Optional[List[int]] = None,
                            qo_lens: Optional[List[int]] = None,
                            spare_pages: int = 3, dtype: str = "bf16",
                            rope_theta: float = 0.0, rope_scale: float = 1.0) -> PrefillWorkload:
    """Small ragged prefill case: KV lengths U{1..max_len} (or given), query
    counts U{1..min(L_b, max_qo)} (or given; 0 allowed), bf16 or an fp8 K/V
    cache (scales 1/64)."""
    rng = np.random.default_rng([seed, 13])
    if lens is None:
        lens = [int(x) for x in rng.integers(1, max_len + 1, size=batch)]
    if qo_lens is None:
        cap = max_qo if max_qo is not None else max_len
        qo_lens = [int(rng.integers(1, max(1, min(L, cap)) + 1)) if L > 0 else 0 for L in lens]
    npg = sum((L + page_size - 1) // page_size for L in lens)
    pool = npg + spare_pages
    ip, ix, lp, un = paged_structure(lens, page_size, pool, rng)
    scale = FP8_SCALE if dtype == "fp8" else 1.0
    return PrefillWorkload(f"prefill_{seed}", 0, len(lens), num_qo_heads, num_kv_heads, head_dim,
                           page_size, dtype, pool, ip, ix, lp, un, 30_000 + seed,
                           qo_indptr=_qo_indptr(qo_lens), causal=causal,
                           k_scale=scale, v_scale=scale, rope_theta=rope_theta,
                           rope_scale=rope_scale)


def workload(config_id: int) -> Workload:
    rng = np.random.default_rng([config_id, 0])
    seed = 1_000_003 * config_id + 1
    if config_id == 1:
        lens = [17, 64, 100, 250]
        ip, ix, lp, un = paged_structure(lens, 16, 40, rng)
        return Workload(CONFIG_NAMES[1], 1, 4, 4, 1, 64, 16, "f32", 40, ip, ix, lp, un, seed)
    if config_id == 2:
        lens = [2048] * 64
        ip, ix, lp, un = paged_structure(lens, 16, 10240, rng)
        return Workload(CONFIG_NAMES[2], 2, 64, 32, 8, 128, 16, "bf16", 10240, ip, ix, lp, un, seed)
    if config_id == 3:
        u = rng.uniform(math.log(32.0), math.log(32768.0), size=64)
        lens = np.clip(np.floor(np.exp(u)).astype(np.int64), 32, 32768)
        pool = int(sum((int(L) + 15) // 16 for L in lens))
        ip, ix, lp, un = paged_structure(lens, 16, pool, rng)
        return Workload(CONFIG_NAMES[3], 3, 64, 32, 8, 128, 16, "bf16", pool, ip, ix, lp, un, seed)
    if config_id == 4:
        lens = [131072, 65536]
        ip, ix, lp, un = paged_structure(lens, 64, 3072, rng)
        return Workload(CONFIG_NAMES[4], 4, 2, 32, 8, 128, 64, "bf16", 3072, ip, ix, lp, un, seed)
    if config_id == 5:
        return _sparse_prefix(rng, seed)
    if config_id == 13:
        return _composed_prefix(seed)
    if config_id in (7, 8, 12, 14):
        return prefill_workload(config_id)
    if config_id == 15:
        return mla_workload(config_id)
    if config_id == 9:  # the skewed batch, K stored before the rotary embedding
        w = workload(3)
        return dataclasses.replace(w, name=CONFIG_NAMES[9], config_id=9, value_seed=seed,
                                   rope_theta=ROPE_THETA)
    if config_id == 11:  # the skewed batch with 64 query heads over 8 KV heads
        w = workload(3)
        return dataclasses.replace(w, name=CONFIG_NAMES[11], config_id=11, num_qo_heads=64,
                                   value_seed=seed)
    if config_id == 10:  # the skewed batch over an fp8 cache of keys before the embedding
        w = workload(6)
        return dataclasses.replace(w, name=CONFIG_NAMES[10], config_id=10,
                                   value_seed=seed, rope_theta=ROPE_THETA)
    if config_id == 6:  # the skewed batch over an fp8 KV cache
        w = workload(3)
        return dataclasses.replace(w, name=CONFIG_NAMES[6], config_id=6, dtype="fp8",
                                   value_seed=seed, k_scale=FP8_SCALE, v_scale=FP8_SCALE)
    raise ValueError(f"unknown config {config_id}")


def _sparse_prefix(rng, seed) -> Workload:
    """32 requests share the same 128 physical prefix pages (8192 tokens at
    P = 64); each has a unique suffix of s_b ~ U{128..1024} tokens cut into
    n_b = ceil(s_b/64) blocks, of which k_b = max(1, floor(n_b/4 + 1/2)) stay
    active: always the newest block (it holds the token being decoded) plus
    k_b - 1 others drawn without replacement, kept in ascending order. The
    inactive suffix blocks stay in the pool (filled with NaN) but are not
    listed."""
    B, P, prefix_pages = 32, 64, 128
    s = rng.integers(128, 1025, size=B)
    nblk = [(int(x) + P - 1) // P for x in s]
    pool = prefix_pages + sum(nblk)
    perm = rng.permutation(pool).astype(np.int32)
    prefix = list(perm[:prefix_pages])
    lists, lens, off = [], [], prefix_pages
    listed = set(prefix)
    for b in range(B):
        n = nblk[b]
        k = max(1, int(math.floor(n / 4.0 + 0.5)))
        others = rng.choice(n - 1, size=k - 1, replace=False) if k > 1 else np.zeros(0, np.int64)
        keep = sorted(int(x) for x in others) + [n - 1]
        phys = [int(perm[off + j]) for j in keep]
        off += n
        listed.update(phys)
        ell = int(s[b]) - P * (n - 1)
        lists.append(prefix + phys)
        lens.append(P * (len(prefix) + len(phys) - 1) + ell)
    ip, ix, lp = _pack(lists, lens, P)
    unused = np.array(sorted(set(range(pool)) - listed), dtype=np.int32)
    return Workload(CONFIG_NAMES[5], 5, B, 32, 8, 128, P, "bf16", pool, ip, ix, lp, unused,
                    seed, shared_pages=prefix_pages)


def random_workload(seed: int, batch: int, max_len: int, num_qo_heads: int,
                    num_kv_heads: int, head_dim: int, page_size: int, dtype: str,
                    empty_every: int = 0, spare_pages: int = 3,
                    lens: Optional[List[int]] = None) -> Workload:
    """Small ragged case for tests: lengths U{1..max_len} (or given), every
    ``empty_every``-th request empty, a few spare pool pages left unused."""
    rng = np.random.default_rng([seed, 7])
    if lens is None:
        lens = [int(x) for x in rng.integers(1, max_len + 1, size=batch)]
        if empty_every:
            for b in range(0, batch, empty_every):
                lens[b] = 0
    npg = sum((L + page_size - 1) // page_size for L in lens)
    pool = npg + spare_pages
    ip, ix, lp, un = paged_structure(lens, page_size, pool, rng)
    scale = FP8_SCALE if dtype == "fp8" else 1.0
    return Workload(f"random_{seed}", 0, batch, num_qo_heads, num_kv_heads, head_dim,
                    page_size, dtype, pool, ip, ix, lp, un, 10_000 + seed,
                    k_scale=scale, v_scale=scale)


def prefix_workload(seed: int, groups: List[tuple], singles: int, suffix_max: int,
                    num_qo_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
                    dtype: str, extra_shared: bool = True) -> Workload:
    """Requests that share prefixes, for cascade tests. ``groups`` lists
    (members, prefix_pages): the members of a group all begin with the same
    prefix_pages physical pages, then a private suffix of U{1..suffix_max}
    tokens. With ``extra_shared`` the first two members of each group also
    share the page after the prefix (so the common run is longer for some
    members than for all). ``singles`` more requests share nothing. The batch
    order is a seeded shuffle, so group members are not adjacent."""
    rng = np.random.default_rng([seed, 11])
    P = page_size
    reqs = []  # (shared page ids, suffix tokens)
    next_page = 0
    for members, prefix_pages in groups:
        prefix = list(range(next_page, next_page + prefix_pages))
        next_page += prefix_pages
        extra = None
        if extra_shared and members >= 2:
            extra = next_page
            next_page += 1
        for m in range(members):
            shared = prefix + ([extra] if extra is not None and m < 2 else [])
            reqs.append((shared, int(rng.integers(1, suffix_max + 1))))
    for _ in range(singles):
        reqs.append(([], int(rng.integers(1, suffix_max + 1))))
    order = rng.permutation(len(reqs))
    reqs = [reqs[i] for i in order]
    lists, lens = [], []
    for shared, suf in reqs:
        n = (suf + P - 1) // P
        own = list(range(next_page, next_page + n))
        next_page += n
        lists.append(shared + own)
        lens.append(P * len(shared) + suf)
    pool = next_page + 3
    perm = rng.permutation(pool).astype(np.int32)  # scatter the ids over the pool
    lists = [[int(perm[x]) for x in pl] for pl in lists]
    ip, ix, lp = _pack(lists, lens, P)
    listed = set(int(x) for x in ix)
    unused = np.array(sorted(set(range(pool)) - listed), dtype=np.int32)
    shared_ids = sum(1 for v in np.unique(ix, return_counts=True)[1] if v > 1)
    return Workload(f"prefix_{seed}", 0, len(lists), num_qo_heads, num_kv_heads, head_dim, P,
                    dtype, pool, ip, ix, lp, unused, 20_000 + seed, shared_pages=shared_ids)


# ------------------------------------------------------ composed formats
@dataclasses.dataclass
class ComposedWorkload(Workload):
    """Requests whose KV is a shared prefix, held once in a second cache with
    its own block size, followed by the request's own tokens in the main
    paged cache. The prefix cache is [num_prefix_pool_pages, H_kv,
    prefix_page_size, d]; prefix g lists blocks prefix_indices[
    prefix_indptr[g] : prefix_indptr[g+1]] (all full but the last, which holds
    prefix_last_page_len[g] tokens); request b begins with prefix
    prefix_of[b] (-1: none). The inherited page table is the requests' own
    tokens."""
    prefix_page_size: int = 0
    num_prefix_pool_pages: int = 0
    prefix_indptr: np.ndarray = None
    prefix_indices: np.ndarray = None
    prefix_last_page_len: np.ndarray = None
    prefix_of: np.ndarray = None
    prefix_unused_pages: np.ndarray = None

    @property
    def num_prefixes(self) -> int:
        return len(self.prefix_indptr) - 1

    def prefix_len(self, g: int) -> int:
        n = int(self.prefix_indptr[g + 1] - self.prefix_indptr[g])
        return 0 if n == 0 else (n - 1) * self.prefix_page_size + int(self.prefix_last_page_len[g])

    def total_kv_lens(self) -> np.ndarray:
        """Tokens each request attends: its prefix and its own."""
        own = self.kv_lens()
        return np.array([own[b] + (self.prefix_len(int(self.prefix_of[b]))
                                   if self.prefix_of[b] >= 0 else 0)
                         for b in range(self.batch)], dtype=np.int64)

    def algorithmic_bytes(self, unique: bool = True) -> int:
        """K and V of every prefix once (``unique``) or once per member, and
        of every request's own tokens, per KV head; plus q and the output."""
        own = int(self.kv_lens().sum())
        if unique:
            used = sorted(set(int(g) for g in self.prefix_of if g >= 0))
            pre = sum(self.prefix_len(g) for g in used)
        else:
            pre = sum(self.prefix_len(int(g)) for g in self.prefix_of if g >= 0)
        kv = 2 * self.num_kv_heads * self.head_dim * (own + pre) * self.kv_elem_bytes
        qo = 2 * self.batch * self.num_qo_heads * self.head_dim * self.elem_bytes
        return kv + qo

    def make_values(self, device="cpu"):
        """(q, k_pool, v_pool, k_prefix, v_prefix): q and the main cache drawn
        as the decode workloads draw them, then the prefix cache's K and V,
        N(0, 1) cast to bf16; unlisted pages and the slots past each last
        page's length hold NaN."""
        import torch

        if self.dtype != "bf16":
            raise ValueError("composed workloads are bf16")
        q, k, v = super().make_values(device)
        g = torch.Generator(device=device)
        g.manual_seed(self.value_seed + 1)
        shape = (self.num_prefix_pool_pages, self.num_kv_heads, self.prefix_page_size,
                 self.head_dim)
        kp = torch.randn(shape, generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)
        vp = torch.randn(shape, generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)
        nan = float("nan")
        for pool in (kp, vp):
            if len(self.prefix_unused_pages):
                idx = torch.as_tensor(self.prefix_unused_pages.astype(np.int64), device=device)
                pool.index_fill_(0, idx, nan)
            for gi in range(self.num_prefixes):
                if self.prefix_indptr[gi + 1] == self.prefix_indptr[gi]:
                    continue
                ell = int(self.prefix_last_page_len[gi])
                if ell < self.prefix_page_size:
                    last = int(self.prefix_indices[self.prefix_indptr[gi + 1] - 1])
                    pool[last, :, ell:, :] = nan
        return q, k, v, kp, vp


def random_composed_workload(seed: int, prefix_lens: List[int], members: List[int],
                             singles: int, own_max: int, num_qo_heads: int, num_kv_heads: int,
                             head_dim: int, page_size: int, prefix_page_size: int,
                             spare_pages: int = 2) -> ComposedWorkload:
    """Small composed case: prefix g has prefix_lens[g] tokens (0 allowed) in
    blocks of prefix_page_size and members[g] requests (0 allowed); ``singles``
    requests have no prefix; every request has U{1..own_max} tokens of its own.
    Batch order, main-cache pages and prefix-cache blocks are seeded
    permutations."""
    rng = np.random.default_rng([seed, 17])
    of = [g for g, m in enumerate(members) for _ in range(m)] + [-1] * singles
    of = [of[i] for i in rng.permutation(len(of))]
    lens = [int(x) for x in rng.integers(1, own_max + 1, size=len(of))]
    npg = sum((L + page_size - 1) // page_size for L in lens)
    ip, ix, lp, un = paged_structure(lens, page_size, npg + spare_pages, rng)
    Pp = prefix_page_size
    nblk = [(L + Pp - 1) // Pp for L in prefix_lens]
    ppool = sum(nblk) + spare_pages
    pip, pix, plp, pun = paged_structure(prefix_lens, Pp, ppool, rng)
    return ComposedWorkload(f"composed_{seed}", 0, len(of), num_qo_heads, num_kv_heads, head_dim,
                            page_size, "bf16", npg + spare_pages, ip, ix, lp, un, 40_000 + seed,
                            prefix_page_size=Pp, num_prefix_pool_pages=ppool,
                            prefix_indptr=pip, prefix_indices=pix, prefix_last_page_len=plp,
                            prefix_of=np.asarray(of, dtype=np.int32), prefix_unused_pages=pun)


def _composed_prefix(seed) -> ComposedWorkload:
    """Config 5's 32 requests with their shared 8192-token prefix held once
    in a second cache as two 4096-token blocks (seeded block order in a
    4-block pool), and each request's own tokens -- the active 64-token
    blocks of its suffix, as config 5 draws them -- in the main paged cache
    (page size 64, the prefix pages removed from every list)."""
    w5 = workload(5)
    P, prefix_pages = w5.page_size, 128
    lists, lens = [], []
    for b in range(w5.batch):
        pages = [int(x) for x in w5.kv_indices[w5.kv_indptr[b]:w5.kv_indptr[b + 1]]]
        lists.append(pages[prefix_pages:])
        lens.append(w5.kv_len(b) - prefix_pages * P)
    # renumber the suffix pages into a pool of their own (the prefix pages
    # leave the main cache)
    used = sorted(set(x for pl in lists for x in pl))
    rng = np.random.default_rng([13, 1])
    spare = 8
    pool = len(used) + spare
    perm = rng.permutation(pool).astype(np.int32)
    remap = {old: int(perm[i]) for i, old in enumerate(used)}
    lists = [[remap[x] for x in pl] for pl in lists]
    ip, ix, lp = _pack(lists, lens, P)
    unused = np.sort(perm[len(used):]).astype(np.int32)
    Pp, nblk, ppool = 4096, 2, 4
    pperm = rng.permutation(ppool).astype(np.int32)
    pip, pix, plp = _pack([list(pperm[:nblk])], [prefix_pages * P], Pp)
    pun = np.sort(pperm[nblk:]).astype(np.int32)
    return ComposedWorkload(CONFIG_NAMES[13], 13, w5.batch, w5.num_qo_heads, w5.num_kv_heads,
                            w5.head_dim, P, "bf16", pool, ip, ix, lp, unused,
                            1_000_003 * 13 + 1, prefix_page_size=Pp, num_prefix_pool_pages=ppool,
                            prefix_indptr=pip, prefix_indices=pix, prefix_last_page_len=plp,
                            prefix_of=np.zeros(w5.batch, dtype=np.int32), prefix_unused_pages=pun)


# ----------------------------------------------------------- latent attention
# Latent width and rotary-key width of the MLA cache (DeepSeek-V2/V3 and
# Kimi K3 geometry), and the pre-absorption query/key head width (128 without
# rotary, 64 with) that sets the softmax scale.
MLA_DC = 512
MLA_DR = 64
MLA_QK_DIM = 192


@dataclasses.dataclass
class MLAWorkload:
    """Multi-head latent attention over a paged latent cache. Request b holds
    the tokens of its listed pages (kv_indptr / kv_indices / last_page_len,
    as for Workload); its query tokens are rows qo_indptr[b] ..
    qo_indptr[b+1]-1 of q_nope [N, H, 512] and q_pe [N, H, 64], its newest
    cached tokens (causal). The pools are ckv [pages, P, 512] and kpe
    [pages, P, 64]."""
    name: str
    config_id: int
    batch: int
    num_heads: int
    page_size: int
    num_pool_pages: int
    kv_indptr: np.ndarray
    kv_indices: np.ndarray
    last_page_len: np.ndarray
    unused_pages: np.ndarray
    value_seed: int
    qo_indptr: np.ndarray
    causal: bool = True
    dtype: str = "bf16"

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(MLA_QK_DIM)

    @property
    def num_qo_tokens(self) -> int:
        return int(self.qo_indptr[-1])

    def qo_lens(self) -> np.ndarray:
        return np.diff(self.qo_indptr).astype(np.int64)

    def kv_len(self, b: int) -> int:
        n = int(self.kv_indptr[b + 1] - self.kv_indptr[b])
        return 0 if n == 0 else (n - 1) * self.page_size + int(self.last_page_len[b])

    def kv_lens(self) -> np.ndarray:
        return np.array([self.kv_len(b) for b in range(self.batch)], dtype=np.int64)

    def visible_pairs(self) -> int:
        tot = 0
        for L, n in zip(self.kv_lens(), self.qo_lens()):
            L, n = int(L), int(n)
            tot += sum(max(0, L - n + i + 1) for i in range(n)) if self.causal else L * n
        return tot

    def flops(self) -> int:
        """Per (query head, visible token): d_c + d_r multiply-adds for the
        score and d_c for the weighted latent sum."""
        return 2 * (2 * MLA_DC + MLA_DR) * self.num_heads * self.visible_pairs()

    def algorithmic_bytes(self) -> int:
        """Every cached latent and rotary key once, plus q read and the output
        written (bf16)."""
        tok = int(self.kv_lens().sum())
        q = self.num_qo_tokens * self.num_heads * (MLA_DC + MLA_DR) * 2
        out = self.num_qo_tokens * self.num_heads * MLA_DC * 2
        return tok * (MLA_DC + MLA_DR) * 2 + q + out

    def make_values(self, device="cpu"):
        """(q_nope, q_pe, ckv_pool, kpe_pool): drawn in that order, N(0, 1)
        float32 cast to bf16; unlisted pages and the slots past each last
        page's length hold NaN."""
        import torch

        g = torch.Generator(device=device)
        g.manual_seed(self.value_seed)
        N, H, P = self.num_qo_tokens, self.num_heads, self.page_size

        def draw(shape):
            return torch.randn(shape, generator=g, dtype=torch.float32, device=device)

        q_nope = draw((N, H, MLA_DC)).to(torch.bfloat16)
        q_pe = draw((N, H, MLA_DR)).to(torch.bfloat16)
        pools = []
        for d in (MLA_DC, MLA_DR):
            x = draw((self.num_pool_pages, P, d))
            if len(self.unused_pages):
                idx = torch.as_tensor(self.unused_pages.astype(np.int64), device=device)
                x.index_fill_(0, idx, float("nan"))
            for b in range(self.batch):
                first, stop = int(self.kv_indptr[b]), int(self.kv_indptr[b + 1])
                ell = int(self.last_page_len[b])
                if stop > first and ell < P:
                    x[int(self.kv_indices[stop - 1]), ell:, :] = float("nan")
            pools.append(x.to(torch.bfloat16))
        return q_nope, q_pe, pools[0], pools[1]


def mla_workload(config_id: int) -> MLAWorkload:
    """15: the skewed batch's 64 history lengths (log-uniform in [32, 32768],
    the same draws as config 3) as a latent cache in 64-token pages, one
    query token per request, 96 heads (Kimi K3's global query heads)."""
    if config_id != 15:
        raise ValueError(f"unknown MLA config {config_id}")
    rng = np.random.default_rng([config_id, 0])
    lens = [int(x) for x in workload(3).kv_lens()]
    P = 64
    pool = sum((L + P - 1) // P for L in lens) + 64
    ip, ix, lp, un = paged_structure(lens, P, pool, rng)
    return MLAWorkload(CONFIG_NAMES[15], 15, len(lens), 96, P, pool, ip, ix, lp, un,
                       1_000_003 * config_id + 1, qo_indptr=_qo_indptr([1] * len(lens)))


def random_mla_workload(seed: int, batch: int, max_len: int, num_heads: int, page_size: int,
                        max_qo: int = 1, lens: Optional[List[int]] = None,
                        qo_lens: Optional[List[int]] = None, causal: bool = True,
                        spare_pages: int = 3) -> MLAWorkload:
    """Small ragged MLA case: history lengths U{1..max_len} (or given; 0
    allowed), query tokens U{1..min(L_b, max_qo)} per request (or given)."""
    rng = np.random.default_rng([seed, 19])
    if lens is None:
        lens = [int(x) for x in rng.integers(1, max_len + 1, size=batch)]
    if qo_lens is None:
        qo_lens = [int(rng.integers(1, max(1, min(L, max_qo)) + 1)) if L > 0 else 0 for L in lens]
    npg = sum((L + page_size - 1) // page_size for L in lens)
    ip, ix, lp, un = paged_structure(lens, page_size, npg + spare_pages, rng)
    return MLAWorkload(f"mla_{seed}", 0, len(lens), num_heads, page_size, npg + spare_pages, ip,
                       ix, lp, un, 40_000 + seed, qo_indptr=_qo_indptr(qo_lens), causal=causal)
