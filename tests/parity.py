"""Comparison of library outputs with the float64 oracle.

Tolerances (max-abs): 2e-3 on outputs, 1e-4 on the float32 natural-log LSE.
A bfloat16 output is compared with the oracle rounded to bfloat16 (nearest
even); an element that misses 2e-3 still passes when it is one of the two
bfloat16 values bracketing the exact result, because rounding an exact value
of magnitude >= 1 to bfloat16 alone moves it by up to 2^-8 > 2e-3. The count of
elements passing only through that second clause is reported.
"""
import numpy as np

from oracle.attention import bf16_neighbors, round_bf16_rne

OUT_TOL = 2e-3
LSE_TOL = 1e-4


def compare(out_gpu, lse_gpu, O, LSE, bf16: bool, what=""):
    """out_gpu, lse_gpu: float64 numpy copies of the library's outputs;
    O, LSE: oracle float64. Raises AssertionError with a summary on failure."""
    out_gpu = np.asarray(out_gpu, dtype=np.float64)
    assert np.all(np.isfinite(out_gpu)), f"{what}: non-finite output"
    stats = {}
    if bf16:
        ref = round_bf16_rne(O)
        diff = np.abs(out_gpu - ref)
        lo, hi = bf16_neighbors(O)
        faithful = (out_gpu == lo) | (out_gpu == hi)
        ok = (diff <= OUT_TOL) | faithful
        stats["faithful_only"] = int(np.sum(~(diff <= OUT_TOL) & faithful))
        stats["max_abs_vs_rounded"] = float(diff.max()) if diff.size else 0.0
    else:
        diff = np.abs(out_gpu - O)
        ok = diff <= OUT_TOL
        stats["max_abs"] = float(diff.max()) if diff.size else 0.0
    stats["max_abs_vs_exact"] = float(np.abs(out_gpu - O).max()) if O.size else 0.0
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} output elements out of tolerance; first at {i}: "
                             f"gpu={out_gpu[i]!r} exact={O[i]!r} stats={stats}")
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    empty = np.isneginf(LSE)
    assert np.array_equal(np.isneginf(lse_gpu), empty), f"{what}: -inf LSE pattern differs"
    if (~empty).any():
        dl = np.abs(lse_gpu[~empty] - LSE[~empty])
        stats["lse_max_abs"] = float(dl.max())
        assert dl.max() <= LSE_TOL, f"{what}: LSE error {dl.max()} > {LSE_TOL}"
    if empty.any():
        assert np.all(out_gpu[empty] == 0), f"{what}: empty request output not zero"
    return stats


def prefill_request(w, b):
    """Request b of a prefill workload as a batch of one over the same pool:
    (first query row, last query row + 1, qo_indptr, kv_indptr, kv_indices,
    last_page_len). The oracle attends per request, so evaluating it on
    these slices one request at a time gives exactly the whole-batch result
    with memory bounded by the largest request."""
    q0, q1 = int(w.qo_indptr[b]), int(w.qo_indptr[b + 1])
    p0, p1 = int(w.kv_indptr[b]), int(w.kv_indptr[b + 1])
    return (q0, q1, np.array([0, q1 - q0]), np.array([0, p1 - p0]),
            np.asarray(w.kv_indices[p0:p1]), np.asarray(w.last_page_len[b:b + 1]))
