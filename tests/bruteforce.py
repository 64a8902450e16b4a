"""Pure-Python brute force of decode attention over a paged KV cache.

Independent of oracle/: plain loops, ``math.fsum`` for every sum, so the only
rounding is one correctly rounded sum per dot product. Used on tiny inputs to
pin the vectorised float64 oracle.
"""
import math


def bruteforce_decode(q, k_pool, v_pool, indptr, indices, last, sm_scale):
    B, Hq, d = q.shape
    Hkv, P = k_pool.shape[1], k_pool.shape[2]
    G = Hq // Hkv
    O = [[[0.0] * d for _ in range(Hq)] for _ in range(B)]
    LSE = [[-math.inf] * Hq for _ in range(B)]
    for b in range(B):
        first, stop = int(indptr[b]), int(indptr[b + 1])
        toks = []
        for j in range(first, stop):
            count = P if j + 1 < stop else int(last[b])
            for slot in range(count):
                toks.append((int(indices[j]), slot))
        for h in range(Hq):
            g = h // G
            if not toks:
                continue
            scores = []
            for (p, s) in toks:
                dot = math.fsum(float(q[b, h, i]) * float(k_pool[p, g, s, i]) for i in range(d))
                scores.append(sm_scale * dot)
            top = max(scores)
            ws = [math.exp(x - top) for x in scores]
            den = math.fsum(ws)
            for i in range(d):
                num = math.fsum(w * float(v_pool[p, g, s, i]) for w, (p, s) in zip(ws, toks))
                O[b][h][i] = num / den
            LSE[b][h] = top + math.log(den)
    return O, LSE
