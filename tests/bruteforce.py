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


def bruteforce_prefill(q, k_pool, v_pool, qo_indptr, indptr, indices, last, sm_scale, causal):
    """Several query tokens per request, written out with plain loops. The
    query tokens of a request are its newest cached tokens: with n queries
    over L cached tokens, query i sits at position L - n + i and (causal)
    sees positions 0 .. L - n + i."""
    N, Hq, d = q.shape
    Hkv, P = k_pool.shape[1], k_pool.shape[2]
    G = Hq // Hkv
    O = [[[0.0] * d for _ in range(Hq)] for _ in range(N)]
    LSE = [[-math.inf] * Hq for _ in range(N)]
    for b in range(len(qo_indptr) - 1):
        toks = []
        first, stop = int(indptr[b]), int(indptr[b + 1])
        for j in range(first, stop):
            count = P if j + 1 < stop else int(last[b])
            toks.extend((int(indices[j]), slot) for slot in range(count))
        n = int(qo_indptr[b + 1]) - int(qo_indptr[b])
        for i in range(n):
            row = int(qo_indptr[b]) + i
            pos = len(toks) - n + i  # this query's own position
            seen = [t for k, t in enumerate(toks) if (k <= pos or not causal)]
            for h in range(Hq):
                g = h // G
                if not seen:
                    continue
                scores = [sm_scale * math.fsum(float(q[row, h, c]) * float(k_pool[p, g, s, c])
                                               for c in range(d)) for (p, s) in seen]
                top = max(scores)
                ws = [math.exp(x - top) for x in scores]
                den = math.fsum(ws)
                for c in range(d):
                    O[row][h][c] = math.fsum(w * float(v_pool[p, g, s, c])
                                             for w, (p, s) in zip(ws, seen)) / den
                LSE[row][h] = top + math.log(den)
    return O, LSE


def rope_rows_loops(rows, positions, theta, scale):
    """Rotary embedding written as plain loops over dim pairs with math.cos
    and math.sin: pair (i, i + d/2) of a row at position p turns by
    (p / scale) * theta ** (-2 i / d)."""
    out = []
    for x, pos in zip(rows, positions):
        d = len(x)
        h = d // 2
        y = [0.0] * d
        for i in range(h):
            ang = (pos / scale) * theta ** (-2.0 * i / d)
            c, s = math.cos(ang), math.sin(ang)
            y[i] = float(x[i]) * c - float(x[i + h]) * s
            y[i + h] = float(x[i + h]) * c + float(x[i]) * s
        out.append(y)
    return out


def bruteforce_mla(q_nope, q_pe, ckv_pool, kpe_pool, qo_indptr, indptr, indices, last, sm_scale,
                   causal):
    """Latent attention written out with plain loops: every head scores a
    token as sm_scale (q_nope . latent + q_pe . rotary key) and averages the
    latents; query i of n over L tokens sits at position L - n + i."""
    N, H, dc = q_nope.shape
    dr = q_pe.shape[2]
    P = ckv_pool.shape[1]
    O = [[[0.0] * dc for _ in range(H)] for _ in range(N)]
    LSE = [[-math.inf] * H for _ in range(N)]
    for b in range(len(qo_indptr) - 1):
        toks = []
        first, stop = int(indptr[b]), int(indptr[b + 1])
        for j in range(first, stop):
            count = P if j + 1 < stop else int(last[b])
            toks.extend((int(indices[j]), slot) for slot in range(count))
        n = int(qo_indptr[b + 1]) - int(qo_indptr[b])
        for i in range(n):
            row = int(qo_indptr[b]) + i
            pos = len(toks) - n + i
            seen = [t for k, t in enumerate(toks) if (k <= pos or not causal)]
            for h in range(H):
                if not seen:
                    continue
                scores = []
                for (p, s) in seen:
                    dot = math.fsum([float(q_nope[row, h, c]) * float(ckv_pool[p, s, c])
                                     for c in range(dc)] +
                                    [float(q_pe[row, h, c]) * float(kpe_pool[p, s, c])
                                     for c in range(dr)])
                    scores.append(sm_scale * dot)
                top = max(scores)
                ws = [math.exp(x - top) for x in scores]
                den = math.fsum(ws)
                for c in range(dc):
                    O[row][h][c] = math.fsum(w * float(ckv_pool[p, s, c])
                                             for w, (p, s) in zip(ws, seen)) / den
                LSE[row][h] = top + math.log(den)
    return O, LSE
