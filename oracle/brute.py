"""Pure-Python brute force for tiny inputs (test infrastructure only).

Triple loops with math.fsum (exactly rounded sums) and no numpy, used to pin
the vectorised oracle in `dense` on inputs with S of a few dozen.  The
quantities are the same plain definitions: the causal normaliser L_d
([P] Section 3.2), the causal attention output, and the column mass
sum_{d >= t + w, same document} exp(s_{d,t} - L_d) ([P] Section 3.1, Eq. 2
before the division by the number of queries; [G] Section 2.2).
"""
from __future__ import annotations

import math


def _docs(S, cu):
    if cu is None:
        return [0] * S, [S] * S
    c = [int(x) for x in cu]
    st, en = [0] * S, [S] * S
    for a, b in zip(c[:-1], c[1:]):
        for i in range(a, b):
            st[i], en[i] = a, b
    return st, en


def brute_attention(q, k, v, cu=None, scale=None, window=0):
    """q, k, v: nested lists [B][H][S][D] of floats.  Returns (lse, out, colmass)
    as nested lists, with lse/colmass [B][Hq][S] and out [B][Hq][S][D]."""
    B, Hq, S, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if not scale else scale
    st, en = _docs(S, cu)
    lse = [[[0.0] * S for _ in range(Hq)] for _ in range(B)]
    out = [[[[0.0] * D for _ in range(S)] for _ in range(Hq)] for _ in range(B)]
    colmass = [[[0.0] * S for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for g in range(Hq):
            h = g // G
            logit = {}
            for d in range(S):
                for t in range(st[d], d + 1):
                    logit[(d, t)] = sc * math.fsum(q[b][g][d][i] * k[b][h][t][i] for i in range(D))
            for d in range(S):
                ts = range(st[d], d + 1)
                L = math.log(math.fsum(math.exp(logit[(d, t)]) for t in ts))
                lse[b][g][d] = L
                for j in range(D):
                    out[b][g][d][j] = math.fsum(math.exp(logit[(d, t)] - L) * v[b][h][t][j] for t in ts)
            for t in range(S):
                colmass[b][g][t] = math.fsum(
                    math.exp(logit[(d, t)] - lse[b][g][d]) for d in range(t + window, en[t]) if d >= t)
    return lse, out, colmass


def brute_future_count(S, cu=None, window=0):
    """N_t of the mean in [P] Section 3.1, Eq. 2, by counting: for every key t,
    the number of query positions d of t's document with d >= t + w, found by
    walking over every position d of the sequence."""
    st, en = _docs(S, cu)
    out = []
    for t in range(S):
        n = 0
        for d in range(S):
            if st[d] == st[t] and d >= t + window:
                n += 1
        out.append(n)
    return out
