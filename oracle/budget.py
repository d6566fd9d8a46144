"""Budget-mask oracle: static ranks, running top-k cutoff, mask rows, masked attention.

Test infrastructure only (see the package docstring).

Definitions ([P] Section 3 overview; [G] Section 2.1):
  each KV head keeps, for query position d,
    * the s sink tokens, i.e. the first s positions ([G] 2.1: the first few
      tokens are always kept),
    * the protected window of the w most recent tokens, (d - w, d],
    * the top-k of the eligible set E_d = [s, d - w] ([P] Section 3.1, Eq. 4:
      tokens outside the sinks and outside the window compete; token d - w has
      just left the window and is newly eligible), ranked by static
      priorities (scores), higher score first, ties to the lower index.
  B = s + w + k ([G] 2.1).

[P] Section 3.2 "Running top-k sparse attention": sort the tokens once by
static priority to get rank(t); as d grows exactly one token (d - w) enters
E_d; insert its rank into a Fenwick tree and find the rank of the k-th best
eligible token by binary lifting; that cutoff c_d keeps exactly the eligible
tokens with rank <= c_d.

Cutoff conventions (the pages leave them open): when |E_d| < k every eligible
token is kept and c_d = CUTOFF_ALL (2^31 - 1); when k = 0 none is and
c_d = CUTOFF_NONE (-1).

Packed sequences (`cu`, document offsets; [P] Section 4 trains on packed
sequences): attention never leaves a document, so the mask of a query is the
mask its document would give on its own: sinks are the first s positions of
the document and E_d = [start(d) + s, d - w] (the pages do not say; this is
the reading under which packing changes nothing).  Ranks are taken over the
whole packed sequence: restricted to one document they order its tokens
exactly as the document's own ranks would, so c_d, the k-th smallest rank in
E_d, selects the same tokens.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .dense import _row_lse, default_scale, doc_bounds

CUTOFF_ALL = 2 ** 31 - 1
CUTOFF_NONE = -1


def static_ranks(scores) -> np.ndarray:
    """rank(t) = position of t in the order (score descending, index ascending).

    -0.0 and +0.0 compare equal (ties go to the lower index); NaN is ranked
    like -inf.  Returns int64 [S], a permutation of 0..S-1.
    """
    s = np.asarray(scores, dtype=np.float64).copy()
    s[np.isnan(s)] = -np.inf
    idx = np.arange(s.shape[0])
    order = np.lexsort((idx, -s))          # primary: -score ascending; secondary: index
    rank = np.empty_like(idx)
    rank[order] = idx
    return rank


class _Fenwick:
    """Fenwick (binary indexed) tree of counts over ranks 0..n-1."""

    def __init__(self, n: int):
        self.n = n
        self.tree = [0] * (n + 1)
        self.log = 1
        while (1 << self.log) <= n:
            self.log += 1

    def insert(self, r: int):
        i = r + 1
        while i <= self.n:
            self.tree[i] += 1
            i += i & (-i)

    def kth(self, k: int) -> int:
        """Smallest rank r such that the count of inserted ranks <= r is >= k
        (binary lifting down the implicit tree).  Requires 1 <= k <= count."""
        pos = 0
        rem = k
        for j in range(self.log, -1, -1):
            nxt = pos + (1 << j)
            if nxt <= self.n and self.tree[nxt] < rem:
                pos = nxt
                rem -= self.tree[nxt]
        return pos          # 1-based position pos+1 -> rank pos


def running_cutoffs(rank, sinks: int, window: int, topk: int, cu=None) -> np.ndarray:
    """c_d for every query position d, by the pages' sequential sweep.

    At step d the token d - w becomes eligible when d - w >= s (positions
    counted from the start of d's document); its rank is inserted into the
    Fenwick tree; then c_d is the k-th smallest inserted rank (binary
    lifting) if at least k are inserted.  The tree starts empty at every
    document start.
    """
    rank = [int(r) for r in rank]
    S = len(rank)
    start, _ = doc_bounds(S, cu)
    fw = None
    count = 0
    out = np.empty(S, dtype=np.int64)
    for d in range(S):
        if d == 0 or start[d] != start[d - 1]:
            fw = _Fenwick(S)
            count = 0
        t_new = d - window
        if t_new >= start[d] + sinks:
            fw.insert(rank[t_new])
            count += 1
        if topk <= 0:
            out[d] = CUTOFF_NONE
        elif count < topk:
            out[d] = CUTOFF_ALL
        else:
            out[d] = fw.kth(topk)
    return out


def mask_rows(rank, cutoff, sinks: int, window: int, rows, cu=None) -> np.ndarray:
    """Membership rows M_d over t (bool [len(rows), S]) from ranks and cutoffs:
    t in d's document, t <= d, and (t < a + s, or d - w < t, or
    (a + s <= t <= d - w and rank(t) <= c_d)), where a is the start of d's
    document (0 without `cu`).  `rank` may be cut short after the last row's
    position; `cu` then still describes the whole sequence."""
    rank = np.asarray(rank)
    S = rank.shape[0]
    rows = np.asarray(rows)
    t = np.arange(S)[None, :]
    d = rows[:, None]
    c = np.asarray(cutoff)[rows][:, None]
    if cu is None:
        a = np.zeros_like(d)
    else:
        c_ = [int(x) for x in cu]
        a = np.asarray([max(x for x in c_[:-1] if x <= int(r)) for r in rows])[:, None]
    sink = t < a + sinks
    win = t > d - window
    elig = (t >= a + sinks) & (t <= d - window)
    return (t >= a) & (t <= d) & (sink | win | (elig & (rank[None, :] <= c)))


def brute_mask_row(scores, d: int, sinks: int, window: int, topk: int, cu=None) -> np.ndarray:
    """The definition for one query, with no ranks and no running structure:
    within d's document (starting at a), the sinks [a, a + s), the window
    (d - w, d], and the k best of E_d = [a + s, d - w] sorted by
    (score desc, index asc)."""
    s = np.asarray(scores, dtype=np.float64)
    S = s.shape[0]
    a = 0 if cu is None else max(int(x) for x in list(cu)[:-1] if int(x) <= d)
    row = np.zeros(S, dtype=bool)
    for t in range(a, min(a + sinks, d + 1)):
        row[t] = True
    for t in range(max(a, d - window + 1), d + 1):
        row[t] = True
    elig = list(range(a + sinks, d - window + 1))
    key = [(-(s[t] if not np.isnan(s[t]) else -np.inf), t) for t in elig]
    key.sort()
    for _, t in key[:max(0, topk)]:
        row[t] = True
    return row


def masked_attention(q, k, v, rank, cutoff, sinks: int, window: int, scale=None,
                     heads: Optional[list] = None, rows: Optional[np.ndarray] = None,
                     row_block: int = 128, cu=None):
    """Attention restricted to the budget mask: for every query row d,
    O_d = sum_{t in M_d} softmax_t(s_{d,t}) v_t and L_d = ln sum_{t in M_d} exp(s_{d,t}).

    The mask is per KV head (the budget is kept per KV head, [P] Section 3)
    and shared by the G query heads of the group.  `rank` and `cutoff` are
    [B, Hkv, S].  Only the columns that some row of a block keeps are
    multiplied (every other column is masked for the whole block).  An empty
    row gives L = -inf and O = 0.  Returns (out [B,Hq,S,D], lse [B,Hq,S]); rows
    not asked for stay NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = default_scale(D, scale)
    out = np.full((B, Hq, S, D), np.nan)
    lse = np.full((B, Hq, S), np.nan)
    all_rows = np.arange(S) if rows is None else np.asarray(sorted(set(int(r) for r in rows)))
    if heads is None:
        heads = [(b, g) for b in range(B) for g in range(Hq)]
    for (b, g) in heads:
        h = g // G
        for i0 in range(0, len(all_rows), row_block):
            rr = all_rows[i0:i0 + row_block]
            M = mask_rows(rank[b, h], cutoff[b, h], sinks, window, rr, cu=cu)
            cols = np.nonzero(M.any(axis=0))[0]
            if cols.size == 0:
                lse[b, g, rr] = -np.inf
                out[b, g, rr] = 0.0
                continue
            logits = sc * (q[b, g, rr] @ k[b, h, cols].T)
            allowed = M[:, cols]
            L = _row_lse(logits, allowed)
            with np.errstate(under="ignore", invalid="ignore"):
                A = np.where(allowed, np.exp(logits - L[:, None]), 0.0)
            lse[b, g, rr] = L
            out[b, g, rr] = A @ v[b, h, cols]
    return out, lse


def budget_reference(scores, sinks: int, window: int, topk: int, cu=None):
    """ranks and cutoffs for scores [B, Hkv, S] (int64 arrays of the same
    shape); with `cu` (batch 1) the cutoffs restart at every document."""
    sc = np.asarray(scores, dtype=np.float64)
    B, H, S = sc.shape
    rank = np.empty((B, H, S), dtype=np.int64)
    cut = np.empty((B, H, S), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            rank[b, h] = static_ranks(sc[b, h])
            cut[b, h] = running_cutoffs(rank[b, h], sinks, window, topk, cu=cu)
    return rank, cut
