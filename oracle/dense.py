"""Dense fp64 oracle: causal attention with LSE, future mass, Eq. 8, target.

Test infrastructure only (see the package docstring).  Everything is computed
from the plain definitions by building the attention matrix explicitly, one
block of query rows at a time ([P] Section 3.1 defines the target through the
dense causal attention probabilities; [P] Section 3.2 notes that the
transposed identity is exact when the dense normaliser is used).

Arrays are numpy float64 with layout [B, H, S, D] (heads major, positions
contiguous).  `cu` is None or an int sequence [n_docs + 1] of document offsets
(batch must then be 1).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

AGG_SUM, AGG_MAX, AGG_NONE = 0, 1, 2


def to_f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (bf16 / f32) or array to numpy float64."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def doc_bounds(S: int, cu=None):
    """Per-position document start (inclusive) and end (exclusive).

    Sequence packing puts several documents in one training sequence ([P]
    Section 4); attention stays inside a document, so each position only sees
    its own document.
    """
    start = np.zeros(S, dtype=np.int64)
    end = np.full(S, S, dtype=np.int64)
    if cu is not None:
        c = [int(x) for x in cu]
        if c[0] != 0 or c[-1] != S or any(c[i + 1] <= c[i] for i in range(len(c) - 1)):
            raise ValueError("cu_seqlens must rise strictly from 0 to S")
        for a, b in zip(c[:-1], c[1:]):
            start[a:b] = a
            end[a:b] = b
    return start, end


def default_scale(D: int, scale: Optional[float]) -> float:
    """Softmax scale: 1/sqrt(D) when not given (the pages speak of the logit
    before the softmax without its scale, [P] Section 3.2; 1/sqrt(D) is
    Qwen3's)."""
    return 1.0 / math.sqrt(D) if (scale is None or scale <= 0) else float(scale)


def _causal_logits(qb: np.ndarray, kh: np.ndarray, rows: np.ndarray, start: np.ndarray, scale: float):
    """Logits sigma * q_d . k_t for a block of rows over columns [c0, r1).

    Returns (logits, allowed, c0) where allowed[d, t] = (t <= d) and t in
    the document of d.
    """
    r0, r1 = int(rows[0]), int(rows[-1]) + 1
    c0 = int(start[r0:r1].min())
    cols = np.arange(c0, r1)
    logits = scale * (qb @ kh[c0:r1].T)
    allowed = (cols[None, :] <= rows[:, None]) & (cols[None, :] >= start[rows][:, None])
    return logits, allowed, c0


def _row_lse(logits: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """L_d = ln sum_{allowed t} exp(s_{d,t}), with the row max taken out."""
    masked = np.where(allowed, logits, -np.inf)
    m = masked.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(under="ignore"):
        ssum = np.exp(masked - m_safe[:, None]).sum(axis=1)
    with np.errstate(divide="ignore"):
        return m_safe + np.log(ssum)


def attention_pass(q, k, v=None, cu=None, scale=None, window: Optional[int] = None,
                   lse_in: Optional[np.ndarray] = None, need_output: bool = True,
                   heads: Optional[list] = None, row_block: int = 256, need_abs_output: bool = False):
    """One pass over the dense causal attention matrix, row block by row block.

    For every (b, g) and query row d it computes the logits s_{d,t} =
    sigma q^g_d . k^h_t over t <= d in the same document, the log-normaliser
    L^g_d (the causal LSE, [P] Section 3.2), the probabilities
    a^g_{d,t} = exp(s_{d,t} - L^g_d) and, when asked,
      * O^g_d = sum_t a^g_{d,t} v^h_t  (dense causal attention output);
      * colmass^g(t) = sum over d >= t + window in the same document of
        a^g_{d,t}  (the column sums of the attention matrix restricted to
        queries at least `window` positions ahead; [P] Section 3.1 Eq. 2
        before its division by the number of such queries; [G] Section 2.2
        writes the condition d >= t + w).

    If `lse_in` is given ([B, Hq, S]) the column sums use exp(s - lse_in)
    instead of the oracle's own L (the pages' sparse-normaliser
    approximation, [P] Section 3.2); O and the returned LSE are still the
    dense ones.

    With `need_abs_output`, also abs_out = sum_t a^g_{d,t} |v^h_t| (used only
    to bound the rounding error of a reduced-precision output).

    Returns dict(lse [B,Hq,S], out [B,Hq,S,D] or None, colmass [B,Hq,S] or
    None, abs_out or None).  `heads` restricts the pass to a list of (b, g)
    pairs (others stay NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    G = Hq // Hkv
    if cu is not None and B != 1:
        raise ValueError("packed sequences need batch 1")
    sc = default_scale(D, scale)
    start, _ = doc_bounds(S, cu)
    lse = np.full((B, Hq, S), np.nan)
    out = np.full((B, Hq, S, D), np.nan) if (need_output and v is not None) else None
    colmass = np.full((B, Hq, S), np.nan) if window is not None else None
    abs_out = np.full((B, Hq, S, D), np.nan) if (need_abs_output and v is not None) else None
    if heads is None:
        heads = [(b, g) for b in range(B) for g in range(Hq)]
    for (b, g) in heads:
        h = g // G
        kh = k[b, h]
        vh = None if v is None else np.asarray(v[b, h], dtype=np.float64)
        if colmass is not None:
            colmass[b, g] = 0.0
        for r0 in range(0, S, row_block):
            rows = np.arange(r0, min(S, r0 + row_block))
            logits, allowed, c0 = _causal_logits(q[b, g, rows], kh, rows, start, sc)
            L = _row_lse(logits, allowed)
            lse[b, g, rows] = L
            if out is not None or colmass is not None or abs_out is not None:
                with np.errstate(under="ignore", invalid="ignore"):
                    A = np.where(allowed, np.exp(logits - L[:, None]), 0.0)
            if out is not None:
                out[b, g, rows] = A @ vh[c0:rows[-1] + 1]
            if abs_out is not None:
                abs_out[b, g, rows] = A @ np.abs(vh[c0:rows[-1] + 1])
            if colmass is not None:
                cols = np.arange(c0, rows[-1] + 1)
                fut = allowed & (cols[None, :] <= rows[:, None] - window)
                if lse_in is not None:
                    Lx = np.asarray(lse_in[b, g, rows], dtype=np.float64)
                    with np.errstate(under="ignore", over="ignore", invalid="ignore"):
                        Af = np.where(fut, np.exp(logits - Lx[:, None]), 0.0)
                else:
                    Af = np.where(fut, A, 0.0)
                colmass[b, g, c0:rows[-1] + 1] += Af.sum(axis=0)
    return {"lse": lse, "out": out, "colmass": colmass, "abs_out": abs_out}


def row_lse(q, k, rows, cu=None, scale=None, heads: Optional[list] = None) -> np.ndarray:
    """The causal log-normaliser L^g_d of attention_pass for the listed query
    positions only, one row at a time (for long sequences, where the whole
    matrix is too large to build).  Returns [B, Hq, S] with NaN outside the
    listed rows and heads."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Hq, S, D = q.shape
    G = Hq // k.shape[1]
    sc = default_scale(D, scale)
    start, _ = doc_bounds(S, cu)
    lse = np.full((B, Hq, S), np.nan)
    if heads is None:
        heads = [(b, g) for b in range(B) for g in range(Hq)]
    for (b, g) in heads:
        for d in sorted(set(int(x) for x in rows)):
            r = np.array([d])
            logits, allowed, _ = _causal_logits(q[b, g, r], k[b, g // G], r, start, sc)
            lse[b, g, d] = _row_lse(logits, allowed)[0]
    return lse


def future_count(S: int, cu, window: int) -> np.ndarray:
    """N_t = number of queries d in t's document with d >= t + w."""
    _, end = doc_bounds(S, cu)
    t = np.arange(S)
    return np.maximum(0, end - t - int(window))


def target_from_colmass(colmass: np.ndarray, n_kv_heads: int, cu, window: int,
                        agg: int = AGG_SUM, mean_over_queries: bool = False,
                        eps: float = 0.0) -> np.ndarray:
    """Future-utility target from the per-query-head column masses.

    m^g(t) = colmass^g(t) / N_t when `mean_over_queries` (the mean of [P]
    Section 3.1 Eq. 2; an empty set gives 0), else colmass^g(t).
      AGG_MAX  : y_h(t) = max_{g in G(h)} ln(m^g(t) + eps)   ([P] Eq. 3 with
                 the max aggregation used in the paper's experiments)
      AGG_SUM  : T_h(t) = ln(sum_{g in G(h)} m^g(t) + eps)   (one log-sum-exp
                 across queries and the query heads of the group)
      AGG_NONE : ln(m^g(t) + eps) per query head.
    Empty sets give ln(eps) (-inf for eps = 0).
    """
    B, Hq, S = colmass.shape
    G = Hq // n_kv_heads
    m = np.array(colmass, dtype=np.float64)
    if mean_over_queries:
        N = future_count(S, cu, window).astype(np.float64)
        with np.errstate(divide="ignore", invalid="ignore"):
            m = np.where(N[None, None, :] > 0, m / np.maximum(N, 1)[None, None, :], 0.0)
    with np.errstate(divide="ignore"):
        if agg == AGG_NONE:
            return np.log(m + eps)
        mg = m.reshape(B, n_kv_heads, G, S)
        if agg == AGG_SUM:
            return np.log(mg.sum(axis=2) + eps)
        if agg == AGG_MAX:
            return np.log(mg + eps).max(axis=2)
    raise ValueError("agg must be AGG_SUM, AGG_MAX or AGG_NONE")


def transposed_lse(q, k, lse: np.ndarray, cu=None, scale=None, window: int = 0,
                   heads: Optional[list] = None, key_block: int = 256, keys=None) -> np.ndarray:
    """The pages' transposed-attention formulation of the first term of Eq. 8.

    [P] Section 3.2: original key positions become queries and original query
    positions become keys; the dot products give back the original logits
    s_{d,t}; the per-query normaliser L_d is subtracted as a score modifier
    and a block mask keeps d >= t + w; the LSE of that attention call, for
    key t, is ln sum_{d >= t+w} exp(s_{d,t} - L_d).  Returns that LSE,
    [B, Hq, S], natural log, -inf where no query qualifies.  Subtracting
    ln N_t gives ln m^g(t) of Eq. 2.  `keys` restricts it to a list of key
    positions (the others stay NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Hq, S, D = q.shape
    G = Hq // k.shape[1]
    sc = default_scale(D, scale)
    start, end = doc_bounds(S, cu)
    res = np.full((B, Hq, S), np.nan)
    if heads is None:
        heads = [(b, g) for b in range(B) for g in range(Hq)]
    for (b, g) in heads:
        h = g // G
        qs = q[b, g]                      # original queries act as keys here
        Lrow = np.asarray(lse[b, g], dtype=np.float64)
        key_list = np.arange(S) if keys is None else np.array(sorted(set(int(x) for x in keys)), dtype=np.int64)
        for t0 in range(0, key_list.size, key_block):
            keys_b = key_list[t0:t0 + key_block]
            scores = sc * (k[b, h, keys_b] @ qs.T) - Lrow[None, :]   # score modifier -L_d
            dcol = np.arange(S)
            block_mask = (dcol[None, :] >= keys_b[:, None] + window) & (dcol[None, :] < end[keys_b][:, None]) \
                & (dcol[None, :] >= start[keys_b][:, None])
            masked = np.where(block_mask, scores, -np.inf)
            mx = masked.max(axis=1)
            mx_safe = np.where(np.isfinite(mx), mx, 0.0)
            with np.errstate(under="ignore", divide="ignore"):
                res[b, g, keys_b] = mx_safe + np.log(np.exp(masked - mx_safe[:, None]).sum(axis=1))
    return res


def reference(q, k, v=None, cu=None, scale=None, window: int = 0, agg: int = AGG_SUM,
              mean_over_queries: bool = False, eps: float = 0.0, need_output: bool = True):
    """Convenience: dense pass + target epilogue.  Returns dict(lse, out, colmass, target)."""
    q64, k64 = to_f64(q), to_f64(k)
    v64 = None if v is None else to_f64(v)
    r = attention_pass(q64, k64, v64, cu=cu, scale=scale, window=window, need_output=need_output)
    r["target"] = target_from_colmass(r["colmass"], k64.shape[1], cu, window, agg,
                                      mean_over_queries, eps)
    return r
