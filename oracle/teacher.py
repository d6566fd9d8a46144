"""Teacher labels at the eviction boundary and the boundary-aware retention
loss: plain CPU reference (test infrastructure only; imported by tests/,
smoke() and bench.py's CPU baseline, never by the library).

KVpop paper, Section 3.1:
  * Eq. 4: at query position d the eligible set is E_d = {t : s <= t <= d-w};
    token d-w has just left the protected window and is newly eligible.
  * Eq. 5: the teacher ranks E_d by effective scores, the target y(t) minus a
    per-head decay lambda times the number of decay steps of size Delta the
    token has aged: y(t) - lambda * floor((d - t) / Delta).  (The formula is
    stripped from the pages; this is the plainest reading of a per-head decay
    factor applied once per decay step, with the stated recency bias.)
  * The teacher keeps the top-k of E_d; the boundary token t_bnd(d) is the
    last retained token under the teacher ranking (Eq. 6 context), and the
    label of the newly eligible token d-w is whether the teacher keeps it.
  * Eq. 7: a pairwise logistic loss at the retention boundary on raw
    predicted scores r: with x_d = (r(d-w) - r(t_bnd(d))) / tau and
    sign_d = +1 for a kept label, -1 otherwise,
        loss_d = omega_d * ln(1 + exp(-sign_d * x_d)).
    (The decay term is the same for the two tokens compared at one d in the
    pages' statement, so the comparison uses raw scores.)

Ordering: effective score descending, ties to the lower index (the same rule
as the budget mask's static ranks).

Section 3.2 turns the per-query top-k into a running threshold over static
priorities, which the pages say holds only approximately because the decay
is applied in whole steps: with the decay written as lambda*(d-t)/Delta the
query-dependent part lambda*d/Delta is shared by all eligible tokens, leaving
the static priority
    pi(t) = y(t) + (lambda / Delta) * t.
`teacher_static` computes that form in float32, operation by operation
(c = lambda / Delta, then c * t, then y + that).  Against the floor form of
Eq. 5 the difference of a token's two scores at query d is a shared term
plus lambda * frac((d-t)/Delta), in [0, lambda (Delta-1)/Delta]: the two
rankings agree whenever static priorities differ by more than that (always
when lambda = 0 or Delta = 1), and only such near-ties can swap otherwise.
tests/test_oracle_teacher.py pins both statements against
`teacher_bruteforce`.
"""
from __future__ import annotations

import math

import numpy as np


def eligible_range(d: int, sinks: int, window: int):
    """E_d = [sinks, d - window] as (lo, hi_inclusive); empty when hi < lo."""
    return sinks, d - window


def teacher_bruteforce(y, sinks: int, window: int, topk: int, lam: float = 0.0, delta: int = 1):
    """Per query position d, sort E_d by the exact effective score of Eq. 5
    (float64) and keep the top-k.  y: [S].  Returns (label[S], boundary[S])
    as int64: label[d] = 1/0 whether token d-w is kept (-1 when d-w < sinks or
    no token is kept), boundary[d] = the last kept token (-1 if none)."""
    y = np.asarray(y, dtype=np.float64)
    S = y.shape[0]
    label = np.full(S, -1, dtype=np.int64)
    bnd = np.full(S, -1, dtype=np.int64)
    for d in range(S):
        lo, hi = eligible_range(d, sinks, window)
        if hi < lo or topk <= 0:
            continue
        toks = list(range(lo, hi + 1))
        eff = {t: y[t] - lam * math.floor((d - t) / delta) for t in toks}
        order = sorted(toks, key=lambda t: (-eff[t], t))
        kept = order[:topk]
        bnd[d] = kept[-1]
        label[d] = 1 if (d - window) in set(kept) else 0
    return label, bnd


def static_priorities(y, lam: float = 0.0, delta: int = 1) -> np.ndarray:
    """pi(t) = y(t) + (lambda/Delta) * t, each operation rounded to float32."""
    y32 = np.asarray(y, dtype=np.float32)
    c = np.float32(lam) / np.float32(delta)
    t = np.arange(y32.shape[-1], dtype=np.float32)
    return (y32 + (c * t).astype(np.float32)).astype(np.float32)


def _ranks(pri) -> np.ndarray:
    """rank(t): position of t when sorted by priority descending, index
    ascending; -0.0 counts as +0.0 and NaN as -inf."""
    p = np.asarray(pri, dtype=np.float64).copy()
    p[np.isnan(p)] = -np.inf
    p[p == 0.0] = 0.0
    order = np.lexsort((np.arange(p.shape[0]), -p))
    rank = np.empty(p.shape[0], dtype=np.int64)
    rank[order] = np.arange(p.shape[0])
    return rank


def teacher_static(y, sinks: int, window: int, topk: int, lam: float = 0.0, delta: int = 1):
    """The running-threshold teacher over static priorities (float32).

    Sweeps d upward, inserting rank(d-w) into a sorted list of the ranks of
    E_d (plain insertion; small sizes only).  The boundary rank is the
    min(k, |E_d|)-th smallest rank of E_d, the boundary token is the token of
    that rank, and the label of d-w is rank(d-w) <= boundary rank.
    Returns (label[S], boundary[S], rank[S], brank[S]) as int64; brank is -1
    where no token is kept."""
    pri = static_priorities(y, lam, delta)
    S = pri.shape[0]
    rank = _ranks(pri)
    token_of_rank = np.empty(S, dtype=np.int64)
    token_of_rank[rank] = np.arange(S)
    label = np.full(S, -1, dtype=np.int64)
    bnd = np.full(S, -1, dtype=np.int64)
    brank = np.full(S, -1, dtype=np.int64)
    elig = []  # sorted ranks of E_d
    import bisect
    for d in range(S):
        lo, hi = eligible_range(d, sinks, window)
        if hi >= lo and hi >= 0:
            bisect.insort(elig, int(rank[hi]))   # token d-w enters
        if not elig or topk <= 0:
            continue
        b = elig[min(topk, len(elig)) - 1]
        brank[d] = b
        bnd[d] = token_of_rank[b]
        label[d] = 1 if rank[d - window] <= b else 0
    return label, bnd, rank, brank


def boundary_loss(pred, label, bnd, window: int, tau: float, weight=None):
    """Eq. 7 per query position and the gradient of the summed loss with
    respect to the raw predicted scores (float64).

    loss[d] = omega_d * softplus(-sign_d * x_d), x_d = (r(d-w) - r(b)) / tau,
    for every d with a label and a boundary (0 elsewhere).  The gradient
    collects +dl/dx / tau on token d-w and -dl/dx / tau on the boundary."""
    r = np.asarray(pred, dtype=np.float64)
    S = r.shape[0]
    w_ = np.ones(S) if weight is None else np.asarray(weight, dtype=np.float64)
    loss = np.zeros(S)
    grad = np.zeros(S)
    for d in range(S):
        if label[d] < 0 or bnd[d] < 0:
            continue
        a, b = d - window, int(bnd[d])
        sgn = 1.0 if label[d] == 1 else -1.0
        x = (r[a] - r[b]) / tau
        z = -sgn * x
        loss[d] = w_[d] * (max(z, 0.0) + math.log1p(math.exp(-abs(z))))   # softplus, stable
        sig = math.exp(min(z, 0.0)) / (1.0 + math.exp(-abs(z)))              # sigmoid(z), stable
        dl_dx = -sgn * w_[d] * sig                                            # omega * sigmoid(z) * dz/dx
        grad[a] += dl_dx / tau
        grad[b] -= dl_dx / tau
    return loss, grad
