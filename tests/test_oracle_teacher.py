"""Pins of the teacher-label and boundary-loss oracle (oracle/teacher.py)
against the pages' definitions (KVpop paper, Section 3.1, Eqs. 4-7),
brute force, closed forms and the budget-mask oracle."""
import math

import numpy as np
import pytest

from oracle import budget, teacher


def test_hand_worked_example():
    """S=9, sinks 1, window 2, top-2, lambda 0.  y by position:
    t : 0    1    2    3    4    5    6    7    8
    y : 9    0.5  3    1    3    -1   2    0    0
    E_d = [1, d-2].  d=3: E={1}: keep {1}, boundary 1, label(1)=1.
    d=4: E={1,2}: both kept (k=2), order 2 (3.0) then 1 (0.5): boundary 1,
    label(2)=1.  d=5: E={1,2,3}: top-2 = {2 (3.0), 3 (1.0)}: boundary 3,
    label(3)=1.  d=6: E adds 4 (3.0, ties with 2 -> lower index 2 first):
    top-2 = {2, 4}, boundary 4, label(4)=1.  d=7: adds 5 (-1): top-2 {2,4},
    boundary 4, label(5)=0.  d=8: adds 6 (2.0): top-2 {2,4}, boundary 4,
    label(6)=0."""
    y = [9, 0.5, 3, 1, 3, -1, 2, 0, 0]
    lab, bnd = teacher.teacher_bruteforce(y, 1, 2, 2)
    assert list(lab) == [-1, -1, -1, 1, 1, 1, 1, 0, 0]
    assert list(bnd) == [-1, -1, -1, 1, 1, 3, 4, 4, 4]
    lab2, bnd2, _, _ = teacher.teacher_static(y, 1, 2, 2)
    assert list(lab2) == list(lab) and list(bnd2) == list(bnd)


@pytest.mark.parametrize("seed", range(6))
def test_static_equals_bruteforce_without_decay(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(5, 80))
    s, w, k = int(rng.integers(0, 5)), int(rng.integers(0, 12)), int(rng.integers(0, 20))
    y = rng.integers(-3, 4, S).astype(np.float64)  # many ties
    lab, bnd = teacher.teacher_bruteforce(y, s, w, k)
    lab2, bnd2, _, _ = teacher.teacher_static(y, s, w, k)
    assert np.array_equal(lab, lab2) and np.array_equal(bnd, bnd2)


@pytest.mark.parametrize("seed", range(6))
def test_static_equals_bruteforce_with_unit_decay_step(seed):
    """Delta = 1: floor((d-t)/1) = d-t, so Eq. 5 equals the static priority
    y(t) + lambda*t minus a term shared by all tokens; with y on a 1/16 grid
    and lambda = 1/4 the float32 priorities are exact."""
    rng = np.random.default_rng(100 + seed)
    S = int(rng.integers(5, 70))
    s, w, k = int(rng.integers(0, 4)), int(rng.integers(0, 10)), int(rng.integers(1, 15))
    y = rng.integers(-40, 40, S) / 16.0
    lab, bnd = teacher.teacher_bruteforce(y, s, w, k, lam=0.25, delta=1)
    lab2, bnd2, _, _ = teacher.teacher_static(y, s, w, k, lam=0.25, delta=1)
    assert np.array_equal(lab, lab2) and np.array_equal(bnd, bnd2)


def test_decay_favours_recent_tokens():
    """With equal targets the decay makes the newest eligible tokens win:
    the kept set is the k most recent eligible tokens, so every newly
    eligible token is kept and the boundary is d-w-k+1."""
    S, s, w, k = 40, 2, 3, 5
    lab, bnd = teacher.teacher_bruteforce(np.zeros(S), s, w, k, lam=0.5, delta=1)
    for d in range(S):
        n = d - w - s + 1
        if n <= 0:
            assert lab[d] == -1 and bnd[d] == -1
        else:
            assert lab[d] == 1
            assert bnd[d] == (s if n < k else d - w - k + 1)


def test_closed_form_decreasing_targets():
    """y strictly decreasing in t, no decay: the first k eligible tokens
    [s, s+k) are kept forever; token d-w is kept iff d-w < s+k."""
    S, s, w, k = 60, 3, 4, 7
    y = -np.arange(S, dtype=np.float64)
    lab, bnd, _, _ = teacher.teacher_static(y, s, w, k)
    for d in range(S):
        a = d - w
        if a < s:
            assert lab[d] == -1
            continue
        assert lab[d] == (1 if a < s + k else 0)
        assert bnd[d] == min(a, s + k - 1)


def test_lambda_zero_agrees_with_the_budget_mask_oracle():
    """Without decay the teacher is the budget mask applied to the targets:
    the boundary rank is the budget cutoff c_d whenever |E_d| >= k, and the
    label of d-w is its membership in mask row d."""
    rng = np.random.default_rng(7)
    S, s, w, k = 300, 4, 16, 25
    y = rng.standard_normal(S)
    lab, bnd, rank, brank = teacher.teacher_static(y, s, w, k)
    y32 = y.astype(np.float32).astype(np.float64)
    rk = budget.static_ranks(y32)
    cut = budget.running_cutoffs(rk, s, w, k)
    assert np.array_equal(rank, rk)
    rows = budget.mask_rows(rk, cut, s, w, np.arange(S))
    for d in range(S):
        n = d - w - s + 1
        if n >= k:
            assert brank[d] == cut[d]
        if d - w >= s:
            assert lab[d] == int(rows[d, d - w])


def test_boundary_loss_closed_forms_and_gradient():
    rng = np.random.default_rng(3)
    S, s, w, k, tau = 50, 2, 4, 6, 0.7
    y = rng.standard_normal(S)
    lab, bnd, _, _ = teacher.teacher_static(y, s, w, k)
    r = rng.standard_normal(S)
    om = rng.uniform(0.5, 2.0, S)
    loss, grad = teacher.boundary_loss(r, lab, bnd, w, tau, om)
    # closed form per term
    for d in range(S):
        if lab[d] < 0:
            assert loss[d] == 0.0
            continue
        x = (r[d - w] - r[bnd[d]]) / tau
        sgn = 1 if lab[d] == 1 else -1
        assert abs(loss[d] - om[d] * math.log(1 + math.exp(-sgn * x))) < 1e-12
    # x = 0 gives omega * ln 2 (the newly eligible token is its own boundary)
    same = [d for d in range(S) if lab[d] >= 0 and bnd[d] == d - w]
    for d in same:
        assert abs(loss[d] - om[d] * math.log(2.0)) < 1e-12
    # central finite differences of the summed loss
    h = 1e-6
    for t in range(S):
        rp, rm = r.copy(), r.copy()
        rp[t] += h
        rm[t] -= h
        fd = (teacher.boundary_loss(rp, lab, bnd, w, tau, om)[0].sum()
              - teacher.boundary_loss(rm, lab, bnd, w, tau, om)[0].sum()) / (2 * h)
        assert abs(fd - grad[t]) < 1e-6
    # the gradient sums to zero (every term moves two scores in opposite directions)
    assert abs(grad.sum()) < 1e-12


def _kept_exact(y, d, s, w, k, lam, delta):
    """The teacher's kept set at query d under Eq. 5's floor form, by sorting
    E_d on (effective score descending, index ascending) in float64."""
    toks = list(range(s, d - w + 1))
    eff = {t: float(y[t]) - lam * math.floor((d - t) / delta) for t in toks}
    return sorted(toks, key=lambda t: (-eff[t], t))[:max(k, 0)]


@pytest.mark.parametrize("delta,lam,seed", [(16, 0.5, 0), (16, 1.5, 1), (8, 0.75, 2), (5, 3.0, 3)])
def test_static_equals_bruteforce_with_separated_priorities(delta, lam, seed):
    """Delta > 1.  Eq. 5's effective score minus the static priority
    pi(t) = y(t) + (lambda/Delta) t is -lambda d/Delta (shared by every token
    at query d) plus lambda * frac((d-t)/Delta), which lies in
    [0, lambda (Delta-1)/Delta].  So when every two static priorities differ
    by more than that, both forms order E_d the same way and the running
    threshold reproduces the floor form exactly.  Priorities here are
    distinct integers times a gap above lambda, and y is derived from them."""
    rng = np.random.default_rng(40 + seed)
    S, s, w, k = 160, 3, 9, 17
    gap = 1.25 * lam + 0.25
    pi = rng.permutation(S).astype(np.float64) * gap
    y = (pi - (lam / delta) * np.arange(S)).astype(np.float32)
    lab, bnd = teacher.teacher_bruteforce(y, s, w, k, lam=lam, delta=delta)
    lab2, bnd2, _, _ = teacher.teacher_static(y, s, w, k, lam=lam, delta=delta)
    assert np.array_equal(lab, lab2) and np.array_equal(bnd, bnd2)


@pytest.mark.parametrize("delta,k,label_differs", [(4, 2, True), (16, 7, True), (16, 13, False), (4, 12, False)])
def test_static_departure_is_confined_to_one_decay_step(delta, k, label_differs):
    """Equal targets, Delta > 1: the floor form ties every token of one
    decay step (ties to the lower index), while the static priorities
    lambda t / Delta put the newest first.  Both keep min(k, |E_d|) tokens,
    and the kept sets differ only inside the decay step of the floor form's
    boundary token; the boundary tokens themselves lie in that step.  Every
    query where the labels differ is recorded and checked against this: the
    newly eligible token d-w is the newest of its step, so the labels differ
    exactly when the top-k ends inside d-w's own step."""
    S, s, w, lam = 120, 2, 5, 0.5
    y = np.zeros(S, dtype=np.float32)
    lab, bnd = teacher.teacher_bruteforce(y, s, w, k, lam=lam, delta=delta)
    lab2, bnd2, _, _ = teacher.teacher_static(y, s, w, k, lam=lam, delta=delta)
    differ = []
    for d in range(S):
        if d - w < s:
            assert lab[d] == lab2[d] == -1
            continue
        ex = _kept_exact(y, d, s, w, k, lam, delta)
        st_kept = sorted(range(s, d - w + 1), key=lambda t: -t)[:k]   # newest first
        assert len(ex) == len(st_kept) == min(k, d - w - s + 1)
        step = lambda t: (d - t) // delta
        bstep = step(ex[-1])
        assert step(bnd2[d]) == bstep == step(bnd[d])
        for t in set(ex) ^ set(st_kept):
            assert step(t) == bstep, (d, t)
        if lab[d] != lab2[d]:
            differ.append(d)
            assert step(d - w) == bstep
    assert bool(differ) == label_differs, differ


@pytest.mark.parametrize("seed", range(4))
def test_static_departure_bound_on_random_targets(seed):
    """For any targets: whenever the floor form keeps a token a that the
    static form drops in favour of b, their static priorities are within
    lambda (Delta-1)/Delta (plus float32 rounding) of each other, i.e. only
    near-ties can swap."""
    rng = np.random.default_rng(70 + seed)
    S, s, w, k, lam, delta = 140, 2, 6, 13, 0.8, 16
    y = rng.standard_normal(S).astype(np.float32)
    pri = teacher.static_priorities(y, lam, delta).astype(np.float64)
    bound = lam * (delta - 1) / delta + 1e-5
    for d in range(s + w, S):
        ex = set(_kept_exact(y, d, s, w, k, lam, delta))
        toks = list(range(s, d - w + 1))
        st_kept = set(sorted(toks, key=lambda t: (-pri[t], t))[:k])
        for a in ex - st_kept:
            for b in st_kept - ex:
                assert abs(pri[a] - pri[b]) <= bound, (d, a, b, pri[a] - pri[b])
