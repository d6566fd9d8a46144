"""Pins for the budget-mask oracle (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import budget, dense

GOLD = os.path.join(os.path.dirname(__file__), "golden", "budget_mask_hand.json")


def _cut(x):
    return budget.CUTOFF_ALL if x == "ALL" else (budget.CUTOFF_NONE if x == "NONE" else int(x))


def test_hand_worked_examples():
    """Rows, ranks and cutoffs derived by hand from the pages' definitions."""
    cases = json.load(open(GOLD))["cases"]
    for c in cases:
        sc = np.array(c["scores"], dtype=np.float64)
        S = sc.shape[0]
        rank = budget.static_ranks(sc)
        assert rank.tolist() == c["rank"], c["name"]
        cut = budget.running_cutoffs(rank, c["sinks"], c["window"], c["topk"])
        assert cut.tolist() == [_cut(x) for x in c["cutoff"]], c["name"]
        rows = budget.mask_rows(rank, cut, c["sinks"], c["window"], np.arange(S))
        for d in range(S):
            assert np.nonzero(rows[d])[0].tolist() == c["rows"][d], (c["name"], d)
            assert np.nonzero(budget.brute_mask_row(sc, d, c["sinks"], c["window"], c["topk"]))[0].tolist() \
                == c["rows"][d]


@settings(max_examples=60, deadline=None)
@given(S=st.integers(1, 120), s=st.integers(0, 6), w=st.integers(0, 20), k=st.integers(0, 40),
       ties=st.booleans(), seed=st.integers(0, 100000))
def test_fenwick_sweep_equals_per_row_selection(S, s, w, k, ties, seed):
    r = np.random.default_rng(seed)
    sc = r.integers(-3, 3, size=S).astype(np.float64) if ties else r.standard_normal(S)
    if ties:
        sc[r.random(S) < 0.3] = -0.0
    rank = budget.static_ranks(sc)
    assert sorted(rank.tolist()) == list(range(S))
    cut = budget.running_cutoffs(rank, s, w, k)
    rows = budget.mask_rows(rank, cut, s, w, np.arange(S))
    for d in range(S):
        assert np.array_equal(rows[d], budget.brute_mask_row(sc, d, s, w, k)), d


@pytest.mark.parametrize("s,w,k", [(4, 16, 30), (0, 1, 5), (2, 0, 7)])
def test_invariants(s, w, k):
    S = 300
    sc = np.random.default_rng(1).standard_normal(S)
    rank = budget.static_ranks(sc)
    cut = budget.running_cutoffs(rank, s, w, k)
    rows = budget.mask_rows(rank, cut, s, w, np.arange(S))
    B = s + w + k
    for d in range(S):
        assert rows[d].sum() == min(d + 1, B)
        if d + 1 < S:
            diff = np.logical_xor(rows[d], rows[d + 1])
            assert diff.sum() <= 2
            if w >= 1:                          # the newest token sits in the window
                assert rows[d + 1][d + 1]
    real = cut[(cut != budget.CUTOFF_ALL)]
    assert np.all(np.diff(real) <= 0)          # the cutoff only falls as d grows
    for t in range(S):                          # each column is one interval of d
        col = np.nonzero(rows[:, t])[0]
        if col.size:
            assert col[0] == t and np.all(np.diff(col) == 1)


@pytest.mark.parametrize("S,s,w,k", [(50, 3, 5, 7), (64, 0, 8, 8)])
def test_monotone_scores_closed_forms(S, s, w, k):
    d = np.arange(S)
    # strictly decreasing (and all-equal) scores: keep [0, s+k) and the window
    for sc in (np.linspace(5, -5, S), np.zeros(S)):
        rank = budget.static_ranks(sc)
        rows = budget.mask_rows(rank, budget.running_cutoffs(rank, s, w, k), s, w, d)
        for q in range(S):
            t = np.arange(S)
            expect = (t <= q) & ((t < s + k) | (t > q - w))
            assert np.array_equal(rows[q], expect)
    # strictly increasing: sinks plus a sliding window of w + k tokens
    sc = np.linspace(-5, 5, S)
    rank = budget.static_ranks(sc)
    rows = budget.mask_rows(rank, budget.running_cutoffs(rank, s, w, k), s, w, d)
    for q in range(S):
        t = np.arange(S)
        expect = (t <= q) & ((t < s) | (t > q - w - k))
        assert np.array_equal(rows[q], expect)


def test_full_budget_equals_dense_causal():
    """S <= B: the mask is the full causal mask, so masked attention equals
    the dense causal oracle."""
    B_, Hq, Hkv, S, D = 1, 4, 2, 40, 8
    r = np.random.default_rng(3)
    q, k, v = (r.standard_normal((B_, Hq, S, D)), r.standard_normal((B_, Hkv, S, D)),
               r.standard_normal((B_, Hkv, S, D)))
    sc = r.standard_normal((B_, Hkv, S))
    rank, cut = budget.budget_reference(sc, 2, 10, 28)
    o, l = budget.masked_attention(q, k, v, rank, cut, 2, 10)
    ref = dense.attention_pass(q, k, v)
    assert np.allclose(o, ref["out"], atol=1e-12)
    assert np.allclose(l, ref["lse"], atol=1e-12)


def test_masked_attention_against_sdpa_with_bool_mask():
    B_, Hq, Hkv, S, D = 1, 4, 2, 90, 16
    r = np.random.default_rng(8)
    q, k, v = (r.standard_normal((B_, Hq, S, D)), r.standard_normal((B_, Hkv, S, D)),
               r.standard_normal((B_, Hkv, S, D)))
    sc = r.standard_normal((B_, Hkv, S))
    s_, w_, k_ = 2, 6, 9
    rank, cut = budget.budget_reference(sc, s_, w_, k_)
    o, l = budget.masked_attention(q, k, v, rank, cut, s_, w_, row_block=16)
    G = Hq // Hkv
    for g in range(Hq):
        h = g // G
        M = torch.from_numpy(np.stack([budget.brute_mask_row(sc[0, h], d, s_, w_, k_) for d in range(S)]))
        qq, kk, vv = (torch.from_numpy(x) for x in (q[0, g], k[0, h], v[0, h]))
        ref = torch.nn.functional.scaled_dot_product_attention(qq[None], kk[None], vv[None], attn_mask=M[None])[0]
        assert np.allclose(o[0, g], ref.numpy(), atol=1e-12)
        logits = (qq @ kk.T) / math.sqrt(D)
        lse = torch.logsumexp(logits.masked_fill(~M, float("-inf")), dim=-1)
        assert np.allclose(l[0, g], lse.numpy(), atol=1e-12)


def test_empty_budget_rows():
    """s = w = k = 0 keeps nothing: L = -inf and O = 0."""
    B_, Hq, Hkv, S, D = 1, 1, 1, 8, 4
    r = np.random.default_rng(0)
    q, k, v = (r.standard_normal((B_, Hq, S, D)), r.standard_normal((B_, Hkv, S, D)),
               r.standard_normal((B_, Hkv, S, D)))
    rank, cut = budget.budget_reference(r.standard_normal((1, 1, S)), 0, 0, 0)
    o, l = budget.masked_attention(q, k, v, rank, cut, 0, 0)
    assert np.all(np.isneginf(l)) and np.all(o == 0)


def test_nan_scores_rank_last():
    sc = np.array([np.nan, 1.0, -np.inf, 0.5, np.nan])
    assert budget.static_ranks(sc).tolist() == [2, 0, 3, 1, 4]


# ---------------------------------------------------------------- packed sequences
def _rand_cu(S, n_docs, r):
    if n_docs <= 1 or S < 2:
        return None
    cuts = sorted(r.choice(np.arange(1, S), size=min(n_docs - 1, S - 1), replace=False).tolist())
    return [0] + cuts + [S]


@settings(max_examples=60, deadline=None)
@given(S=st.integers(1, 120), docs=st.integers(1, 6), s=st.integers(0, 5), w=st.integers(0, 20),
       k=st.integers(0, 30), ties=st.booleans(), seed=st.integers(0, 100000))
def test_packed_sweep_equals_per_row_selection(S, docs, s, w, k, ties, seed):
    """With documents, the sweep over global ranks that restarts at every
    document gives, row by row, the per-row definition inside the row's
    document (its own sinks, window and top-k)."""
    r = np.random.default_rng(seed)
    sc = r.integers(-3, 3, size=S).astype(np.float64) if ties else r.standard_normal(S)
    cu = _rand_cu(S, docs, r)
    rank = budget.static_ranks(sc)
    cut = budget.running_cutoffs(rank, s, w, k, cu=cu)
    rows = budget.mask_rows(rank, cut, s, w, np.arange(S), cu=cu)
    for d in range(S):
        assert np.array_equal(rows[d], budget.brute_mask_row(sc, d, s, w, k, cu=cu)), d


@pytest.mark.parametrize("cu,s,w,k", [([0, 30, 47, 120], 3, 5, 9), ([0, 1, 2, 60, 61, 90], 2, 4, 6),
                                      ([0, 64, 128], 0, 8, 20), ([0, 10, 90], 4, 0, 12)])
def test_packed_equals_documents_alone(cu, s, w, k):
    """Each document of a packed sequence gets exactly the mask, the output
    and the LSE it gets when run alone (its own ranks, cutoffs and
    positions from 0); rows of a packed sequence never reach another
    document."""
    S = cu[-1]
    r = np.random.default_rng(sum(cu) + s + w + k)
    sc = r.integers(-4, 4, size=(1, 1, S)).astype(np.float64)
    Hq, D = 2, 8
    q, kk, v = r.standard_normal((1, Hq, S, D)), r.standard_normal((1, 1, S, D)), r.standard_normal((1, 1, S, D))
    rank, cut = budget.budget_reference(sc, s, w, k, cu=cu)
    rows = budget.mask_rows(rank[0, 0], cut[0, 0], s, w, np.arange(S), cu=cu)
    o, l = budget.masked_attention(q, kk, v, rank, cut, s, w, cu=cu, row_block=7)
    for a, b in zip(cu[:-1], cu[1:]):
        ra, ca = budget.budget_reference(sc[:, :, a:b], s, w, k)
        alone = budget.mask_rows(ra[0, 0], ca[0, 0], s, w, np.arange(b - a))
        assert not rows[a:b, :a].any() and not rows[a:b, b:].any()
        assert np.array_equal(rows[a:b, a:b], alone)
        oa, la = budget.masked_attention(q[:, :, a:b], kk[:, :, a:b], v[:, :, a:b], ra, ca, s, w)
        assert np.allclose(o[:, :, a:b], oa, atol=1e-12) and np.allclose(l[:, :, a:b], la, atol=1e-12)
        # row size: min(pos + 1, s + w + k) inside each document
        assert np.array_equal(rows[a:b].sum(axis=1), np.minimum(np.arange(b - a) + 1, s + w + k))
