"""Pins for the dense oracle (CPU only).

Each test ties the oracle to something other than itself: a pure-Python
brute force, a closed form, a library routine, the pages' own transposed
construction (Eq. 8), or an invariant of the definitions.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import brute, dense
from oracle.dense import AGG_MAX, AGG_NONE, AGG_SUM

rng = np.random.default_rng(1234)


def rand_problem(B, Hq, Hkv, S, D, seed, scale_k=1.0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, S, D))
    k = r.standard_normal((B, Hkv, S, D)) * scale_k
    v = r.standard_normal((B, Hkv, S, D))
    return q, k, v


def rand_cu(S, n_docs, seed):
    if n_docs <= 1:
        return None
    r = np.random.default_rng(seed)
    cuts = sorted(r.choice(np.arange(1, S), size=n_docs - 1, replace=False).tolist())
    return [0] + cuts + [S]


def harmonic(n):
    return math.fsum(1.0 / i for i in range(1, n + 1))


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("S,docs,w", [(40, 1, 0), (40, 1, 5), (64, 3, 4), (33, 2, 40)])
def test_zero_queries_closed_form(S, docs, w):
    """Q = 0 makes every logit 0: a_{d,t} = 1/(pos(d)+1), L_d = ln(pos(d)+1),
    and the column mass of key t is H_n - H_{pos(t)+w} (harmonic numbers) for
    a document of length n."""
    B, Hq, Hkv, D = 1, 4, 2, 8
    _, k, v = rand_problem(B, Hq, Hkv, S, D, 7)
    q = np.zeros((B, Hq, S, D))
    cu = rand_cu(S, docs, 3)
    r = dense.attention_pass(q, k, v, cu=cu, window=w)
    start, end = dense.doc_bounds(S, cu)
    for t in range(S):
        pos = t - start[t]
        n = end[t] - start[t]
        assert np.allclose(r["lse"][0, :, t], math.log(pos + 1), atol=1e-13)
        expect = harmonic(n) - harmonic(min(n, pos + w)) if pos + w < n else 0.0
        assert np.allclose(r["colmass"][0, :, t], expect, atol=1e-12), (t, expect)
    # SUM over the G = 2 identical heads adds ln 2; MAX with the mean gives ln(mean + eps)
    tsum = dense.target_from_colmass(r["colmass"], Hkv, cu, w, AGG_SUM)
    tnone = dense.target_from_colmass(r["colmass"], Hkv, cu, w, AGG_NONE)
    fin = np.isfinite(tnone[0, 0])
    assert np.allclose(tsum[0, 0][fin], tnone[0, 0][fin] + math.log(2), atol=1e-12)
    eps = 1e-6
    tmax = dense.target_from_colmass(r["colmass"], Hkv, cu, w, AGG_MAX, True, eps)
    N = dense.future_count(S, cu, w)
    for t in range(S):
        cm = r["colmass"][0, 0, t]
        expect = math.log((cm / N[t] if N[t] > 0 else 0.0) + eps)
        assert abs(tmax[0, 0, t] - expect) < 1e-12


# ---------------------------------------------------------------- brute force
@settings(max_examples=25, deadline=None)
@given(S=st.integers(1, 24), D=st.sampled_from([2, 4]), G=st.sampled_from([1, 2]),
       docs=st.integers(1, 3), w=st.integers(0, 26), seed=st.integers(0, 10_000))
def test_against_brute_force(S, D, G, docs, w, seed):
    Hkv = 1
    q, k, v = rand_problem(1, G * Hkv, Hkv, S, D, seed, scale_k=1.5)
    cu = rand_cu(S, min(docs, S), seed + 1)
    r = dense.attention_pass(q, k, v, cu=cu, window=w, row_block=5)
    bl, bo, bc = brute.brute_attention(q.tolist(), k.tolist(), v.tolist(), cu=cu, window=w)
    assert np.allclose(r["lse"], np.array(bl), rtol=1e-12, atol=1e-12)
    assert np.allclose(r["out"], np.array(bo), rtol=1e-11, atol=1e-12)
    assert np.allclose(r["colmass"], np.array(bc), rtol=1e-11, atol=1e-14)


@settings(max_examples=20, deadline=None)
@given(S=st.integers(1, 24), D=st.sampled_from([2, 4]), G=st.sampled_from([1, 2]),
       docs=st.integers(1, 3), w=st.integers(0, 26), seed=st.integers(0, 10_000))
def test_row_and_key_subsets_against_brute_force(S, D, G, docs, w, seed):
    """The subset forms used for long sequences: row_lse on a few query rows,
    and transposed_lse on a few keys fed with the dense L (ln of the column
    mass by Eq. 8), against the pure-Python double sums; other entries NaN."""
    q, k, v = rand_problem(1, G, 1, S, D, seed, scale_k=1.5)
    cu = rand_cu(S, min(docs, S), seed + 1)
    bl, _, bc = brute.brute_attention(q.tolist(), k.tolist(), v.tolist(), cu=cu, window=w)
    bl = np.array(bl)
    r = np.random.default_rng(seed)
    rows = r.choice(S, size=min(S, 5), replace=False)
    got = dense.row_lse(q, k, rows, cu=cu)
    assert np.allclose(got[:, :, rows], bl[:, :, rows], rtol=1e-12, atol=1e-12)
    assert np.all(np.isnan(np.delete(got, rows, axis=2)))
    keys = r.choice(S, size=min(S, 5), replace=False)
    tl = dense.transposed_lse(q, k, bl, cu=cu, window=w, keys=keys)
    with np.errstate(divide="ignore"):
        want = np.log(np.array(bc))
    assert np.allclose(tl[:, :, keys], want[:, :, keys], rtol=1e-11, atol=1e-12)
    assert np.all(np.isnan(np.delete(tl, keys, axis=2)))


# ---------------------------------------------------------------- library routine
@pytest.mark.parametrize("docs", [1, 3])
def test_against_torch_sdpa(docs):
    """torch's scaled_dot_product_attention in float64 with the same
    block-diagonal causal mask gives O; torch.logsumexp of the masked logits
    gives L."""
    B, Hq, Hkv, S, D = 1, 4, 2, 96, 16
    q, k, v = rand_problem(B, Hq, Hkv, S, D, 11)
    cu = rand_cu(S, docs, 5)
    r = dense.attention_pass(q, k, v, cu=cu, window=0, row_block=17)
    start, _ = dense.doc_bounds(S, cu)
    t = torch.arange(S)
    mask = (t[None, :] <= t[:, None]) & (t[None, :] >= torch.from_numpy(start)[:, None])
    G = Hq // Hkv
    kk = torch.from_numpy(k).repeat_interleave(G, dim=1)
    vv = torch.from_numpy(v).repeat_interleave(G, dim=1)
    qq = torch.from_numpy(q)
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)
    assert np.allclose(r["out"], o.numpy(), atol=1e-12)
    logits = (qq @ kk.transpose(-1, -2)) / math.sqrt(D)
    lse = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1)
    assert np.allclose(r["lse"], lse.numpy(), atol=1e-12)


# ---------------------------------------------------------------- Eq. 8 (pages' construction)
@pytest.mark.parametrize("docs,w", [(1, 0), (1, 7), (4, 3), (2, 100)])
def test_transposed_formulation_eq8(docs, w):
    """[P] Section 3.2: the column reduction equals the LSE of the transposed
    attention call (keys as queries, score modifier -L_d, mask d >= t + w)."""
    B, Hq, Hkv, S, D = 2 if docs == 1 else 1, 4, 2, 80, 8
    q, k, v = rand_problem(B, Hq, Hkv, S, D, 21)
    cu = rand_cu(S, docs, 9)
    r = dense.attention_pass(q, k, v, cu=cu, window=w, row_block=13)
    tl = dense.transposed_lse(q, k, r["lse"], cu=cu, window=w, key_block=11)
    with np.errstate(divide="ignore"):
        lc = np.log(r["colmass"])
    assert np.array_equal(np.isneginf(lc), np.isneginf(tl))
    fin = np.isfinite(lc)
    assert np.allclose(lc[fin], tl[fin], atol=1e-10)


def test_transposed_with_external_lse():
    """With an arbitrary normaliser passed in (the sparse-LSE approximation,
    [P] Section 3.2) both formulations still agree."""
    B, Hq, Hkv, S, D = 1, 2, 1, 50, 8
    q, k, v = rand_problem(B, Hq, Hkv, S, D, 2)
    L = np.random.default_rng(4).uniform(0.0, 3.0, size=(B, Hq, S))
    r = dense.attention_pass(q, k, None, window=2, lse_in=L, need_output=False)
    tl = dense.transposed_lse(q, k, L, window=2)
    with np.errstate(divide="ignore"):
        lc = np.log(r["colmass"])
    fin = np.isfinite(lc)
    assert np.array_equal(fin, np.isfinite(tl))
    assert np.allclose(lc[fin], tl[fin], atol=1e-10)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("docs", [1, 3])
def test_rows_sum_to_one_and_total_mass(docs):
    """Every attention row sums to 1, so at w = 0 the column masses of one
    query head add up to the number of query positions, and the SUM target
    of a group adds up (in exp) to G times that."""
    B, Hq, Hkv, S, D = 1, 4, 1, 70, 8
    q, k, v = rand_problem(B, Hq, Hkv, S, D, 5, scale_k=2.0)
    cu = rand_cu(S, docs, 8)
    ones = np.ones_like(v)
    r = dense.attention_pass(q, k, ones, cu=cu, window=0)
    assert np.allclose(r["out"], 1.0, atol=1e-12)
    assert np.allclose(r["colmass"].sum(axis=-1), S, rtol=1e-12)
    T = dense.target_from_colmass(r["colmass"], Hkv, cu, 0, AGG_SUM)
    assert np.isclose(np.exp(T).sum(), Hq * S, rtol=1e-12)


@pytest.mark.parametrize("docs", [1, 3])
def test_empty_sets_monotone_and_saturation(docs):
    B, Hq, Hkv, S, D = 1, 2, 1, 60, 8
    q, k, v = rand_problem(B, Hq, Hkv, S, D, 6)
    cu = rand_cu(S, docs, 2)
    lengths = np.diff(cu) if cu is not None else [S]
    prev = None
    for w in [0, 1, 5, 17]:
        r = dense.attention_pass(q, k, None, cu=cu, window=w, need_output=False)
        T = dense.target_from_colmass(r["colmass"], Hkv, cu, w, AGG_NONE)
        # number of -inf per head = sum over documents of min(n_doc, w)
        assert np.isneginf(T[0, 0]).sum() == sum(min(int(n), w) for n in lengths)
        if prev is not None:
            fin = np.isfinite(T)
            assert np.all(T[fin] <= prev[fin] + 1e-12)     # fewer queries, less mass
        prev = T
    wmax = int(max(lengths))
    r = dense.attention_pass(q, k, None, cu=cu, window=wmax, need_output=False)
    assert np.all(np.isneginf(dense.target_from_colmass(r["colmass"], Hkv, cu, wmax, AGG_SUM)))


def test_duplicated_heads_sum_equals_none_plus_log_g():
    B, Hkv, G, S, D = 1, 2, 4, 40, 8
    q1, k, v = rand_problem(B, Hkv, Hkv, S, D, 3)
    q = np.repeat(q1, G, axis=1).reshape(B, Hkv * G, S, D)   # heads of a group identical
    r = dense.attention_pass(q, k, None, window=3, need_output=False)
    ts = dense.target_from_colmass(r["colmass"], Hkv, None, 3, AGG_SUM)
    tn = dense.target_from_colmass(r["colmass"], Hkv, None, 3, AGG_NONE)
    tm = dense.target_from_colmass(r["colmass"], Hkv, None, 3, AGG_MAX)
    fin = np.isfinite(ts)
    assert np.allclose(ts[fin], tn[:, ::G][fin] + math.log(G), atol=1e-12)
    assert np.allclose(tm[fin], tn[:, ::G][fin], atol=1e-12)


# ---------------------------------------------------------------- N_t of the mean (Eq. 2)
@settings(max_examples=80, deadline=None)
@given(S=st.integers(1, 40), docs=st.integers(1, 5), w=st.integers(0, 45), seed=st.integers(0, 10_000))
def test_future_count_against_counting(S, docs, w, seed):
    """N_t (the number of future queries the mean of Eq. 2 divides by)
    against an explicit count over all positions, including windows longer
    than a document."""
    cu = rand_cu(S, min(docs, S), seed)
    got = dense.future_count(S, cu, w)
    assert got.tolist() == brute.brute_future_count(S, cu, w)


@pytest.mark.parametrize("S,docs,w", [(40, 1, 0), (40, 1, 5), (64, 3, 4), (33, 2, 40), (50, 4, 13)])
def test_zero_queries_mean_closed_form(S, docs, w):
    """Q = 0 with the mean of Eq. 2: every probability of query d is
    1/(pos(d)+1), so the mean future mass of key t is
    (sum over d in [t+w, docend) of 1/(pos(d)+1)) / len([t+w, docend)),
    written here from the positions alone.  AGG_MAX with eps = 0 gives its
    log (the G heads are identical), -inf for an empty range."""
    B, Hq, Hkv, D = 1, 4, 2, 8
    _, k, v = rand_problem(B, Hq, Hkv, S, D, 9)
    q = np.zeros((B, Hq, S, D))
    cu = rand_cu(S, docs, 4)
    r = dense.attention_pass(q, k, None, cu=cu, window=w, need_output=False)
    got = dense.target_from_colmass(r["colmass"], Hkv, cu, w, AGG_MAX, True, 0.0)
    starts = [0] if cu is None else list(cu[:-1])
    ends = [S] if cu is None else list(cu[1:])
    for t in range(S):
        m = max(i for i in range(len(starts)) if starts[i] <= t)
        ds, de = starts[m], ends[m]
        fut = range(t + w, de)
        if len(fut) == 0:
            assert np.all(np.isneginf(got[0, :, t])), t
            continue
        mean = math.fsum(1.0 / (d - ds + 1) for d in fut) / len(fut)
        assert np.allclose(got[0, :, t], math.log(mean), atol=1e-12), (t, mean)


def test_max_aggregation_matches_per_head_max():
    B, Hq, Hkv, S, D = 1, 4, 2, 50, 8
    q, k, v = rand_problem(B, Hq, Hkv, S, D, 13)
    r = dense.attention_pass(q, k, None, window=4, need_output=False)
    tn = dense.target_from_colmass(r["colmass"], Hkv, None, 4, AGG_NONE, True, 1e-6)
    tm = dense.target_from_colmass(r["colmass"], Hkv, None, 4, AGG_MAX, True, 1e-6)
    assert np.allclose(tm, tn.reshape(B, Hkv, 2, S).max(axis=2))


def test_docs_are_independent():
    """A packed sequence gives the same results as running each document alone."""
    B, Hq, Hkv, S, D = 1, 2, 1, 45, 8
    q, k, v = rand_problem(B, Hq, Hkv, S, D, 17)
    cu = [0, 12, 30, 45]
    r = dense.attention_pass(q, k, v, cu=cu, window=3)
    for a, b in zip(cu[:-1], cu[1:]):
        rs = dense.attention_pass(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], window=3)
        assert np.allclose(r["lse"][..., a:b], rs["lse"], atol=1e-12)
        assert np.allclose(r["out"][:, :, a:b], rs["out"], atol=1e-12)
        assert np.allclose(r["colmass"][..., a:b], rs["colmass"], atol=1e-12)


def test_bf16_inputs_are_upcast_exactly():
    x = torch.randn(3, 5).to(torch.bfloat16)
    y = dense.to_f64(x)
    assert y.dtype == np.float64
    assert np.array_equal(y, x.float().numpy().astype(np.float64))


def test_invalid_cu_rejected():
    with pytest.raises(ValueError):
        dense.doc_bounds(10, [0, 5, 5, 10])
    with pytest.raises(ValueError):
        dense.doc_bounds(10, [0, 5, 9])


def test_transposed_lse_with_sparse_normaliser_matches_brute_force():
    """The paper's training target (Eq. 9): the transposed formulation fed with
    the budget-masked normaliser L~ equals the plain double sum
    ln sum_{d >= t+w} exp(s_{d,t} - L~_d), evaluated term by term in pure
    Python, on a tiny input.  L~ comes from an independent per-row loop over
    the mask rows."""
    import math
    from oracle import budget
    rng = np.random.default_rng(11)
    S, D, s, w, kk = 23, 8, 2, 3, 4
    q = rng.standard_normal((1, 1, S, D))
    k = rng.standard_normal((1, 1, S, D))
    scores = rng.standard_normal((1, 1, S))
    rank, cut = budget.budget_reference(scores, s, w, kk)
    M = budget.mask_rows(rank[0, 0], cut[0, 0], s, w, np.arange(S))
    sc = 1.0 / math.sqrt(D)
    Ls = np.empty(S)
    for d in range(S):
        terms = [sc * float(np.dot(q[0, 0, d], k[0, 0, t])) for t in range(S) if M[d, t]]
        m = max(terms)
        Ls[d] = m + math.log(math.fsum(math.exp(x - m) for x in terms))
    got = dense.transposed_lse(q, k, Ls.reshape(1, 1, S), window=w)
    for t in range(S):
        terms = [sc * float(np.dot(q[0, 0, d], k[0, 0, t])) - Ls[d] for d in range(t + w, S)]
        if not terms:
            assert np.isneginf(got[0, 0, t])
            continue
        want = math.log(math.fsum(math.exp(x) for x in terms))
        assert abs(got[0, 0, t] - want) < 1e-12
