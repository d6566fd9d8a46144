"""GPU parity of the fixed-budget sparse forward: ranks and cutoffs
bit-exact against the oracle's sort and Fenwick sweep; output and LSE within
tolerance of the oracle's masked attention.  Runs on an MI355X."""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import budget, dense
from tests.parity import assert_lse_close, assert_out_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ws_int32(ws_cpu, offset, n):
    return ws_cpu[offset: offset + 4 * n].view(torch.int32).numpy()


def check_lists(kv, q, k, s, w, topk, ws, r_rank, r_cut, cu=None):
    """The key lists the sparse forward gathered, read back from its
    workspace, against the oracle's mask rows, for every query block of every
    (batch row, KV head):
      * status 0: nothing dropped at the capacity, shared count as laid out;
      * no key listed twice, and the listed set is the union of the block's
        mask rows (every key some query keeps), plus, with a zero window
        only, positions inside the block that no query keeps (the list
        covers the block's own positions whole; the mask drops them);
      * the shared segment (attended without a mask in whole tiles) is
        exactly the keys every query of the block keeps, outside the
        positions (d0-w, d1-w], which are masked per query instead;
      * the span [lo, hi) of every key in a masked tile (from the last
        whole tile of the shared segment on) holds exactly the block's
        queries whose mask row keeps it, and the padding to whole tiles is
        position S, kept by no query."""
    lay = kv.budget_lists_layout(q, k, s, w, topk, cu_seqlens=cu)
    B, Hkv, S = r_rank.shape
    nqb, QB, cap = lay["n_query_blocks"], lay["query_block"], lay["capacity"]
    wsc = ws.cpu()
    lists = ws_int32(wsc, lay["lists_offset"], B * Hkv * nqb * cap).reshape(B * Hkv, nqb, cap)
    spans = ws_int32(wsc, lay["spans_offset"], 2 * B * Hkv * nqb * cap).reshape(B * Hkv, nqb, cap, 2)
    KT = lay["tile_keys"]
    lens = ws_int32(wsc, lay["lens_offset"], B * Hkv * nqb).reshape(B * Hkv, nqb)
    lens_full = ws_int32(wsc, lay["lens_full_offset"], B * Hkv * nqb).reshape(B * Hkv, nqb)
    status = ws_int32(wsc, lay["status_offset"], B * Hkv * nqb).reshape(B * Hkv, nqb)
    assert np.all(status == 0), f"list status set for {np.count_nonzero(status)} blocks"
    assert np.all(lens <= cap) and np.all(lens_full <= lens)
    for bh in range(B * Hkv):
        b, h = divmod(bh, Hkv)
        rk, ct = r_rank[b, h], r_cut[b, h]
        for qb in range(nqb):
            d0, d1 = qb * QB, min(S - 1, qb * QB + QB - 1)
            rows = budget.mask_rows(rk[:d1 + 1], ct, s, w, np.arange(d0, d1 + 1), cu=cu)
            lst = lists[bh, qb, :lens[bh, qb]]
            assert np.unique(lst).size == lst.size, (bh, qb, "duplicate keys")
            union = np.nonzero(rows.any(axis=0))[0]
            extra = np.setdiff1d(lst, union)
            assert np.setdiff1d(union, lst).size == 0, (bh, qb, "kept keys missing from the list")
            assert extra.size == 0 or (w == 0 and np.all((extra > d0) & (extra <= d1))), (bh, qb, "listed set")
            t = np.arange(d1 + 1)
            shared = rows.all(axis=0) & ((t <= d0 - w) | (t > d1 - w))
            full = lists[bh, qb, :lens_full[bh, qb]]
            assert np.array_equal(np.sort(full), np.nonzero(shared)[0]), (bh, qb, "shared segment")
            n = lens[bh, qb]
            j0 = lens_full[bh, qb] // KT * KT
            sp = spans[bh, qb, j0:n]
            d = np.arange(d0, d1 + 1)[:, None]
            by_span = (d >= sp[None, :, 0]) & (d < sp[None, :, 1])
            assert np.array_equal(by_span, rows[:, lst[j0:]]), (bh, qb, "spans")
            n_pad = -(-n // KT) * KT
            assert np.all(lists[bh, qb, n:n_pad] == S), (bh, qb, "padding")
            assert np.all(spans[bh, qb, n:n_pad, 0] == 2 ** 31 - 1), (bh, qb, "padding spans")


def check_budget(kv, q, k, v, scores, s, w, topk, heads=None, rows=None, cu=None):
    """cu: None, or the document offsets as a list (batch 1)."""
    cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int32)
    need = kv.workspace_size(kv.CALL_BUDGET_MASK_FWD, q, k, cu_seqlens=cu_t, sinks=s, window=w, topk=topk)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    o, lse, rank, cut = kv.budget_mask_fwd(q, k, v, scores, s, w, topk, workspace=ws, cu_seqlens=cu_t)
    torch.cuda.synchronize()
    r_rank, r_cut = budget.budget_reference(scores.cpu().numpy(), s, w, topk, cu=cu)
    assert np.array_equal(rank.cpu().numpy(), r_rank), "ranks differ"
    assert np.array_equal(cut.cpu().numpy(), r_cut), "cutoffs differ"
    check_lists(kv, q, k, s, w, topk, ws, r_rank, r_cut, cu=cu)
    ro, rl = budget.masked_attention(dense.to_f64(q), dense.to_f64(k), dense.to_f64(v), r_rank, r_cut, s, w,
                                     heads=heads, rows=rows, cu=cu)
    if heads is None:
        heads = [(b, g) for b in range(q.shape[0]) for g in range(q.shape[1])]
    rr = np.arange(q.shape[2]) if rows is None else np.asarray(sorted(set(int(x) for x in rows)))
    for (b, g) in heads:
        assert_lse_close(lse[b, g, rr], rl[b, g, rr], what=f"lse b{b} g{g}")
        ref_o = ro[b, g, rr]
        if np.all(ref_o == 0):
            assert torch.all(o[b, g, rr].float() == 0)
        else:
            assert_out_close(o[b, g, rr], ref_o, what=f"out b{b} g{g}")
    return o, lse, rank, cut


SMALL = [
    # S, Hq, Hkv, D, dtype, s, w, k, score kind
    (300, 4, 1, 128, "bf16", 4, 16, 40, "normal"),
    (700, 8, 2, 128, "bf16", 2, 64, 100, "ties"),
    (513, 4, 4, 64, "bf16", 0, 1, 7, "normal"),
    (450, 2, 1, 128, "bf16", 3, 0, 30, "normal"),
    (260, 4, 1, 128, "bf16", 4, 8, 0, "normal"),       # k = 0: sinks and window only
    (200, 4, 1, 128, "bf16", 8, 64, 150, "normal"),    # S <= B: full causal
    (333, 4, 1, 64, "f32", 2, 9, 20, "normal"),
    (2500, 4, 1, 128, "bf16", 4, 128, 300, "decreasing"),
    (2500, 4, 1, 128, "bf16", 4, 128, 300, "increasing"),
    (640, 6, 2, 128, "bf16", 4, 32, 90, "normal"),     # G = 3: 128-query blocks, three per KV head
    (520, 12, 2, 64, "bf16", 2, 16, 60, "ties"),       # G = 6: 64-query blocks, three per KV head
    (600, 16, 2, 128, "bf16", 4, 32, 90, "normal"),    # G = 8: 32-query blocks, two per KV head
    (450, 5, 1, 64, "bf16", 2, 16, 40, "ties"),        # G = 5: 128-query blocks, five per KV head
]


@pytest.mark.parametrize("S,Hq,Hkv,D,dt,s,w,kk,kind", SMALL)
def test_budget_small(kvpop_lib, S, Hq, Hkv, D, dt, s, w, kk, kind):
    say(f"budget S={S} Hq={Hq} Hkv={Hkv} D={D} {dt} s={s} w={w} k={kk} {kind}")
    t = synth.make_qkv(1, S, Hq, Hkv, D, dt, 1000 + S + kk, device=DEV, with_scores=True)
    sc = t["scores"]
    if kind == "ties":
        sc = torch.round(sc * 2) / 2
        sc[sc == 0] = -0.0
    elif kind == "decreasing":
        sc = torch.linspace(3, -3, S, device=DEV).expand(1, Hkv, S).contiguous()
    elif kind == "increasing":
        sc = torch.linspace(-3, 3, S, device=DEV).expand(1, Hkv, S).contiguous()
    check_budget(kvpop_lib, t["q"], t["k"], t["v"], sc.contiguous(), s, w, kk)


@pytest.mark.parametrize("kind", ["rising", "jumps", "negative"])
def test_budget_running_maximum(kvpop_lib, kind):
    """The sparse forward on logit sequences that steer its running maximum
    (see the dense forward's test of the same name)."""
    S = 1500
    say(f"budget running maximum: {kind}")
    t = synth.make_leveled_qkv(S, 4, 1, 128, "bf16", 21, synth.key_levels(kind, S), device=DEV,
                               with_scores=True)
    check_budget(kvpop_lib, t["q"], t["k"], t["v"], t["scores"], 4, 64, 200)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_budget_batch_of_sequences(kvpop_lib, dt):
    """Three batch rows in one call: each row's ranks and cutoffs come from its
    own scores, and its output from its own keys."""
    say(f"budget batch B=3 {dt}")
    D = 128 if dt == "bf16" else 64    # the fp32 budget forward takes head_dim 64 only
    t = synth.make_qkv(3, 900, 8, 2, D, dt, 55, device=DEV, with_scores=True)
    check_budget(kvpop_lib, t["q"], t["k"], t["v"], t["scores"], 4, 32, 120)


def test_budget_full_causal_equals_dense(kvpop_lib):
    """S <= s + w + k: the budget mask is the full causal mask.  Both paths
    against the oracle's dense attention at the per-row output tolerance, and
    their LSEs within 1e-4 of each other."""
    t = synth.make_qkv(1, 500, 8, 2, 128, "bf16", 3, device=DEV, with_scores=True)
    o, lse, _, _ = kvpop_lib.budget_mask_fwd(t["q"], t["k"], t["v"], t["scores"], 4, 128, 400)
    od, ld = kvpop_lib.attn_fwd_lse(t["q"], t["k"], t["v"])
    torch.cuda.synchronize()
    r = dense.attention_pass(dense.to_f64(t["q"]), dense.to_f64(t["k"]), dense.to_f64(t["v"]))
    assert torch.allclose(lse, ld, atol=1e-4)
    assert_lse_close(lse, r["lse"], what="budget lse")
    assert_out_close(o, r["out"], what="budget out")
    assert_out_close(od, r["out"], what="dense out")


# Q = 0: every logit is 0, so each query's LSE is ln |M_d| and its output the
# mean of V over M_d.  The count pins how many keys the kernel attended for
# every row; the fp32 mean pins which (one key swapped for another moves the
# mean by |v_a - v_b| / |M_d|, ~1e-3 at |M_d| = 2048, against fp32 rounding
# of ~1e-7).
ZERO_Q = [
    # S, Hq, Hkv, D, dtype, s, w, k, score kind
    (700, 8, 2, 128, "bf16", 2, 64, 100, "ties"),
    (2500, 4, 1, 128, "bf16", 4, 128, 300, "normal"),
    (513, 4, 4, 64, "f32", 0, 1, 7, "normal"),
    (1500, 4, 2, 64, "f32", 4, 32, 200, "ties"),
    (900, 4, 1, 64, "f32", 3, 0, 150, "increasing"),
]


def _scores(t, kind, S, Hkv):
    sc = t["scores"]
    if kind == "ties":
        sc = torch.round(sc * 2) / 2
    elif kind == "increasing":
        sc = torch.linspace(-3, 3, S, device=DEV).expand(1, Hkv, S)
    return sc.contiguous()


def check_zero_q(kv, t, sc, s, w, kk, mean_checks=None, cu=None):
    q = torch.zeros_like(t["q"])
    k, v = t["k"], t["v"]
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int32)
    o, lse, rank, cut = kv.budget_mask_fwd(q, k, v, sc, s, w, kk, cu_seqlens=cu_t)
    torch.cuda.synchronize()
    r_rank, r_cut = budget.budget_reference(sc.cpu().numpy(), s, w, kk, cu=cu)
    assert np.array_equal(cut.cpu().numpy(), r_cut)
    count = np.exp(lse.cpu().double().numpy())
    start, _ = dense.doc_bounds(S, cu)
    want = np.minimum(np.arange(S) - start + 1, s + w + kk)   # row size, pinned on the oracle
    # fp32 logarithm: relative error ~1e-6, against 1/|M_d| >= 4.9e-4 for one key more or less
    rel = np.abs(count / want - 1.0)
    assert rel.max() <= 2e-5, f"keys per row: worst relative deviation {rel.max():.3g}"
    if t["q"].dtype == torch.float32:
        # (heads, rows) pairs to compare; default every head on every row
        for heads, mrows in (mean_checks or [([(0, g) for g in range(Hq)], None)]):
            ro, _ = budget.masked_attention(np.zeros((B, Hq, S, D)), dense.to_f64(k), dense.to_f64(v), r_rank,
                                            r_cut, s, w, heads=heads, rows=mrows, cu=cu)
            rr = np.arange(S) if mrows is None else np.asarray(sorted(set(int(x) for x in mrows)))
            for (b, g) in heads:
                err = np.abs(o[b, g, rr].cpu().double().numpy() - ro[b, g, rr]).max()
                assert err <= 1e-5, f"mean of V over the mask: head {g} max |delta| {err:.3g}"


@pytest.mark.parametrize("S,Hq,Hkv,D,dt,s,w,kk,kind", ZERO_Q)
def test_budget_zero_queries_membership(kvpop_lib, S, Hq, Hkv, D, dt, s, w, kk, kind):
    say(f"budget Q=0 S={S} Hq={Hq} Hkv={Hkv} D={D} {dt} s={s} w={w} k={kk} {kind}")
    t = synth.make_qkv(1, S, Hq, Hkv, D, dt, 300 + S, device=DEV, with_scores=True)
    check_zero_q(kvpop_lib, t, _scores(t, kind, S, Hkv), s, w, kk)


def test_budget32k_zero_queries_membership(kvpop_lib):
    """The budget workload's shape (S=32768, 32q/8kv, s=4, w=128, k=1916) with
    Q = 0: every row of every query head attends exactly min(d+1, 2048) keys
    (bf16, D=128); and in fp32 at D=64 the output is the mean of V over
    exactly the oracle's mask: every row of two KV heads' first query heads,
    and 512 rows (first and last 64, 384 random) of one query head of each
    other KV head."""
    t = synth.make_workload("budget32k", device=DEV)
    say("budget32k Q=0 bf16 count")
    check_zero_q(kvpop_lib, t, t["scores"], t["sinks"], t["window"], t["topk"])
    say("budget32k Q=0 fp32 D=64 mean")
    t32 = synth.make_qkv(1, 32768, 32, 8, 64, "f32", 77, device=DEV, with_scores=True)
    rng = np.random.default_rng(1)
    rows = np.concatenate([np.arange(64), np.arange(32768 - 64, 32768), rng.integers(0, 32768, 384)])
    check_zero_q(kvpop_lib, t32, t32["scores"], 4, 128, 1916,
                 mean_checks=[([(0, 0), (0, 20)], None), ([(0, 4 * h + h % 4) for h in (1, 2, 3, 4, 6, 7)], rows)])


def test_budget_empty_rows(kvpop_lib):
    """s = w = k = 0 keeps nothing: LSE -inf and O = 0."""
    t = synth.make_qkv(1, 130, 4, 1, 64, "bf16", 4, device=DEV, with_scores=True)
    o, lse, _, cut = kvpop_lib.budget_mask_fwd(t["q"], t["k"], t["v"], t["scores"], 0, 0, 0)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(lse))
    assert torch.all(o.float() == 0)
    assert torch.all(cut == kvpop_lib.CUTOFF_NONE)


def test_budget32k(kvpop_lib):
    """S=32768, 32q/8kv/128, s=4, w=128, k=1916 (B=2048): ranks and cutoffs of
    every KV head bit-exact; output and LSE of every query head on sampled rows."""
    t = synth.make_workload("budget32k", device=DEV)
    q, k, v, sc = t["q"], t["k"], t["v"], t["scores"]
    rng = np.random.default_rng(0)
    rows = np.concatenate([np.arange(64), np.arange(32768 - 64, 32768), rng.integers(0, 32768, 384)])
    say("budget32k: gpu + oracle")
    check_budget(kvpop_lib, q, k, v, sc, t["sinks"], t["window"], t["topk"],
                 heads=[(0, g) for g in range(32)], rows=rows)


@pytest.mark.parametrize("S,packed", [(40000, False), (36000, True)])
def test_budget_long_sequence(kvpop_lib, S, packed):
    """Past 32768 eligible tokens (S=40000 minus 4 sinks; or packed, where the
    wavelet matrix spans the whole sequence) the wavelet matrix is built by
    the sequential global-memory kernel instead of in LDS.  Ranks, cutoffs
    and the key lists of every block exactly; output and LSE of every query
    head on sampled rows."""
    Hq, Hkv = 4, 1
    cu = [0, 9000, 9100, 30000, S] if packed else None
    say(f"budget long sequence S={S} packed={packed}")
    t = synth.make_qkv(1, S, Hq, Hkv, 128, "bf16", 40 + S, device=DEV, with_scores=True)
    r = np.random.default_rng(S)
    rows = np.concatenate([np.arange(32), np.arange(S - 32, S), r.integers(0, S, 192)])
    if packed:
        rows = np.concatenate([rows, [8999, 9000, 9099, 9100, 29999, 30000]])
    check_budget(kvpop_lib, t["q"], t["k"], t["v"], t["scores"], 4, 128, 1916,
                 heads=[(0, g) for g in range(Hq)], rows=rows, cu=cu)


def test_budget_packed_block_order_limit(kvpop_lib):
    """Packed S=32768 at 4 query heads per KV head: 1024 query blocks per
    head, the most the budget forward still runs in list-length order (one
    more block and it keeps the plain order, as at S=36000 above).  Ranks,
    cutoffs and the key lists of every block exactly; output and LSE of
    every query head on sampled rows."""
    S, Hq, Hkv = 32768, 8, 2
    cu = [0, 700, 13000, 13032, 20000, S]
    say(f"budget packed S={S} docs={np.diff(cu).tolist()} Hq={Hq} Hkv={Hkv}")
    t = synth.make_qkv(1, S, Hq, Hkv, 128, "bf16", 77, device=DEV, with_scores=True)
    r = np.random.default_rng(S + 1)
    rows = np.concatenate([np.arange(32), np.arange(S - 32, S), r.integers(0, S, 128),
                           [699, 700, 12999, 13000, 13031, 13032, 19999, 20000]])
    check_budget(kvpop_lib, t["q"], t["k"], t["v"], t["scores"], 4, 128, 1916,
                 heads=[(0, g) for g in range(Hq)], rows=rows, cu=cu)


# Packed documents: each document keeps what it would keep alone (sinks and
# window counted from its start).  Document lengths include ones shorter
# than a query block (32 positions), than the sinks plus window, and one.
PACKED = [
    # lengths, Hq, Hkv, D, dtype, s, w, k, score kind
    ([700, 300, 1000], 8, 2, 128, "bf16", 4, 64, 100, "normal"),
    ([5, 1, 40, 17, 250, 3, 90, 31, 63], 4, 1, 128, "bf16", 2, 16, 20, "ties"),
    ([1200, 1300], 4, 2, 64, "f32", 3, 32, 150, "normal"),
    ([333, 200, 480], 4, 1, 128, "bf16", 0, 0, 40, "normal"),
    ([900, 100, 1000], 4, 1, 128, "bf16", 4, 128, 300, "increasing"),
]


def _cu(lengths):
    return [0] + np.cumsum(lengths).tolist()


@pytest.mark.parametrize("lengths,Hq,Hkv,D,dt,s,w,kk,kind", PACKED)
def test_budget_packed(kvpop_lib, lengths, Hq, Hkv, D, dt, s, w, kk, kind):
    S = sum(lengths)
    say(f"budget packed docs={lengths} Hq={Hq} Hkv={Hkv} D={D} {dt} s={s} w={w} k={kk} {kind}")
    t = synth.make_qkv(1, S, Hq, Hkv, D, dt, 500 + S + kk, device=DEV, with_scores=True)
    check_budget(kvpop_lib, t["q"], t["k"], t["v"], _scores(t, kind, S, Hkv), s, w, kk, cu=_cu(lengths))


@pytest.mark.parametrize("lengths,dt", [([700, 300, 1000], "bf16"), ([5, 1, 40, 17, 250, 3, 90, 31, 63], "f32"),
                                        ([1200, 1300], "f32")])
def test_budget_packed_zero_queries_membership(kvpop_lib, lengths, dt):
    S = sum(lengths)
    say(f"budget packed Q=0 docs={lengths} {dt}")
    D = 128 if dt == "bf16" else 64
    t = synth.make_qkv(1, S, 8, 2, D, dt, 600 + S, device=DEV, with_scores=True)
    check_zero_q(kvpop_lib, t, _scores(t, "ties", S, 2), 3, 24, 60, cu=_cu(lengths))


def test_budget_packed16k(kvpop_lib):
    """The pages' training shape: S=16384 packed as 6 documents, 32q/8kv/128,
    with the budget s=4, w=128, k=1916: ranks, cutoffs and the key lists of
    every block of every KV head exactly, output and LSE of every query head
    on 512 sampled rows."""
    t = synth.make_workload("packed16k", device=DEV)
    cu = t["cu_seqlens"].tolist()
    g = torch.Generator(device=DEV).manual_seed(16)
    sc = torch.randn(1, 8, 16384, generator=g, device=DEV)
    rng = np.random.default_rng(2)
    rows = np.concatenate([np.arange(64), np.arange(16384 - 64, 16384), rng.integers(0, 16384, 384)])
    say("budget packed16k docs", synth.doc_lengths_of(t["cu_seqlens"], 16384))
    check_budget(kvpop_lib, t["q"], t["k"], t["v"], sc, 4, 128, 1916, heads=[(0, g_) for g_ in range(32)],
                 rows=rows, cu=cu)


def test_budget_mask_alone(kvpop_lib):
    """With no outputs the call builds the mask alone: the same ranks,
    cutoffs, list status and key lists as the whole call, packed or not."""
    kv = kvpop_lib
    for cu in (None, [0, 700, 1000, 2000]):
        t = synth.make_qkv(1, 2000, 8, 2, 128, "bf16", 71, device=DEV, with_scores=True)
        q, k, v, sc = t["q"], t["k"], t["v"], t["scores"]
        cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int32)
        need = kv.workspace_size(kv.CALL_BUDGET_MASK_FWD, q, k, cu_seqlens=cu_t, sinks=4, window=64, topk=300)
        ws1 = torch.zeros(need, dtype=torch.uint8, device=DEV)
        ws2 = torch.zeros(need, dtype=torch.uint8, device=DEV)
        _, _, r1, c1 = kv.budget_mask_fwd(q, k, v, sc, 4, 64, 300, workspace=ws1, cu_seqlens=cu_t)
        o2, l2, r2, c2 = kv.budget_mask_fwd(q, k, v, sc, 4, 64, 300, workspace=ws2, cu_seqlens=cu_t,
                                            need_output=False)
        torch.cuda.synchronize()
        assert o2 is None and l2 is None
        assert torch.equal(r1, r2) and torch.equal(c1, c2)
        lay = kv.budget_lists_layout(q, k, 4, 64, 300, cu_seqlens=cu_t)
        a, b = lay["lists_offset"], lay["status_offset"] + 4 * 2 * lay["n_query_blocks"]
        assert torch.equal(ws1[a:b], ws2[a:b]), "lists differ"
