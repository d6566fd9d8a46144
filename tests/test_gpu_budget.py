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


def check_budget(kv, q, k, v, scores, s, w, topk, heads=None, rows=None):
    o, lse, rank, cut = kv.budget_mask_fwd(q, k, v, scores, s, w, topk)
    torch.cuda.synchronize()
    r_rank, r_cut = budget.budget_reference(scores.cpu().numpy(), s, w, topk)
    assert np.array_equal(rank.cpu().numpy(), r_rank), "ranks differ"
    assert np.array_equal(cut.cpu().numpy(), r_cut), "cutoffs differ"
    ro, rl = budget.masked_attention(dense.to_f64(q), dense.to_f64(k), dense.to_f64(v), r_rank, r_cut, s, w,
                                     heads=heads, rows=rows)
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
    """S <= s + w + k: the budget mask is the full causal mask."""
    t = synth.make_qkv(1, 500, 8, 2, 128, "bf16", 3, device=DEV, with_scores=True)
    o, lse, _, _ = kvpop_lib.budget_mask_fwd(t["q"], t["k"], t["v"], t["scores"], 4, 128, 400)
    od, ld = kvpop_lib.attn_fwd_lse(t["q"], t["k"], t["v"])
    torch.cuda.synchronize()
    assert torch.allclose(lse, ld, atol=1e-4)
    assert torch.allclose(o.float(), od.float(), atol=2e-2)


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
