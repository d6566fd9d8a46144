"""GPU parity of fixed-budget decoding (kvpop_decode_init / kvpop_decode_step):
feeding the tokens of a sequence one by one, the output and LSE of every
step's query must equal row d of the oracle's budget-masked attention with
the same static scores (KVpop paper, Section 3 and Section 3.2: the retained
slots at step d are exactly the mask row d).  Tolerances as for the masked
forward: LSE |delta| <= 2e-3, output per row max |delta| <= 2e-2 * RMS.
Runs on an MI355X."""
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


CASES = [
    # S, Hq, Hkv, D, dtype, s, w, k
    (400, 4, 1, 128, "bf16", 4, 32, 50),
    (300, 8, 2, 64, "bf16", 2, 16, 30),
    (200, 4, 2, 128, "bf16", 0, 0, 20),     # no sinks, no window: every token competes at once
    (260, 2, 1, 64, "f32", 3, 8, 0),        # k = 0: sinks and window only
    (150, 4, 1, 128, "bf16", 4, 64, 300),   # budget larger than the sequence: dense causal
    (700, 4, 1, 128, "bf16", 4, 128, 200),  # several attention chunks
    (220, 8, 1, 128, "bf16", 2, 16, 40),    # 8 query heads per KV head
    (180, 3, 3, 64, "f32", 1, 8, 25),       # one query head per KV head
    (240, 6, 2, 128, "bf16", 4, 16, 60),    # 3 query heads per KV head
    (1300, 2, 1, 64, "bf16", 4, 64, 1100),  # ten chunks, the last one ragged
    (300, 2, 1, 64, "bf16", 1, 8, 1),       # one top-k slot: an eviction leaves no other key
    (250, 4, 2, 128, "bf16", 0, 1, 5),      # one-token window: a ring of two slots
    (600, 8, 2, 128, "f32", 4, 32, 150),    # fp32 at head_dim 128, several chunks
    (230, 5, 1, 64, "bf16", 2, 16, 30),     # 5 query heads per KV head
    (260, 12, 2, 128, "bf16", 3, 8, 40),    # 6 query heads per KV head
    (210, 7, 1, 64, "bf16", 1, 4, 90),      # 7 query heads per KV head
]


@pytest.mark.parametrize("S,Hq,Hkv,D,dt,s,w,kk", CASES)
def test_decode_matches_masked_attention(kvpop_lib, S, Hq, Hkv, D, dt, s, w, kk):
    say(f"decode S={S} Hq={Hq} Hkv={Hkv} D={D} {dt} s={s} w={w} k={kk}")
    t = synth.make_qkv(1, S, Hq, Hkv, D, dt, 900 + S, device=DEV, heavy_hitters=True, with_scores=True)
    q, k, v, sc = t["q"], t["k"], t["v"], t["scores"]
    cache = kvpop_lib.DecodeCache(1, Hq, Hkv, D, q.dtype, s, w, kk)
    outs, lses = [], []
    for d in range(S):
        o, l = cache.step(q[:, :, d].contiguous(), k[:, :, d].contiguous(), v[:, :, d].contiguous(),
                          sc[:, :, d].contiguous())
        outs.append(o)
        lses.append(l)
    o = torch.stack(outs, dim=2)
    l = torch.stack(lses, dim=2)
    torch.cuda.synchronize()
    r_rank, r_cut = budget.budget_reference(sc.cpu().numpy(), s, w, kk)
    ro, rl = budget.masked_attention(dense.to_f64(q), dense.to_f64(k), dense.to_f64(v), r_rank, r_cut, s, w)
    assert_lse_close(l, rl, what="decode lse")
    assert_out_close(o, ro, what="decode out")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_batch_of_sequences(kvpop_lib, dt):
    """Three sequences decoded side by side in one cache: each keeps its own
    budget state, so every sequence matches its own masked attention."""
    Bn, S, Hq, Hkv, D, s, w, kk = 3, 500, 8, 2, 128, 2, 24, 90
    say(f"decode batch B={Bn} S={S} {dt}")
    t = synth.make_qkv(Bn, S, Hq, Hkv, D, dt, 77, device=DEV, heavy_hitters=True, with_scores=True)
    q, k, v, sc = t["q"], t["k"], t["v"], t["scores"]
    cache = kvpop_lib.DecodeCache(Bn, Hq, Hkv, D, q.dtype, s, w, kk)
    outs, lses = [], []
    for d in range(S):
        o, l = cache.step(q[:, :, d].contiguous(), k[:, :, d].contiguous(), v[:, :, d].contiguous(),
                          sc[:, :, d].contiguous())
        outs.append(o)
        lses.append(l)
    o = torch.stack(outs, dim=2)
    l = torch.stack(lses, dim=2)
    torch.cuda.synchronize()
    r_rank, r_cut = budget.budget_reference(sc.cpu().numpy(), s, w, kk)
    ro, rl = budget.masked_attention(dense.to_f64(q), dense.to_f64(k), dense.to_f64(v), r_rank, r_cut, s, w)
    assert_lse_close(l, rl, what="decode lse")
    assert_out_close(o, ro, what="decode out")


def test_decode_cache_is_bounded_and_reusable(kvpop_lib):
    """The state size depends on the budget, not on the sequence length, and
    a re-initialised cache reproduces the same outputs bitwise."""
    a = kvpop_lib.DecodeCache(1, 4, 1, 128, torch.bfloat16, 4, 32, 64)
    b = kvpop_lib.DecodeCache(1, 4, 1, 128, torch.bfloat16, 4, 32, 64)
    assert a.state.numel() == b.state.numel()
    t = synth.make_qkv(1, 120, 4, 1, 128, "bf16", 3, device=DEV, with_scores=True)
    r1, r2 = [], []
    for d in range(120):
        args = (t["q"][:, :, d].contiguous(), t["k"][:, :, d].contiguous(), t["v"][:, :, d].contiguous(),
                t["scores"][:, :, d].contiguous())
        r1.append(a.step(*args)[0])
        r2.append(b.step(*args)[0])
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(r1, r2))


def test_decode_at_the_bench_shape(kvpop_lib):
    """The decode workload bench.py times (batch 1, 32q/8kv, D=128, bf16,
    budget 4 + 128 + 1916 = 2048), fed 2600 tokens so that the top-k fills at
    d = 2047 and evicts from then on: every query head's output and LSE at
    sampled steps (early, around the fill, and the last ones) against the
    oracle's masked attention row of the same step."""
    S, Hq, Hkv, D, s, w, kk = 2600, 32, 8, 128, 4, 128, 1916
    say(f"decode bench shape S={S}")
    t = synth.make_qkv(1, S, Hq, Hkv, D, "bf16", 4096, device=DEV, heavy_hitters=True, with_scores=True)
    q, k, v, sc = t["q"], t["k"], t["v"], t["scores"]
    steps = np.array(sorted(set([0, 1, 5, 130, 131, 500, 2046, 2047, 2048, 2049, 2100] + list(range(S - 6, S)))))
    cache = kvpop_lib.DecodeCache(1, Hq, Hkv, D, q.dtype, s, w, kk)
    got = {}
    for d in range(S):
        o, l = cache.step(q[:, :, d].contiguous(), k[:, :, d].contiguous(), v[:, :, d].contiguous(),
                          sc[:, :, d].contiguous())
        if d in steps:
            got[d] = (o.clone(), l.clone())
    torch.cuda.synchronize()
    say("decode bench shape: oracle rows")
    r_rank, r_cut = budget.budget_reference(sc.cpu().numpy(), s, w, kk)
    ro, rl = budget.masked_attention(dense.to_f64(q), dense.to_f64(k), dense.to_f64(v), r_rank, r_cut, s, w,
                                     rows=steps)
    for d in steps:
        o, l = got[int(d)]
        assert_lse_close(l, rl[:, :, d], what=f"decode lse step {d}")
        assert_out_close(o, ro[:, :, d], what=f"decode out step {d}")
