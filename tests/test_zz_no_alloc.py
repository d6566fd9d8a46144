"""kvpop_future_target_noalloc, the target without a workspace (a fixed
per-GPU scratch array instead), through the C ABI: bit for bit the results
of kvpop_future_target on the same inputs, for consecutive calls that leave
the shared scratch holding the previous call's data (the second call is
smaller than the first), at the metric layer's size, and a clear error for a
shape whose scratch need exceeds the array.  Runs on an MI355X."""
import sys

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def same(a, b):
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


def both(kv, q, k, w, agg, mean, eps, cu):
    _, lse = kv.attn_fwd_lse(q, k, torch.zeros_like(k), cu_seqlens=cu, need_output=False)
    ref = kv.future_target(q, k, lse, w, agg=agg, mean_over_queries=mean, eps=eps, cu_seqlens=cu)
    Hout = q.shape[1] if agg == "none" else k.shape[1]
    out = torch.full((q.shape[0], Hout, q.shape[2]), float("nan"), device=DEV)
    kv.future_target_noalloc(q, k, lse, w, out, agg=agg, mean_over_queries=mean, eps=eps, cu_seqlens=cu)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_matches_workspace_entry_point(kvpop_lib):
    kv = kvpop_lib
    # 1: S=4096, 32q/8kv, two documents, per-head partials (MAX with the mean): 8.9 MB of scratch
    t = synth.make_qkv(1, 4096, 32, 8, 128, "bf16", 41, device=DEV, heavy_hitters=True)
    cu = torch.tensor([0, 1500, 4096], dtype=torch.int32)
    say("no-alloc call 1: S=4096 packed, max + mean")
    ref, out = both(kv, t["q"], t["k"], 64, "max", True, 1e-6, cu)
    assert same(ref, out), "first call differs from kvpop_future_target"
    # 2: smaller, right after: the scratch still holds call 1's partials
    t2 = synth.make_qkv(1, 1000, 8, 2, 64, "bf16", 42, device=DEV)
    cu2 = torch.tensor([0, 333, 1000], dtype=torch.int32)
    say("no-alloc call 2: S=1000, sum")
    ref2, out2 = both(kv, t2["q"], t2["k"], 16, "sum", False, 0.0, cu2)
    assert same(ref2, out2), "second (smaller) call differs from kvpop_future_target"
    # 3: the same small call per head, fp32 inputs
    t3 = synth.make_qkv(1, 700, 4, 2, 64, "f32", 43, device=DEV)
    say("no-alloc call 3: S=700 fp32, none")
    ref3, out3 = both(kv, t3["q"], t3["k"], 9, "none", False, 0.0, None)
    assert same(ref3, out3), "third call differs from kvpop_future_target"


def test_noalloc_at_the_metric_layer_size(kvpop_lib):
    """B=2, S=16384, 32q/8kv/128, w=128 with the SUM aggregation (21 MB of
    scratch); per-head partials at that size (71 MB) are refused."""
    kv = kvpop_lib
    t = synth.make_workload("stack36", layer=3, device=DEV)
    say("no-alloc metric layer: sum")
    ref, out = both(kv, t["q"], t["k"], t["window"], "sum", False, 0.0, None)
    assert same(ref, out)
    _, lse = kv.attn_fwd_lse(t["q"], t["k"], t["v"], need_output=False)
    bad = torch.empty(2, 32, 16384, device=DEV)
    with pytest.raises(kv.KvpopError) as ei:
        kv.future_target_noalloc(t["q"], t["k"], lse, t["window"], bad, agg="none")
    assert ei.value.status == kv.EUNSUPPORTED and "scratch" in str(ei.value)
