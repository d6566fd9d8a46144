"""Guard regions around every output and workspace: each entry point writes
into views of larger buffers whose margins before and after hold a sentinel
byte pattern, and the margins must be untouched after the call; the outputs
must equal those of the same call on plain allocations, bit for bit.  Ragged
shapes (lengths that are not multiples of any tile), packed documents and
odd group sizes put the kernels' last tiles at the edges of their buffers.
Runs on an MI355X."""
import sys

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
MARGIN = 4096          # bytes before and after each guarded buffer (keeps 256-byte alignment)
SENTINEL = 0xA7


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Guarded:
    """A contiguous tensor of `shape` and `dtype` inside a byte buffer with
    MARGIN sentinel bytes on each side."""

    def __init__(self, shape, dtype, fill=None):
        n = 1
        for x in shape:
            n *= int(x)
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((MARGIN + nbytes + MARGIN,), SENTINEL, dtype=torch.uint8, device=DEV)
        self.t = self.buf[MARGIN:MARGIN + nbytes].view(dtype).view(*shape)
        if fill is not None:
            self.t.copy_(fill)
        self.nbytes = nbytes

    def intact(self):
        head = self.buf[:MARGIN]
        tail = self.buf[MARGIN + self.nbytes:]
        return bool(torch.all(head == SENTINEL)) and bool(torch.all(tail == SENTINEL))


def same(a, b):
    """Bitwise equality (NaN and -inf patterns included)."""
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


SHAPES = [
    # B, S, Hq, Hkv, D, dtype, docs, w
    (1, 333, 4, 1, 128, "bf16", 1, 17),
    (2, 1000, 6, 3, 64, "bf16", 1, 64),
    (1, 777, 8, 2, 128, "bf16", 3, 5),
    (1, 301, 4, 2, 64, "f32", 2, 9),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,dt,docs,w", SHAPES)
def test_forward_and_target_stay_in_bounds(kvpop_lib, B, S, Hq, Hkv, D, dt, docs, w):
    kv = kvpop_lib
    say(f"canary fwd/target B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} {dt} docs={docs} w={w}")
    t = synth.make_qkv(B, S, Hq, Hkv, D, dt, 5 + S, device=DEV, heavy_hitters=True)
    q, k, v = t["q"], t["k"], t["v"]
    cu = synth.cu_seqlens_from_lengths(synth.doc_lengths(S, docs, 10, S)) if docs > 1 else None
    o0, l0 = kv.attn_fwd_lse(q, k, v, cu_seqlens=cu)
    og, lg = Guarded(q.shape, q.dtype), Guarded((B, Hq, S), torch.float32)
    kv.attn_fwd_lse(q, k, v, cu_seqlens=cu, out=og.t, lse=lg.t)
    for agg in ("sum", "none"):
        t0 = kv.future_target(q, k, l0, w, agg=agg, cu_seqlens=cu)
        need = kv.workspace_size(kv.CALL_FUTURE_TARGET, q, k, cu_seqlens=cu, window=w)
        Hout = Hq if agg == "none" else Hkv
        tgg, wsg = Guarded((B, Hout, S), torch.float32), Guarded((max(need, 1),), torch.uint8)
        kv.future_target(q, k, lg.t, w, agg=agg, cu_seqlens=cu, out=tgg.t, workspace=wsg.t)
        torch.cuda.synchronize()
        assert tgg.intact() and wsg.intact(), f"target ({agg}) wrote outside its buffers"
        assert same(tgg.t, t0), f"target ({agg}) differs with guarded buffers"
    assert og.intact() and lg.intact(), "forward wrote outside its buffers"
    assert same(og.t, o0) and same(lg.t, l0)


BUDGET = [
    # S, Hq, Hkv, D, dtype, s, w, k
    (333, 4, 1, 128, "bf16", 4, 16, 40),
    (1025, 8, 2, 128, "bf16", 2, 64, 300),
    (517, 4, 4, 64, "f32", 0, 1, 7),
    (2049, 4, 1, 64, "bf16", 4, 128, 1916),
]


@pytest.mark.parametrize("S,Hq,Hkv,D,dt,s,w,kk", BUDGET)
def test_budget_stays_in_bounds(kvpop_lib, S, Hq, Hkv, D, dt, s, w, kk):
    kv = kvpop_lib
    say(f"canary budget S={S} Hq={Hq} Hkv={Hkv} D={D} {dt} s={s} w={w} k={kk}")
    t = synth.make_qkv(1, S, Hq, Hkv, D, dt, 9 + S, device=DEV, with_scores=True)
    q, k, v, sc = t["q"], t["k"], t["v"], t["scores"]
    o0, l0, r0, c0 = kv.budget_mask_fwd(q, k, v, sc, s, w, kk)
    need = kv.workspace_size(kv.CALL_BUDGET_MASK_FWD, q, k, sinks=s, window=w, topk=kk)
    og, lg = Guarded(q.shape, q.dtype), Guarded((1, Hq, S), torch.float32)
    wsg = Guarded((need,), torch.uint8)
    o1, l1, r1, c1 = kv.budget_mask_fwd(q, k, v, sc, s, w, kk, out=og.t, lse=lg.t, workspace=wsg.t)
    torch.cuda.synchronize()
    assert og.intact() and lg.intact() and wsg.intact(), "budget forward wrote outside its buffers"
    assert same(og.t, o0) and same(lg.t, l0) and torch.equal(r1, r0) and torch.equal(c1, c0)


def test_decode_stays_in_bounds(kvpop_lib):
    kv = kvpop_lib
    S, Hq, Hkv, D, s, w, kk = 300, 6, 2, 128, 2, 16, 40
    say("canary decode")
    t = synth.make_qkv(1, S, Hq, Hkv, D, "bf16", 17, device=DEV, with_scores=True)
    q, k, v, sc = t["q"], t["k"], t["v"], t["scores"]
    plain = kv.DecodeCache(1, Hq, Hkv, D, q.dtype, s, w, kk)
    guarded = kv.DecodeCache(1, Hq, Hkv, D, q.dtype, s, w, kk)
    sg = Guarded((guarded.state.numel(),), torch.uint8)
    sg.t.copy_(guarded.state)
    guarded.state = sg.t
    for d in range(S):
        args = (q[:, :, d].contiguous(), k[:, :, d].contiguous(), v[:, :, d].contiguous(),
                sc[:, :, d].contiguous())
        o0, l0 = plain.step(*args)
        og, lg = Guarded((1, Hq, D), q.dtype), Guarded((1, Hq), torch.float32)
        guarded.step(*args, out=og.t, lse=lg.t)
        if d % 37 == 0 or d == S - 1:
            torch.cuda.synchronize()
            assert og.intact() and lg.intact() and sg.intact(), f"decode step {d} wrote outside its buffers"
            assert same(og.t, o0) and same(lg.t, l0), f"decode step {d} differs"
