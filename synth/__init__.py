"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module draws random tensors and nothing else: it contains none of the
method's arithmetic (no logits, no softmax, no masks, no ranks).  Both the CPU
oracle and the HIP path receive the very same tensors produced here.

Workloads (sizes follow the KVpop pages: Qwen3-4B attention shape of 32 query
heads, 8 KV heads, head_dim 128; packed training sequences of 16384 tokens,
KVpop paper, Section 4 "Setup"; per-head budget B = s + w + k, Section 3):

  tiny      1 x 1q/1kv x S=512 x D=64, fp32, K scaled by 1.5, w=16, seed 0
  qwen4k    1 x 32q/8kv x S=4096 x D=128, bf16, 1% heavy-hitter keys, w=64, seed 2
  packed16k 1 x 32q/8kv x S=16384 (6 documents, each >= 512) x D=128, bf16,
            1% heavy hitters, w=128, seed 3
  stack36   36 layers x (2 x 32q/8kv x S=16384 x D=128), bf16, 1% heavy
            hitters, w=128, layer l uses seed 4000+l
  budget32k 1 x 32q/8kv x S=32768 x D=128, bf16, scores [1,8,S] fp32 N(0,1),
            sinks 4, window 128, top-k 1916 (budget 2048), seed 5

Recipe (fixed order of draws from one torch.Generator seeded per workload):
Q, K, V ~ N(0,1) float32; then, where enabled, heavy hitters: for every
(batch, KV head) a direction u ~ N(0, I_D) is drawn, scaled to norm 4, and added
to round(0.01*S) key positions drawn without replacement; then scores ~ N(0,1)
float32 where needed; finally bf16 workloads are rounded to bfloat16 with
round-to-nearest-even (torch's conversion).  Generation runs on whichever
device is asked for; CPU and GPU draws differ, so a test always hands the same
materialised tensors to both sides.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str            # "bf16" or "f32"
    window: int
    seed: int
    k_scale: float = 1.0
    heavy_hitters: bool = False
    n_docs: int = 1       # >1: packed via cu_seqlens (batch must be 1)
    min_doc: int = 0
    layers: int = 1
    sinks: int = 0
    topk: int = 0
    with_scores: bool = False

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS = {
    "tiny": Workload("tiny", 1, 512, 1, 1, 64, "f32", 16, 0, k_scale=1.5),
    "qwen4k": Workload("qwen4k", 1, 4096, 32, 8, 128, "bf16", 64, 2, heavy_hitters=True),
    "packed16k": Workload("packed16k", 1, 16384, 32, 8, 128, "bf16", 128, 3,
                          heavy_hitters=True, n_docs=6, min_doc=512),
    "stack36": Workload("stack36", 2, 16384, 32, 8, 128, "bf16", 128, 4000,
                        heavy_hitters=True, layers=36),
    "budget32k": Workload("budget32k", 1, 32768, 32, 8, 128, "bf16", 128, 5,
                          sinks=4, topk=1916, with_scores=True),
}


def doc_lengths(seqlen: int, n_docs: int, min_doc: int, seed: int) -> list[int]:
    """Seeded random document lengths summing to seqlen, each >= min_doc + 1.

    Draws n_docs-1 distinct cut points in [1, extra-1] where
    extra = seqlen - n_docs*min_doc, and adds min_doc to each gap.
    """
    extra = seqlen - n_docs * min_doc
    if n_docs == 1:
        return [seqlen]
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(extra - 1, generator=g)[: n_docs - 1] + 1
    cuts = sorted(int(c) for c in perm)
    bounds = [0] + cuts + [extra]
    return [min_doc + (bounds[i + 1] - bounds[i]) for i in range(n_docs)]


def cu_seqlens_from_lengths(lengths) -> torch.Tensor:
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return torch.tensor(out, dtype=torch.int32)


def _to_dtype(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x.contiguous()
    raise ValueError(dtype)


def make_qkv(batch: int, seqlen: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
             dtype: str, seed: int, device="cpu", k_scale: float = 1.0,
             heavy_hitters: bool = False, with_scores: bool = False):
    """Draw Q [B,Hq,S,D], K, V [B,Hkv,S,D] (and scores [B,Hkv,S] fp32 if asked).

    Returns a dict with q, k, v (and scores) on `device`, in `dtype`.
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev).manual_seed(int(seed))
    f32 = torch.float32
    q = torch.randn(batch, n_q_heads, seqlen, head_dim, generator=g, device=dev, dtype=f32)
    k = torch.randn(batch, n_kv_heads, seqlen, head_dim, generator=g, device=dev, dtype=f32)
    v = torch.randn(batch, n_kv_heads, seqlen, head_dim, generator=g, device=dev, dtype=f32)
    if k_scale != 1.0:
        k.mul_(k_scale)
    if heavy_hitters:
        n_hh = int(round(0.01 * seqlen))
        for b in range(batch):
            for h in range(n_kv_heads):
                u = torch.randn(head_dim, generator=g, device=dev, dtype=f32)
                u = u * (4.0 / torch.linalg.vector_norm(u))
                pos = torch.randperm(seqlen, generator=g, device=dev)[:n_hh]
                k[b, h, pos] += u
    out = {"q": _to_dtype(q, dtype), "k": _to_dtype(k, dtype), "v": _to_dtype(v, dtype)}
    if with_scores:
        out["scores"] = torch.randn(batch, n_kv_heads, seqlen, generator=g, device=dev, dtype=f32)
    return out


def make_leveled_qkv(seqlen: int, n_q_heads: int, n_kv_heads: int, head_dim: int, dtype: str,
                     seed: int, key_level, device="cpu", with_scores: bool = False):
    """Q and K nearly aligned, with K's magnitude set per position.

    Every query is 1 + 0.05 N(0,1) per element and key t is
    key_level[t] * (1 + 0.05 N(0,1)) per element, so a logit is close to
    key_level[t] * head_dim / sqrt(head_dim): the sequence of levels shapes
    how each row's maximum evolves along the keys.  V is N(0,1).  Batch 1.
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev).manual_seed(int(seed))
    f32 = torch.float32
    lvl = torch.as_tensor(key_level, dtype=f32, device=dev).reshape(1, 1, seqlen, 1)
    q = 1.0 + 0.05 * torch.randn(1, n_q_heads, seqlen, head_dim, generator=g, device=dev, dtype=f32)
    k = lvl * (1.0 + 0.05 * torch.randn(1, n_kv_heads, seqlen, head_dim, generator=g, device=dev, dtype=f32))
    v = torch.randn(1, n_kv_heads, seqlen, head_dim, generator=g, device=dev, dtype=f32)
    out = {"q": _to_dtype(q, dtype), "k": _to_dtype(k, dtype), "v": _to_dtype(v, dtype)}
    if with_scores:
        out["scores"] = torch.randn(1, n_kv_heads, seqlen, generator=g, device=dev, dtype=f32)
    return out


def key_levels(kind: str, seqlen: int):
    """Per-position key levels for make_leveled_qkv (natural-log logits near
    level * sqrt(head_dim)): 'rising' climbs steadily; 'jumps' steps up twice
    by more than 100 natural-log units (beyond fp32 exp range); 'falling'
    decreases; 'negative' keeps every logit near -226 at head_dim 128."""
    t = torch.arange(seqlen, dtype=torch.float64)
    if kind == "rising":
        return 0.02 + t * (3.0 / seqlen)
    if kind == "jumps":
        return torch.where(t < seqlen // 3, 0.05, torch.where(t < 2 * seqlen // 3, 10.0, 21.0))
    if kind == "falling":
        return 3.0 - t * (3.0 / seqlen)
    if kind == "negative":
        return torch.full((seqlen,), -20.0, dtype=torch.float64)
    raise ValueError(kind)


def make_workload(name: str, layer: int = 0, device="cpu", seqlen: Optional[int] = None):
    """Materialise one layer of a named workload.

    Returns dict(q, k, v, [scores], cu_seqlens (int32 CPU tensor or None),
    window, sinks, topk, spec).  `seqlen` overrides S for scaled-down tests
    (document lengths are then redrawn for the smaller S).
    """
    w = WORKLOADS[name]
    S = w.seqlen if seqlen is None else int(seqlen)
    seed = w.seed + layer
    cu = None
    if w.n_docs > 1:
        min_doc = w.min_doc if seqlen is None else max(1, min(w.min_doc, S // (2 * w.n_docs)))
        cu = cu_seqlens_from_lengths(doc_lengths(S, w.n_docs, min_doc, seed))
    t = make_qkv(w.batch, S, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype, seed,
                 device=device, k_scale=w.k_scale, heavy_hitters=w.heavy_hitters,
                 with_scores=w.with_scores)
    t.update(cu_seqlens=cu, window=w.window, sinks=w.sinks, topk=w.topk, spec=w)
    return t


def doc_lengths_of(cu_seqlens, seqlen: int):
    if cu_seqlens is None:
        return [seqlen]
    c = [int(x) for x in cu_seqlens]
    return [c[i + 1] - c[i] for i in range(len(c) - 1)]


__all__ = ["Workload", "WORKLOADS", "make_qkv", "make_workload", "doc_lengths",
           "cu_seqlens_from_lengths", "doc_lengths_of"]
