"""Argument checks of the Python binding that need no GPU: K and V must have
q's batch, sequence length, head dimension and dtype (the kernels take those
from q and would otherwise read past K/V), and every tensor must match.  The
checks run before any device access, so CPU tensors exercise them here."""
import pytest
import torch

import attention_target_amd as kv


def qkv(B=1, Hq=4, Hkv=2, S=64, D=64, dtype=torch.bfloat16):
    q = torch.zeros(B, Hq, S, D, dtype=dtype)
    k = torch.zeros(B, Hkv, S, D, dtype=dtype)
    return q, k, torch.zeros_like(k)


BAD_K = [
    ("half the sequence", lambda q, k: torch.zeros(1, 2, 32, 64, dtype=q.dtype)),
    ("other batch", lambda q, k: torch.zeros(2, 2, 64, 64, dtype=q.dtype)),
    ("other head_dim", lambda q, k: torch.zeros(1, 2, 64, 128, dtype=q.dtype)),
    ("BSHD layout", lambda q, k: torch.zeros(1, 64, 2, 64, dtype=q.dtype)),
    ("3-D", lambda q, k: torch.zeros(2, 64, 64, dtype=q.dtype)),
    ("other dtype", lambda q, k: torch.zeros(1, 2, 64, 64, dtype=torch.float32)),
]


@pytest.mark.parametrize("what,make", BAD_K, ids=[b[0] for b in BAD_K])
def test_mismatched_k_is_rejected(what, make):
    q, k, v = qkv()
    bad = make(q, k)
    lse = torch.zeros(1, 4, 64)
    sc = torch.zeros(1, 2, 64)
    pat = "k must|multiple of n_kv_heads"
    with pytest.raises(ValueError, match=pat):
        kv.attn_fwd_lse(q, bad, v)
    with pytest.raises(ValueError, match=pat):
        kv.future_target(q, bad, lse, 4)
    with pytest.raises(ValueError, match=pat):
        kv.budget_mask_fwd(q, bad, v, sc, 1, 4, 8)


def test_mismatched_v_is_rejected():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="v must"):
        kv.attn_fwd_lse(q, k, torch.zeros(1, 2, 32, 64, dtype=q.dtype))
    with pytest.raises(ValueError, match="v must"):
        kv.budget_mask_fwd(q, k, torch.zeros(1, 2, 64, 128, dtype=q.dtype), torch.zeros(1, 2, 64), 1, 4, 8)


def test_group_size_must_divide():
    q, _, _ = qkv(Hq=4)
    k = torch.zeros(1, 3, 64, 64, dtype=q.dtype)
    with pytest.raises(ValueError, match="multiple"):
        kv.attn_fwd_lse(q, k, torch.zeros_like(k))


def test_other_tensors_are_checked_by_shape():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="lse must"):
        kv.future_target(q, k, torch.zeros(1, 4, 63), 4)
    with pytest.raises(ValueError, match="scores must"):
        kv.budget_mask_fwd(q, k, v, torch.zeros(1, 4, 64), 1, 4, 8)
    with pytest.raises(ValueError, match="out must"):
        kv.attn_fwd_lse(q, k, v, out=torch.zeros(1, 4, 64, 32, dtype=q.dtype))
    with pytest.raises(ValueError, match="out must"):
        kv.future_target(q, k, torch.zeros(1, 4, 64), 4, out=torch.zeros(1, 4, 64))   # SUM: [B, Hkv, S]
    with pytest.raises(ValueError, match="lse must"):
        kv.budget_mask_fwd(q, k, v, torch.zeros(1, 2, 64), 1, 4, 8, lse=torch.zeros(1, 4, 64, dtype=torch.float64))


def test_cpu_tensors_are_rejected_after_the_shape_checks():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="CUDA"):
        kv.attn_fwd_lse(q, k, v)
