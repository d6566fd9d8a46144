"""GPU parity of the teacher labels at the eviction boundary (kvpop_teacher_labels)
and the boundary-aware retention loss (kvpop_boundary_loss) against the CPU
oracle (oracle/teacher.py; KVpop paper, Section 3.1, Eqs. 4-7).

Labels, boundary tokens, ranks and boundary ranks are integers decided by
float32 priorities computed the same way on both sides: bit-exact.  The loss
and its gradient are float32 on the GPU against float64 in the oracle:
|delta| <= 1e-5 * (1 + |ref|) for the per-position loss, and for the gradient
1e-5 * (1 + sum of |terms| reaching that token), the rounding of an fp32 sum.
Runs on an MI355X."""
import sys

import numpy as np
import pytest
import torch

from oracle import dense, teacher

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_teacher(y, s, w, k, lam, delta):
    B, H, S = y.shape
    out = [np.empty((B, H, S), dtype=np.int64) for _ in range(4)]
    for b in range(B):
        for h in range(H):
            lh = 0.0 if lam is None else float(lam[h])
            lab, bnd, rank, brank = teacher.teacher_static(y[b, h], s, w, k, lh, delta)
            for o, v in zip(out, (lab, bnd, rank, brank)):
                o[b, h] = v
    return out


CASES = [
    # B, H, S, s, w, k, lam, delta, kind
    (1, 1, 300, 4, 16, 20, None, 1, "normal"),
    (2, 3, 1000, 2, 64, 100, None, 1, "ties"),
    (1, 2, 777, 0, 0, 50, [0.25, 0.0], 1, "grid"),
    (1, 2, 1500, 4, 32, 64, [0.5, 0.125], 8, "normal"),
    (1, 1, 400, 4, 8, 0, None, 1, "normal"),          # k = 0: no labels
    (1, 1, 200, 4, 8, 500, None, 1, "normal"),        # k > |E_d| everywhere
    (1, 2, 8192, 4, 128, 1916, [0.01, 0.02], 16, "normal"),
]


def make_y(B, H, S, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "ties":
        y = rng.integers(-4, 5, (B, H, S)).astype(np.float32)
    elif kind == "grid":
        y = (rng.integers(-64, 64, (B, H, S)) / 16.0).astype(np.float32)
    else:
        y = rng.standard_normal((B, H, S)).astype(np.float32)
    return y


@pytest.mark.parametrize("B,H,S,s,w,k,lam,delta,kind", CASES)
def test_teacher_labels_bit_exact(kvpop_lib, B, H, S, s, w, k, lam, delta, kind):
    say(f"teacher B={B} H={H} S={S} s={s} w={w} k={k} lam={lam} delta={delta} {kind}")
    y = make_y(B, H, S, kind, S + k)
    lam_t = None if lam is None else torch.tensor(lam, dtype=torch.float32, device=DEV)
    lab, bnd, rank, brank = kvpop_lib.teacher_labels(torch.from_numpy(y).to(DEV), s, w, k, decay_lambda=lam_t,
                                                    decay_step=delta, return_ranks=True)
    torch.cuda.synchronize()
    r_lab, r_bnd, r_rank, r_brank = oracle_teacher(y, s, w, k, lam, delta)
    assert np.array_equal(rank.cpu().numpy(), r_rank), "ranks differ"
    assert np.array_equal(brank.cpu().numpy(), r_brank), "boundary ranks differ"
    assert np.array_equal(bnd.cpu().numpy(), r_bnd), "boundary tokens differ"
    assert np.array_equal(lab.cpu().numpy(), r_lab), "labels differ"


def check_loss(kv, y, s, w, k, tau, with_weight, seed):
    B, H, S = y.shape
    rng = np.random.default_rng(seed)
    pred = rng.standard_normal((B, H, S)).astype(np.float32)
    om = rng.uniform(0.5, 2.0, (B, H, S)).astype(np.float32) if with_weight else None
    lab, bnd = kv.teacher_labels(torch.from_numpy(y).to(DEV), s, w, k)
    loss, grad = kv.boundary_loss(torch.from_numpy(pred).to(DEV), lab, bnd, s, w, k, tau,
                                  weight=None if om is None else torch.from_numpy(om).to(DEV))
    torch.cuda.synchronize()
    g_loss, g_grad = loss.cpu().double().numpy(), grad.cpu().double().numpy()
    r_lab, r_bnd, _, _ = oracle_teacher(y, s, w, k, None, 1)
    for b in range(B):
        for h in range(H):
            rl, rg = teacher.boundary_loss(pred[b, h], r_lab[b, h], r_bnd[b, h], w, tau,
                                           None if om is None else om[b, h])
            # magnitude of the terms that reach each token
            scale = np.zeros(S)
            for d in range(S):
                if r_lab[b, h, d] >= 0 and r_bnd[b, h, d] >= 0:
                    mag = abs(rl[d]) + 1.0
                    scale[d - w] += mag
                    scale[r_bnd[b, h, d]] += mag
            assert np.all(np.abs(g_loss[b, h] - rl) <= 1e-5 * (1 + np.abs(rl))), "loss differs"
            err = np.abs(g_grad[b, h] - rg)
            assert np.all(err <= 1e-5 * (1 + scale) * max(1.0, 1.0 / tau)), \
                f"grad differs: max {err.max():.3g}"
            assert abs(g_grad[b, h].sum()) <= 1e-4 * (1 + scale.sum())


@pytest.mark.parametrize("S,s,w,k,tau,wt", [(500, 4, 16, 40, 1.0, False), (3000, 2, 64, 300, 0.5, True),
                                            (200, 4, 8, 500, 2.0, True),
                                            # long runs of one boundary token across many 64-position waves
                                            (5000, 4, 32, 2000, 1.0, False), (4096, 0, 64, 1000, 0.5, True)])
def test_boundary_loss_and_gradient(kvpop_lib, S, s, w, k, tau, wt):
    say(f"boundary loss S={S} s={s} w={w} k={k} tau={tau} weight={wt}")
    y = make_y(1, 2, S, "normal", 7 * S)
    check_loss(kvpop_lib, y, s, w, k, tau, wt, 11 * S)


def test_chain_from_oracle_targets(kvpop_lib):
    """The paper's chain on a small layer: the target y (max over the GQA
    group of ln(mean future mass + eps), Eq. 3) computed by the oracle, then
    the teacher and the loss on both sides from that same y."""
    rng = np.random.default_rng(5)
    S, Hq, Hkv, D, w, s, k = 600, 4, 2, 64, 32, 4, 60
    q = rng.standard_normal((1, Hq, S, D))
    kk = rng.standard_normal((1, Hkv, S, D))
    r = dense.reference(q, kk, None, window=w, agg=dense.AGG_MAX, mean_over_queries=True, eps=1e-6,
                        need_output=False)
    y = r["target"].astype(np.float32)
    lab, bnd, rank, brank = kvpop_lib.teacher_labels(torch.from_numpy(y).to(DEV), s, w, k, return_ranks=True)
    torch.cuda.synchronize()
    r_lab, r_bnd, r_rank, _ = oracle_teacher(y, s, w, k, None, 1)
    assert np.array_equal(lab.cpu().numpy(), r_lab) and np.array_equal(bnd.cpu().numpy(), r_bnd)
    check_loss(kvpop_lib, y, s, w, k, 1.0, False, 3)
