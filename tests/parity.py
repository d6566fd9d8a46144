"""Parity checks between the HIP library and the CPU oracle (test helpers).

Tolerances:
  LSE                 |delta| <= 2e-3 (natural log)
  target              |delta| <= 2e-2 where the oracle value > -30 (mass > e^-30);
                      -inf exactly where the oracle is -inf (empty set);
                      -inf or <= -30 + 2e-2 where the oracle is finite but <= -30;
                      never NaN or +inf
  sparse output       per output row (one query, one head): max |delta| <= 2e-2 * RMS of the
                      oracle row, beyond each element's own final rounding to the output
                      format (half an ulp of the reference element); bf16 rounding is
                      relative to each element's own magnitude
  dense output        per element |delta O| <= 2^-7 * sum_t a_{d,t} |v_t| + 1e-6: P and O
                      rounded to bf16 (unit roundoff 2^-8 each); fp32 outputs: 2^-16;
                      and the sparse output's per-row bound as well, each element
                      allowed its own final rounding (half an ulp of the reference)
  ranks, cutoffs      bit-exact
"""
import numpy as np

LSE_TOL = 2e-3
TARGET_TOL = 2e-2
TARGET_FLOOR = -30.0
OUT_REL_TOL = 2e-2


def report(what, quantity, value, bar):
    """One line per check with its worst case against its bar; pytest shows
    these for passing tests with -rP."""
    print(f"[parity] {what}: {quantity} = {value:.3g} (bar {bar:g})", flush=True)


def as_np(x):
    import torch
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def assert_lse_close(gpu, ref, tol=LSE_TOL, what="lse"):
    g, r = as_np(gpu), as_np(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    ninf = np.isneginf(r)
    assert np.array_equal(np.isneginf(g), ninf), f"{what}: -inf pattern differs"
    fin = ~ninf
    assert np.all(np.isfinite(g[fin])), f"{what}: non-finite values"
    err = np.abs(g[fin] - r[fin]).max() if fin.any() else 0.0
    report(what, "lse max |delta|", err, tol)
    assert err <= tol, f"{what}: max |delta| = {err:.3g} > {tol}"
    return err


def assert_target_close(gpu, ref, tol=TARGET_TOL, floor=TARGET_FLOOR, what="target"):
    g, r = as_np(gpu), as_np(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert not np.isnan(g).any(), f"{what}: NaN"
    assert not np.isposinf(g).any(), f"{what}: +inf"
    empty = np.isneginf(r)
    assert np.all(np.isneginf(g[empty])), f"{what}: {(~np.isneginf(g[empty])).sum()} empty sets not -inf"
    big = np.isfinite(r) & (r > floor)
    assert np.all(np.isfinite(g[big])), f"{what}: {(~np.isfinite(g[big])).sum()} non-empty keys are -inf"
    err = np.abs(g[big] - r[big]).max() if big.any() else 0.0
    report(what, "target max |delta|", err, tol)
    assert err <= tol, f"{what}: max |delta| = {err:.3g} > {tol}"
    small = np.isfinite(r) & (r <= floor)
    if small.any():
        gs = g[small]
        assert np.all(np.isneginf(gs) | (gs <= floor + tol)), f"{what}: tiny masses out of range"
    return err


def assert_out_bounded(gpu, ref, abs_ref, u=2.0 ** -8, what="out"):
    """Element-wise rounding bound of an attention output computed with P
    and O rounded to a format of unit roundoff u (bf16: 2^-8):
    |delta O_dj| <= 2u * sum_t a_{d,t} |v_tj| + 1e-6."""
    g, r, a = as_np(gpu), as_np(ref), as_np(abs_ref)
    assert g.shape == r.shape == a.shape, (what, g.shape, r.shape, a.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    err = np.abs(g - r)
    bound = 2.0 * u * a + 1e-6
    worst = float((err / bound).max())
    report(what, "out error / rounding bound", worst, 1.0)
    assert worst <= 1.0, f"{what}: error reaches {worst:.3g} of the bf16 rounding bound"
    return worst


OUT_ROUND = {"torch.bfloat16": 2.0 ** -8, "torch.float32": 2.0 ** -24}


def assert_out_close(gpu, ref, rel=OUT_REL_TOL, what="out", out_round=None):
    """Per output row (the head_dim vector O_d of one query of one head):
    max_j (|delta O_dj| - h_dj) <= rel * RMS_j(O_ref,dj), where h_dj is the
    output format's own rounding of that element, half an ulp of the
    reference value (`out_round` is the format's unit roundoff; by default
    taken from the GPU tensor's dtype).  Rows whose reference is exactly zero
    (nothing attended) must be exactly zero.  Returns the largest ratio over
    rows."""
    if out_round is None:
        out_round = OUT_ROUND.get(str(getattr(gpu, "dtype", "")), 0.0)
    g, r = as_np(gpu), as_np(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    D = r.shape[-1]
    g2, r2 = g.reshape(-1, D), r.reshape(-1, D)
    rms = np.sqrt(np.mean(r2 * r2, axis=1))
    with np.errstate(divide="ignore"):
        half_ulp = out_round * np.exp2(np.floor(np.log2(np.abs(r2))))
    err = np.maximum(np.abs(g2 - r2) - half_ulp, 0.0).max(axis=1)
    zero = rms == 0
    assert np.all(err[zero] == 0), f"{what}: rows that attend nothing are not zero"
    ratio = err[~zero] / rms[~zero]
    worst = float(ratio.max()) if ratio.size else 0.0
    i = int(np.argmax(ratio)) if ratio.size else 0
    report(what, "out row error / row RMS", worst, rel)
    assert worst <= rel, (f"{what}: row max |delta| / row RMS = {worst:.3g} > {rel} "
                          f"(row {i}: err {err[~zero][i]:.3g}, rms {rms[~zero][i]:.3g})")
    return worst


def assert_dense_out(gpu, ref, abs_ref, u=2.0 ** -8, what="out"):
    """The dense forward's output under both bounds: the element-wise
    rounding bound and the per-row bound of the sparse output.  Returns the
    worst ratio of each."""
    return (assert_out_bounded(gpu, ref, abs_ref, u=u, what=what),
            assert_out_close(gpu, ref, what=what))
