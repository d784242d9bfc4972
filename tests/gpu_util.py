"""Helpers shared by the GPU parity tests: device inputs, host copies of the
exact input bits, and the comparison policy against the oracle.

Comparison policy:
  - argmax, renoise/init tokens: bit-exact;
  - entropy: |H_gpu - H_oracle| <= 1e-4 absolute (the measured maximum is
    reported);
  - sample: bit-exact except near-ties, i.e. rows where the oracle's two best
    Gumbel-perturbed scores (block level or in-block level) differ by less
    than 1e-6 * max(1, |score|); such rows are counted and reported;
  - acceptance/stop against the oracle's: exact except at a near-tie that the
    measured entropy error can flip (accept_tie_clause, stop_tie_clause:
    the bound slack within k * max|dH|, a boundary gap within 2 max|dH|, the
    mean entropy within max|dH| of the threshold; each capped at 1e-4), which
    is counted and named; in addition the GPU's decisions must obey the rules
    as properties of the GPU's own outputs (check_decision_rules, which uses
    no oracle code);
  - logits from the LM head (fp32 accumulation) differ from the oracle's
    exact products by a measured per-row error e; an argmax or sample mismatch
    is then a near-tie when the oracle's competing scores are within 2e/T of
    each other (compare_stats's logit_err).
"""
import numpy as np
import pytest
import torch

from oracle import sampler as O

H_TOL = 1e-4
NEAR_TIE_REL = 1e-6

gpu = pytest.mark.gpu


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def seeds_tensor(seeds, device="cuda"):
    """int64 tensor holding the two's-complement bits of uint64 seeds."""
    vals = [(int(s) & (2**64 - 1)) - (2**64 if (int(s) & (2**64 - 1)) >= 2**63 else 0) for s in seeds]
    return torch.tensor(vals, dtype=torch.int64, device=device)


def host_values(t):
    """Exact fp64 values of a bf16/fp32 tensor (widening is exact)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def near_tie(best, gap):
    return gap < NEAR_TIE_REL * np.maximum(1.0, np.abs(best))


def compare_stats(z_host, temp, seed, positions, step, h_gpu, am_gpu, smp_gpu, report=None,
                  logit_err=None):
    """Compares one canvas's GPU statistics (rows `positions` of z_host) with
    the oracle. logit_err (per row, optional): how far the logits the GPU
    consumed may be from z_host. Returns a dict of measured errors and counts."""
    z = np.asarray(z_host, dtype=np.float64)
    oh = O.entropy(z, temp)
    oam = O.argmax_raw(z)
    osmp, bbest, bgap, ebest, egap = O.sample_two_level_detail(z, temp, seed, positions, step)
    dh = np.abs(np.asarray(h_gpu, dtype=np.float64) - oh)
    out = dict(max_dh=float(dh.max()) if dh.size else 0.0, rows=len(positions))
    assert out["max_dh"] <= H_TOL, f"entropy error {out['max_dh']:.3g} > {H_TOL}"
    am_gpu = np.asarray(am_gpu)
    bad_am = np.flatnonzero(am_gpu != oam)
    if logit_err is not None and bad_am.size:
        err = np.broadcast_to(np.asarray(logit_err, dtype=np.float64), (len(positions),))
        gap = z[bad_am, oam[bad_am]] - z[bad_am, am_gpu[bad_am]]
        excused = gap <= 2 * err[bad_am]
        out["argmax_near_ties"] = int(excused.sum())
        bad_am = bad_am[~excused]
    assert bad_am.size == 0, f"argmax differs at rows {bad_am[:10]} (gpu {am_gpu[bad_am[:5]]}, oracle {oam[bad_am[:5]]})"
    mism = np.asarray(smp_gpu) != osmp
    ties = near_tie(bbest, bgap) | near_tie(ebest, egap)
    if logit_err is not None:
        slack = 2 * np.asarray(logit_err, dtype=np.float64) / float(temp)
        ties = ties | (bgap < slack) | (egap < slack)
    hard = np.flatnonzero(mism & ~ties)
    assert hard.size == 0, (f"sample differs at rows {hard[:10]} that are not near-ties: gpu "
                            f"{np.asarray(smp_gpu)[hard[:5]]}, oracle {osmp[hard[:5]]}, block gaps "
                            f"{bgap[hard[:5]]}, element gaps {egap[hard[:5]]}")
    out["sample_near_ties"] = int((mism & ties).sum())
    out["near_tie_rows"] = int(ties.sum())
    if report is not None:
        report.append(out)
    return out


# A slack or gap larger than this never excuses a difference, however large
# the measured entropy error (it stays well below it in every configuration).
ACCEPT_SLACK_CAP = 1e-4


def _fp64_prefix_rounding(n, total):
    """Bound on the rounding of an n-term fp64 sum of non-negative terms that
    add up to `total` (either side's prefix sums)."""
    return 2.0 * n * 2.0 ** -53 * max(float(total), 0.0) + 1e-300


def accept_tie_clause(h_oracle, bound, dh):
    """Names the near-tie through which entropies within dh of the oracle's
    (per row) can change the oracle's acceptance, or returns None.

    With pi the (H, position) order, EX_i the sum of the i smallest entropies
    and k the oracle's count (EX_i <= b exactly for i < k): entropies off by
    at most dh move each sorted value by at most dh and EX_i by at most
    i * dh. So the count can change only when EX_k - b <= k * dh (one more
    position fits) or b - EX_{k-1} < (k - 1) * dh (the last accepted one no
    longer fits), and the accepted set can change at an equal count only when
    H_pi(k) - H_pi(k-1) <= 2 * dh (the two boundary positions trade places).
    Every slack also allows both sides' fp64 rounding of the prefix sums and
    is capped at ACCEPT_SLACK_CAP."""
    h = np.asarray(h_oracle, dtype=np.float64)
    L = len(h)
    order = np.lexsort((np.arange(L), h))
    hs = h[order]
    _, k = O.accept(h, bound)
    ex = np.concatenate([[0.0], np.cumsum(hs)])
    cap = ACCEPT_SLACK_CAP
    if k < L:
        slack = ex[k] - bound
        tol = min(k * dh + _fp64_prefix_rounding(k, ex[k]), cap)
        if slack <= tol:
            return f"one more position fits: EX_k - b = {slack:.3g} <= k*dH = {tol:.3g} (k = {k})"
        gap = hs[k] - hs[k - 1]
        tol = min(2 * dh, cap)
        if gap <= tol:
            return f"boundary positions trade places: H gap {gap:.3g} <= 2 dH = {tol:.3g} (k = {k})"
    if k > 1:
        slack = bound - ex[k - 1]
        tol = min((k - 1) * dh + _fp64_prefix_rounding(k - 1, ex[k - 1]), cap)
        if slack < tol:
            return f"last position no longer fits: b - EX_(k-1) = {slack:.3g} < (k-1)*dH = {tol:.3g} (k = {k})"
    return None


def stop_tie_clause(mean_h_oracle, threshold, dh):
    """Names the near-tie through which a mean entropy off by at most dh (plus
    fp32 rounding of the GPU's mean) can flip the strict test mean < threshold,
    or returns None."""
    m = float(mean_h_oracle)
    tol = min(dh + 2.0 ** -23 * max(m, float(threshold)), ACCEPT_SLACK_CAP)
    if abs(m - float(threshold)) <= tol:
        return f"mean entropy {m:.6g} within {tol:.3g} of the stop threshold {float(threshold):.6g}"
    return None


def check_decision_rules(h, accept, n_accept, sample, canvas, renoise, mean_h, stop, prev_argmax,
                         argmax, bound, threshold):
    """The acceptance, renoise and stop rules as properties of one canvas's
    GPU outputs (no oracle code): the accepted positions are the n_accept
    lowest by (entropy, position); the entropy of the accepted prefix without
    its last element stays within the bound and one more position would break
    it (fp64 sums; boundary cases closer than 1e-12 are not judged); accepted
    positions take the sample, the others the given renoise tokens; the mean
    entropy is the fp64 mean; the stop needs a previous argmax canvas equal to
    this one and a mean entropy below the threshold."""
    h = np.asarray(h, dtype=np.float64)
    L = len(h)
    order = np.lexsort((np.arange(L), h))
    k = int(n_accept)
    assert 1 <= k <= L, f"n_accept {k} outside 1..{L}"
    want = np.zeros(L, dtype=bool)
    want[order[:k]] = True
    assert np.array_equal(np.asarray(accept).astype(bool), want), "accepted set is not the lowest-entropy prefix"
    hs = h[order]
    ex = np.concatenate([[0.0], np.cumsum(hs)])
    assert ex[k - 1] <= bound + 1e-12, f"accepted prefix exceeds the bound: {ex[k - 1]} > {bound}"
    if k < L:
        assert ex[k] > bound - 1e-12, f"one more position fits the bound: {ex[k]} <= {bound}"
    assert np.array_equal(np.asarray(canvas), np.where(want, np.asarray(sample), np.asarray(renoise)))
    mh = float(np.mean(h))
    assert abs(float(mean_h) - mh) <= 1e-6 * max(1.0, mh)
    stable = prev_argmax is not None and np.array_equal(np.asarray(argmax), np.asarray(prev_argmax))
    if abs(mh - float(threshold)) > 1e-6:
        assert bool(stop) == (stable and mh < float(threshold))
    return k
