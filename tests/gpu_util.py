"""Helpers shared by the GPU parity tests: device inputs, host copies of the
exact input bits, and the comparison policy against the oracle.

Comparison policy:
  - argmax, renoise/init tokens: bit-exact;
  - entropy: |H_gpu - H_oracle| <= 1e-4 absolute (the measured maximum is
    reported);
  - sample: bit-exact except near-ties, i.e. rows where the oracle's two best
    Gumbel-perturbed scores (block level or in-block level) differ by less
    than 1e-6 * max(1, |score|); such rows are counted and reported;
  - acceptance/stop from the GPU's own entropies: exact (the decision rule is
    checked in isolation); from the oracle's entropies: exact except when an
    entropy gap or the bound slack at the acceptance boundary is below the
    measured entropy error.
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


def compare_stats(z_host, temp, seed, positions, step, h_gpu, am_gpu, smp_gpu, report=None):
    """Compares one canvas's GPU statistics (rows `positions` of z_host) with
    the oracle. Returns a dict of measured errors and counts."""
    z = np.asarray(z_host, dtype=np.float64)
    oh = O.entropy(z, temp)
    oam = O.argmax_raw(z)
    osmp, bbest, bgap, ebest, egap = O.sample_two_level_detail(z, temp, seed, positions, step)
    dh = np.abs(np.asarray(h_gpu, dtype=np.float64) - oh)
    out = dict(max_dh=float(dh.max()) if dh.size else 0.0, rows=len(positions))
    assert out["max_dh"] <= H_TOL, f"entropy error {out['max_dh']:.3g} > {H_TOL}"
    bad_am = np.flatnonzero(np.asarray(am_gpu) != oam)
    assert bad_am.size == 0, f"argmax differs at rows {bad_am[:10]} (gpu {np.asarray(am_gpu)[bad_am[:5]]}, oracle {oam[bad_am[:5]]})"
    mism = np.asarray(smp_gpu) != osmp
    ties = near_tie(bbest, bgap) | near_tie(ebest, egap)
    hard = np.flatnonzero(mism & ~ties)
    assert hard.size == 0, (f"sample differs at rows {hard[:10]} that are not near-ties: gpu "
                            f"{np.asarray(smp_gpu)[hard[:5]]}, oracle {osmp[hard[:5]]}, block gaps "
                            f"{bgap[hard[:5]]}, element gaps {egap[hard[:5]]}")
    out["sample_near_ties"] = int((mism & ties).sum())
    out["near_tie_rows"] = int(ties.sum())
    if report is not None:
        report.append(out)
    return out


def accept_near_tie(h_oracle, bound, tol):
    """True when the acceptance decision of the oracle's entropies could flip
    under entropy errors up to tol: an entropy gap at the boundary or the bound
    slack of the boundary prefix sums is within the error."""
    L = len(h_oracle)
    order = np.lexsort((np.arange(L), h_oracle))
    hs = h_oracle[order]
    _, k = O.accept(h_oracle, bound)
    ex = np.concatenate([[0.0], np.cumsum(hs)])[:-1]
    slack_tol = max(1e-6, 4 * L * tol)
    near = False
    if k < L:
        near |= abs(ex[k] - bound) < slack_tol or abs(hs[k] - hs[k - 1]) < max(1e-6, 4 * tol)
    near |= abs(ex[k - 1] - bound) < slack_tol
    return near
