"""Host-side analysis of comparison results (numpy, no GPU).

Turns the per-row outputs and the margin-bin report of the library into the
quantities the logit-diffing page reasons with ("在 agent 时代如何快速验证 kernel
对精度的影响"):

  flip_probability      the Gaussian flip model of the appendix (附录：公式的来历):
                        Phi(-margin / (sqrt(2) sigma)) and its tail bound
                        exp(-margin^2 / (4 sigma^2))
  model_flip_rates      that model averaged over the rows of each margin bin,
                        to set beside the measured flip rates
  flip_rates            measured flips / count per bin, from the bin report
  group_quantiles       per-group KL medians and quantiles (the page compares
                        KL medians per context depth and per code / prose)
  empirical_cdf         points of a KL CDF
  perplexity            exp(-mean ln q(target)) per group (section perplexity
                        看不出这一级的差别)
  total_variation       half the L1 distance of two distributions
  accuracy_gap_bound    the loose bound of section 和 GSM8K 的关系:
                        |Acc_base - Acc_cand| <= sqrt(1/2 sum_t KL_t)
  kl_per_step_for_gap   the mean per-step KL that the bound needs for a gap
"""
from __future__ import annotations

import math

import numpy as np


def _phi(x):
    """Standard normal CDF (elementwise)."""
    x = np.asarray(x, np.float64)
    return 0.5 * np.vectorize(math.erfc)(-x / math.sqrt(2.0))


def flip_probability(margin, sigma: float):
    """Probability that the runner-up overtakes the leader when both logits
    carry independent N(0, sigma^2) noise: Phi(-margin / (sqrt(2) sigma)).
    Returns (probability, upper bound exp(-margin^2 / (4 sigma^2)))."""
    m = np.asarray(margin, np.float64)
    if sigma <= 0:
        raise ValueError("sigma must be positive")
    p = _phi(-m / (math.sqrt(2.0) * sigma))
    bound = np.exp(-(m * m) / (4.0 * sigma * sigma))
    return p, bound


def model_flip_rates(margin, edges, sigma: float, status=None):
    """Mean model flip probability of the rows in each half-open margin bin
    [edges[j-1], edges[j]) (edges[-1] = 0), rows with a nonzero status left
    out.  Returns (rates [n_edges], counts [n_edges]); NaN for an empty bin."""
    m = np.asarray(margin, np.float64)
    keep = np.ones(m.shape, bool) if status is None else np.asarray(status) == 0
    m = m[keep]
    e = np.asarray(edges, np.float64)
    j = np.searchsorted(e, m, side="right")  # first edge strictly above m
    p, _ = flip_probability(m, sigma)
    rates = np.full(e.size, np.nan)
    counts = np.zeros(e.size, np.int64)
    for b in range(e.size):
        sel = j == b
        counts[b] = int(sel.sum())
        if counts[b]:
            rates[b] = float(p[sel].mean())
    return rates, counts


def flip_rates(bins):
    """Measured flip rate per bin (flips / count; NaN for an empty bin) from the
    structured bin records of lcmp_bin_report (fields count, flips)."""
    c = np.asarray(bins["count"], np.float64)
    f = np.asarray(bins["flips"], np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(c > 0, f / np.where(c > 0, c, 1), np.nan)


def group_quantiles(values, groups=None, qs=(0.5,), status=None):
    """Quantiles of `values` (e.g. kl_full) per group id.  Returns
    {group: array of quantiles}; rows with a nonzero status are left out."""
    v = np.asarray(values, np.float64)
    g = np.zeros(v.shape, np.int64) if groups is None else np.asarray(groups)
    keep = np.ones(v.shape, bool) if status is None else np.asarray(status) == 0
    out = {}
    for gid in np.unique(g[keep]):
        sel = keep & (g == gid)
        out[int(gid)] = np.quantile(v[sel], qs)
    return out


def empirical_cdf(values, points=None):
    """(x, F(x)) of the empirical CDF at `points` (default: the sorted values)."""
    v = np.sort(np.asarray(values, np.float64))
    x = v if points is None else np.asarray(points, np.float64)
    return x, np.searchsorted(v, x, side="right") / max(v.size, 1)


def perplexity(logp, groups=None):
    """exp(-mean ln q(target)) per group ({group: perplexity}); NaN rows are
    left out."""
    lp = np.asarray(logp, np.float64)
    g = np.zeros(lp.shape, np.int64) if groups is None else np.asarray(groups)
    ok = ~np.isnan(lp)
    return {int(gid): float(np.exp(-lp[ok & (g == gid)].mean())) for gid in np.unique(g[ok])}


def total_variation(p, q) -> float:
    """Total-variation distance of two distributions: half the L1 distance."""
    p = np.asarray(p, np.float64)
    q = np.asarray(q, np.float64)
    return 0.5 * float(np.abs(p - q).sum())


def accuracy_gap_bound(kl_per_step) -> float:
    """Upper bound on |Acc_base - Acc_cand| for answers sampled from the
    baseline: total variation of the whole-answer distributions, bounded by
    Pinsker through the chain rule: sqrt(1/2 * sum_t KL_t) (capped at 1)."""
    total = float(np.sum(np.asarray(kl_per_step, np.float64)))
    return min(1.0, math.sqrt(0.5 * total))


def kl_per_step_for_gap(gap: float, steps: int) -> float:
    """Mean per-step KL at which the bound above first allows an accuracy gap
    `gap` over `steps` steps: 2 gap^2 / steps."""
    return 2.0 * gap * gap / steps
