"""Host analytics (CPU only): the flip model, the accuracy-gap bound, total
variation, per-group quantiles and perplexity, pinned to the numbers the page
"在 agent 时代如何快速验证 kernel 对精度的影响" prints (tests/golden/flip_phi.txt,
tests/golden/tv_pinsker.txt), to closed forms, to a Monte-Carlo run of the noise
model itself, and to the oracle's margin binning."""
import math
import os

import numpy as np
import pytest

from logit_distribution_diffing_amd import analytics as A

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_flip_probability_matches_page():
    for sigma, margin, page, rtol in _rows("flip_phi.txt"):
        p, bound = A.flip_probability(float(margin), float(sigma))
        assert abs(float(p) - float(page)) <= float(rtol) * float(page), (margin, float(p))
        assert float(p) <= float(bound)


def test_flip_probability_special_values():
    p, bound = A.flip_probability(np.array([0.0, 1e-3, 10.0]), 0.1)
    assert p[0] == 0.5 and bound[0] == 1.0          # a tie flips half the time
    assert 0.49 < p[1] < 0.5
    assert p[2] < 1e-200
    # scale invariance: only margin / sigma matters
    assert np.allclose(A.flip_probability(0.3, 0.2)[0], A.flip_probability(0.03, 0.02)[0])
    with pytest.raises(ValueError):
        A.flip_probability(0.1, 0.0)


def test_flip_model_matches_monte_carlo_per_bin():
    """The model rate per bin equals the flip rate of a simulation of the model's
    own assumption (independent Gaussian noise on the top two logits) within
    binomial error, and the rows per bin equal the oracle's bin counts."""
    import oracle
    rng = np.random.default_rng(7)
    sigma, n = 0.1, 400_000
    margin = rng.exponential(0.2, n)
    noise = rng.normal(0.0, sigma, (n, 2))
    flip = (margin + noise[:, 0] - noise[:, 1] < 0).astype(np.uint8)
    edges = [0.02, 0.05, 0.1, 0.2, 0.5, 1.0]
    rates, counts = A.model_flip_rates(margin, edges, sigma)
    zeros = np.zeros(n)
    bins, _ = oracle.bin_report(margin, flip, zeros, zeros, edges)
    assert np.array_equal(counts, bins[0]["count"])
    measured = A.flip_rates(bins[0])
    for b in range(len(edges)):
        se = math.sqrt(max(rates[b] * (1 - rates[b]), 1e-12) / counts[b])
        assert abs(measured[b] - rates[b]) <= 5 * se + 1e-6, (b, measured[b], rates[b])
    # a status-flagged row leaves its bin, as in the bin report
    st = np.zeros(n, np.uint8)
    st[np.argmin(margin)] = 1
    _, c2 = A.model_flip_rates(margin, edges, sigma, status=st)
    assert c2[0] == counts[0] - 1


def test_flip_rates_of_empty_bin_is_nan():
    bins = np.zeros(3, dtype=[("count", np.int64), ("flips", np.int64)])
    bins["count"] = [4, 0, 10]
    bins["flips"] = [1, 0, 0]
    r = A.flip_rates(bins)
    assert r[0] == 0.25 and math.isnan(r[1]) and r[2] == 0.0


def test_accuracy_gap_bound_and_tv_match_page():
    for kind, a, b, page, rtol in _rows("tv_pinsker.txt"):
        page, rtol = float(page), float(rtol)
        if kind == "bound":
            got = A.accuracy_gap_bound(np.full(int(a), float(b)))
            # the page rounds sqrt(0.175) = 0.418 down to 0.4
            assert abs(got - math.sqrt(0.175)) < 1e-12
            assert round(got, 1) == page
        elif kind == "gap":
            got = A.kl_per_step_for_gap(float(a), int(b))
            assert abs(got - page) <= rtol * page
        else:
            p = [float(x) for x in a.split(",")]
            q = [float(x) for x in b.split(",")]
            assert abs(A.total_variation(p, q) - page) <= rtol + 1e-15


def test_bound_inverts_and_caps():
    kl = A.kl_per_step_for_gap(0.05, 300)
    assert abs(A.accuracy_gap_bound(np.full(300, kl)) - 0.05) < 1e-12
    assert A.accuracy_gap_bound([10.0]) == 1.0
    assert A.accuracy_gap_bound([]) == 0.0


def test_pinsker_holds_on_random_distributions():
    """TV <= sqrt(KL / 2) for random pairs; equality fails only by rounding."""
    rng = np.random.default_rng(3)
    for _ in range(200):
        p = rng.dirichlet(np.full(50, 0.3))
        q = rng.dirichlet(np.full(50, 0.3))
        q = 0.9 * q + 0.1 * p
        kl = float(np.sum(p * (np.log(p) - np.log(q))))
        assert A.total_variation(p, q) <= math.sqrt(0.5 * kl) + 1e-12
    assert A.total_variation([1, 0], [0, 1]) == 1.0


def test_group_quantiles_and_cdf():
    v = np.array([5.0, 1.0, 3.0, 2.0, 4.0, 100.0, 7.0])
    g = np.array([0, 0, 0, 1, 1, 1, 0])
    st = np.array([0, 0, 0, 0, 0, 1, 0], np.uint8)
    q = A.group_quantiles(v, g, qs=(0.0, 0.5, 1.0), status=st)
    assert list(q[0]) == [1.0, 4.0, 7.0]       # 1, 3, 5, 7
    assert list(q[1]) == [2.0, 3.0, 4.0]       # the flagged 100 is left out
    x, F = A.empirical_cdf(v)
    assert np.all(np.diff(F) > 0) and F[-1] == 1.0 and x[0] == 1.0
    _, F2 = A.empirical_cdf(v, [0.0, 3.0, 1e9])
    assert list(F2) == [0.0, 3 / 7, 1.0]


def test_perplexity_closed_forms():
    v = 151936
    lp = np.full(1000, -math.log(v))            # uniform over the vocabulary
    assert abs(A.perplexity(lp)[0] - v) < 1e-6 * v
    lp2 = np.array([math.log(0.5), math.log(0.125), float("nan")])
    g = np.array([0, 0, 1])
    assert abs(A.perplexity(lp2, g)[0] - 4.0) < 1e-12   # geometric mean of 1/p
    assert 1 not in A.perplexity(lp2, g)
