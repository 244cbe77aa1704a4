"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties an oracle function to something other than the oracle itself:
values the logit page prints for its worked examples (tests/golden/), library
routines for special cases (scipy rel_entr / softmax, torch kl_div), closed
forms, invariants, brute force on tiny inputs and known answers by
construction.  All run on the CPU.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _kv(name):
    return {r[0]: r[1:] for r in _golden(name)}


def _logits(p):
    return np.log(np.asarray(p, np.float64)).astype(np.float32)[None, :]


# ------------------------------------------------------------------ KL pins
def test_cat_dog_kl_matches_page():
    g = _kv("cat_dog.txt")
    p = np.array(g["p"], float)
    q = np.array(g["q"], float)
    r = oracle.compare(_logits(p), _logits(q), k=20)
    assert r["status"][0] == 0
    assert abs(r["kl_full"][0] - float(g["kl"][0])) <= float(g["tol"][0])
    # the other direction or another log base would miss the page's value
    assert abs(r["kl_full"][0] - 0.12) < 0.005
    # library special case on the widened float32 inputs
    pf = scipy.special.softmax(_logits(p).astype(np.float64)[0])
    qf = scipy.special.softmax(_logits(q).astype(np.float64)[0])
    assert r["kl_full"][0] == pytest.approx(scipy.special.rel_entr(pf, qf).sum(), rel=1e-12)
    # k covers the vocabulary: the top-k form is the full KL
    assert r["kl_topk"][0] == pytest.approx(r["kl_full"][0], rel=1e-12)


def test_cat_dog_top2_plus_other_is_merged_kl():
    """Top-2 + other is the KL of the 3-bucket merged distributions (library rel_entr)."""
    g = _kv("cat_dog.txt")
    p = np.array(g["p"], float)
    q = np.array(g["q"], float)
    r = oracle.compare(_logits(p), _logits(q), k=2)
    pf = scipy.special.softmax(_logits(p).astype(np.float64)[0])
    qf = scipy.special.softmax(_logits(q).astype(np.float64)[0])
    pm = np.array([pf[0], pf[1], pf[2] + pf[3]])
    qm = np.array([qf[0], qf[1], qf[2] + qf[3]])
    assert list(r["topk_idx"][0]) == [0, 1]
    assert r["kl_topk"][0] == pytest.approx(scipy.special.rel_entr(pm, qm).sum(), rel=1e-12)
    assert r["kl_topk"][0] < r["kl_full"][0]


def _long_tail_rows():
    g = _kv("long_tail.txt")
    n_tail = int(g["tail_tokens"][0])
    tp = float(g["tail_p"][0])
    n_up, p_up = int(g["moved_up"][0]), float(g["moved_up"][1])
    n_dn, p_dn = int(g["moved_down"][0]), float(g["moved_down"][1])
    head = 20
    hp = (1.0 - n_tail * tp) / head
    p = np.array([hp] * head + [tp] * n_tail)
    q = np.array([hp] * head + [p_up] * n_up + [p_dn] * n_dn)
    return g, p, q


def test_long_tail_full_kl_matches_page_and_topk_ignores_it():
    g, p, q = _long_tail_rows()
    r = oracle.compare(_logits(p), _logits(q), k=20)
    assert abs(r["kl_full"][0] - float(g["kl_full"][0])) <= float(g["tol"][0])
    # closed form of the example: 0.005 * ln(4/3); float32 logits cost ~1e-8
    assert r["kl_full"][0] == pytest.approx(0.005 * math.log(4.0 / 3.0), rel=2e-5)
    # head unchanged and the tail total unchanged: top-20 + other sees nothing
    assert abs(r["kl_topk"][0]) < 1e-9
    assert sorted(r["topk_idx"][0]) == list(range(20))


# ------------------------------------------------------------------ margin pins
def test_two_way_margin_probabilities_match_page():
    for m, p_page, tol in _golden("margin_two_way.txt"):
        m, p_page, tol = float(m), float(p_page), float(tol)
        a = np.array([[m, 0.0]], np.float32)
        r = oracle.compare(a, a.copy(), k=1)
        p_top = math.exp(float(a[0, 0]) - r["lse_base"][0])
        assert abs(p_top - p_page) <= tol
        assert p_top == pytest.approx(scipy.special.expit(float(a[0, 0])), rel=1e-12)
        assert r["margin"][0] == float(a[0, 0])
        assert (r["top1_base"][0], r["top2_base"][0]) == (0, 1)


# ------------------------------------------------------------------ flip model
def test_phi_flip_model_values_match_page():
    for sigma, m, page, rtol in _golden("flip_phi.txt"):
        sigma, m, page, rtol = map(float, (sigma, m, page, rtol))
        phi = scipy.stats.norm.cdf(-m / (math.sqrt(2.0) * sigma))
        assert abs(phi - page) <= rtol * page
        assert phi <= math.exp(-m * m / (4.0 * sigma * sigma))


@pytest.mark.parametrize("margin,rows", [(0.1, 100000), (0.3, 100000), (0.5, 400000)])
def test_monte_carlo_flip_rate_tracks_phi(margin, rows):
    """Two-token rows with independent N(0, sigma^2) noise on both logits: the
    oracle's flip rate matches Phi(-m / (sqrt(2) sigma)) within binomial error."""
    sigma = 0.1
    z = synth.normals(0xF11B, 7, int(margin * 1000), 2 * rows).reshape(rows, 2)
    a = np.tile(np.array([margin, 0.0], np.float32), (rows, 1))
    b = (a.astype(np.float64) + sigma * z).astype(np.float32)
    r = oracle.compare(a, b, k=2)
    rate = r["flip"].mean()
    p = scipy.stats.norm.cdf(-float(a[0, 0]) / (math.sqrt(2.0) * sigma))
    sd = math.sqrt(p * (1 - p) / rows)
    assert abs(rate - p) <= 5 * sd + 1.0 / rows


# ------------------------------------------------------------------ small-delta pin
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_small_delta_variance_approximation(seed):
    """KL ~= 1/2 (sum p d^2 - (sum p d)^2) for small Gaussian logit errors d."""
    v = 2000
    x = synth.normals(seed, 8, 0, v)
    d = 1e-3 * synth.normals(seed, 9, 0, v)
    a = x.astype(np.float32)[None]
    b = (x - d).astype(np.float32)[None]
    r = oracle.compare(a, b, k=20)
    dd = a[0].astype(np.float64) - b[0].astype(np.float64)
    p = scipy.special.softmax(a[0].astype(np.float64))
    approx = 0.5 * (np.sum(p * dd * dd) - np.sum(p * dd) ** 2)
    assert r["kl_full"][0] == pytest.approx(approx, rel=1e-3)


# ------------------------------------------------------------------ library cross-checks
@pytest.mark.parametrize("seed", range(5))
def test_full_kl_against_scipy_and_torch(seed):
    import torch
    rng = np.random.default_rng(seed)
    n, v = 8, 300
    a = (2.0 * rng.standard_normal((n, v))).astype(np.float32)
    b = (a + 0.3 * rng.standard_normal((n, v))).astype(np.float32)
    r = oracle.compare(a, b, k=20)
    for i in range(n):
        pf = scipy.special.softmax(a[i].astype(np.float64))
        qf = scipy.special.softmax(b[i].astype(np.float64))
        ref = scipy.special.rel_entr(pf, qf).sum()
        assert r["kl_full"][i] == pytest.approx(ref, rel=1e-10)
        lp = torch.log_softmax(torch.from_numpy(a[i].astype(np.float64)), 0)
        lq = torch.log_softmax(torch.from_numpy(b[i].astype(np.float64)), 0)
        tk = torch.nn.functional.kl_div(lq, lp, reduction="sum", log_target=True).item()
        assert r["kl_full"][i] == pytest.approx(tk, rel=1e-10)
        assert r["lse_base"][i] == pytest.approx(
            scipy.special.logsumexp(a[i].astype(np.float64)), rel=1e-14)


# ------------------------------------------------------------------ top-k brute force
def _brute_topk(x, k):
    left = list(range(len(x)))
    out = []
    for _ in range(min(k, len(x))):
        best = left[0]
        for i in left:
            if x[i] > x[best]:
                best = i
        out.append(best)
        left.remove(best)
    return out


def test_topk_and_argmax_brute_force_with_ties():
    rng = np.random.default_rng(11)
    for trial in range(400):
        v = int(rng.integers(2, 13))
        k = int(rng.integers(1, 14))
        a = rng.integers(0, 3, v).astype(np.float32)[None]
        b = rng.integers(0, 3, v).astype(np.float32)[None]
        r = oracle.compare(a, b, k=k)
        ref = _brute_topk(list(a[0]), k)
        got = [i for i in r["topk_idx"][0] if i >= 0]
        assert got == ref, (a, k)
        assert all(i == -1 for i in r["topk_idx"][0][len(ref):])
        ref_b = _brute_topk(list(b[0]), 1)[0]
        assert r["top1_cand"][0] == ref_b
        assert r["flip"][0] == int(ref_b != ref[0])
        top2 = _brute_topk(list(a[0]), 2)
        assert (r["top1_base"][0], r["top2_base"][0]) == (top2[0], top2[1])
        assert r["margin"][0] == float(a[0, top2[0]]) - float(a[0, top2[1]])


def test_topk_against_sort_on_larger_rows():
    rng = np.random.default_rng(12)
    a = rng.integers(-20, 20, (16, 5000)).astype(np.float32)  # many ties
    r = oracle.compare(a, a + 1, k=64)
    for i in range(16):
        ref = np.lexsort((np.arange(5000), -a[i]))[:64]
        assert np.array_equal(r["topk_idx"][i], ref)


def test_negative_zero_ties_with_positive_zero():
    a = np.array([[-0.0, 0.0, -1.0]], np.float32)
    r = oracle.compare(a, a.copy(), k=2)
    assert list(r["topk_idx"][0]) == [0, 1]
    assert r["margin"][0] == 0.0
    assert r["top1_cand"][0] == 0


# ------------------------------------------------------------------ invariants
def test_identical_inputs_give_exact_zero():
    a, _ = synth.tiny(synth.SEED_BASE, 0, 16, 1024)
    r = oracle.compare(a, a.copy(), k=20)
    assert np.all(r["kl_full"] == 0.0) and np.all(r["kl_topk"] == 0.0)
    assert np.all(r["flip"] == 0)
    bd = oracle.bitdiff(a, a.copy())
    assert np.all(bd["ndiff"] == 0) and np.all(bd["first_diff"] == -1)
    assert np.all(bd["max_ulp"] == 0) and np.all(bd["max_abs"] == 0.0)


def test_kl_nonnegative_and_topk_below_full():
    a, b = synth.tiny(synth.SEED_BASE, 0, 64, 1024)
    for k in (1, 2, 5, 20, 100):
        r = oracle.compare(a, b, k=k)
        assert np.all(r["kl_full"] > 0) and np.all(r["kl_topk"] >= -1e-15)
        assert np.all(r["kl_topk"] <= r["kl_full"] * (1 + 1e-12))


def test_topk_equals_full_when_bucket_holds_at_most_one_token():
    a, b = synth.tiny(synth.SEED_BASE, 0, 8, 64)
    for k in (63, 64, 200):
        r = oracle.compare(a, b, k=k)
        assert np.allclose(r["kl_topk"], r["kl_full"], rtol=1e-12, atol=0)


def test_exact_shift_leaves_everything_but_lse_unchanged():
    a, b = synth.tiny(synth.SEED_BASE, 0, 8, 1024)
    r0 = oracle.compare(a, b, k=20)
    # power-of-two scale of a shift keeps the float32 values exact here
    r1 = oracle.compare(a + np.float32(4.0), b - np.float32(2.0), k=20)
    assert np.array_equal(r0["topk_idx"], r1["topk_idx"])
    assert np.array_equal(r0["top1_cand"], r1["top1_cand"])
    assert np.allclose(r0["kl_full"], r1["kl_full"], rtol=1e-6)
    assert np.allclose(r0["kl_topk"], r1["kl_topk"], rtol=1e-5, atol=1e-12)


def test_flagged_and_infinite_rows():
    v = 16
    a = np.zeros((5, v), np.float32)
    b = np.zeros((5, v), np.float32)
    a[0, 3] = np.nan
    b[1, 4] = np.inf
    a[2, :] = -np.inf
    b[3, 5] = -np.inf  # candidate excludes a token the baseline keeps -> KL = inf
    a[4, 7:] = -np.inf  # baseline excludes tokens: they add nothing
    b[4, 7:] = 1.0
    r = oracle.compare(a, b, k=4)
    assert list(r["status"]) == [1, 1, 2, 0, 0]
    assert np.isnan(r["kl_full"][0]) and r["top1_base"][0] == -1
    assert np.all(r["topk_idx"][2] == -1)
    assert r["kl_full"][3] == np.inf
    # token 5 lies in the "other" bucket, which keeps candidate mass: finite
    pm = np.array([1 / 16] * 4 + [12 / 16])
    qm = np.array([1 / 15] * 4 + [11 / 15])
    assert r["kl_topk"][3] == pytest.approx(scipy.special.rel_entr(pm, qm).sum(), rel=1e-12)
    r5 = oracle.compare(a[3:4], b[3:4], k=6)  # now token 5 is in the head
    assert r5["kl_topk"][0] == np.inf
    p = np.full(7, 1 / 7)
    q = np.exp(np.zeros(7)) / (7 + 9 * math.e)
    assert r["kl_full"][4] == pytest.approx(np.sum(p * np.log(p / q)), rel=1e-12)


# ------------------------------------------------------------------ bitwise pins
def _f32(vals):
    return np.array([vals], np.float32)


def test_bitdiff_hand_cases_fp32():
    one = np.float32(1.0)
    nxt = np.nextafter(one, np.float32(2.0))
    a = _f32([1.0, 0.0, 1.0, 3.0, -2.0])
    b = _f32([nxt, -0.0, 1.0, 3.0, -2.0])
    bd = oracle.bitdiff(a, b)[0]
    assert bd["ndiff"] == 2 and bd["first_diff"] == 0
    assert bd["max_ulp"] == 1  # next float, and +0 vs -0
    assert bd["max_abs"] == pytest.approx(float(nxt) - 1.0, rel=0)
    # opposite signs: distance through zero
    bd = oracle.bitdiff(_f32([1.0]), _f32([-1.0]))[0]
    assert bd["max_ulp"] == 2 * 0x3F800000 + 1
    assert bd["rel_l2"] == 2.0 and bd["mean_abs"] == 2.0


def test_bitdiff_hand_cases_bf16_and_norms():
    # bf16 patterns: 1.0 = 0x3f80; next = 0x3f81; -0 = 0x8000
    a = np.array([[0x3F80, 0x0000, 0x4040, 0x4080]], np.uint16)
    b = np.array([[0x3F80, 0x8000, 0x4041, 0x4080]], np.uint16)
    bd = oracle.bitdiff(a, b)[0]
    assert bd["ndiff"] == 2 and bd["first_diff"] == 1 and bd["max_ulp"] == 1
    # norms: values 1, 0, 3, 4 vs 1, -0, 3.015625, 4
    assert bd["max_abs"] == pytest.approx(0.015625)
    assert bd["sum_sq_base"] == pytest.approx(1 + 9 + 16)
    assert bd["rel_l2"] == pytest.approx(0.015625 / math.sqrt(26))
    assert bd["mean_abs"] == pytest.approx(0.015625 / 4)


def test_bitdiff_nonfinite_counted_and_excluded():
    a = _f32([np.inf, 1.0, np.nan, 2.0])
    b = _f32([np.inf, 1.0, 1.0, -np.inf])
    bd = oracle.bitdiff(a, b)[0]
    assert bd["nonfinite_a"] == 2 and bd["nonfinite_b"] == 2
    assert bd["ndiff"] == 2 and bd["first_diff"] == 2
    assert bd["max_abs"] == 0.0 and bd["sum_sq_base"] == 1.0  # only column 1 counts


def test_bitdiff_mixed_dtypes_compare_in_fp32():
    a = _f32([1.0, 1.00390625, 2.0])  # 1 + 2^-8 is not a bf16 value
    b = np.array([[0x3F80, 0x3F80, 0x4000]], np.uint16)
    bd = oracle.bitdiff(a, b)[0]
    assert bd["ndiff"] == 1 and bd["first_diff"] == 1
    assert bd["max_ulp"] == 2 ** 15  # 2^-8 is 2^15 fp32 units above 1.0


@pytest.mark.parametrize("t", [1, 17, 65, 1024])
def test_bitdiff_known_answers_by_construction(t):
    """ULP injections: per-row count, first column and largest step are known."""
    cols = 5120
    seed = synth.WORKLOADS["sweep"]["seed"]
    a = synth.bf16_normal(seed, 0, t, cols)
    b, pos, steps = synth.inject_ulp(seed, t, a, 0.001)
    assert pos.size == round(0.001 * t * cols)
    bd = oracle.bitdiff(a, b)
    rows = pos // cols
    for r in range(t):
        sel = rows == r
        assert bd["ndiff"][r] == sel.sum()
        assert bd["first_diff"][r] == (pos[sel].min() % cols if sel.any() else -1)
        assert bd["max_ulp"][r] == (np.abs(steps[sel]).max() if sel.any() else 0)


# ------------------------------------------------------------------ bins
def test_bin_report_hand_counted():
    edges = np.array(synth.DEFAULT_EDGES)
    margin = np.array([0.0, 0.0, 0.05, 0.1, 0.3, 0.99, 1.0, 1.5, 3.0, 2.0, 0.2])
    flip = np.array([1, 0, 1, 0, 1, 1, 1, 1, 0, 1, 0], np.uint8)
    kl = np.arange(11, dtype=np.float64) * 0.01
    klf = kl * 2
    status = np.zeros(11, np.uint8)
    status[10] = 1
    bins, summ = oracle.bin_report(margin, flip, kl, klf, edges, status=status)
    b = bins[0]
    # [0,.1): rows 0,1,2   [.1,.25): row 3   [.25,.5): row 4   [.5,1): row 5
    # [1,2): rows 6,7      [2,inf): rows 8,9          row 10 excluded
    assert list(b["count"]) == [3, 1, 1, 1, 2, 2]
    assert list(b["flips"]) == [2, 0, 1, 1, 2, 1]
    assert list(b["ties"]) == [2, 0, 0, 0, 0, 0]
    assert list(b["tie_flips"]) == [1, 0, 0, 0, 0, 0]
    assert b["sum_kl_topk"][0] == pytest.approx(0.00 + 0.01 + 0.02)
    assert b["sum_kl_full"][4] == pytest.approx(2 * (0.06 + 0.07))
    assert b["max_kl_topk"][5] == pytest.approx(0.09)
    # flips strictly above margin 1: rows 7 (1.5) and 9 (2.0); row 6 sits at 1.0
    assert summ[0]["big_margin_flips"] == 2
    assert summ[0]["excluded"] == 1 and summ[0]["unbinned"] == 0


def test_bin_report_without_full_kl():
    """A comparison against a record has no full KL: the counts and top-k sums
    are those of the report with it, and sum_kl_full is NaN exactly in the bins
    that hold rows."""
    edges = np.array(synth.DEFAULT_EDGES)
    margin = np.array([0.0, 0.05, 0.3, 1.5, 3.0])
    flip = np.array([1, 0, 1, 1, 0], np.uint8)
    kl = np.arange(5, dtype=np.float64) * 0.01
    b1, s1 = oracle.bin_report(margin, flip, kl, kl * 2, edges)
    b0, s0 = oracle.bin_report(margin, flip, kl, None, edges)
    for f in ("count", "flips", "ties", "tie_flips", "sum_kl_topk", "max_kl_topk"):
        assert np.array_equal(b0[f], b1[f]), f
    assert s0.tobytes() == s1.tobytes()
    held = b0["count"][0] > 0
    assert np.all(np.isnan(b0["sum_kl_full"][0][held]))
    assert np.all(b0["sum_kl_full"][0][~held] == 0.0)


def test_bin_report_groups_and_unbinned():
    edges = np.array([0.5, 1.0])
    margin = np.array([0.2, 0.7, 5.0, 0.2, np.inf])
    flip = np.array([1, 0, 1, 0, 1], np.uint8)
    kl = np.ones(5)
    group = np.array([0, 1, 1, 7, 0], np.int32)  # group 7 is out of range: skipped
    bins, summ = oracle.bin_report(margin, flip, kl, kl, edges, group=group, n_groups=2)
    assert list(bins[0]["count"]) == [1, 0] and list(bins[1]["count"]) == [0, 1]
    assert summ[1]["unbinned"] == 1 and summ[1]["big_margin_flips"] == 1
    assert summ[0]["unbinned"] == 1 and summ[0]["big_margin_flips"] == 1
    assert np.isneginf(bins[0]["max_kl_topk"][1])


# ------------------------------------------------------------------ target log-probability
def test_target_logprob_cat_dog_is_log_of_page_probabilities():
    """With logits ln p, the log-probability of each token is ln p_t (the page's
    cat/dog numbers), on both sides."""
    g = _kv("cat_dog.txt")
    p = np.array(g["p"], float)
    q = np.array(g["q"], float)
    a, b = np.repeat(_logits(p), 4, 0), np.repeat(_logits(q), 4, 0)
    r = oracle.target_logprob(a, b, np.arange(4, dtype=np.int32))
    assert np.allclose(r["logp_base"], np.log(p), rtol=0, atol=1e-6)
    assert np.allclose(r["logp_cand"], np.log(q), rtol=0, atol=1e-6)


@pytest.mark.parametrize("seed", [0, 1])
def test_target_logprob_against_torch_log_softmax(seed):
    import torch
    rng = np.random.default_rng(seed)
    n, v = 6, 777
    a = (2.0 * rng.standard_normal((n, v))).astype(np.float32)
    b = (a + 0.05 * rng.standard_normal((n, v))).astype(np.float32)
    t = rng.integers(0, v, n).astype(np.int32)
    r = oracle.target_logprob(a, b, t)
    la = torch.log_softmax(torch.from_numpy(a).double(), dim=1).numpy()
    lb = torch.log_softmax(torch.from_numpy(b).double(), dim=1).numpy()
    assert np.allclose(r["logp_base"], la[np.arange(n), t], rtol=0, atol=1e-12)
    assert np.allclose(r["logp_cand"], lb[np.arange(n), t], rtol=0, atol=1e-12)


def test_target_logprob_shift_invariant_and_edge_cases():
    rng = np.random.default_rng(3)
    n, v = 8, 64
    a = rng.standard_normal((n, v)).astype(np.float32)
    b = a.copy()
    t = np.array([0, 63, 5, -1, 64, 7, 9, 11], np.int32)
    a[5, 7] = -np.inf      # the target itself has probability 0
    b[6, 3] = np.nan       # flagged row
    r = oracle.target_logprob(a, b, t)
    shifted = oracle.target_logprob(a + 4.0, b - 2.0, t)
    ok = [0, 1, 2, 7]
    assert np.allclose(r["logp_base"][ok], shifted["logp_base"][ok], rtol=0, atol=1e-6)
    assert np.array_equal(r["logp_base"][ok], r["logp_cand"][ok])  # identical rows
    assert np.all(np.isnan(r["logp_base"][[3, 4, 6]]))             # out of range, flagged
    assert r["logp_base"][5] == -np.inf
    # perplexity of a row set is exp(-mean ln q(target)); identical sides agree
    assert np.exp(-r["logp_base"][ok].mean()) == np.exp(-r["logp_cand"][ok].mean())


# ------------------------------------------------------------------ precision perturbations
def _bf16_patterns_sample():
    hi = np.arange(0, 1 << 16, 7, dtype=np.uint32)
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    u = ((hi[:, None] << 16) | lows[None, :]).ravel()
    f = u.view(np.float32)
    return f[np.isfinite(f)]


def test_keep_7_mantissa_bits_is_bf16_rounding():
    """fp32 and bf16 share the exponent range, so keeping 7 fraction bits is the
    bf16 cast (torch, round to nearest even)."""
    import torch
    x = _bf16_patterns_sample()
    ours = oracle.perturb(x, oracle.PERTURB_MANTISSA, 7)[0]
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    as_bf16 = oracle.perturb(x, oracle.PERTURB_MANTISSA, 7, out_bf16=True)[0]
    assert np.array_equal(synth.bf16_to_f32(as_bf16).view(np.uint32), ref.view(np.uint32))


def test_e4m3_against_torch_float8_in_range():
    import torch
    rng = np.random.default_rng(5)
    x = np.concatenate([_bf16_patterns_sample(),
                        (rng.standard_normal(200000) * 10 ** rng.uniform(-5, 2.6, 200000))])
    x = x.astype(np.float32)
    x = x[np.abs(x) <= 448.0]
    ours = oracle.perturb(x, oracle.PERTURB_E4M3)[0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_constants_match_page():
    g = _kv("e4m3.txt")
    tiny = np.float32(2.0 ** -9)
    x = np.array([tiny, 2.0 ** -10, np.nextafter(np.float32(2.0 ** -10), np.float32(1)),
                  np.float32(2.0 ** -11), 448.0, 460.0, 470.0, 1e6, -1e6], np.float32)
    r = oracle.perturb(x, oracle.PERTURB_E4M3)[0]
    assert r[0] == tiny and abs(float(tiny) - float(g["min_subnormal_approx"][0])) \
        <= float(g["min_subnormal_tol"][0])
    assert r[1] == 0.0 and r[3] == 0.0          # half of the smallest and below: 0
    assert r[2] == tiny                         # just above half: the smallest value
    assert r[4] == 448.0 and r[5] == 448.0      # 460 < 464: rounds to 448
    assert r[6] == 448.0 and r[7] == 448.0 and r[8] == -448.0   # saturate
    assert float(g["max_finite"][0]) == 448.0
    # scaling by 448 first: the smallest weight that survives is near 2^-10 / 448
    s = oracle.perturb(np.array([2.3e-6, 2.1e-6], np.float32), oracle.PERTURB_E4M3_SCALED)[0]
    assert s[0] > 0.0 and s[1] == 0.0
    assert 2.0 ** -10 / 448 < float(g["scaled_threshold_max"][0])


@pytest.mark.parametrize("m", [0, 4, 7, 10, 13, 16, 22, 23])
def test_keep_mantissa_closed_forms(m):
    rng = np.random.default_rng(m)
    x = (rng.standard_normal(100000) * 10 ** rng.uniform(-44, 38, 100000)).astype(np.float32)
    x = np.concatenate([x, np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, 3.4e38], np.float32)])
    x = x[np.isfinite(x) | np.isinf(x)]
    r = oracle.perturb(x, oracle.PERTURB_MANTISSA, m)[0]
    fin = np.isfinite(x) & np.isfinite(r)
    if m == 23:
        assert np.array_equal(r.view(np.uint32), x.view(np.uint32))
    # error at most half a quantum 2^(E - m), E = max(floor(log2 |x|), -126)
    xd = x[fin].astype(np.float64)
    E = np.maximum(np.floor(np.log2(np.abs(np.where(xd == 0, 1.0, xd)))), -126)
    assert np.all(np.abs(r[fin] - xd) <= np.ldexp(0.5, (E - m).astype(int)) * (1 + 1e-12))
    # idempotent, odd, monotone
    assert np.array_equal(oracle.perturb(r, oracle.PERTURB_MANTISSA, m)[0].view(np.uint32),
                          r.view(np.uint32))
    assert np.array_equal(oracle.perturb(-x, oracle.PERTURB_MANTISSA, m)[0], -r)
    order = np.argsort(x, kind="stable")
    assert np.all(np.diff(r[order][np.isfinite(r[order])]) >= 0)


# ------------------------------------------------------------------ compact record pins
_REC_INT = ("top1_base", "top2_base", "top1_cand", "flip", "topk_idx", "status")


def _assert_record_matches_full(base, cand, k, k_rec, target=None):
    """The record path must give what the full compare (pinned above) gives:
    the record is a sufficient statistic of the top-k + other comparison."""
    full = oracle.compare(base, cand, k=k)
    rec = oracle.record(base, k=k_rec, target=target)
    r = oracle.compare_record(rec, cand, k=k, target=target)
    for f in _REC_INT:
        assert np.array_equal(full[f], r[f]), f
    ok = full["status"] == 0
    for f in ("kl_topk", "margin", "lse_base", "lse_cand"):
        a, b = full[f][ok], r[f][ok]
        fin = np.isfinite(a)
        assert np.array_equal(fin, np.isfinite(b)) and np.array_equal(a[~fin], b[~fin]), f
        assert np.all(np.abs(a[fin] - b[fin]) <= 1e-12 + 1e-8 * np.abs(a[fin])), f
        assert np.all(np.isnan(r[f][~ok])), f
    if target is not None:
        lp = oracle.target_logprob(base, cand, target)
        for f in ("logp_base", "logp_cand"):
            a, b = lp[f], r[f]
            assert np.array_equal(np.isnan(a), np.isnan(b)), f
            m = ~np.isnan(a)
            assert np.all(np.abs(a[m] - b[m]) <= 1e-12 * (1 + np.abs(a[m]))), f
    return rec, r


@pytest.mark.parametrize("k,k_rec", [(1, 2), (2, 2), (5, 20), (20, 20), (20, 64), (64, 64)])
def test_record_path_equals_full_compare(k, k_rec):
    a, b = synth.tiny(11, 0, 48, 700)
    target = (np.arange(48, dtype=np.int32) * 37) % 700
    target[3] = -1
    target[4] = 700
    _assert_record_matches_full(a, b, k, k_rec, target)


def test_record_path_equals_full_compare_on_corpus_and_bf16_rows():
    a, b = synth.corpus(5, 0, 24, 4099, 1000)          # fp32 baseline, bf16 candidate
    _assert_record_matches_full(a, b, 20, 20)
    sa, sb = synth.stream(6, 0, 24, 3001)              # both bf16
    _assert_record_matches_full(sa, sb, 20, 32)


def test_record_path_with_ties_and_small_vocabularies():
    rng = np.random.default_rng(2)
    a = rng.integers(-3, 3, (64, 40)).astype(np.float32)   # many equal logits
    b = (a + rng.integers(-1, 2, a.shape)).astype(np.float32)
    _assert_record_matches_full(a, b, 20, 20)
    for v in (2, 3, 5):                                    # v <= k: nothing left over
        rec, r = _assert_record_matches_full(a[:, :v].copy(), b[:, :v].copy(), 20, 20)
        assert np.all(rec["lse_rest"] == -np.inf)
        assert np.all(rec["idx"][:, v:] == -1) and np.all(rec["val"][:, v:] == -np.inf)


def test_record_flagged_and_infinite_rows():
    v = 16
    a = np.zeros((7, v), np.float32)
    b = np.zeros((7, v), np.float32)
    a[0, 3] = np.nan                 # baseline NaN: the record itself is flagged
    b[1, 4] = np.inf                 # candidate +inf outside the head
    a[2, :] = -np.inf                # baseline empty
    b[3, 5] = -np.inf                # candidate -inf in the bucket: finite top-k KL
    b[4, :] = -np.inf                # candidate empty
    b[5, 0] = np.nan                 # candidate NaN on a head token
    a[6, 7:] = -np.inf               # baseline -inf tokens add nothing
    b[6, 7:] = 1.0
    rec, r = _assert_record_matches_full(a, b, 4, 8)
    assert list(rec["status"]) == [1, 0, 2, 0, 0, 0, 0]
    assert np.isnan(rec["lse_rest"][0]) and np.all(rec["idx"][0] == -1)
    assert list(r["status"]) == [1, 1, 2, 0, 2, 1, 0]
    r6 = oracle.compare_record(oracle.record(a[3:4], k=6), b[3:4], k=6)
    assert r6["kl_topk"][0] == np.inf    # token 5 now in the head, candidate -inf


def test_record_long_tail_example_and_merged_buckets():
    """The page's long-tail example seen through a record: head unchanged and
    tail total unchanged, so top-20 + other is zero; and with k = 2 of a record
    of 4, top-2 + other is the KL of the merged 3-bucket distributions."""
    g, p, q = _long_tail_rows()
    r = oracle.compare_record(oracle.record(_logits(p), k=20), _logits(q), k=20)
    assert abs(r["kl_topk"][0]) < 1e-9
    g = _kv("cat_dog.txt")
    p = np.array(g["p"], float)
    q = np.array(g["q"], float)
    r = oracle.compare_record(oracle.record(_logits(p), k=4), _logits(q), k=2)
    pf = scipy.special.softmax(_logits(p).astype(np.float64)[0])
    qf = scipy.special.softmax(_logits(q).astype(np.float64)[0])
    pm = np.array([pf[0], pf[1], pf[2] + pf[3]])
    qm = np.array([qf[0], qf[1], qf[2] + qf[3]])
    assert r["kl_topk"][0] == pytest.approx(scipy.special.rel_entr(pm, qm).sum(), rel=1e-12)


def test_record_rest_mass_closed_form():
    """lse_rest of a uniform row of v equal logits with k taken is ln(v - k)."""
    v, k = 1000, 20
    rec = oracle.record(np.zeros((2, v), np.float32), k=k)
    assert np.allclose(rec["lse_rest"], math.log(v - k), rtol=0, atol=1e-12)
    assert np.array_equal(rec["idx"][0], np.arange(k))   # ties: lowest indices
