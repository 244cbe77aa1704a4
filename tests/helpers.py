"""Shared helpers of the GPU parity tests: device round trips through the C ABI
and element-by-element comparison against the oracle with the stated bar.

Tolerances (derived in the design notes from the arithmetic of the kernels):
  KL (full and top-k)   |gpu - oracle| <= 1e-7 + 1e-4 |oracle|
  lse_base / lse_cand   |gpu - oracle| <= 2e-6 * max(1, |oracle|)
  error norms           relative 1e-6 (absolute 1e-300 floor for zeros)
  indices, flips, margins, status, bitwise counts: bit-exact
"""
import numpy as np

KL_ABS, KL_REL = 1e-7, 1e-4
LSE_REL = 2e-6
NORM_REL = 1e-6


def to_device(arr: np.ndarray, device="cuda"):
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(arr).to(device)


def gpu_compare(base: np.ndarray, cand: np.ndarray, k=20, with_bitdiff=False, v=None):
    import torch
    import logit_distribution_diffing_amd as L
    tb, tc = to_device(base), to_device(cand)
    out = L.lcmp_compare_logits(tb, tc, k=k, with_bitdiff=with_bitdiff, v=v)
    torch.cuda.synchronize()
    res = {key: val.cpu().numpy() for key, val in out.items() if key != "bitdiff"}
    if with_bitdiff:
        res["bitdiff"] = L.unpack_bitdiff(out["bitdiff"])
    return res


def assert_kl_close(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf), f"{what}: infinities differ"
    fin = ~inf
    err = np.abs(got[fin] - ref[fin])
    tol = KL_ABS + KL_REL * np.abs(ref[fin])
    bad = np.flatnonzero(err > tol)
    assert bad.size == 0, (f"{what}: {bad.size} rows out of tolerance, worst row "
                           f"{np.flatnonzero(fin)[bad[np.argmax(err[bad] / tol[bad])]]} "
                           f"err/tol={np.max(err[bad] / tol[bad]):.3g}")


def assert_compare_equal(g: dict, o: dict, rows=None):
    """GPU outputs g (all rows or the subset `rows`) against oracle outputs o."""
    sel = slice(None) if rows is None else rows
    gs = {kk: vv[sel] for kk, vv in g.items() if kk != "bitdiff"}
    assert np.array_equal(gs["status"], o["status"]), "status differs"
    ok = o["status"] == 0
    for f in ("topk_idx", "top1_base", "top2_base", "top1_cand", "flip"):
        assert np.array_equal(gs[f], o[f]), f"{f} differs at rows {np.flatnonzero((gs[f] != o[f]).reshape(len(ok), -1).any(1))[:8]}"
    assert np.array_equal(gs["margin"][ok], o["margin"][ok]), "margin not bit-exact"
    assert_kl_close(gs["kl_full"][ok], o["kl_full"][ok], "kl_full")
    assert_kl_close(gs["kl_topk"][ok], o["kl_topk"][ok], "kl_topk")
    for f in ("lse_base", "lse_cand"):
        err = np.abs(gs[f][ok] - o[f][ok])
        tol = LSE_REL * np.maximum(1.0, np.abs(o[f][ok]))
        assert np.all(err <= tol), f"{f}: worst err/tol {np.max(err / tol):.3g}"
    bad = ~ok
    if bad.any():
        assert np.all(np.isnan(gs["kl_full"][bad])) and np.all(gs["top1_base"][bad] == -1)


def assert_bitdiff_equal(g, o):
    for f in ("ndiff", "first_diff", "nonfinite_a", "nonfinite_b", "max_ulp"):
        assert np.array_equal(g[f], o[f]), f"{f} differs at rows {np.flatnonzero(g[f] != o[f])[:8]}"
    for f in ("max_abs", "sum_abs", "sum_sq_diff", "sum_sq_base", "mean_abs", "rel_l2"):
        gv, ov = g[f].astype(np.float64), o[f].astype(np.float64)
        same_inf = np.isinf(gv) == np.isinf(ov)
        assert same_inf.all(), f"{f}: infinities differ"
        fin = ~np.isinf(ov)
        err = np.abs(gv[fin] - ov[fin])
        tol = NORM_REL * np.abs(ov[fin]) + 1e-300
        assert np.all(err <= tol), f"{f}: worst rel err {np.max(err / np.maximum(np.abs(ov[fin]), 1e-300)):.3g}"
