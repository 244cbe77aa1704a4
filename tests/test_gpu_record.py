"""GPU parity of the compact baseline record: lcmp_record_baseline against the
oracle's record, and lcmp_compare_record against the oracle's comparison with a
record, both on records made on the GPU and on records made by the oracle
(uploaded), so each half is checked on its own.  Full-size corpus rows are
checked on a sample of positions, plus the identity with the full compare on
every row (same indices, flips, margins; KL and normalisers to tolerance)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import KL_ABS, KL_REL, LSE_REL, assert_kl_close, to_device

pytestmark = pytest.mark.gpu

INT_FIELDS = ("topk_idx", "top1_base", "top2_base", "top1_cand", "flip")


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _np(d):
    return {k: v.cpu().numpy() for k, v in d.items()}


def gpu_record(base, k_rec, target=None):
    import torch
    import logit_distribution_diffing_amd as L
    t = None if target is None else torch.from_numpy(np.ascontiguousarray(target, np.int32)).cuda()
    rec = L.lcmp_record_baseline(to_device(base), k_rec=k_rec, target=t)
    torch.cuda.synchronize()
    return rec


def gpu_compare_record(rec, cand, k=None, target=None):
    import torch
    import logit_distribution_diffing_amd as L
    t = None if target is None else torch.from_numpy(np.ascontiguousarray(target, np.int32)).cuda()
    out = L.lcmp_compare_record(rec, to_device(cand), k=k, target=t)
    torch.cuda.synchronize()
    return _np(out)


def upload_record(orec):
    import torch
    d = dict(topk_idx=torch.from_numpy(orec["idx"]).cuda(),
             topk_val=torch.from_numpy(orec["val"]).cuda(),
             lse_rest=torch.from_numpy(orec["lse_rest"]).cuda(),
             status=torch.from_numpy(orec["status"]).cuda())
    if "logp_target" in orec:
        d["logp_target"] = torch.from_numpy(orec["logp_target"]).cuda()
    return d


def _close(got, ref, what, rel=LSE_REL):
    assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{what}: NaNs differ"
    assert np.array_equal(np.isinf(got), np.isinf(ref)), f"{what}: infinities differ"
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)]), f"{what}: infinity signs"
    m = np.isfinite(ref)
    err = np.abs(got[m] - ref[m])
    tol = rel * np.maximum(1.0, np.abs(ref[m]))
    assert np.all(err <= tol), f"{what}: worst err/tol {np.max(err / tol):.3g}"


def assert_record_equal(g, o):
    g = _np(g)
    assert np.array_equal(g["status"], o["status"]), "status differs"
    assert np.array_equal(g["topk_idx"], o["idx"]), "topk_idx differs"
    assert np.array_equal(g["topk_val"].view(np.uint32), o["val"].view(np.uint32)), "topk_val"
    _close(g["lse_rest"], o["lse_rest"], "lse_rest")
    if "logp_target" in o:
        _close(g["logp_target"], o["logp_target"], "logp_target")


def assert_compare_record_equal(g, o):
    assert np.array_equal(g["status"], o["status"]), "status differs"
    ok = o["status"] == 0
    for f in INT_FIELDS:
        assert np.array_equal(g[f], o[f]), f"{f} differs"
    assert np.array_equal(g["margin"][ok], o["margin"][ok]), "margin not bit-exact"
    assert_kl_close(g["kl_topk"][ok], o["kl_topk"][ok], "kl_topk")
    for f in ("lse_base", "lse_cand", "logp_base", "logp_cand"):
        if f in o:
            _close(g[f], o[f], f)
    bad = ~ok
    if bad.any():
        assert np.all(np.isnan(g["kl_topk"][bad])) and np.all(g["top1_base"][bad] == -1)


def check_both(base, cand, k, k_rec, target=None):
    """GPU record vs oracle record; GPU compare on the GPU record and on the
    uploaded oracle record vs the oracle's compare."""
    orec = oracle.record(base, k=k_rec, target=target)
    grec = gpu_record(base, k_rec, target)
    assert_record_equal(grec, orec)
    ocmp = oracle.compare_record(orec, cand, k=k, target=target)
    assert_compare_record_equal(gpu_compare_record(grec, cand, k, target), ocmp)
    assert_compare_record_equal(gpu_compare_record(upload_record(orec), cand, k, target), ocmp)
    return grec


def test_tiny_workload_record_parity():
    w = synth.WORKLOADS["tiny"]
    _case("record tiny 64x1024 f32/f32")
    a, b = synth.tiny(w["seed"], 0, w["n"], w["v"])
    target = (np.arange(w["n"], dtype=np.int32) * 53) % w["v"]
    target[5] = -1
    check_both(a, b, 20, 20, target)


@pytest.mark.parametrize("v", [2, 3, 19, 20, 21, 511, 512, 513, 1023, 1024, 1025, 2047, 2049,
                               4097, 20001])
@pytest.mark.parametrize("k,k_rec", [(1, 2), (20, 20), (5, 64), (64, 64)])
def test_ragged_vocab_sizes(v, k, k_rec):
    _case(f"record ragged v={v} k={k} k_rec={k_rec}")
    rng = np.random.default_rng(v * 7 + k)
    n = 7
    a = (1.5 * rng.standard_normal((n, v))).astype(np.float32)
    b = (a + 0.05 * rng.standard_normal((n, v))).astype(np.float32)
    target = rng.integers(0, v, n).astype(np.int32)
    check_both(a, b, k, k_rec, target)


@pytest.mark.parametrize("tb,tc", [("f32", "f32"), ("f32", "bf16"), ("bf16", "f32"),
                                   ("bf16", "bf16")])
def test_dtype_combinations(tb, tc):
    _case(f"record dtypes {tb}/{tc}")
    import torch
    rng = np.random.default_rng(15)
    n, v = 33, 5000
    x = (1.5 * rng.standard_normal((n, v))).astype(np.float32)
    y = (x + 0.02 * rng.standard_normal((n, v))).astype(np.float32)

    def conv(t, arr):
        if t == "f32":
            return arr
        return torch.from_numpy(arr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    check_both(conv(tb, x), conv(tc, y), 20, 32)


def test_unaligned_rows_take_the_checked_path():
    """Row strides that are not a multiple of 16 bytes stream through the
    bounds-checked loads instead of the LDS ring."""
    import torch
    import logit_distribution_diffing_amd as L
    _case("record unaligned rows")
    rng = np.random.default_rng(4)
    n, v = 9, 3001
    a = (2.0 * rng.standard_normal((n, v + 1))).astype(np.float32)
    b = (a + 0.03 * rng.standard_normal((n, v + 1))).astype(np.float32)
    da, db = to_device(a), to_device(b)
    rec = L.lcmp_record_baseline(da, k_rec=20, v=v)          # ld = v + 1
    out = _np(L.lcmp_compare_record(rec, db, v=v))
    torch.cuda.synchronize()
    orec = oracle.record(a, k=20, v=v)
    assert_record_equal(rec, orec)
    assert_compare_record_equal(out, oracle.compare_record(orec, b, k=20, v=v))


def test_ties_and_signed_zeros():
    _case("record ties")
    rng = np.random.default_rng(19)
    n, v = 12, 3000
    a = rng.integers(-3, 3, (n, v)).astype(np.float32)
    b = rng.integers(-3, 3, (n, v)).astype(np.float32)
    a[0] = 0.0
    a[1] = -0.0
    a[1, ::2] = 0.0
    b[2] = 5.0
    b[3] = -0.0
    b[3, 1::3] = 0.0
    check_both(a, b, 20, 64)


def test_flagged_and_infinite_rows():
    _case("record flagged rows")
    v = 3000
    a = np.zeros((10, v), np.float32)
    a[:, :50] = np.linspace(3, 1, 50, dtype=np.float32)
    b = a.copy()
    a[0, 3] = np.nan                 # baseline NaN: record flagged
    b[1, 2000] = np.inf              # candidate +inf outside the head
    a[2, :] = -np.inf                # baseline empty
    b[3, 2500] = -np.inf             # candidate -inf in the bucket
    b[4, :] = -np.inf                # candidate empty
    b[5, 0] = np.nan                 # candidate NaN on a head token
    b[6, 1] = np.inf                 # candidate +inf on a head token
    b[7, 2] = -np.inf                # candidate -inf on a head token: KL = inf
    a[8, 100:] = -np.inf             # baseline -inf tokens add nothing
    b[8, 100:] = 1.0
    b[9, 1500] = np.nan              # candidate NaN outside the head
    check_both(a, b, 20, 20)


def test_adversarial_rows():
    """Ascending rows move the reference every step; a head far above the rest
    (more than 87 nats) must leave the rest mass finite; huge logits; a
    candidate whose maximum sits in a later chunk."""
    _case("record adversarial rows")
    rng = np.random.default_rng(23)
    v = 151936
    rows = []
    rows.append(np.sort(rng.standard_normal(v)).astype(np.float32))            # ascending
    rows.append(np.sort(rng.standard_normal(v))[::-1].astype(np.float32))      # descending
    r = (0.1 * rng.standard_normal(v)).astype(np.float32)
    r[rng.choice(v, 20, replace=False)] = 200.0                                # head >> rest
    rows.append(r)
    rows.append((1e30 + 1e23 * rng.standard_normal(v)).astype(np.float32))     # huge values
    rows.append((rng.standard_normal(v) * 30).astype(np.float32))               # wide spread
    a = np.stack(rows)
    b = (a + 0.01 * rng.standard_normal(a.shape).astype(np.float32)).astype(np.float32)
    b[0, -1] = 100.0
    grec = check_both(a, b, 20, 20)
    assert np.isfinite(grec["lse_rest"].cpu().numpy()[2])


def test_far_apart_normalisers_against_a_record():
    """The candidate rows of the full compare's far-apart test against a
    stored baseline: shifts of +-40 (KL 0), spikes outside and on the head, a
    candidate far below except on a few tokens, the head kept while the rest
    drops by 20 or 60 nats, an unrelated and a reversed candidate."""
    _case("record far-apart normalisers")
    rng = np.random.default_rng(13)
    v = 30011
    a = (1.5 * rng.standard_normal((10, v))).astype(np.float32)
    a[:, 7] += 9.0
    a[8:10, 100:120] += 8.0
    b = (a + 0.01 * rng.standard_normal(a.shape)).astype(np.float32)
    b[0] = a[0] + 40.0
    b[1] = a[1] - 40.0
    b[2] = a[2] + 0.5
    b[3, 123] = a[3].max() + 40.0
    b[4, 7] = a[4, 7] + 40.0
    b[5] = a[5] - 60.0
    b[5, [3, 99, 2000]] = a[5, [3, 99, 2000]]
    b[6] = a[6] + 25.0 * rng.standard_normal(v).astype(np.float32)
    b[7] = -a[7]
    rest = np.ones(v, bool)
    rest[100:120] = False
    b[8, rest] -= 20.0
    b[9, rest] -= 60.0
    check_both(a, b, 20, 20)
    check_both(a, b, 5, 20)


def test_record_compare_matches_full_compare_on_corpus_rows():
    """2048 corpus rows (fp32 baseline, bf16 candidate): the record path gives
    the full compare's indices, flips and margins bit for bit, and its top-k KL
    and normalisers within the parity tolerance of each other."""
    import torch
    import logit_distribution_diffing_amd as L
    w = synth.WORKLOADS["corpus"]
    n = 2048
    _case(f"record vs full compare, corpus {n}x{w['v']}")
    a, b = synth.corpus(w["seed"], 0, n, w["v"], w["n"], w["swap_frac"])
    da, db = to_device(a), to_device(b)
    full = _np(L.lcmp_compare_logits(da, db, k=20))
    rec = L.lcmp_record_baseline(da, k_rec=20)
    cr = _np(L.lcmp_compare_record(rec, db))
    torch.cuda.synchronize()
    for f in INT_FIELDS + ("status",):
        assert np.array_equal(cr[f], full[f]), f
    assert np.array_equal(cr["margin"], full["margin"])
    err = np.abs(cr["kl_topk"] - full["kl_topk"])
    assert np.all(err <= 2 * (KL_ABS + KL_REL * np.abs(full["kl_topk"])))
    for f in ("lse_base", "lse_cand"):
        assert np.all(np.abs(cr[f] - full[f]) <= 2 * LSE_REL * np.maximum(1.0, np.abs(full[f])))
    # sampled rows against the oracle
    rows = np.unique(np.concatenate([[0, 1, n - 1], np.random.default_rng(2).choice(n, 40)]))
    orec = oracle.record(a[rows], k=20)
    o = oracle.compare_record(orec, b[rows], k=20)
    assert_compare_record_equal({k: v[rows] for k, v in cr.items()}, o)


def test_corpus_full_size_sampled_rows():
    """10240 x 151936 at full size in the timed configuration (record made
    once, candidate compared against it), sampled rows against the oracle."""
    import torch
    import logit_distribution_diffing_amd as L
    w = synth.WORKLOADS["corpus"]
    _case("record corpus 10240x151936 f32 record, bf16 candidate")
    n, v = w["n"], w["v"]
    base = torch.empty((n, v), dtype=torch.float32, device="cuda")
    cand = torch.empty((n, v), dtype=torch.bfloat16, device="cuda")
    rng = np.random.default_rng(31)
    keep = set(int(r) for r in np.concatenate([rng.choice(n, 64, replace=False),
                                               [0, 4095, 4096, n - 1]]))
    ka, kb = {}, {}
    for r0 in range(0, n, 1024):
        a, b = synth.corpus(w["seed"], r0, 1024, v, n, w["swap_frac"])
        for r in keep:
            if r0 <= r < r0 + 1024:
                ka[r], kb[r] = a[r - r0].copy(), b[r - r0].copy()
        base[r0:r0 + 1024].copy_(to_device(a))
        cand[r0:r0 + 1024].copy_(to_device(b))
        print(f"[gen] corpus rows {r0 + 1024}/{n}", flush=True)
    rec = L.lcmp_record_baseline(base, k_rec=20)
    del base
    torch.cuda.empty_cache()
    out = _np(L.lcmp_compare_record(rec, cand))
    out2 = _np(L.lcmp_compare_record(rec, cand))
    grec = _np(rec)
    torch.cuda.synchronize()
    rows = np.array(sorted(keep))
    ha = np.stack([ka[r] for r in rows])
    hb = np.stack([kb[r] for r in rows])
    orec = oracle.record(ha, k=20)
    assert np.array_equal(grec["topk_idx"][rows], orec["idx"])
    _close(grec["lse_rest"][rows], orec["lse_rest"], "lse_rest")
    assert_compare_record_equal({k: v[rows] for k, v in out.items()},
                                oracle.compare_record(orec, hb, k=20))
    for key in out:  # repeatable bit for bit
        assert np.array_equal(out[key].view(np.uint8), out2[key].view(np.uint8)), key
    swaps = synth.swap_rows(w["seed"], n, w["swap_frac"])
    assert np.all(out["flip"][swaps] == 1) and np.all(out["margin"][swaps] > 1.0)
