"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments on the host before any launch (CPU only: no call here reaches a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lcmp.h")


@pytest.fixture(scope="module")
def L():
    import runpy
    runpy.run_path(os.path.join(ROOT, "logit_distribution_diffing_amd", "build.py"))["build"]()
    import logit_distribution_diffing_amd as mod
    return mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lcmp_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 8
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(L.EXPORTED)


def test_version_and_strerror(L):
    lib = L.lib()
    assert lib.lcmp_abi_version() == 4
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert len(lib.lcmp_strerror(st)) > 0
    assert lib.lcmp_strerror(-99) == b"unknown status"


def test_workspace_queries(L):
    lib = L.lib()
    assert lib.lcmp_compare_workspace_bytes(10240, 151936, 20, 0) > 0
    for args in ((10240, 151936, 20, 1), (7, 1000, 64, 0), (10, 1, 20, 0), (-1, 100, 20, 0)):
        assert lib.lcmp_workspace_bytes(*args) == lib.lcmp_compare_workspace_bytes(*args)
    a = lib.lcmp_compare_workspace_bytes(512, 151936, 20, 0)
    b = lib.lcmp_compare_workspace_bytes(512, 151936, 20, 1)
    assert b > a
    assert lib.lcmp_compare_workspace_bytes(10, 1, 20, 0) == 0      # v < 2
    assert lib.lcmp_compare_workspace_bytes(10, 100, 0, 0) == 0     # k < 1
    assert lib.lcmp_compare_workspace_bytes(10, 100, 65, 0) == 0    # k > 64
    assert lib.lcmp_compare_workspace_bytes(-1, 100, 20, 0) == 0
    assert lib.lcmp_compare_workspace_bytes(1 << 31, 100, 20, 0) == 0   # one block per row
    assert lib.lcmp_compare_workspace_bytes((1 << 31) - 1, 100, 20, 0) > 0
    assert lib.lcmp_bitdiff_workspace_bytes(1 << 31, 10) == 0
    assert lib.lcmp_compare_record_workspace_bytes(1 << 31, 100) == 0
    assert lib.lcmp_bitdiff_workspace_bytes(4096, 5120) > 0
    assert lib.lcmp_bitdiff_workspace_bytes(4, 0) == 0
    assert lib.lcmp_bin_workspace_bytes(65536, 1, 6) > 0
    assert lib.lcmp_bin_workspace_bytes(10, 0, 6) == 0
    assert lib.lcmp_bin_workspace_bytes(10, 16, 17) == 0            # more than 256 bins
    assert lib.lcmp_bin_workspace_bytes((1 << 36) + 1, 1, 6) == 0   # more rows than the limit


FAKE = 0x10000  # a non-null address that is never dereferenced: every call below fails validation


def _compare(L, **kw):
    args = dict(base=FAKE, tb=0, ld_base=100, cand=FAKE, tc=0, ld_cand=100, n=4, v=100, k=20,
                flags=0, out=L.RowOut(), bd=None, ws=FAKE, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    out = args["out"]
    return L.lib().lcmp_compare_logits(args["base"], args["tb"], args["ld_base"], args["cand"],
                                       args["tc"], args["ld_cand"], args["n"], args["v"], args["k"],
                                       args["flags"], None if out is None else ctypes.byref(out),
                                       args["bd"], args["ws"], args["ws_bytes"], args["stream"])


def test_compare_argument_errors(L):
    assert _compare(L, tb=7) == -2
    assert _compare(L, tc=-1) == -2
    assert _compare(L, n=-1) == -1
    assert _compare(L, flags=2) == -1
    assert _compare(L, out=None) == -1
    assert _compare(L, v=1) == -3
    assert _compare(L, k=0) == -3
    assert _compare(L, k=65) == -3
    assert _compare(L, ld_base=99) == -3
    assert _compare(L, ld_cand=50) == -3
    assert _compare(L, flags=1, bd=None) == -1          # bitwise stats need a destination
    assert _compare(L, base=None) == -1
    assert _compare(L, ws=None) == -4
    assert _compare(L, ws_bytes=16) == -4
    assert _compare(L, ws=FAKE + 4) == -1                # misaligned workspace
    assert _compare(L, n=0) == 0                         # empty batch: nothing to do
    assert _compare(L, n=0, flags=1, bd=None, base=None, ws=None) == 0  # and nothing is read
    assert _compare(L, n=1 << 31) == -3                  # more rows than LCMP_MAX_ROWS
    ro = L.RowOut()
    ro.logp_cand = FAKE
    assert _compare(L, out=ro) == -1                     # target log-probabilities need targets


def test_bitdiff_argument_errors(L):
    lib = L.lib()

    def call(**kw):
        a = dict(a=FAKE, ta=1, lda=10, b=FAKE, tb=1, ldb=10, rows=2, cols=10, out=FAKE, ws=FAKE,
                 ws_bytes=1 << 20, stream=None)
        a.update(kw)
        return lib.lcmp_bitdiff(a["a"], a["ta"], a["lda"], a["b"], a["tb"], a["ldb"], a["rows"],
                                a["cols"], a["out"], a["ws"], a["ws_bytes"], a["stream"])

    assert call(ta=3) == -2
    assert call(rows=-2) == -1
    assert call(cols=0) == -3
    assert call(lda=9) == -3
    assert call(out=None) == -1
    assert call(ws=None) == -4
    assert call(ws_bytes=1) == -4
    assert call(rows=0) == 0


def test_bin_report_argument_errors(L):
    lib = L.lib()

    def call(edges=(0.1, 0.5, float("inf")), **kw):
        e = (ctypes.c_double * len(edges))(*edges)
        a = dict(margin=FAKE, flip=FAKE, kt=FAKE, kf=FAKE, status=None, group=None, ng=1, n=10,
                 ne=len(edges), big=1.0, bins=FAKE, summ=FAKE, ws=FAKE, ws_bytes=1 << 20)
        a.update(kw)
        return lib.lcmp_bin_report(a["margin"], a["flip"], a["kt"], a["kf"], a["status"], a["group"],
                                   a["ng"], a["n"], e, a["ne"], a["big"], a["bins"], a["summ"],
                                   a["ws"], a["ws_bytes"], None)

    assert call(edges=(0.5, 0.1)) == -6                    # not ascending
    assert call(edges=(0.0, 1.0)) == -6                    # not positive
    assert call(edges=(0.1, float("nan"))) == -6
    assert call(edges=(0.1, 0.1)) == -6
    assert call(ng=0) == -3
    assert call(ng=300) == -3
    assert call(ng=100, edges=(0.1, 0.5, 1.0)) == -3       # 300 bins
    assert call(n=-1) == -1
    assert call(n=(1 << 36) + 1) == -3                     # more rows than LCMP_MAX_BIN_ROWS
    assert call(bins=None) == -1
    assert call(margin=None) == -1
    assert call(ws=None) == -4
    assert call(big=float("nan")) == -1


def test_binding_rejects_unsupported_dtype(L):
    """Only float32 and bfloat16 tensors are accepted."""
    import torch
    with pytest.raises(TypeError):
        L.lcmp_compare_logits(torch.zeros(2, 4, dtype=torch.float64),
                              torch.zeros(2, 4, dtype=torch.float64))


def test_perturb_argument_errors(L):
    lib = L.lib()

    def call(**kw):
        a = dict(src=FAKE, ts=0, lds=10, dst=FAKE, td=0, ldd=10, rows=2, cols=10, mode=0, param=7)
        a.update(kw)
        return lib.lcmp_perturb(a["src"], a["ts"], a["lds"], a["dst"], a["td"], a["ldd"],
                                a["rows"], a["cols"], a["mode"], a["param"], None)

    assert call(ts=2) == -2
    assert call(mode=3) == -1
    assert call(param=24) == -1
    assert call(param=-1) == -1
    assert call(td=1, param=8) == -2            # 8 fraction bits do not fit bf16
    assert call(td=1, mode=2) == -2             # scaled e4m3 results are not bf16 values
    assert call(lds=9) == -3
    assert call(src=None) == -1
    assert call(rows=-1) == -1
    assert call(rows=0) == 0



def _record(L, **kw):
    r = L.Record(topk_idx=FAKE, topk_val=FAKE, lse_rest=FAKE, status=FAKE, logp_target=None)
    for key, val in kw.items():
        setattr(r, key, val)
    return r


def test_record_workspace_queries(L):
    lib = L.lib()
    assert lib.lcmp_record_workspace_bytes(1000, 151936, 20) > lib.lcmp_compare_record_workspace_bytes(1000, 151936)
    assert lib.lcmp_record_workspace_bytes(10, 100, 1) == 0       # k_rec < 2
    assert lib.lcmp_record_workspace_bytes(10, 100, 65) == 0
    assert lib.lcmp_record_workspace_bytes(10, 1, 20) == 0
    assert lib.lcmp_compare_record_workspace_bytes(10, 1) == 0
    assert lib.lcmp_compare_record_workspace_bytes(-1, 100) == 0
    assert lib.lcmp_compare_record_workspace_bytes(0, 100) > 0


def test_record_baseline_argument_errors(L):
    lib = L.lib()

    def call(rec=None, **kw):
        a = dict(base=FAKE, tb=0, ld=100, n=4, v=100, k_rec=20, target=None, ws=FAKE,
                 ws_bytes=1 << 30)
        a.update(kw)
        r = _record(L) if rec is None else rec
        return lib.lcmp_record_baseline(a["base"], a["tb"], a["ld"], a["n"], a["v"], a["k_rec"],
                                        a["target"], ctypes.byref(r), a["ws"], a["ws_bytes"], None)

    assert call(tb=2) == -2
    assert call(n=-1) == -1
    assert call(k_rec=1) == -3
    assert call(k_rec=65) == -3
    assert call(ld=99) == -3
    assert call(v=1) == -3
    assert call(rec=_record(L, logp_target=FAKE)) == -1     # target log-probability needs targets
    assert call(base=None) == -1
    assert call(rec=_record(L, lse_rest=None)) == -1
    assert call(ws=None) == -4
    assert call(ws_bytes=8) == -4
    assert call(n=0) == 0


def test_compare_record_argument_errors(L):
    lib = L.lib()

    def call(rec=None, out=None, **kw):
        a = dict(k_rec=20, cand=FAKE, tc=0, ld=100, n=4, v=100, k=20, ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        r = _record(L) if rec is None else rec
        o = L.RowOut() if out is None else out
        return lib.lcmp_compare_record(ctypes.byref(r), a["k_rec"], a["cand"], a["tc"], a["ld"],
                                       a["n"], a["v"], a["k"], ctypes.byref(o), a["ws"],
                                       a["ws_bytes"], None)

    assert call(tc=5) == -2
    assert call(n=-1) == -1
    assert call(k=21) == -3                       # more entries than the record holds
    assert call(k=0) == -3
    assert call(k_rec=1, k=1) == -3
    assert call(ld=50) == -3
    ro = L.RowOut()
    ro.kl_full = FAKE
    assert call(out=ro) == -1                     # the full KL needs the baseline rows
    ro = L.RowOut()
    ro.logp_cand = FAKE
    assert call(out=ro) == -1                     # needs targets
    ro.target = FAKE
    ro.logp_base = FAKE
    assert call(out=ro) == -1                     # the record holds no target log-probability
    assert call(cand=None) == -1
    assert call(ws=None) == -4
    assert call(ws_bytes=8) == -4
    assert call(ws=FAKE + 8) == -1
    assert call(n=0) == 0


def test_binding_checks_tensors_before_any_call(L):
    """Tensors too small, of the wrong type, or not on the GPU are rejected in
    the binding, before a pointer reaches the library (CPU tensors here)."""
    import torch
    base = torch.zeros(4, 100)
    with pytest.raises(ValueError, match="cand"):
        L.lcmp_compare_logits(base, torch.zeros(3, 100))          # row counts differ
    with pytest.raises(ValueError, match="base"):
        L.lcmp_compare_logits(base, base, v=101)                  # v beyond the columns
    small = {"kl_topk": torch.zeros(3, dtype=torch.float64)}
    with pytest.raises(ValueError, match="kl_topk"):
        L.lcmp_compare_logits(base, base, out=small)
    with pytest.raises(ValueError):
        L.lcmp_compare_logits(base, base)                         # host memory
    rec = {"topk_idx": torch.zeros(4, 20, dtype=torch.int32),
           "topk_val": torch.zeros(4, 20, dtype=torch.float64),  # wrong element type
           "lse_rest": torch.zeros(4, dtype=torch.float64), "status": torch.zeros(4, dtype=torch.uint8)}
    with pytest.raises(ValueError):
        L.lcmp_compare_record(rec, base)
    with pytest.raises(ValueError, match="margin"):
        L.lcmp_bin_report(torch.zeros(10), torch.zeros(10, dtype=torch.uint8),
                          torch.zeros(10, dtype=torch.float64), None, (0.5, 1.0))
    with pytest.raises(ValueError):
        L.lcmp_perturb(base, 0, 7)
