"""Double-precision CPU oracle for the teacher-forced logit comparison.

TEST INFRASTRUCTURE ONLY.  The parity tests, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` are the only permitted users; the GPU
library never imports, links or calls anything here, and nothing here reads
the GPU library.

Arrays are numpy: float32 for fp32 tensors, uint16 bit patterns for bf16.
Every function follows a plain definition from the logit-diffing page (see the
header of ``oracle.c`` for the citations and the readings taken).

Pins (tests/test_oracle_pins.py): the cat/dog and long-tail examples of the
logit page, the two-way margin probabilities, the small-delta variance
approximation, the Monte-Carlo flip rate against Phi, brute-force top-k on
tiny vocabularies, library cross-checks (scipy rel_entr, torch kl_div),
bitwise known answers by construction and hand-countable margin bins.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1
ROW_NONFINITE, ROW_EMPTY = 1, 2


class BitdiffRow(ctypes.Structure):
    _fields_ = [("ndiff", ctypes.c_int64), ("first_diff", ctypes.c_int64),
                ("nonfinite_a", ctypes.c_int64), ("nonfinite_b", ctypes.c_int64),
                ("max_ulp", ctypes.c_uint32), ("pad_", ctypes.c_uint32),
                ("max_abs", ctypes.c_double), ("sum_abs", ctypes.c_double),
                ("sum_sq_diff", ctypes.c_double), ("sum_sq_base", ctypes.c_double),
                ("mean_abs", ctypes.c_double), ("rel_l2", ctypes.c_double)]


class Bin(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int64), ("flips", ctypes.c_int64),
                ("ties", ctypes.c_int64), ("tie_flips", ctypes.c_int64),
                ("sum_kl_topk", ctypes.c_double), ("sum_kl_full", ctypes.c_double),
                ("max_kl_topk", ctypes.c_double)]


class GroupSummary(ctypes.Structure):
    _fields_ = [("big_margin_flips", ctypes.c_int64), ("excluded", ctypes.c_int64),
                ("unbinned", ctypes.c_int64)]


BITDIFF_DTYPE = np.dtype([(n, t) for n, t in (
    ("ndiff", np.int64), ("first_diff", np.int64), ("nonfinite_a", np.int64),
    ("nonfinite_b", np.int64), ("max_ulp", np.uint32), ("pad_", np.uint32),
    ("max_abs", np.float64), ("sum_abs", np.float64), ("sum_sq_diff", np.float64),
    ("sum_sq_base", np.float64), ("mean_abs", np.float64), ("rel_l2", np.float64))])
BIN_DTYPE = np.dtype([("count", np.int64), ("flips", np.int64), ("ties", np.int64),
                      ("tie_flips", np.int64), ("sum_kl_topk", np.float64),
                      ("sum_kl_full", np.float64), ("max_kl_topk", np.float64)])
SUMMARY_DTYPE = np.dtype([("big_margin_flips", np.int64), ("excluded", np.int64),
                          ("unbinned", np.int64)])


def build(force: bool = False) -> str:
    """Compile liboracle.so (gcc, -O2, OpenMP over rows)."""
    if force or not os.path.exists(_SO):
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", _SO,
               os.path.join(_HERE, "oracle.c"), "-lm"]
        subprocess.run(cmd, check=True)
    return _SO


def _L():
    global _lib
    if _lib is None:
        # ORACLE_LIB names another build of oracle.c (the mutation tests load
        # deliberately broken copies through it); by default the in-tree build
        path = os.environ.get("ORACLE_LIB")
        if not path:
            build()
            path = _SO
        lib = ctypes.CDLL(path)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.orc_compare.restype = ci
        lib.orc_compare.argtypes = [vp, ci, i64, vp, ci, i64, i64, i64, ci] + [vp] * 11 + [ci]
        lib.orc_target_logprob.restype = ci
        lib.orc_target_logprob.argtypes = [vp, ci, i64, vp, ci, i64, i64, i64, vp, vp, vp, ci]
        lib.orc_record.restype = ci
        lib.orc_record.argtypes = [vp, ci, i64, i64, i64, ci, vp, vp, vp, vp, vp, vp, ci]
        lib.orc_compare_record.restype = ci
        lib.orc_compare_record.argtypes = [vp, vp, vp, vp, vp, ci, vp, ci, i64, i64, i64, ci,
                                           vp] + [vp] * 12 + [ci]
        lib.orc_perturb.restype = ci
        lib.orc_perturb.argtypes = [vp, ci, i64, vp, ci, i64, i64, i64, ci, ci]
        lib.orc_bitdiff.restype = ci
        lib.orc_bitdiff.argtypes = [vp, ci, i64, vp, ci, i64, i64, i64, vp, ci]
        lib.orc_bin_report.restype = ci
        lib.orc_bin_report.argtypes = [vp, vp, vp, vp, vp, vp, ci, i64, vp, ci,
                                       ctypes.c_double, vp, vp]
        _lib = lib
    return _lib


def dtype_code(arr: np.ndarray) -> int:
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.uint16:
        return BF16
    raise TypeError(f"unsupported dtype {arr.dtype} (float32 or uint16 bf16 patterns)")


def _p(a):
    return None if a is None else a.ctypes.data


def compare(base: np.ndarray, cand: np.ndarray, k: int = 20, v: int | None = None,
            nthreads: int = 0) -> dict:
    """Per-row comparison of baseline and candidate logits ([n, ld] arrays; the
    first v columns are the vocabulary).  Returns a dict of numpy arrays."""
    assert base.ndim == 2 and cand.ndim == 2 and base.shape[0] == cand.shape[0]
    base = np.ascontiguousarray(base)
    cand = np.ascontiguousarray(cand)
    n = base.shape[0]
    v = base.shape[1] if v is None else v
    out = dict(kl_topk=np.empty(n), kl_full=np.empty(n), margin=np.empty(n),
               lse_base=np.empty(n), lse_cand=np.empty(n),
               top1_base=np.empty(n, np.int32), top2_base=np.empty(n, np.int32),
               top1_cand=np.empty(n, np.int32), flip=np.empty(n, np.uint8),
               topk_idx=np.empty((n, k), np.int32), status=np.empty(n, np.uint8))
    rc = _L().orc_compare(base.ctypes.data, dtype_code(base), base.shape[1], cand.ctypes.data,
                          dtype_code(cand), cand.shape[1], n, v, k,
                          *[_p(out[f]) for f in ("kl_topk", "kl_full", "margin", "lse_base",
                                                 "lse_cand", "top1_base", "top2_base",
                                                 "top1_cand", "flip", "topk_idx", "status")],
                          nthreads)
    if rc != 0:
        raise ValueError("orc_compare rejected its arguments")
    return out


def target_logprob(base: np.ndarray, cand: np.ndarray, target, v: int | None = None,
                   nthreads: int = 0) -> dict:
    """ln p(target) and ln q(target) per row (NaN for flagged rows and targets
    outside [0, v)); `target` is one int32 id per row."""
    assert base.ndim == 2 and cand.ndim == 2 and base.shape[0] == cand.shape[0]
    base = np.ascontiguousarray(base)
    cand = np.ascontiguousarray(cand)
    n = base.shape[0]
    v = base.shape[1] if v is None else v
    target = np.ascontiguousarray(target, dtype=np.int32)
    assert target.shape == (n,)
    out = dict(logp_base=np.empty(n), logp_cand=np.empty(n))
    rc = _L().orc_target_logprob(base.ctypes.data, dtype_code(base), base.shape[1],
                                 cand.ctypes.data, dtype_code(cand), cand.shape[1], n, v,
                                 target.ctypes.data, out["logp_base"].ctypes.data,
                                 out["logp_cand"].ctypes.data, nthreads)
    if rc != 0:
        raise ValueError("orc_target_logprob rejected its arguments")
    return out


def record(base: np.ndarray, k: int = 20, target=None, v: int | None = None,
           nthreads: int = 0) -> dict:
    """Compact ground-truth record of baseline rows: the k largest logits
    (idx [n, k] int32, val [n, k] float32), lse_rest [n] (ln of the mass outside
    them), status [n], and logp_target [n] when `target` is given."""
    assert base.ndim == 2
    base = np.ascontiguousarray(base)
    n = base.shape[0]
    v = base.shape[1] if v is None else v
    out = dict(idx=np.empty((n, k), np.int32), val=np.empty((n, k), np.float32),
               lse_rest=np.empty(n), status=np.empty(n, np.uint8))
    tg = None
    if target is not None:
        tg = np.ascontiguousarray(target, dtype=np.int32)
        assert tg.shape == (n,)
        out["logp_target"] = np.empty(n)
    rc = _L().orc_record(base.ctypes.data, dtype_code(base), base.shape[1], n, v, k, _p(tg),
                         out["idx"].ctypes.data, out["val"].ctypes.data,
                         out["lse_rest"].ctypes.data, out["status"].ctypes.data,
                         _p(out.get("logp_target")), nthreads)
    if rc != 0:
        raise ValueError("orc_record rejected its arguments")
    return out


def compare_record(rec: dict, cand: np.ndarray, k: int | None = None, target=None,
                   v: int | None = None, nthreads: int = 0) -> dict:
    """Compare candidate rows against a record (from record()) using its first
    k entries; returns the outputs of compare() except kl_full, plus logp_base /
    logp_cand when `target` is given (logp_base needs a record with targets)."""
    assert cand.ndim == 2
    cand = np.ascontiguousarray(cand)
    n = cand.shape[0]
    v = cand.shape[1] if v is None else v
    k_rec = rec["idx"].shape[1]
    k = k_rec if k is None else k
    idx = np.ascontiguousarray(rec["idx"], np.int32)
    val = np.ascontiguousarray(rec["val"], np.float32)
    lse_rest = np.ascontiguousarray(rec["lse_rest"], np.float64)
    st = np.ascontiguousarray(rec["status"], np.uint8)
    assert idx.shape[0] == n
    out = dict(kl_topk=np.empty(n), margin=np.empty(n), lse_base=np.empty(n),
               lse_cand=np.empty(n), top1_base=np.empty(n, np.int32),
               top2_base=np.empty(n, np.int32), top1_cand=np.empty(n, np.int32),
               flip=np.empty(n, np.uint8), topk_idx=np.empty((n, k), np.int32),
               status=np.empty(n, np.uint8))
    tg = rl = None
    if target is not None:
        tg = np.ascontiguousarray(target, dtype=np.int32)
        assert tg.shape == (n,)
        out["logp_cand"] = np.empty(n)
        if "logp_target" in rec:
            rl = np.ascontiguousarray(rec["logp_target"], np.float64)
            out["logp_base"] = np.empty(n)
    rc = _L().orc_compare_record(idx.ctypes.data, val.ctypes.data, lse_rest.ctypes.data,
                                 st.ctypes.data, _p(rl), k_rec, cand.ctypes.data,
                                 dtype_code(cand), cand.shape[1], n, v, k, _p(tg),
                                 *[_p(out.get(f)) for f in (
                                     "kl_topk", "margin", "lse_base", "lse_cand", "top1_base",
                                     "top2_base", "top1_cand", "flip", "topk_idx", "status",
                                     "logp_base", "logp_cand")],
                                 nthreads)
    if rc != 0:
        raise ValueError("orc_compare_record rejected its arguments")
    return out


PERTURB_MANTISSA, PERTURB_E4M3, PERTURB_E4M3_SCALED = 0, 1, 2


def perturb(src: np.ndarray, mode: int, param: int = 0, out_bf16: bool = False) -> np.ndarray:
    """Precision perturbation of a [rows, cols] array (float32 or uint16 bf16
    patterns): keep `param` fraction bits, or round to e4m3 (optionally after
    scaling by 448).  Returns float32, or uint16 bf16 patterns with out_bf16."""
    src = np.ascontiguousarray(src)
    if src.ndim == 1:
        src = src[None, :]
    rows, cols = src.shape
    dst = np.empty((rows, cols), np.uint16 if out_bf16 else np.float32)
    rc = _L().orc_perturb(src.ctypes.data, dtype_code(src), cols, dst.ctypes.data,
                          BF16 if out_bf16 else F32, cols, rows, cols, mode, param)
    if rc != 0:
        raise ValueError("orc_perturb rejected its arguments")
    return dst


def bitdiff(a: np.ndarray, b: np.ndarray, cols: int | None = None, nthreads: int = 0) -> np.ndarray:
    """Per-row bitwise / ULP statistics; returns a structured array (BITDIFF_DTYPE)."""
    assert a.ndim == 2 and b.ndim == 2 and a.shape[0] == b.shape[0]
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    rows = a.shape[0]
    cols = a.shape[1] if cols is None else cols
    out = np.zeros(rows, dtype=BITDIFF_DTYPE)
    rc = _L().orc_bitdiff(a.ctypes.data, dtype_code(a), a.shape[1], b.ctypes.data, dtype_code(b),
                          b.shape[1], rows, cols, out.ctypes.data, nthreads)
    if rc != 0:
        raise ValueError("orc_bitdiff rejected its arguments")
    return out


def bin_report(margin, flip, kl_topk, kl_full, edges, status=None, group=None, n_groups=1,
               big_margin: float = 1.0):
    """Margin-binned flip counts and KL sums.  Returns (bins [n_groups, n_edges],
    summary [n_groups]) as structured arrays."""
    margin = np.ascontiguousarray(margin, np.float64)
    flip = np.ascontiguousarray(flip, np.uint8)
    kl_topk = np.ascontiguousarray(kl_topk, np.float64)
    kl_full = None if kl_full is None else np.ascontiguousarray(kl_full, np.float64)
    edges = np.ascontiguousarray(edges, np.float64)
    st = None if status is None else np.ascontiguousarray(status, np.uint8)
    gr = None if group is None else np.ascontiguousarray(group, np.int32)
    n = margin.shape[0]
    bins = np.zeros((n_groups, edges.size), dtype=BIN_DTYPE)
    summ = np.zeros(n_groups, dtype=SUMMARY_DTYPE)
    rc = _L().orc_bin_report(margin.ctypes.data, flip.ctypes.data, kl_topk.ctypes.data,
                             _p(kl_full), _p(st), _p(gr), n_groups, n, edges.ctypes.data,
                             edges.size, big_margin, bins.ctypes.data, summ.ctypes.data)
    if rc != 0:
        raise ValueError("orc_bin_report rejected its arguments")
    return bins, summ
