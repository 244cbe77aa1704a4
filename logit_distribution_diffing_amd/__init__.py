"""Teacher-forced logit comparison on AMD MI355X (gfx950): Python binding.

Thin ctypes layer over ``liblcmp.so`` (see ``include/lcmp.h`` for the C ABI).
It only marshals arguments: torch is used for device memory and streams, and
every step of the comparison runs in the library's HIP kernels.  There is no
CPU fallback: importing this module raises if the library has not been built
(``python -m logit_distribution_diffing_amd.build``).

Entry points (same names as the C ABI):
  lcmp_compare_logits(base, cand, k=20, with_bitdiff=False)  -> dict of tensors
  lcmp_bitdiff(a, b)                                         -> structured tensor
  lcmp_bin_report(margin, flip, kl_topk, kl_full, edges, ...) -> (bins, summary)
  lcmp_perturb(src, mode, param)                             -> perturbed tensor
  lcmp_record_baseline(base, k_rec=20, target=None)          -> record (dict of tensors)
  lcmp_compare_record(record, cand, k=None, target=None)     -> dict of tensors
"""
from __future__ import annotations

import ctypes
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblcmp.so")

LCMP_F32, LCMP_BF16 = 0, 1
LCMP_WITH_BITDIFF = 1
LCMP_ROW_NONFINITE, LCMP_ROW_EMPTY = 1, 2
LCMP_MAX_K = 64
LCMP_NOALLOC_SCRATCH_BYTES = 64 << 20
ABI_VERSION = 4
LCMP_PERTURB_MANTISSA, LCMP_PERTURB_E4M3, LCMP_PERTURB_E4M3_SCALED = 0, 1, 2
STATUS_NAMES = {0: "LCMP_OK", -1: "LCMP_EINVAL", -2: "LCMP_EDTYPE", -3: "LCMP_ESHAPE",
                -4: "LCMP_EWORKSPACE", -5: "LCMP_EHIP", -6: "LCMP_EEDGES"}

EXPORTED = ("lcmp_abi_version", "lcmp_strerror", "lcmp_compare_workspace_bytes",
            "lcmp_workspace_bytes",
            "lcmp_compare_logits", "lcmp_compare_logits_timed", "lcmp_bitdiff_workspace_bytes",
            "lcmp_bitdiff", "lcmp_bin_workspace_bytes", "lcmp_bin_report", "lcmp_perturb",
            "lcmp_record_workspace_bytes", "lcmp_record_baseline",
            "lcmp_compare_record_workspace_bytes", "lcmp_compare_record",
            "lcmp_compare_record_timed", "lcmp_bitdiff_timed", "lcmp_read_probe",
            "lcmp_compare_logits_noalloc")


class LcmpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.lcmp_strerror(status).decode() if _lib is not None else ""
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({msg})")


ROW_OUT_FIELDS = ("kl_topk", "kl_full", "margin", "lse_base", "lse_cand", "top1_base",
                  "top2_base", "top1_cand", "flip", "status", "topk_idx", "target", "logp_base",
                  "logp_cand")


class RowOut(ctypes.Structure):
    """lcmp_row_out: device pointers, NULL to skip (target is an input)."""
    _fields_ = [(n, ctypes.c_void_p) for n in ROW_OUT_FIELDS]


RECORD_FIELDS = ("topk_idx", "topk_val", "lse_rest", "status", "logp_target")


class Record(ctypes.Structure):
    """lcmp_record: device arrays of a compact baseline record (logp_target may be NULL)."""
    _fields_ = [(n, ctypes.c_void_p) for n in RECORD_FIELDS]


# record sizes of the C structs (int64 x4, uint32 x2, double x6) etc.
BITDIFF_ROW_BYTES = 4 * 8 + 2 * 4 + 6 * 8
BIN_BYTES = 4 * 8 + 3 * 8
GROUP_SUMMARY_BYTES = 3 * 8

_lib = None


def _load():
    global _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing; build it with `python -m logit_distribution_diffing_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, ci, u32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32,
                            ctypes.c_size_t)
    lib.lcmp_abi_version.restype = ci
    lib.lcmp_abi_version.argtypes = []
    lib.lcmp_strerror.restype = ctypes.c_char_p
    lib.lcmp_strerror.argtypes = [ci]
    lib.lcmp_compare_workspace_bytes.restype = sz
    lib.lcmp_compare_workspace_bytes.argtypes = [i64, i64, ci, u32]
    lib.lcmp_workspace_bytes.restype = sz
    lib.lcmp_workspace_bytes.argtypes = [i64, i64, ci, u32]
    lib.lcmp_compare_logits.restype = ci
    lib.lcmp_compare_logits.argtypes = [vp, ci, i64, vp, ci, i64, i64, i64, ci, u32,
                                        ctypes.POINTER(RowOut), vp, vp, sz, vp]
    lib.lcmp_compare_logits_timed.restype = ci
    lib.lcmp_compare_logits_timed.argtypes = lib.lcmp_compare_logits.argtypes + [vp, vp]
    lib.lcmp_compare_logits_noalloc.restype = ci
    lib.lcmp_compare_logits_noalloc.argtypes = [vp, ci, i64, vp, ci, i64, i64, i64, ci, u32,
                                                ctypes.POINTER(RowOut), vp, vp]
    lib.lcmp_bitdiff_workspace_bytes.restype = sz
    lib.lcmp_bitdiff_workspace_bytes.argtypes = [i64, i64]
    lib.lcmp_bitdiff.restype = ci
    lib.lcmp_bitdiff.argtypes = [vp, ci, i64, vp, ci, i64, i64, i64, vp, vp, sz, vp]
    lib.lcmp_bitdiff_timed.restype = ci
    lib.lcmp_bitdiff_timed.argtypes = lib.lcmp_bitdiff.argtypes + [vp, vp]
    lib.lcmp_read_probe.restype = ci
    lib.lcmp_read_probe.argtypes = [vp, ci, i64, vp, ci, i64, i64, i64, vp, sz, vp, vp, vp]
    lib.lcmp_bin_workspace_bytes.restype = sz
    lib.lcmp_bin_workspace_bytes.argtypes = [i64, ci, ci]
    lib.lcmp_perturb.restype = ci
    lib.lcmp_perturb.argtypes = [vp, ci, i64, vp, ci, i64, i64, i64, ci, ci, vp]
    lib.lcmp_bin_report.restype = ci
    lib.lcmp_bin_report.argtypes = [vp, vp, vp, vp, vp, vp, ci, i64,
                                    ctypes.POINTER(ctypes.c_double), ci, ctypes.c_double,
                                    vp, vp, vp, sz, vp]
    lib.lcmp_record_workspace_bytes.restype = sz
    lib.lcmp_record_workspace_bytes.argtypes = [i64, i64, ci]
    lib.lcmp_record_baseline.restype = ci
    lib.lcmp_record_baseline.argtypes = [vp, ci, i64, i64, i64, ci, vp, ctypes.POINTER(Record),
                                         vp, sz, vp]
    lib.lcmp_compare_record_workspace_bytes.restype = sz
    lib.lcmp_compare_record_workspace_bytes.argtypes = [i64, i64]
    lib.lcmp_compare_record.restype = ci
    lib.lcmp_compare_record.argtypes = [ctypes.POINTER(Record), ci, vp, ci, i64, i64, i64, ci,
                                        ctypes.POINTER(RowOut), vp, sz, vp]
    lib.lcmp_compare_record_timed.restype = ci
    lib.lcmp_compare_record_timed.argtypes = lib.lcmp_compare_record.argtypes + [vp, vp]
    if lib.lcmp_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI {lib.lcmp_abi_version()}, this binding expects "
                          f"{ABI_VERSION}; rebuild it")
    _lib = lib
    return lib


_load()


def lib() -> ctypes.CDLL:
    return _lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LCMP_F32
    if t.dtype == torch.bfloat16:
        return LCMP_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _ld(t: torch.Tensor) -> int:
    if t.dim() == 2 and t.numel() == 0:
        return t.size(1)  # no element is read: any layout will do
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit stride along the vocabulary")
    return t.stride(0) if t.size(0) > 1 else max(t.stride(0), t.size(1))


def _torch_stream(stream):
    """The torch stream object of `stream`: None is the current stream, a raw
    hipStream_t handle is wrapped without taking ownership."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.ExternalStream(handle)


def _stream(stream) -> int:
    return _torch_stream(stream).cuda_stream


def _on_stream(fn):
    """Run a binding call with its launch stream as torch's current stream, so
    every tensor the call allocates (a workspace or outputs the caller did not
    pass) belongs to the stream its kernels run on.  The caching allocator then
    cannot hand such a block to work on another stream while the kernels still
    use it, also after the call has dropped its own reference."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kw):
        if not torch.cuda.is_available():  # the call's own checks reject host tensors
            return fn(*args, stream=stream, **kw)
        ts = _torch_stream(stream)
        with torch.cuda.stream(ts):
            return fn(*args, stream=ts, **kw)
    return wrapper


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(rc: int, where: str):
    if rc != 0:
        raise LcmpError(rc, where)


# ----------------------------------------------------------------------------- checks
# The C side checks sizes and strides it is given; these checks make sure the
# tensors behind the pointers are as large as those sizes say, of the right
# element type and on the GPU, before any pointer reaches a kernel.

# output field -> (dtype, elements per row; "k" = k per row)
_OUT_SPEC = {
    "kl_topk": (torch.float64, 1), "kl_full": (torch.float64, 1), "margin": (torch.float64, 1),
    "lse_base": (torch.float64, 1), "lse_cand": (torch.float64, 1),
    "logp_base": (torch.float64, 1), "logp_cand": (torch.float64, 1),
    "top1_base": (torch.int32, 1), "top2_base": (torch.int32, 1), "top1_cand": (torch.int32, 1),
    "flip": (torch.uint8, 1), "status": (torch.uint8, 1), "topk_idx": (torch.int32, "k"),
    "bitdiff": (torch.uint8, BITDIFF_ROW_BYTES),
}


def _on_gpu(*named):
    """(name, tensor) pairs; None tensors are skipped.  Run after the shape and
    type checks, so those are reported first."""
    for what, t in named:
        if t is not None and t.device.type != "cuda":
            raise ValueError(f"{what} must be a GPU tensor")


def _check_buffer(t, dtype, numel: int, what: str):
    if t.dtype != dtype or not t.is_contiguous() or t.numel() < numel:
        raise ValueError(f"{what} must be a contiguous {dtype} tensor of at least {numel} "
                         f"elements (got {t.dtype}, {t.numel()}, contiguous={t.is_contiguous()})")


def _check_rows(t, n: int, v: int, what: str):
    if t.dim() != 2 or t.size(0) != n or t.size(1) < v:
        raise ValueError(f"{what} must be [n={n}, >= v={v}] (got {tuple(t.shape)})")
    _dtype_code(t)


def _check_out(out: dict, n: int, k: int, allowed=None):
    for key, t in out.items():
        if key not in _OUT_SPEC or (allowed is not None and key not in allowed):
            raise ValueError(f"unexpected output field {key!r}")
        dtype, per = _OUT_SPEC[key]
        _check_buffer(t, dtype, n * (k if per == "k" else per), f"out[{key!r}]")


def _check_workspace(ws):
    """A caller's workspace is passed on as given: one that is too small comes
    back from the library as LCMP_EWORKSPACE instead of being replaced here."""
    if ws is not None:
        _check_buffer(ws, torch.uint8, 0, "workspace")


def compare_workspace_bytes(n: int, v: int, k: int = 20, with_bitdiff: bool = False) -> int:
    return int(_lib.lcmp_compare_workspace_bytes(n, v, k, LCMP_WITH_BITDIFF if with_bitdiff else 0))


def alloc_compare_outputs(n: int, k: int, device, with_bitdiff: bool = False,
                          with_target: bool = False) -> dict:
    f64 = dict(dtype=torch.float64, device=device)
    i32 = dict(dtype=torch.int32, device=device)
    u8 = dict(dtype=torch.uint8, device=device)
    out = dict(kl_topk=torch.empty(n, **f64), kl_full=torch.empty(n, **f64),
               margin=torch.empty(n, **f64), lse_base=torch.empty(n, **f64),
               lse_cand=torch.empty(n, **f64), top1_base=torch.empty(n, **i32),
               top2_base=torch.empty(n, **i32), top1_cand=torch.empty(n, **i32),
               flip=torch.empty(n, **u8), status=torch.empty(n, **u8),
               topk_idx=torch.empty((n, k), **i32))
    if with_bitdiff:
        out["bitdiff"] = torch.empty((n, BITDIFF_ROW_BYTES), **u8)
    if with_target:
        out["logp_base"] = torch.empty(n, **f64)
        out["logp_cand"] = torch.empty(n, **f64)
    return out


@_on_stream
def lcmp_compare_logits(base: torch.Tensor, cand: torch.Tensor, k: int = 20,
                        with_bitdiff: bool = False, v: int | None = None, out: dict | None = None,
                        workspace: torch.Tensor | None = None, stream=None,
                        events: tuple | None = None,
                        target: torch.Tensor | None = None) -> dict:
    """Compare baseline and candidate logits row by row (device tensors [n, >=v]).

    Returns a dict of device tensors (kl_topk, kl_full, margin, lse_base, lse_cand,
    top1_base, top2_base, top1_cand, flip, status, topk_idx and, with
    with_bitdiff, a raw [n, 88] uint8 `bitdiff` record tensor; see unpack_bitdiff).
    `target` (int32 device [n], the teacher-forced next tokens) adds logp_base
    and logp_cand.  `events`, a pair of raw hipEvent_t handles, selects
    lcmp_compare_logits_timed."""
    n = base.size(0)
    v = base.size(1) if v is None else v
    _check_rows(base, n, v, "base")
    _check_rows(cand, n, v, "cand")
    flags = LCMP_WITH_BITDIFF if with_bitdiff else 0
    _check_target(target, n)
    _check_workspace(workspace)
    if out is None:
        out = alloc_compare_outputs(n, k, base.device, with_bitdiff, target is not None)
    _check_out(out, n, k)
    if with_bitdiff and "bitdiff" not in out:
        raise ValueError("with_bitdiff needs out['bitdiff']")
    _on_gpu(("base", base), ("cand", cand), ("target", target), ("workspace", workspace),
            *[(f"out[{key!r}]", t) for key, t in out.items()])
    ws_bytes = int(_lib.lcmp_compare_workspace_bytes(n, v, k, flags))
    if ws_bytes == 0:
        raise LcmpError(-3, "lcmp_compare_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=base.device)
    ptrs = dict(out, target=target)
    ro = RowOut(*[_ptr(ptrs.get(f)) for f in ROW_OUT_FIELDS])
    args = (base.data_ptr(), _dtype_code(base), _ld(base), cand.data_ptr(), _dtype_code(cand),
            _ld(cand), n, v, k, flags, ctypes.byref(ro), _ptr(out.get("bitdiff")),
            workspace.data_ptr(), workspace.numel(), _stream(stream))
    if events is None:
        rc = _lib.lcmp_compare_logits(*args)
    else:
        rc = _lib.lcmp_compare_logits_timed(*args, events[0], events[1])
    _check(rc, "lcmp_compare_logits")
    return out


@_on_stream
def lcmp_compare_logits_noalloc(base: torch.Tensor, cand: torch.Tensor, out: dict, k: int = 20,
                                with_bitdiff: bool = False, v: int | None = None,
                                target: torch.Tensor | None = None, stream=None) -> dict:
    """lcmp_compare_logits without a workspace and without any allocation: the
    caller passes every output tensor in `out` (see alloc_compare_outputs), and
    the library's per-device scratch array serves as the workspace.  Calls that
    overlap on one device race; sizes beyond the array raise LCMP_EWORKSPACE."""
    n = base.size(0)
    v = base.size(1) if v is None else v
    _check_rows(base, n, v, "base")
    _check_rows(cand, n, v, "cand")
    flags = LCMP_WITH_BITDIFF if with_bitdiff else 0
    _check_target(target, n)
    _check_out(out, n, k)
    if with_bitdiff and "bitdiff" not in out:
        raise ValueError("with_bitdiff needs out['bitdiff']")
    _on_gpu(("base", base), ("cand", cand), ("target", target),
            *[(f"out[{key!r}]", t) for key, t in out.items()])
    ptrs = dict(out, target=target)
    ro = RowOut(*[_ptr(ptrs.get(f)) for f in ROW_OUT_FIELDS])
    rc = _lib.lcmp_compare_logits_noalloc(base.data_ptr(), _dtype_code(base), _ld(base),
                                          cand.data_ptr(), _dtype_code(cand), _ld(cand), n, v, k,
                                          flags, ctypes.byref(ro), _ptr(out.get("bitdiff")),
                                          _stream(stream))
    _check(rc, "lcmp_compare_logits_noalloc")
    return out


def _check_target(target, n):
    if target is not None:
        if target.dtype != torch.int32 or target.numel() != n or not target.is_contiguous():
            raise ValueError("target must be a contiguous int32 tensor of one id per row")


_RECORD_SPEC = {"topk_idx": torch.int32, "topk_val": torch.float32, "lse_rest": torch.float64,
                "status": torch.uint8, "logp_target": torch.float64}


def _check_record(record: dict, n: int, k_rec: int):
    for key in ("topk_idx", "topk_val", "lse_rest", "status"):
        if key not in record:
            raise ValueError(f"record lacks {key!r}")
    for key, t in record.items():
        if key not in _RECORD_SPEC:
            raise ValueError(f"unexpected record field {key!r}")
        if t is None:
            continue
        per = k_rec if key in ("topk_idx", "topk_val") else 1
        _check_buffer(t, _RECORD_SPEC[key], n * per, f"record[{key!r}]")


@_on_stream
def lcmp_record_baseline(base: torch.Tensor, k_rec: int = 20, target: torch.Tensor | None = None,
                         v: int | None = None, workspace: torch.Tensor | None = None,
                         stream=None) -> dict:
    """Compact record of baseline rows (device [n, >=v]): a dict of device
    tensors topk_idx [n, k_rec] int32, topk_val [n, k_rec] float32, lse_rest [n]
    float64, status [n] uint8, and logp_target [n] float64 when `target` is given."""
    n = base.size(0)
    v = base.size(1) if v is None else v
    _check_rows(base, n, v, "base")
    _check_target(target, n)
    _check_workspace(workspace)
    _on_gpu(("base", base), ("target", target), ("workspace", workspace))
    dev = base.device
    rec = dict(topk_idx=torch.empty((n, k_rec), dtype=torch.int32, device=dev),
               topk_val=torch.empty((n, k_rec), dtype=torch.float32, device=dev),
               lse_rest=torch.empty(n, dtype=torch.float64, device=dev),
               status=torch.empty(n, dtype=torch.uint8, device=dev))
    if target is not None:
        rec["logp_target"] = torch.empty(n, dtype=torch.float64, device=dev)
    ws_bytes = int(_lib.lcmp_record_workspace_bytes(n, v, k_rec))
    if ws_bytes == 0:
        raise LcmpError(-3, "lcmp_record_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    r = Record(*[_ptr(rec.get(f)) for f in RECORD_FIELDS])
    rc = _lib.lcmp_record_baseline(base.data_ptr(), _dtype_code(base), _ld(base), n, v, k_rec,
                                   _ptr(target), ctypes.byref(r), workspace.data_ptr(),
                                   workspace.numel(), _stream(stream))
    _check(rc, "lcmp_record_baseline")
    return rec


@_on_stream
def lcmp_compare_record(record: dict, cand: torch.Tensor, k: int | None = None,
                        target: torch.Tensor | None = None, v: int | None = None,
                        out: dict | None = None, workspace: torch.Tensor | None = None,
                        stream=None, events: tuple | None = None) -> dict:
    """Compare candidate rows (device [n, >=v]) against a record from
    lcmp_record_baseline, using its first k entries (default all).  Returns the
    outputs of lcmp_compare_logits except kl_full (and bitdiff); with `target`,
    logp_cand, plus logp_base when the record holds logp_target."""
    n = cand.size(0)
    v = cand.size(1) if v is None else v
    _check_rows(cand, n, v, "cand")
    if record["topk_idx"].dim() != 2 or record["topk_idx"].size(0) != n:
        raise ValueError("the record and the candidate need the same number of rows")
    k_rec = record["topk_idx"].size(1)
    k = k_rec if k is None else k
    _check_record(record, n, k_rec)
    _check_target(target, n)
    _check_workspace(workspace)
    if out is None:
        out = alloc_compare_outputs(n, k, cand.device)
        del out["kl_full"]
        if target is not None:
            out["logp_cand"] = torch.empty(n, dtype=torch.float64, device=cand.device)
            if record.get("logp_target") is not None:
                out["logp_base"] = torch.empty(n, dtype=torch.float64, device=cand.device)
    _check_out(out, n, k, allowed=set(_OUT_SPEC) - {"kl_full", "bitdiff"})
    _on_gpu(("cand", cand), ("target", target), ("workspace", workspace),
            *[(f"record[{key!r}]", t) for key, t in record.items()],
            *[(f"out[{key!r}]", t) for key, t in out.items()])
    ws_bytes = int(_lib.lcmp_compare_record_workspace_bytes(n, v))
    if ws_bytes == 0:
        raise LcmpError(-3, "lcmp_compare_record_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=cand.device)
    r = Record(*[_ptr(record.get(f)) for f in RECORD_FIELDS])
    ptrs = dict(out, target=target)
    ro = RowOut(*[_ptr(ptrs.get(f)) for f in ROW_OUT_FIELDS])
    args = (ctypes.byref(r), k_rec, cand.data_ptr(), _dtype_code(cand), _ld(cand), n, v, k,
            ctypes.byref(ro), workspace.data_ptr(), workspace.numel(), _stream(stream))
    if events is None:
        rc = _lib.lcmp_compare_record(*args)
    else:
        rc = _lib.lcmp_compare_record_timed(*args, events[0], events[1])
    _check(rc, "lcmp_compare_record")
    return out


@_on_stream
def lcmp_bitdiff(a: torch.Tensor, b: torch.Tensor, cols: int | None = None,
                 out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 stream=None, events: tuple | None = None) -> torch.Tensor:
    """Per-row bitwise / ULP statistics; returns a raw [rows, 88] uint8 record
    tensor.  `events`, a pair of raw hipEvent_t handles, selects
    lcmp_bitdiff_timed."""
    rows = a.size(0)
    cols = a.size(1) if cols is None else cols
    _check_rows(a, rows, cols, "a")
    _check_rows(b, rows, cols, "b")
    _check_workspace(workspace)
    if out is None:
        out = torch.empty((rows, BITDIFF_ROW_BYTES), dtype=torch.uint8, device=a.device)
    _check_buffer(out, torch.uint8, rows * BITDIFF_ROW_BYTES, "out")
    _on_gpu(("a", a), ("b", b), ("out", out), ("workspace", workspace))
    ws_bytes = int(_lib.lcmp_bitdiff_workspace_bytes(rows, cols))
    if ws_bytes == 0:
        raise LcmpError(-3, "lcmp_bitdiff_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=a.device)
    args = (a.data_ptr(), _dtype_code(a), _ld(a), b.data_ptr(), _dtype_code(b), _ld(b), rows,
            cols, out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(stream))
    if events is None:
        rc = _lib.lcmp_bitdiff(*args)
    else:
        rc = _lib.lcmp_bitdiff_timed(*args, events[0], events[1])
    _check(rc, "lcmp_bitdiff")
    return out


@_on_stream
def lcmp_read_probe(base: torch.Tensor, cand: torch.Tensor, v: int | None = None,
                    workspace: torch.Tensor | None = None, stream=None,
                    events: tuple | None = None) -> None:
    """Read-only reference stream over the row pairs in the comparison's own
    access pattern (measurement only; see lcmp.h)."""
    n = base.size(0)
    v = base.size(1) if v is None else v
    _check_rows(base, n, v, "base")
    _check_rows(cand, n, v, "cand")
    _check_workspace(workspace)
    _on_gpu(("base", base), ("cand", cand), ("workspace", workspace))
    if workspace is None:
        ws_bytes = int(_lib.lcmp_compare_workspace_bytes(n, v, 1, 0))
        if ws_bytes == 0:
            raise LcmpError(-3, "lcmp_compare_workspace_bytes")
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=base.device)
    ev = (None, None) if events is None else events
    rc = _lib.lcmp_read_probe(base.data_ptr(), _dtype_code(base), _ld(base), cand.data_ptr(),
                              _dtype_code(cand), _ld(cand), n, v, workspace.data_ptr(),
                              workspace.numel(), _stream(stream), ev[0], ev[1])
    _check(rc, "lcmp_read_probe")


@_on_stream
def lcmp_bin_report(margin, flip, kl_topk, kl_full, edges, status=None, group=None,
                    n_groups: int = 1, big_margin: float = 1.0, workspace=None, stream=None,
                    bins=None, summary=None):
    """Margin-bin report; returns raw (bins [n_groups*n_edges, 56] uint8,
    summary [n_groups, 24] uint8) device tensors (see unpack_bins)."""
    n = margin.numel()
    edges = [float(e) for e in edges]
    ne = len(edges)
    dev = margin.device
    for what, t, dtype in (("margin", margin, torch.float64), ("flip", flip, torch.uint8),
                           ("kl_topk", kl_topk, torch.float64), ("kl_full", kl_full, torch.float64),
                           ("status", status, torch.uint8), ("group", group, torch.int32)):
        if t is not None:
            _check_buffer(t, dtype, n, what)
    _check_workspace(workspace)
    if bins is None:
        bins = torch.empty((n_groups * ne, BIN_BYTES), dtype=torch.uint8, device=dev)
    if summary is None:
        summary = torch.empty((n_groups, GROUP_SUMMARY_BYTES), dtype=torch.uint8, device=dev)
    _check_buffer(bins, torch.uint8, n_groups * ne * BIN_BYTES, "bins")
    _check_buffer(summary, torch.uint8, n_groups * GROUP_SUMMARY_BYTES, "summary")
    _on_gpu(("margin", margin), ("flip", flip), ("kl_topk", kl_topk), ("kl_full", kl_full),
            ("status", status), ("group", group), ("workspace", workspace), ("bins", bins),
            ("summary", summary))
    summ = summary
    ws_bytes = int(_lib.lcmp_bin_workspace_bytes(n, n_groups, ne))
    if ws_bytes == 0:
        raise LcmpError(-3, "lcmp_bin_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    e_arr = (ctypes.c_double * ne)(*edges)
    rc = _lib.lcmp_bin_report(_ptr(margin), _ptr(flip), _ptr(kl_topk), _ptr(kl_full),
                              _ptr(status), _ptr(group), n_groups, n, e_arr, ne, big_margin,
                              bins.data_ptr(), summ.data_ptr(), workspace.data_ptr(),
                              workspace.numel(), _stream(stream))
    _check(rc, "lcmp_bin_report")
    return bins, summ


@_on_stream
def lcmp_perturb(src: torch.Tensor, mode: int, param: int = 0, out: torch.Tensor | None = None,
                 out_dtype: torch.dtype | None = None, stream=None) -> torch.Tensor:
    """Precision perturbation of a [rows, cols] fp32 / bf16 device tensor (keep
    `param` fraction bits, or e4m3, or e4m3 after x448); returns `out`, by
    default a new fp32 tensor (bf16 with out_dtype=torch.bfloat16)."""
    if src.dim() == 1:
        src = src.view(1, -1)
    rows, cols = src.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=out_dtype or torch.float32, device=src.device)
    elif out.dim() == 1:
        out = out.view(1, -1)
    if out.shape[0] != rows or out.shape[1] < cols:
        raise ValueError("out must hold [rows, cols]")
    _dtype_code(src)
    _dtype_code(out)
    _on_gpu(("src", src), ("out", out))
    rc = _lib.lcmp_perturb(src.data_ptr(), _dtype_code(src), _ld(src), out.data_ptr(),
                           _dtype_code(out), _ld(out), rows, cols, mode, param, _stream(stream))
    _check(rc, "lcmp_perturb")
    return out


# ----------------------------------------------------------------------------- unpacking
def _np():
    import numpy as np
    return np


def bitdiff_dtype():
    np = _np()
    return np.dtype([("ndiff", np.int64), ("first_diff", np.int64), ("nonfinite_a", np.int64),
                     ("nonfinite_b", np.int64), ("max_ulp", np.uint32), ("pad_", np.uint32),
                     ("max_abs", np.float64), ("sum_abs", np.float64),
                     ("sum_sq_diff", np.float64), ("sum_sq_base", np.float64),
                     ("mean_abs", np.float64), ("rel_l2", np.float64)])


def bin_dtype():
    np = _np()
    return np.dtype([("count", np.int64), ("flips", np.int64), ("ties", np.int64),
                     ("tie_flips", np.int64), ("sum_kl_topk", np.float64),
                     ("sum_kl_full", np.float64), ("max_kl_topk", np.float64)])


def summary_dtype():
    np = _np()
    return np.dtype([("big_margin_flips", np.int64), ("excluded", np.int64),
                     ("unbinned", np.int64)])


def unpack_bitdiff(raw: torch.Tensor):
    """[rows, 88] uint8 device/host tensor -> numpy structured array."""
    return raw.cpu().numpy().reshape(-1).view(bitdiff_dtype())


def unpack_bins(bins: torch.Tensor, summ: torch.Tensor, n_groups: int = 1):
    b = bins.cpu().numpy().reshape(-1).view(bin_dtype()).reshape(n_groups, -1)
    s = summ.cpu().numpy().reshape(-1).view(summary_dtype())
    return b, s
