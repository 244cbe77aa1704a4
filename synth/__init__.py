"""Seeded synthetic inputs for the logit-comparison workloads.

Thin ctypes wrapper over ``synth.c``.  This module produces input bytes only;
it contains none of the comparison arithmetic, so both the HIP path and the
oracle may be fed from it.  bf16 tensors are returned as ``uint16`` bit
patterns.

Workloads (shapes follow the teacher-forced scoring setup of the logit
distribution-diffing page: N scored positions x vocabulary V):

  tiny     N=64,    V=1024,   fp32/fp32   a = 2Z + U[0,8] peak, b = a + 0.05Z'
  segment  N=512,   V=151936, fp32/fp32   code/prose rows, b = bf16(a) widened
  corpus   N=10240, V=151936, fp32/bf16   5 depths x 4 segments x 512 positions,
                                          b = bf16(a + 0.02Z'), 0.5% top-1/top-2 swaps
  sweep    bf16 [T,5120] for 8 values of T plus fp32 [512,151936], 0.1% of the
           elements moved by +-1..3 ULP
  stream   N=65536, V=151936, bf16/bf16   b = bf16(a + 0.01Z')
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

SEED_BASE = 0x5EED0000
V_FULL = 151936

WORKLOADS = {
    "tiny": dict(n=64, v=1024, base="f32", cand="f32", k=20, seed=SEED_BASE + 0),
    "segment": dict(n=512, v=V_FULL, base="f32", cand="f32", k=20, seed=SEED_BASE + 1),
    "corpus": dict(n=10240, v=V_FULL, base="f32", cand="bf16", k=20, seed=SEED_BASE + 2,
                   swap_frac=0.005),
    "sweep": dict(t_list=(1, 17, 65, 1024, 1502, 1777, 4095, 4096), cols=5120,
                  logit_rows=512, v=V_FULL, frac=0.001, seed=SEED_BASE + 3),
    "stream": dict(n=65536, v=V_FULL, base="bf16", cand="bf16", k=20, seed=SEED_BASE + 4),
}

DEFAULT_EDGES = (0.1, 0.25, 0.5, 1.0, 2.0, float("inf"))


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (OpenMP)."""
    if force or not os.path.exists(_SO):
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", _SO,
               os.path.join(_HERE, "synth.c"), "-lm"]
        subprocess.run(cmd, check=True)
    return _SO


def _L():
    global _lib
    if _lib is None:
        # SYNTH_LIB names another build of synth.c (the sanitizer test loads an
        # instrumented one through it); by default the in-tree build
        path = os.environ.get("SYNTH_LIB")
        if not path:
            build()
            path = _SO
        lib = ctypes.CDLL(path)
        u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        lib.synth_key.restype = u64
        lib.synth_key.argtypes = [u64, u64]
        lib.synth_u64.restype = u64
        lib.synth_u64.argtypes = [u64, u64]
        lib.synth_bf16_rne.restype = ctypes.c_uint16
        lib.synth_bf16_rne.argtypes = [ctypes.c_float]
        for name in ("synth_tiny", "synth_segment"):
            getattr(lib, name).argtypes = [u64, i64, i64, i64, vp, vp]
        lib.synth_corpus.argtypes = [u64, i64, i64, i64, vp, vp, vp]
        lib.synth_stream.argtypes = [u64, i64, i64, i64, vp, vp]
        lib.synth_bf16_normal.argtypes = [u64, i64, i64, i64, vp]
        lib.synth_logit_rows.argtypes = [u64, i64, i64, i64, vp]
        lib.synth_pick_hash.argtypes = [u64, u64, i64, i64, vp]
        lib.synth_ulp_step.restype = ctypes.c_int
        lib.synth_ulp_step.argtypes = [u64, i64]
        lib.synth_ulp_move.restype = ctypes.c_uint32
        lib.synth_ulp_move.argtypes = [ctypes.c_uint32, ctypes.c_int, ctypes.c_int]
        lib.synth_apply_ulp.argtypes = [vp, ctypes.c_int, vp, vp, i64]
        lib.synth_normals.argtypes = [u64, u64, i64, i64, vp]
        _lib = lib
    return _lib


def _ptr(x) -> int:
    """Address of a numpy array or of a CPU torch tensor."""
    if isinstance(x, np.ndarray):
        assert x.flags["C_CONTIGUOUS"]
        return x.ctypes.data
    return int(x.data_ptr())


def _out(shape, dtype, out):
    if out is None:
        return np.empty(shape, dtype=dtype)
    return out


# ----------------------------------------------------------------------------- scalars
def bf16_rne(f: float) -> int:
    return int(_L().synth_bf16_rne(ctypes.c_float(f)))


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 (exact)."""
    return (h.astype(np.uint32) << 16).view(np.float32)


def normals(seed: int, stream: int, row: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _L().synth_normals(seed, stream, row, n, _ptr(out))
    return out


# ----------------------------------------------------------------------------- rows
def tiny(seed: int, r0: int, nr: int, v: int, out_a=None, out_b=None):
    a = _out((nr, v), np.float32, out_a)
    b = _out((nr, v), np.float32, out_b)
    _L().synth_tiny(seed, r0, nr, v, _ptr(a), _ptr(b))
    return a, b


def segment(seed: int, r0: int, nr: int, v: int, out_a=None, out_b=None):
    a = _out((nr, v), np.float32, out_a)
    b = _out((nr, v), np.float32, out_b)
    _L().synth_segment(seed, r0, nr, v, _ptr(a), _ptr(b))
    return a, b


def pick_subset(seed: int, stream: int, numel: int, m: int) -> np.ndarray:
    """Uniform random m-subset of range(numel): the m smallest selection hashes (sorted)."""
    if m <= 0:
        return np.zeros(0, dtype=np.int64)
    h = np.empty(numel, dtype=np.uint64)
    _L().synth_pick_hash(seed, stream, 0, numel, _ptr(h))
    if m >= numel:
        return np.arange(numel, dtype=np.int64)
    sel = np.argpartition(h, m - 1)[:m]
    return np.sort(sel.astype(np.int64))


def swap_rows(seed: int, n: int, frac: float = 0.005) -> np.ndarray:
    """Rows of the corpus workload that carry a constructed top-1/top-2 exchange."""
    return pick_subset(seed, 2, n, int(np.floor(frac * n)))


def corpus(seed: int, r0: int, nr: int, v: int, n_total: int, frac: float = 0.005,
           out_a=None, out_b=None):
    a = _out((nr, v), np.float32, out_a)
    b = _out((nr, v), np.uint16, out_b)
    rows = swap_rows(seed, n_total, frac)
    flags = np.zeros(nr, dtype=np.uint8)
    sel = rows[(rows >= r0) & (rows < r0 + nr)] - r0
    flags[sel] = 1
    _L().synth_corpus(seed, r0, nr, v, _ptr(flags), _ptr(a), _ptr(b))
    return a, b


CORPUS_DEPTHS = 5
CORPUS_GROUPS = 2 * CORPUS_DEPTHS


def corpus_groups(n: int = 10240) -> np.ndarray:
    """Row group of each corpus position, for per-group margin bins: context
    depth * 2 + 1 for a prose segment (0 for code).  Row r is depth*2048 +
    segment*512 + position; segments 0-1 are code-like, 2-3 prose-like."""
    r = np.arange(n, dtype=np.int64)
    depth = r // 2048
    prose = ((r // 512) % 4) >= 2
    return (2 * depth + prose).astype(np.int32)


def stream(seed: int, r0: int, nr: int, v: int, out_a=None, out_b=None):
    a = _out((nr, v), np.uint16, out_a)
    b = _out((nr, v), np.uint16, out_b)
    _L().synth_stream(seed, r0, nr, v, _ptr(a), _ptr(b))
    return a, b


def bf16_normal(seed: int, r0: int, nr: int, cols: int, out=None):
    a = _out((nr, cols), np.uint16, out)
    _L().synth_bf16_normal(seed, r0, nr, cols, _ptr(a))
    return a


def logit_rows(seed: int, r0: int, nr: int, v: int, out=None):
    a = _out((nr, v), np.float32, out)
    _L().synth_logit_rows(seed, r0, nr, v, _ptr(a))
    return a


def ulp_steps(seed: int, m: int) -> np.ndarray:
    L = _L()
    return np.array([L.synth_ulp_step(seed, j) for j in range(m)], dtype=np.int32)


def inject_ulp(seed: int, stream_id: int, base: np.ndarray, frac: float = 0.001):
    """Copy of `base` (uint16 bf16 or float32/uint32 patterns) with round(frac*numel)
    distinct uniformly chosen elements moved by +-1..3 units in the ordered-integer
    view of the format.  Returns (perturbed, flat positions, steps)."""
    width = 16 if base.dtype == np.uint16 else 32
    bits = base.view(np.uint16 if width == 16 else np.uint32)
    m = int(round(frac * bits.size))
    pos = pick_subset(seed, stream_id, bits.size, m)
    steps = ulp_steps(seed * 31 + stream_id, m)
    out = np.ascontiguousarray(bits.copy())
    _L().synth_apply_ulp(_ptr(out), width, _ptr(pos), _ptr(steps), m)
    return out.view(base.dtype), pos, steps


def ulp_move(u: int, step: int, width: int) -> int:
    return int(_L().synth_ulp_move(u, step, width))
