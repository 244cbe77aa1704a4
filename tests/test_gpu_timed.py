"""The instrumented entry points (lcmp_compare_logits_timed, lcmp_bitdiff_timed,
lcmp_compare_record_timed, lcmp_read_probe with events).

The two events ride on the streaming kernel's dispatch: the results must equal
those of the plain call bit for bit, a launch must show a positive duration,
and a call with no rows must still record both events (back to back), so that
a caller can read an elapsed time for every call it timed."""
import ctypes

import numpy as np
import pytest

from helpers import to_device

pytestmark = pytest.mark.gpu

DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence


def _case(msg):
    print(f"[case] {msg}", flush=True)


class _Events:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def pair(self, flags):
        out = []
        for _ in range(2):
            e = ctypes.c_void_p()
            assert self.lib.hipEventCreateWithFlags(ctypes.byref(e), flags) == 0
            self.made.append(e.value)
            out.append(e.value)
        return tuple(out)

    def ms(self, pair):
        t = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(t), pair[0], pair[1])
        assert rc == 0, f"hipEventElapsedTime returned {rc}"
        return t.value

    def close(self):
        for e in self.made:
            self.lib.hipEventDestroy(e)


@pytest.fixture
def events():
    ev = _Events()
    yield ev
    ev.close()


def _inputs(seed, n, v):
    rng = np.random.default_rng(seed)
    a = (1.5 * rng.standard_normal((n, v))).astype(np.float32)
    b = (a + 0.03 * rng.standard_normal((n, v))).astype(np.float32)
    return a, b


def _bytes(d):
    return {k: v.detach().cpu().numpy().tobytes() for k, v in d.items()}


@pytest.mark.parametrize("n", [0, 37])
@pytest.mark.parametrize("flags", [0, DISABLE_SYSTEM_FENCE])
def test_compare_timed(events, n, flags):
    import torch
    import logit_distribution_diffing_amd as L
    v, k = 20001, 20
    _case(f"compare timed n={n} flags={flags:#x}")
    a, b = _inputs(5 + n, n, v)
    da, db = to_device(a), to_device(b).to(torch.bfloat16)
    plain = L.lcmp_compare_logits(da, db, k=k, with_bitdiff=True)
    ev = events.pair(flags)
    timed = L.lcmp_compare_logits(da, db, k=k, with_bitdiff=True, events=ev)
    torch.cuda.synchronize()
    assert _bytes(plain) == _bytes(timed)
    ms = events.ms(ev)
    assert ms > 0.0 if n else ms >= 0.0


@pytest.mark.parametrize("rows", [0, 65])
def test_bitdiff_timed(events, rows):
    import torch
    import logit_distribution_diffing_amd as L
    cols = 5120
    _case(f"bitdiff timed rows={rows}")
    a, b = _inputs(9 + rows, rows, cols)
    da, db = to_device(a).to(torch.bfloat16), to_device(b).to(torch.bfloat16)
    plain = L.lcmp_bitdiff(da, db)
    ev = events.pair(DISABLE_SYSTEM_FENCE)
    timed = L.lcmp_bitdiff(da, db, events=ev)
    torch.cuda.synchronize()
    assert plain.cpu().numpy().tobytes() == timed.cpu().numpy().tobytes()
    ms = events.ms(ev)
    assert ms > 0.0 if rows else ms >= 0.0


@pytest.mark.parametrize("n", [0, 29])
def test_compare_record_timed(events, n):
    import torch
    import logit_distribution_diffing_amd as L
    v, k = 30001, 20
    _case(f"compare against a record, timed n={n}")
    a, b = _inputs(13 + n, n, v)
    da, db = to_device(a), to_device(b).to(torch.bfloat16)
    rec = L.lcmp_record_baseline(da, k_rec=k)
    plain = L.lcmp_compare_record(rec, db, k=k)
    ev = events.pair(DISABLE_SYSTEM_FENCE)
    timed = L.lcmp_compare_record(rec, db, k=k, events=ev)
    torch.cuda.synchronize()
    assert _bytes(plain) == _bytes(timed)
    ms = events.ms(ev)
    assert ms > 0.0 if n else ms >= 0.0


@pytest.mark.parametrize("n", [0, 16])
def test_read_probe_timed(events, n):
    import torch
    import logit_distribution_diffing_amd as L
    v = 151936
    _case(f"read probe timed n={n}")
    a, b = _inputs(17 + n, n, v)
    da, db = to_device(a), to_device(b)
    ev = events.pair(DISABLE_SYSTEM_FENCE)
    L.lcmp_read_probe(da, db, events=ev)
    torch.cuda.synchronize()
    ms = events.ms(ev)
    assert ms > 0.0 if n else ms >= 0.0
