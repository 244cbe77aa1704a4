"""The allocation-free compare (lcmp_compare_logits_noalloc) against the
compare with a caller's workspace (lcmp_compare_logits): identical outputs,
bit for bit, on two calls in a row whose second input is smaller, with rows
that send work to the bucket pass, so the shared scratch array holds the first
call's records and list when the second call starts."""
import numpy as np
import pytest

from helpers import to_device

pytestmark = pytest.mark.gpu


def _inputs(seed, n, v, tb, tc):
    import torch
    rng = np.random.default_rng(seed)
    a = (1.5 * rng.standard_normal((n, v))).astype(np.float32)
    b = (a + 0.03 * rng.standard_normal((n, v))).astype(np.float32)
    b[1, (int(np.argmax(a[1])) + 1) % v] = a[1].max() + 1.0     # a flip
    b[2] = a[2] - 30.0                                          # far-apart normalisers
    b[3, :] -= 40.0                                             # a listed bucket row
    b[3, np.argsort(a[3])[-20:]] += 40.0

    def conv(t, x):
        if t == "f32":
            return x
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    return conv(tb, a), conv(tc, b)


def _snap(out):
    return {key: val.cpu().numpy().copy() for key, val in out.items()}


@pytest.mark.parametrize("first,second", [
    ((2048, 151936, "f32", "bf16", 20, True), (96, 30011, "bf16", "bf16", 7, True)),
    ((512, 151936, "f32", "f32", 20, True), (33, 5000, "f32", "bf16", 64, False)),
])
def test_noalloc_matches_workspace_call(first, second):
    import torch
    import logit_distribution_diffing_amd as L
    for seed, (n, v, tb, tc, k, bits) in enumerate((first, second)):
        print(f"[case] noalloc call {seed + 1}: {n}x{v} {tb}/{tc} k={k} bits={bits}", flush=True)
        a, b = _inputs(100 + seed, n, v, tb, tc)
        da, db = to_device(a), to_device(b)
        ref = L.lcmp_compare_logits(da, db, k=k, with_bitdiff=bits)
        out = L.alloc_compare_outputs(n, k, "cuda", with_bitdiff=bits)
        for t in out.values():
            t.fill_(7)
        torch.cuda.synchronize()
        L.lcmp_compare_logits_noalloc(da, db, out, k=k, with_bitdiff=bits)
        torch.cuda.synchronize()
        want, got = _snap(ref), _snap(out)
        assert want.keys() == got.keys()
        for key in want:
            assert got[key].tobytes() == want[key].tobytes(), key


def test_noalloc_rejects_sizes_beyond_the_array():
    """Refused on the host, before any launch, with LCMP_EWORKSPACE."""
    import ctypes
    import logit_distribution_diffing_amd as L
    lib = L.lib()
    n, v, k = 262144, 151936, 20
    assert lib.lcmp_compare_workspace_bytes(n, v, k, 1) > L.LCMP_NOALLOC_SCRATCH_BYTES
    fake = 0x10000   # never dereferenced: the size check comes first
    rc = lib.lcmp_compare_logits_noalloc(fake, 1, v, fake, 1, v, n, v, k, 1,
                                         ctypes.byref(L.RowOut()), fake, None)
    assert rc == -4
    assert lib.lcmp_compare_logits_noalloc(fake, 1, v, fake, 1, v, 73728, v, k, 1,
                                           None, fake, None) == -1   # no out struct
