"""GPU parity of lcmp_perturb (precision perturbations) against the oracle, bit for bit."""
import numpy as np
import pytest

import oracle
import synth
from helpers import to_device

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _values(rows, cols, seed):
    """Wide-range fp32 values with the special ones: zeros, subnormals, the
    largest finite, infinities, NaNs with payloads in either half, ties."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * 10 ** rng.uniform(-44, 38, (rows, cols)))
    x = x.astype(np.float32)
    flat = x.reshape(-1)
    special = np.array([0x00000000, 0x80000000, 0x00000001, 0x807fffff, 0x7f7fffff, 0xff7fffff,
                        0x7f800000, 0xff800000, 0x7fc00000, 0x7f800001, 0xffc00123, 0x3f808000,
                        0x3f818000, 0x3a800000, 0x3a800001, 0x3b000000, 0x43e00000, 0x43e80000,
                        0x43f00000], np.uint32).view(np.float32)
    flat[:special.size] = special[: min(special.size, flat.size)]
    return x


def _gpu(src, mode, param, out_bf16=False, ld_pad=0):
    import torch
    import logit_distribution_diffing_amd as L
    t = to_device(src)
    if ld_pad:
        wide = torch.zeros((t.shape[0], t.shape[1] + ld_pad), dtype=t.dtype, device="cuda")
        wide[:, : t.shape[1]] = t
        t = wide[:, : src.shape[1]]
    out = L.lcmp_perturb(t, mode, param, out_dtype=torch.bfloat16 if out_bf16 else None)
    torch.cuda.synchronize()
    if out_bf16:
        return out.view(torch.int16).cpu().numpy().view(np.uint16)
    return out.cpu().numpy()


def _same_bits(g, o):
    gb = g.view(np.uint16 if g.dtype == np.uint16 else np.uint32)
    ob = o.view(np.uint16 if o.dtype == np.uint16 else np.uint32)
    bad = np.flatnonzero(gb.ravel() != ob.ravel())
    assert bad.size == 0, f"{bad.size} elements differ, first at {bad[:5]}: " \
                          f"{gb.ravel()[bad[:5]]} vs {ob.ravel()[bad[:5]]}"


@pytest.mark.parametrize("m", [0, 1, 3, 4, 7, 10, 13, 16, 22, 23])
def test_keep_mantissa_bits(m):
    _case(f"mantissa {m}")
    x = _values(7, 3001, m)
    _same_bits(_gpu(x, oracle.PERTURB_MANTISSA, m), oracle.perturb(x, oracle.PERTURB_MANTISSA, m))
    if m <= 7:
        _same_bits(_gpu(x, oracle.PERTURB_MANTISSA, m, out_bf16=True),
                   oracle.perturb(x, oracle.PERTURB_MANTISSA, m, out_bf16=True))


@pytest.mark.parametrize("mode", [1, 2])
def test_e4m3_modes(mode):
    _case(f"e4m3 mode {mode}")
    rng = np.random.default_rng(mode)
    wide = _values(5, 4099, 40 + mode)
    probs = rng.random((5, 4099)).astype(np.float32) ** 6   # softmax-like weights in [0, 1]
    for x in (wide, probs):
        _same_bits(_gpu(x, mode, 0), oracle.perturb(x, mode))
        if mode == 1:
            _same_bits(_gpu(x, mode, 0, out_bf16=True), oracle.perturb(x, mode, out_bf16=True))


@pytest.mark.parametrize("cols,ld_pad", [(1, 0), (3, 0), (4, 0), (1023, 0), (1024, 0), (1025, 0),
                                         (5000, 1), (5000, 3), (2049, 4)])
def test_ragged_and_unaligned_rows(cols, ld_pad):
    _case(f"ragged cols={cols} pad={ld_pad}")
    x = _values(6, cols, cols)
    for mode, m in ((0, 5), (1, 0), (2, 0)):
        _same_bits(_gpu(x, mode, m, ld_pad=ld_pad), oracle.perturb(x, mode, m))


def test_bf16_input_and_in_place():
    import torch
    import logit_distribution_diffing_amd as L
    _case("bf16 input, in place")
    a = synth.bf16_normal(synth.SEED_BASE + 3, 0, 9, 5120)
    _same_bits(_gpu(a, 0, 4, out_bf16=True), oracle.perturb(a, 0, 4, out_bf16=True))
    _same_bits(_gpu(a, 1, 0), oracle.perturb(a, 1))
    x = _values(4, 3000, 9)
    t = torch.from_numpy(x).cuda()
    L.lcmp_perturb(t, 0, 9, out=t)
    torch.cuda.synchronize()
    _same_bits(t.cpu().numpy(), oracle.perturb(x, 0, 9))


def test_logit_rows_at_vocabulary_size():
    """The segment-shaped logits (512 x 151936 fp32) rounded to 7 bits: the bf16
    candidate of the segment workload."""
    _case("512 x 151936 keep 7 bits")
    w = synth.WORKLOADS["segment"]
    a, b = synth.segment(w["seed"], 0, 512, w["v"])
    g = _gpu(a, 0, 7)
    _same_bits(g, b)                                  # the generator's own bf16 rounding
    rows = [0, 1, 255, 511]
    _same_bits(g[rows], oracle.perturb(a[rows], 0, 7))
