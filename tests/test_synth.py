"""Checks of the synthetic input generators (CPU)."""
import numpy as np
import pytest
import torch

import oracle
import synth


def test_bf16_rne_against_torch_on_every_high_half():
    """All 65536 upper halves x the low halves that decide the rounding (zero, one,
    just below / at / above the tie, all ones, and a few others), through the C
    routine, against torch's float32 -> bfloat16 cast."""
    import ctypes
    L = synth._L()
    f = ctypes.c_float
    lows = np.array([0, 1, 0x1234, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF], np.uint32)
    hi = np.arange(1 << 16, dtype=np.uint32)
    u = ((hi[:, None] << 16) | lows[None, :]).ravel()
    fv = u.view(np.float32)
    ref = torch.from_numpy(fv).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    fn = L.synth_bf16_rne
    ours = np.fromiter((fn(f(x)) for x in fv.tolist()), np.uint16, count=fv.size)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all((ours[nan] & 0x7F) != 0)


def test_rows_independent_of_block_and_threads():
    a1, b1 = synth.segment(synth.SEED_BASE + 1, 0, 6, 4096)
    a2, b2 = synth.segment(synth.SEED_BASE + 1, 3, 3, 4096)
    assert np.array_equal(a1[3:], a2) and np.array_equal(b1[3:], b2)
    c1, d1 = synth.corpus(synth.SEED_BASE + 2, 500, 30, 4096, 10240)
    c2, d2 = synth.corpus(synth.SEED_BASE + 2, 510, 10, 4096, 10240)
    assert np.array_equal(c1[10:20], c2) and np.array_equal(d1[10:20], d2)


def test_segment_candidate_is_bf16_rounding_of_baseline():
    a, b = synth.segment(synth.SEED_BASE + 1, 0, 4, 4096)
    ref = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    assert np.array_equal(b, ref)


def test_normals_are_standard_and_bounded():
    z = synth.normals(123, 1, 0, 1 << 20)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    assert np.abs(z).max() <= 8.58


def test_corpus_swap_rows_have_constructed_big_margin_flip():
    w = synth.WORKLOADS["corpus"]
    rows = synth.swap_rows(w["seed"], w["n"], w["swap_frac"])
    assert rows.size == 51 and np.unique(rows).size == 51
    v = 8192
    sel = rows[:4]
    for r in sel:
        a, b = synth.corpus(w["seed"], int(r), 1, v, w["n"], w["swap_frac"])
        res = oracle.compare(a, b, k=20)
        assert res["margin"][0] > 1.25 and res["flip"][0] == 1
    # a neighbouring ordinary row cannot flip at a margin above 1
    a, b = synth.corpus(w["seed"], int(sel[0]) + 1, 1, v, w["n"], w["swap_frac"])
    res = oracle.compare(a, b, k=20)
    assert not (res["flip"][0] == 1 and res["margin"][0] > 1)


def test_ulp_move_round_trip_and_order():
    for width in (16, 32):
        for u in (0, 1, 0x3F80, 0x8000, 0x8001, 0x7F7F) if width == 16 else \
                (0, 1, 0x3F800000, 0x80000000, 0x80000001, 0x7F7FFFFF):
            for s in (-3, -1, 1, 3):
                m = synth.ulp_move(u, s, width)
                assert synth.ulp_move(m, -s, width) == u
    # +0 moved down by one is -0
    assert synth.ulp_move(0, -1, 32) == 0x80000000
    assert synth.ulp_move(0x3F800000, 1, 32) == 0x3F800001


def test_injection_counts_and_bounds():
    a = synth.bf16_normal(7, 0, 65, 5120)
    b, pos, steps = synth.inject_ulp(7, 65, a, 0.001)
    assert pos.size == round(0.001 * a.size) and np.unique(pos).size == pos.size
    assert set(np.abs(steps)) <= {1, 2, 3}
    diff = np.flatnonzero(a.ravel() != b.ravel())
    assert np.array_equal(diff, pos)
    assert np.all(np.isfinite(synth.bf16_to_f32(b)))
