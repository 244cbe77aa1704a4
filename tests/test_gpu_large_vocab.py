"""GPU parity at vocabularies beyond the workloads' V = 151936.

- A few rows of V = 1,000,003 (ragged): the chunk choice splits each row into
  the most chunks it allows, and the merge reads that many chunk records.
- 4096 rows of V = 262,181: one chunk per row, so each wave runs 513 steps,
  folding its float partials and 16-bit differing counters over a chunk
  almost twice as long as the workloads'.  Sampled rows (first, last, and
  random ones) are compared with the oracle element by element.

Inputs are seeded: numpy for the small case, a seeded torch generator on the
device for the large one (the sampled rows are copied back to the host, so
both sides see the same values)."""
import numpy as np
import pytest

import oracle
from helpers import assert_bitdiff_equal, assert_compare_equal, gpu_compare

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _bf16(x: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("pair", [("f32", "f32"), ("f32", "bf16"), ("bf16", "bf16")])
def test_million_token_vocab(pair):
    n, v, k = 3, 1_000_003, 20
    _case(f"v={v} n={n} {pair[0]}/{pair[1]}")
    rng = np.random.default_rng(1_000_003)
    a = (1.5 * rng.standard_normal((n, v))).astype(np.float32)
    a[np.arange(n), rng.integers(0, v, n)] += np.float32(9.0)
    b = (a + 0.01 * rng.standard_normal((n, v))).astype(np.float32)
    ha = _bf16(a) if pair[0] == "bf16" else a
    hb = _bf16(b) if pair[1] == "bf16" else b
    g = gpu_compare(ha, hb, k=k, with_bitdiff=True)
    assert_compare_equal(g, oracle.compare(ha, hb, k=k))
    assert_bitdiff_equal(g["bitdiff"], oracle.bitdiff(ha, hb))


@pytest.mark.parametrize("base_t", ["bf16", "f32"])
def test_long_chunks(base_t):
    import torch
    import logit_distribution_diffing_amd as L
    n, v, k = 4096, 262_181, 20
    _case(f"long chunks n={n} v={v} {base_t}/bf16")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(262_181)
    a32 = 1.5 * torch.randn((n, v), generator=gen, device="cuda")
    b = (a32 + 0.01 * torch.randn((n, v), generator=gen, device="cuda")).to(torch.bfloat16)
    a = a32.to(torch.bfloat16) if base_t == "bf16" else a32
    del a32
    out = L.lcmp_compare_logits(a, b, k=k, with_bitdiff=True)
    torch.cuda.synchronize()
    g = {key: val.cpu().numpy() for key, val in out.items() if key != "bitdiff"}
    g["bitdiff"] = L.unpack_bitdiff(out["bitdiff"])
    rows = np.unique(np.concatenate([[0, 1, n - 2, n - 1],
                                     np.random.default_rng(7).choice(n, 44, replace=False)]))

    def host(t):
        t = t[torch.from_numpy(rows).cuda()].contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    ha, hb = host(a), host(b)
    sub = {key: val[rows] for key, val in g.items() if key != "bitdiff"}
    assert_compare_equal(sub, oracle.compare(ha, hb, k=k))
    assert_bitdiff_equal(g["bitdiff"][rows], oracle.bitdiff(ha, hb))
    assert np.all(g["status"] == 0)
