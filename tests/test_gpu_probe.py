"""The read-only reference stream (lcmp_read_probe) reads every input word
once: the XOR of everything it writes equals the XOR of all words of both
inputs, computed on the host.  Full steps XOR whole 32-bit words (two bf16
elements each); the ragged last step XORs single elements."""
import numpy as np
import pytest

from helpers import to_device

pytestmark = pytest.mark.gpu


def _host_xor(x: np.ndarray) -> int:
    v = x.shape[1]
    full = v - v % 512
    if x.dtype == np.float32:
        return int(np.bitwise_xor.reduce(x.view(np.uint32), axis=None))
    h = x.astype(np.uint32)
    even = np.bitwise_xor.reduce(h[:, 0:full:2], axis=None)
    odd = np.bitwise_xor.reduce(h[:, 1:full:2], axis=None)
    tail = np.bitwise_xor.reduce(h[:, full:], axis=None) if full < v else 0
    return int((even ^ tail) | (odd << 16))


def _bf16(x):
    import torch
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("tb,tc,n,v", [("f32", "f32", 40, 151936), ("f32", "bf16", 300, 151936),
                                       ("bf16", "bf16", 64, 151936), ("bf16", "f32", 7, 5000),
                                       ("bf16", "bf16", 3, 1528)])
def test_probe_reads_every_word(tb, tc, n, v):
    import torch
    import logit_distribution_diffing_amd as L
    print(f"[case] read probe {tb}/{tc} {n}x{v}", flush=True)
    rng = np.random.default_rng(n + v)
    x = rng.standard_normal((n, v)).astype(np.float32)
    y = rng.standard_normal((n, v)).astype(np.float32)
    a = x if tb == "f32" else _bf16(x)
    b = y if tc == "f32" else _bf16(y)
    ws = torch.zeros(int(L.lib().lcmp_compare_workspace_bytes(n, v, 1, 0)), dtype=torch.uint8,
                     device="cuda")
    L.lcmp_read_probe(to_device(a), to_device(b), workspace=ws)
    torch.cuda.synchronize()
    words = ws.cpu().numpy().view(np.uint32)
    assert int(np.bitwise_xor.reduce(words)) == _host_xor(a) ^ _host_xor(b)
