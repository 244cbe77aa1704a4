"""The comparison path under HIP graph capture and on concurrent streams.

The library allocates nothing and enqueues no memset, so a whole step
(compare + margin bins, or the comparison against a record) can be captured in
a HIP graph.  Each replay runs on new inputs copied into the captured buffers,
with eager work and synchronisations between replays, and must give the eager
results bit for bit.  Calls on two streams with their own workspaces must give
the same results as one after the other."""
import numpy as np
import pytest

import synth
from helpers import to_device

pytestmark = pytest.mark.gpu

EDGES = synth.DEFAULT_EDGES


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _inputs(seed, n, v):
    rng = np.random.default_rng(seed)
    a = (1.5 * rng.standard_normal((n, v))).astype(np.float32)
    b = (a + 0.03 * rng.standard_normal((n, v))).astype(np.float32)
    c = (int(np.argmax(a[3])) + 1) % v
    b[3, c] = a[3].max() + 1.0                       # one constructed flip
    b[5] = a[5] - 30.0                               # far-apart normalisers: the
    b[6, :] -= 40.0                                  # bucket pass has rows to redo
    b[6, np.argsort(a[6])[-20:]] += 40.0
    return a, b


def _snapshot(out, bins, summ):
    d = {k: v.detach().cpu().numpy().copy() for k, v in out.items()}
    d["bins"] = bins.cpu().numpy().copy()
    d["summ"] = summ.cpu().numpy().copy()
    return d


def _assert_same(x, y):
    assert x.keys() == y.keys()
    for k in x:
        assert x[k].tobytes() == y[k].tobytes(), k


def test_compare_step_replays_in_a_hip_graph():
    import torch
    import logit_distribution_diffing_amd as L
    n, v, k = 256, 20001, 20
    _case(f"graph compare {n}x{v}")
    base = torch.empty((n, v), dtype=torch.float32, device="cuda")
    cand = torch.empty((n, v), dtype=torch.bfloat16, device="cuda")
    out = L.alloc_compare_outputs(n, k, "cuda", with_bitdiff=True)
    ws = torch.empty(L.compare_workspace_bytes(n, v, k, True), dtype=torch.uint8, device="cuda")
    bws = torch.empty(int(L.lib().lcmp_bin_workspace_bytes(n, 1, len(EDGES))), dtype=torch.uint8,
                      device="cuda")
    bins = torch.empty((len(EDGES), L.BIN_BYTES), dtype=torch.uint8, device="cuda")
    summ = torch.empty((1, L.GROUP_SUMMARY_BYTES), dtype=torch.uint8, device="cuda")

    def step():
        L.lcmp_compare_logits(base, cand, k=k, with_bitdiff=True, out=out, workspace=ws)
        L.lcmp_bin_report(out["margin"], out["flip"], out["kl_topk"], out["kl_full"], EDGES,
                          status=out["status"], workspace=bws, bins=bins, summary=summ)

    sets = [_inputs(s, n, v) for s in (1, 2, 3)]
    eager = []
    for a, b in sets:
        base.copy_(to_device(a))
        cand.copy_(to_device(b).to(torch.bfloat16))
        step()
        torch.cuda.synchronize()
        eager.append(_snapshot(out, bins, summ))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(2):
        for (a, b), want in zip(sets, eager):
            base.copy_(to_device(a))
            cand.copy_(to_device(b).to(torch.bfloat16))
            for key in out:      # eager work between replays: poison the outputs
                out[key].fill_(7)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            _assert_same(_snapshot(out, bins, summ), want)
    assert eager[0]["flip"][3] == 1


def test_record_comparison_replays_in_a_hip_graph():
    import torch
    import logit_distribution_diffing_amd as L
    n, v, k = 192, 9000, 20
    _case(f"graph record {n}x{v}")
    a, _ = _inputs(4, n, v)
    rec = L.lcmp_record_baseline(to_device(a), k_rec=k)
    cand = torch.empty((n, v), dtype=torch.float32, device="cuda")
    out = L.alloc_compare_outputs(n, k, "cuda")
    del out["kl_full"]
    ws = torch.empty(int(L.lib().lcmp_compare_record_workspace_bytes(n, v)), dtype=torch.uint8,
                     device="cuda")

    def step():
        L.lcmp_compare_record(rec, cand, k=k, out=out, workspace=ws)

    cands = [_inputs(s, n, v)[1] for s in (5, 6)]
    eager = []
    for b in cands:
        cand.copy_(to_device(b))
        step()
        torch.cuda.synchronize()
        eager.append({kk: vv.cpu().numpy().copy() for kk, vv in out.items()})
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(2):
        for b, want in zip(cands, eager):
            cand.copy_(to_device(b))
            for key in out:
                out[key].fill_(3)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = {kk: vv.cpu().numpy() for kk, vv in out.items()}
            _assert_same(got, want)


def test_two_streams_with_their_own_workspaces():
    import torch
    import logit_distribution_diffing_amd as L
    n, v, k = 300, 30011, 20
    _case(f"two streams {n}x{v}")
    (a1, b1), (a2, b2) = _inputs(8, n, v), _inputs(9, n, v)
    t = [(to_device(a1), to_device(b1)), (to_device(a2), to_device(b2))]
    ref = []
    for da, db in t:
        o = L.lcmp_compare_logits(da, db, k=k, with_bitdiff=True)
        torch.cuda.synchronize()
        ref.append({kk: vv.cpu().numpy().copy() for kk, vv in o.items()})
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    outs = [L.alloc_compare_outputs(n, k, "cuda", with_bitdiff=True) for _ in range(2)]
    wss = [torch.empty(L.compare_workspace_bytes(n, v, k, True), dtype=torch.uint8,
                       device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    for rep in range(3):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                L.lcmp_compare_logits(t[i][0], t[i][1], k=k, with_bitdiff=True, out=outs[i],
                                      workspace=wss[i], stream=streams[i])
        torch.cuda.synchronize()
        for i in range(2):
            _assert_same({kk: vv.cpu().numpy() for kk, vv in outs[i].items()}, ref[i])


def test_side_stream_without_workspace():
    """A call on a side stream that brings no workspace and no outputs: what the
    binding allocates belongs to that stream, so memory allocated and filled on
    the current stream right after the call (before any synchronisation) cannot
    land on a block the side stream's kernels still use."""
    import torch
    import logit_distribution_diffing_amd as L
    n, v, k = 1024, 151936, 20
    _case(f"side stream, internal workspace {n}x{v}")
    a, b = _inputs(11, n, v)
    da, db = to_device(a), to_device(b)
    ref = L.lcmp_compare_logits(da, db, k=k, with_bitdiff=True)
    torch.cuda.synchronize()
    ref = {kk: vv.cpu().numpy().copy() for kk, vv in ref.items()}
    ws_bytes = L.compare_workspace_bytes(n, v, k, True)
    side = torch.cuda.Stream()   # default priority
    for rep in range(3):
        torch.cuda.synchronize()
        out = L.lcmp_compare_logits(da, db, k=k, with_bitdiff=True, stream=side)
        junk = [torch.empty(ws_bytes, dtype=torch.uint8, device="cuda").fill_(0xA5)
                for _ in range(4)]
        junk += [torch.full((n, k), -7, dtype=torch.int32, device="cuda")]
        torch.cuda.synchronize()
        del junk
        _assert_same({kk: vv.cpu().numpy() for kk, vv in out.items()}, ref)
