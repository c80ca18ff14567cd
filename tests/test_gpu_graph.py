"""The fused scan + top-k step (plan, then fathom_scan_topk), alone and
followed by fathom_sparse_attention, captured into a
HIP graph: every replay, with the program's own eager calls and
synchronisations between replays, gives the eager call's results; the
library enqueues only kernels (no copy, memset, allocation or
synchronisation), which is what makes the capture possible."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    import sparse_top_key_amd as fathom
    fathom.lib()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return fathom


@pytest.mark.parametrize("group", [1, 4])
def test_graph_replays_equal_eager(F, group):
    dev = torch.device("cuda:0")
    n, hkv, hq, k, B = 150000, 2, 8, 512, 68
    print(f"graph replay group={group}", flush=True)
    layers = []
    for l in range(2):
        keys = synth.keys(81, l, n, hkv, 128, torch.float16, 4, device=dev)
        p = F.pack(keys)
        q = synth.queries(81, l, hq, 128, device=dev)
        layers.append((p, q))
    ws = torch.empty(F.scan_topk_workspace_bytes([n], hkv, hq, group, k), dtype=torch.uint8,
                     device=dev)
    plan = torch.empty((hq, 128), dtype=torch.uint8, device=dev)
    idx = torch.empty((hq // group, k), dtype=torch.int32, device=dev)
    vals = torch.empty((hq // group, k), dtype=torch.float32, device=dev)

    def step(p, q):
        F.plan(q, p.sigma2, B, out=plan)
        F.scan_topk(p.planes, p.lo, p.hi, n, q, plan, k, group, ws=ws, idx=idx, vals=vals)

    eager = []
    for p, q in layers:
        step(p, q)
        torch.cuda.synchronize()
        eager.append((idx.clone(), vals.clone()))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(*layers[0])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(*layers[0])
    for r in range(4):
        idx.fill_(-7)
        vals.fill_(0.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, eager[0][0]) and torch.equal(vals, eager[0][1]), r
        step(*layers[1])                      # eager work on other data in between
        torch.cuda.synchronize()
        assert torch.equal(idx, eager[1][0]) and torch.equal(vals, eager[1][1]), r


@pytest.mark.parametrize("group", [1, 4])
def test_graph_decode_step_with_attention_replays_equal_eager(F, group):
    """plan -> scan_topk -> sparse_attention captured as one graph: every
    replay gives the eager step's selected keys, attention output and lse;
    eager steps on another layer run between the replays."""
    dev = torch.device("cuda:0")
    n, hkv, hq, k, B = 70000, 2, 8, 256, 92
    print(f"graph decode step group={group}", flush=True)
    layers = []
    for l in range(2):
        keys = synth.keys(83, l, n, hkv, 128, torch.float16, 4, device=dev)
        vals_kv = synth.keys(84, l, n, hkv, 128, torch.float16, 0, device=dev)
        p = F.pack(keys)
        q = synth.queries(83, l, hq, 128, device=dev)
        layers.append((p, q, keys, vals_kv))
    ws = torch.empty(F.scan_topk_workspace_bytes([n], hkv, hq, group, k), dtype=torch.uint8,
                     device=dev)
    aws = torch.empty(F.attention_workspace_bytes(hq, k), dtype=torch.uint8, device=dev)
    plan = torch.empty((hq, 128), dtype=torch.uint8, device=dev)
    idx = torch.empty((hq // group, k), dtype=torch.int32, device=dev)
    vals = torch.empty((hq // group, k), dtype=torch.float32, device=dev)
    out = torch.empty((hq, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((hq,), dtype=torch.float32, device=dev)

    def step(p, q, kc, vc):
        F.plan(q, p.sigma2, B, out=plan)
        F.scan_topk(p.planes, p.lo, p.hi, n, q, plan, k, group, ws=ws, idx=idx, vals=vals)
        F.sparse_attention(q, kc, vc, idx, group, out=out, lse=lse, ws=aws)

    def state():
        return idx.clone(), out.clone(), lse.clone()

    eager = []
    for layer in layers:
        step(*layer)
        torch.cuda.synchronize()
        eager.append(state())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(*layers[0])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(*layers[0])
    for r in range(4):
        idx.fill_(-7)
        out.fill_(float("nan"))
        lse.fill_(0.0)
        g.replay()
        torch.cuda.synchronize()
        got = state()
        assert all(torch.equal(a, b) for a, b in zip(got, eager[0])), r
        step(*layers[1])                      # eager work on other data in between
        torch.cuda.synchronize()
        got = state()
        assert all(torch.equal(a, b) for a, b in zip(got, eager[1])), r
