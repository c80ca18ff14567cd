"""GPU parity of the multi-session calls (bit-identical to the one-session
calls and within tolerance of the oracle) and of the whole path at the 1M-key
layer size in the launch configuration the bench times, spot-checked against
the oracle."""
import numpy as np
import pytest
import torch

import synth
from parity import assert_logits_close, assert_topk_tie_tolerant, logit_scale

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    import sparse_top_key_amd as fathom
    fathom.lib()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return fathom


def dev():
    return torch.device("cuda:0")


def build_sessions(F, lengths, budgets, hkv=8, hq=32, k=1024, host=False, seed=300):
    sess = []
    for s, (n, B) in enumerate(zip(lengths, budgets)):
        keys = synth.keys(seed, 0, max(n, 1), hkv, 128, torch.float16, 4, device=dev(),
                          session=s)[:n]
        q = synth.queries(seed, 0, hq, 128, device=dev(), session=s)
        if n > 0:
            p = F.pack(keys)
            planes, lo, hi, s2 = p.planes, p.lo, p.hi, p.sigma2
        else:
            planes = torch.zeros((hkv, 128, 4, 0), dtype=torch.int32, device=dev())
            lo = torch.zeros((hkv, 128), device=dev())
            hi = torch.ones((hkv, 128), device=dev())
            s2 = torch.ones((hkv, 128), device=dev())
        if host:
            hp = torch.empty(planes.shape, dtype=planes.dtype, pin_memory=True)
            hp.copy_(planes)
            planes = hp
        plan = F.plan(q, s2, B)
        logits = torch.full((hq, max(n, 1) + 5), 3.0, device=dev())
        idx = torch.empty((hq // 4, k), dtype=torch.int32, device=dev())
        vals = torch.empty((hq // 4, k), device=dev())
        sess.append(F.Session(planes, lo, hi, n, q, plan, logits, idx, vals))
    torch.cuda.synchronize()
    return sess


def test_batched_equals_single_calls(F, orc):
    lengths = [5000, 17001, 1, 0, 40000, 2048]
    budgets = [68, 92, 136, 92, 91, 7]
    sess = build_sessions(F, lengths, budgets)
    F.scan_batched(sess)
    F.topk_batched(sess, 1024, group=4)
    torch.cuda.synchronize()
    for s in sess:
        print(f"batched session n={s.n}", flush=True)
        if s.n == 0:
            assert torch.all(s.idx == -1)
            continue
        single = F.scan(s.planes, s.lo, s.hi, s.n, s.q, s.plan)
        idx, vals = F.topk(single, 1024, group=4)
        torch.cuda.synchronize()
        assert torch.equal(s.logits[:, :s.n], single)
        assert torch.all(s.logits[:, s.n:] == 3.0)
        assert torch.equal(s.idx, idx) and torch.equal(s.vals, vals)
        ref = orc.scan(s.planes.cpu().numpy().view(np.uint32), s.lo.cpu().numpy(),
                       s.hi.cpu().numpy(), s.n, s.q.cpu().numpy(), s.plan.cpu().numpy())
        A = logit_scale(s.q.cpu().numpy(), s.lo.cpu().numpy(), s.hi.cpu().numpy(), 4)
        assert_logits_close(single.cpu().numpy(), ref, A)
        ridx, _ = orc.topk(single.cpu().numpy(), 1024, 4)
        np.testing.assert_array_equal(s.idx.cpu().numpy(), ridx)


def test_batched_many_sessions_host_resident(F, orc):
    w = synth.SESSIONS_16
    rng = np.random.default_rng(0)
    lengths = [int(x) for x in rng.integers(2000, 30000, 20)]     # > 16: two launches
    budgets = [w.budget_set[i % 3] for i in range(20)]
    sess = build_sessions(F, lengths, budgets, host=True, seed=301)
    F.scan_batched(sess)
    F.topk_batched(sess, 1024, group=4)
    torch.cuda.synchronize()
    for s in sess[::5]:
        ref = orc.scan(s.planes.numpy().view(np.uint32), s.lo.cpu().numpy(),
                       s.hi.cpu().numpy(), s.n, s.q.cpu().numpy(), s.plan.cpu().numpy())
        A = logit_scale(s.q.cpu().numpy(), s.lo.cpu().numpy(), s.hi.cpu().numpy(), 4)
        assert_logits_close(s.logits[:, :s.n].cpu().numpy(), ref, A)
        ridx, _ = orc.topk(s.logits[:, :s.n].cpu().numpy(), 1024, 4)
        np.testing.assert_array_equal(s.idx.cpu().numpy(), ridx)


@pytest.mark.parametrize("resident", ["hbm", "host"])
def test_full_layer_1m_spot_checks(F, orc, resident):
    """The 1M-key Qwen3-8B-shaped layer, B = 92, k = 2048: pack, plan, scan and
    top-k as the bench runs them, checked at sampled keys / rows."""
    w = synth.LAYER_1M
    n = w.n
    keys = synth.keys(w.seed, 0, n, w.hkv, 128, w.dtype, w.outliers, device=dev())
    q = synth.queries(w.seed, 0, w.hq, 128, device=dev())
    p = F.pack(keys)
    del keys
    planes = p.planes
    if resident == "host":
        planes = torch.empty(p.planes.shape, dtype=p.planes.dtype, pin_memory=True)
        planes.copy_(p.planes)
    plan = F.plan(q, p.sigma2, w.budget)
    logits = F.scan(planes, p.lo, p.hi, n, q, plan)
    idx, vals = F.topk(logits, w.k)
    gidx, gvals = F.topk(logits, w.k, group=4)
    torch.cuda.synchronize()
    print(f"full layer {resident}: n={n}", flush=True)
    planes_np = p.planes.cpu().numpy().view(np.uint32)
    lo, hi = p.lo.cpu().numpy(), p.hi.cpu().numpy()
    qn, pn = q.cpu().numpy(), plan.cpu().numpy()
    np.testing.assert_array_equal(pn, orc.plan(qn, p.sigma2.cpu().numpy(), w.budget))
    rng = np.random.default_rng(1)
    pick = np.unique(np.concatenate([rng.integers(0, n, 1500), np.arange(n - 40, n),
                                     np.arange(0, 40), idx[:, :4].cpu().numpy().ravel()]))
    ref = orc.scan_at(planes_np, lo, hi, n, qn, pn, pick)
    A = logit_scale(qn, lo, hi, 4)
    L = logits.cpu().numpy()
    assert_logits_close(L[:, pick], ref, A)
    # top-k of the GPU logits, bit-exact against the oracle's sort (4 rows, 1 group)
    for r in (0, 17):
        ridx, rvals = orc.topk(L[r:r + 1], w.k)
        np.testing.assert_array_equal(idx[r:r + 1].cpu().numpy(), ridx)
        np.testing.assert_array_equal(vals[r:r + 1].cpu().numpy(), rvals)
    ridx, rvals = orc.topk(L[8:12], w.k, 4)
    np.testing.assert_array_equal(gidx[2:3].cpu().numpy(), ridx)
    # and every selected key's oracle score beats (within tolerance) the k-th
    sel = idx[0].cpu().numpy()
    sref = orc.scan_at(planes_np[:1], lo[:1], hi[:1], n, qn[:1], pn[:1], sel)[0]
    assert np.all(sref >= vals[0, -1].item() - 2e-5 * A[0])


@pytest.mark.parametrize("layer", [0, 17, 35])
def test_step_36_layers_spot_parity(F, orc, layer):
    """Spot parity of the 36-layer decode step's own layers (its seeded keys
    and queries): the plan bit-exact, sampled logits within tolerance, the
    fused scan + top-k bit-identical to scan then top-k, and two rows' top-k
    bit-exact against the oracle's sort of the GPU logits."""
    w = synth.STEP_36L_1M
    n = w.n
    print(f"36-layer step, layer {layer}", flush=True)
    keys = synth.keys(w.seed, layer, n, w.hkv, 128, w.dtype, w.outliers, device=dev())
    q = synth.queries(w.seed, layer, w.hq, 128, device=dev())
    p = F.pack(keys)
    del keys
    plan = F.plan(q, p.sigma2, w.budget)
    logits = F.scan(p.planes, p.lo, p.hi, n, q, plan)
    idx, vals = F.topk(logits, w.k)
    fidx, fvals = F.scan_topk(p.planes, p.lo, p.hi, n, q, plan, w.k, 1)
    torch.cuda.synchronize()
    assert torch.equal(fidx, idx) and torch.equal(fvals, vals)
    planes_np = p.planes.cpu().numpy().view(np.uint32)
    lo, hi = p.lo.cpu().numpy(), p.hi.cpu().numpy()
    qn, pn = q.cpu().numpy(), plan.cpu().numpy()
    np.testing.assert_array_equal(pn, orc.plan(qn, p.sigma2.cpu().numpy(), w.budget))
    rng = np.random.default_rng(layer)
    pick = np.unique(np.concatenate([rng.integers(0, n, 1000), np.arange(n - 20, n)]))
    ref = orc.scan_at(planes_np, lo, hi, n, qn, pn, pick)
    A = logit_scale(qn, lo, hi, 4)
    L = logits.cpu().numpy()
    assert_logits_close(L[:, pick], ref, A)
    for r in (layer % 32, 31 - layer % 32):
        ridx, rvals = orc.topk(L[r:r + 1], w.k)
        np.testing.assert_array_equal(idx[r:r + 1].cpu().numpy(), ridx)
        np.testing.assert_array_equal(vals[r:r + 1].cpu().numpy(), rvals)


@pytest.mark.parametrize("layer", [5, 30])
def test_step_36_layers_spot_parity_host_resident(F, orc, layer):
    """The 36-layer step's host leg: the same layer's planes in pinned host
    memory (read zero-copy by the scan): sampled logits within tolerance of
    the oracle, scan_topk bit-identical to scan then top-k on those planes,
    and two rows' top-k bit-exact against the oracle's sort of the GPU
    logits."""
    w = synth.STEP_36L_1M
    n = w.n
    print(f"36-layer step, host-resident layer {layer}", flush=True)
    keys = synth.keys(w.seed, layer, n, w.hkv, 128, w.dtype, w.outliers, device=dev())
    q = synth.queries(w.seed, layer, w.hq, 128, device=dev())
    p = F.pack(keys)
    del keys
    hplanes = torch.empty(p.planes.shape, dtype=p.planes.dtype, pin_memory=True)
    hplanes.copy_(p.planes)
    plan = F.plan(q, p.sigma2, w.budget)
    logits = F.scan(hplanes, p.lo, p.hi, n, q, plan)
    idx, vals = F.topk(logits, w.k)
    fidx, fvals = F.scan_topk(hplanes, p.lo, p.hi, n, q, plan, w.k, 1)
    torch.cuda.synchronize()
    assert torch.equal(fidx, idx) and torch.equal(fvals, vals)
    planes_np = hplanes.numpy().view(np.uint32)
    lo, hi = p.lo.cpu().numpy(), p.hi.cpu().numpy()
    qn, pn = q.cpu().numpy(), plan.cpu().numpy()
    np.testing.assert_array_equal(pn, orc.plan(qn, p.sigma2.cpu().numpy(), w.budget))
    rng = np.random.default_rng(100 + layer)
    pick = np.unique(np.concatenate([rng.integers(0, n, 1000), np.arange(n - 20, n)]))
    ref = orc.scan_at(planes_np, lo, hi, n, qn, pn, pick)
    A = logit_scale(qn, lo, hi, 4)
    L = logits.cpu().numpy()
    assert_logits_close(L[:, pick], ref, A)
    for r in (layer % 32, 31 - layer % 32):
        ridx, rvals = orc.topk(L[r:r + 1], w.k)
        np.testing.assert_array_equal(idx[r:r + 1].cpu().numpy(), ridx)
        np.testing.assert_array_equal(vals[r:r + 1].cpu().numpy(), rvals)
