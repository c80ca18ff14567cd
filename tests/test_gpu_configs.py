"""GPU parity at the stated sizes of every workload, in the launch
configurations the benchmark times:

  * the 131,072-key Qwen3-8B-shaped layer (planes in HBM) at B = 68, 92 and
    136 with k = 1024, per query head and per GQA group;
  * 16 ragged sessions of 64K..512K keys with per-session budgets and k = 1024,
    planes in pinned host memory, through the batched calls;
  * the 1M-key layer's fixed-136 baseline (r = 32 channels plus the 8-bit side
    stream) with planes in pinned host memory;
  * the 1M-key layer's fused scan + top-k compared directly with the oracle's
    own top-k of its own logits (tie-tolerant), per head and per group;
  * rows whose top keys cluster in one 2048-key tile (more candidates than one
    scan block's share of the candidate store), per head and per group.

Checks: plans bit-exact against the oracle; logits at sampled keys within
1e-5 * A_h of the oracle (A_h = sum_c |q_c| max(|lo_c|, |hi_c|)); top-k rows
bit-exact against the oracle's sort of the GPU logits; the fused call
bit-identical to scan then top-k; and on whole rows, the top-k of the GPU
against the top-k of the oracle's logits, identical except for keys whose
oracle score lies within 2e-5 * A_h of the oracle's k-th score."""
import numpy as np
import pytest
import torch

import synth
from parity import assert_logits_close, assert_topk_tie_tolerant, group_scores, logit_scale

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


def oracle_rows(orc, planes_np, lo, hi, n, qn, pn, heads, group):
    """Oracle logits of whole rows of the given query heads: [len(heads)][n]."""
    out = []
    for h in heads:
        g = h // group
        out.append(orc.scan(planes_np[g:g + 1], lo[g:g + 1], hi[g:g + 1], n, qn[h:h + 1],
                            pn[h:h + 1])[0])
    return np.stack(out)


@pytest.fixture(scope="module")
def layer_128k(F):
    w = synth.LAYER_128K
    keys = synth.keys(w.seed, 0, w.n, w.hkv, 128, w.dtype, w.outliers, device=dev())
    q = synth.queries(w.seed, 0, w.hq, 128, device=dev())
    p = F.pack(keys)
    torch.cuda.synchronize()
    return w, p, q


@pytest.mark.parametrize("B", [68, 92, 136])
def test_layer_128k_budgets(F, orc, layer_128k, B):
    w, p, q = layer_128k
    n, k, G = w.n, w.k, w.hq // w.hkv
    print(f"128K layer B={B}", flush=True)
    plan = F.plan(q, p.sigma2, B)
    logits = F.scan(p.planes, p.lo, p.hi, n, q, plan)
    idx, vals = F.topk(logits, k)
    gidx, gvals = F.topk(logits, k, group=G)
    fidx, fvals = F.scan_topk(p.planes, p.lo, p.hi, n, q, plan, k, 1)
    fgidx, fgvals = F.scan_topk(p.planes, p.lo, p.hi, n, q, plan, k, G)
    torch.cuda.synchronize()
    assert torch.equal(fidx, idx) and torch.equal(fvals, vals)
    assert torch.equal(fgidx, gidx) and torch.equal(fgvals, gvals)
    planes_np = p.planes.cpu().numpy().view(np.uint32)
    lo, hi = p.lo.cpu().numpy(), p.hi.cpu().numpy()
    qn, pn = q.cpu().numpy(), plan.cpu().numpy()
    np.testing.assert_array_equal(pn, orc.plan(qn, p.sigma2.cpu().numpy(), B))
    rng = np.random.default_rng(B)
    pick = np.unique(np.concatenate([rng.integers(0, n, 2000), np.arange(n - 30, n),
                                     idx[:, :3].cpu().numpy().ravel()]))
    A = logit_scale(qn, lo, hi, G)
    L = logits.cpu().numpy()
    assert_logits_close(L[:, pick], orc.scan_at(planes_np, lo, hi, n, qn, pn, pick), A)
    for r in (B % 32, 31 - B % 32):
        ridx, rvals = orc.topk(L[r:r + 1], k)
        np.testing.assert_array_equal(idx[r:r + 1].cpu().numpy(), ridx)
        np.testing.assert_array_equal(vals[r:r + 1].cpu().numpy(), rvals)
    g = (B // 4) % w.hkv
    ridx, rvals = orc.topk(L[G * g:G * g + G], k, G)
    np.testing.assert_array_equal(gidx[g:g + 1].cpu().numpy(), ridx)
    np.testing.assert_array_equal(gvals[g:g + 1].cpu().numpy(), rvals)
    # whole rows: the fused top-k against the oracle's own top-k
    heads = [3, 20]
    R = oracle_rows(orc, planes_np, lo, hi, n, qn, pn, heads, G)
    ridx, _ = orc.topk(R, k)
    assert_topk_tie_tolerant(fidx[heads].cpu().numpy(), ridx, R, A[heads], n, k)
    heads = list(range(G * g, G * g + G))
    R = oracle_rows(orc, planes_np, lo, hi, n, qn, pn, heads, G)
    ridx, _ = orc.topk(R, k, G)
    Rg = group_scores(R, G)
    assert_topk_tie_tolerant(fgidx[g:g + 1].cpu().numpy(), ridx, Rg,
                             np.array([A[heads].sum()]), n, k)


def test_sessions_16_host_resident(F, orc):
    """16 sessions at their seeded lengths (64K..512K) and budgets, planes in
    pinned host memory: batched scan + top-k and the batched fused call (which
    scans host planes into its workspace), spot-checked per session."""
    w = synth.SESSIONS_16
    lengths = synth.session_lengths(w)
    budgets = synth.session_budgets(w)
    print(f"16 sessions: {sum(lengths)} keys, budgets {budgets}", flush=True)
    sess, packs = [], []
    for s, (n, B) in enumerate(zip(lengths, budgets)):
        keys = synth.keys(w.seed, 0, n, w.hkv, 128, w.dtype, w.outliers, device=dev(),
                          session=s)
        p = F.pack(keys)
        del keys
        host = torch.empty(p.planes.shape, dtype=p.planes.dtype, pin_memory=True)
        host.copy_(p.planes)
        p.planes = None
        q = synth.queries(w.seed, 0, w.hq, 128, device=dev(), session=s)
        plan = F.plan(q, p.sigma2, B)
        sess.append(F.Session(host, p.lo, p.hi, n, q, plan,
                              torch.empty((w.hq, n), device=dev()),
                              torch.empty((w.hq, w.k), dtype=torch.int32, device=dev()),
                              torch.empty((w.hq, w.k), device=dev())))
        packs.append(p)
    F.scan_batched(sess)
    F.topk_batched(sess, w.k, group=1)
    fused = [F.Session(S.planes, S.lo, S.hi, S.n, S.q, S.plan, None,
                       torch.empty((w.hq, w.k), dtype=torch.int32, device=dev()),
                       torch.empty((w.hq, w.k), device=dev())) for S in sess]
    F.scan_topk_batched(fused, w.k, group=1)
    torch.cuda.synchronize()
    G = w.hq // w.hkv
    for s, (S, Fs, p, B) in enumerate(zip(sess, fused, packs, budgets)):
        print(f"session {s}: n={S.n} B={B}", flush=True)
        assert torch.equal(Fs.idx, S.idx) and torch.equal(Fs.vals, S.vals)
        planes_np = S.planes.numpy().view(np.uint32)
        lo, hi = S.lo.cpu().numpy(), S.hi.cpu().numpy()
        qn, pn = S.q.cpu().numpy(), S.plan.cpu().numpy()
        np.testing.assert_array_equal(pn, orc.plan(qn, p.sigma2.cpu().numpy(), B))
        rng = np.random.default_rng(s)
        pick = np.unique(np.concatenate([rng.integers(0, S.n, 300), np.arange(S.n - 10, S.n)]))
        A = logit_scale(qn, lo, hi, G)
        L = S.logits.cpu().numpy()
        assert_logits_close(L[:, pick], orc.scan_at(planes_np, lo, hi, S.n, qn, pn, pick), A)
        r = s % w.hq
        ridx, rvals = orc.topk(L[r:r + 1], w.k)
        np.testing.assert_array_equal(S.idx[r:r + 1].cpu().numpy(), ridx)
        np.testing.assert_array_equal(S.vals[r:r + 1].cpu().numpy(), rvals)
        if s % 4 == 0:
            R = oracle_rows(orc, planes_np, lo, hi, S.n, qn, pn, [r], G)
            ridx, _ = orc.topk(R, w.k)
            assert_topk_tie_tolerant(S.idx[r:r + 1].cpu().numpy(), ridx, R, A[[r]], S.n, w.k)


@pytest.fixture(scope="module")
def layer_1m(F):
    w = synth.LAYER_1M
    keys = synth.keys(w.seed, 0, w.n, w.hkv, 128, w.dtype, w.outliers, device=dev())
    q = synth.queries(w.seed, 0, w.hq, 128, device=dev())
    p = F.pack(keys)
    torch.cuda.synchronize()
    return w, keys, p, q


def test_layer_1m_fixed136_host(F, orc, layer_1m):
    """The fixed-136 baseline of the 1M-key layer (top-32 |q_c| channels at 4
    bits plus the 8-bit side stream) with planes in pinned host memory."""
    w, _, p, q = layer_1m
    n, G = w.n, w.hq // w.hkv
    print("1M fixed-136, host planes", flush=True)
    host = torch.empty(p.planes.shape, dtype=p.planes.dtype, pin_memory=True)
    host.copy_(p.planes)
    meta = synth.side_stream(w.seed, 0, w.hkv, n, device=dev())
    ms = 0.01
    plan = F.plan_fixed(q, 32)
    logits = F.scan(host, p.lo, p.hi, n, q, plan, meta=meta, meta_scale=ms)
    idx, vals = F.topk(logits, w.k)
    fidx, fvals = F.scan_topk(host, p.lo, p.hi, n, q, plan, w.k, 1, meta=meta, meta_scale=ms)
    torch.cuda.synchronize()
    assert torch.equal(fidx, idx) and torch.equal(fvals, vals)
    planes_np = host.numpy().view(np.uint32)
    lo, hi = p.lo.cpu().numpy(), p.hi.cpu().numpy()
    qn, pn = q.cpu().numpy(), plan.cpu().numpy()
    mn = meta.cpu().numpy()
    np.testing.assert_array_equal(pn, orc.plan_fixed(qn, 32))
    rng = np.random.default_rng(136)
    pick = np.unique(np.concatenate([rng.integers(0, n, 1500), np.arange(n - 30, n),
                                     np.arange(0, 30)]))
    A = logit_scale(qn, lo, hi, G, ms)
    L = logits.cpu().numpy()
    assert_logits_close(L[:, pick],
                        orc.scan_at(planes_np, lo, hi, n, qn, pn, pick, meta=mn, meta_scale=ms), A)
    for r in (5, 30):
        ridx, rvals = orc.topk(L[r:r + 1], w.k)
        np.testing.assert_array_equal(idx[r:r + 1].cpu().numpy(), ridx)
        np.testing.assert_array_equal(vals[r:r + 1].cpu().numpy(), rvals)
    g = r // G
    R = orc.scan(planes_np[g:g + 1], lo[g:g + 1], hi[g:g + 1], n, qn[r:r + 1], pn[r:r + 1],
                 meta=mn[g:g + 1], meta_scale=ms)
    ridx, _ = orc.topk(R, w.k)
    assert_topk_tie_tolerant(idx[r:r + 1].cpu().numpy(), ridx, R, A[[r]], n, w.k)


@pytest.mark.parametrize("group", [1, 4])
def test_layer_1m_fused_against_oracle(F, orc, layer_1m, group):
    """The 1M-key layer's fused call (planes in HBM, B = 92, k = 2048) against
    the oracle's own top-k of whole rows."""
    w, _, p, q = layer_1m
    n, G = w.n, w.hq // w.hkv
    print(f"1M fused vs oracle, group {group}", flush=True)
    plan = F.plan(q, p.sigma2, w.budget)
    fidx, fvals = F.scan_topk(p.planes, p.lo, p.hi, n, q, plan, w.k, group)
    torch.cuda.synchronize()
    planes_np = p.planes.cpu().numpy().view(np.uint32)
    lo, hi = p.lo.cpu().numpy(), p.hi.cpu().numpy()
    qn, pn = q.cpu().numpy(), plan.cpu().numpy()
    A = logit_scale(qn, lo, hi, G)
    if group == 1:
        for h in (0, 13, 31):
            R = oracle_rows(orc, planes_np, lo, hi, n, qn, pn, [h], G)
            ridx, _ = orc.topk(R, w.k)
            assert_topk_tie_tolerant(fidx[h:h + 1].cpu().numpy(), ridx, R, A[[h]], n, w.k)
            # the returned scores are the GPU logits of the returned keys
            sref = orc.scan_at(planes_np[h // G:h // G + 1], lo[h // G:h // G + 1],
                               hi[h // G:h // G + 1], n, qn[h:h + 1], pn[h:h + 1],
                               fidx[h].cpu().numpy())[0]
            assert np.all(np.abs(sref - fvals[h].cpu().numpy()) <= 1e-5 * A[h])
    else:
        g = 5
        heads = list(range(G * g, G * g + G))
        R = oracle_rows(orc, planes_np, lo, hi, n, qn, pn, heads, G)
        ridx, _ = orc.topk(R, w.k, G)
        assert_topk_tie_tolerant(fidx[g:g + 1].cpu().numpy(), ridx, group_scores(R, G),
                                 np.array([A[heads].sum()]), n, w.k)


def _planted_layer(F, w, keys, q, group, tile, m, head):
    """The 1M-key layer with keys tile*2048 .. tile*2048+m-1 of kv head
    head // 4 replaced by one vector aligned with the query (per head) or
    with the group's summed query (group 4): those m keys score far above
    every other key of the rows that read them."""
    G = w.hq // w.hkv
    g = head // G
    k2 = keys.clone()
    sd = keys[:, g, :].float().std(0)
    qd = q[head] if group == 1 else q[G * g:G * g + G].sum(0)
    v = (3.0 * sd * torch.sign(qd)).to(keys.dtype)
    t0 = tile * 2048
    k2[t0:t0 + m, g, :] = v
    # a little spread inside the cluster, so that its scores are not all equal
    k2[t0:t0 + m, g, 0] = (v[0].float() + 0.01 * sd[0] * torch.arange(
        m, device=keys.device, dtype=torch.float32) / m).to(keys.dtype)
    p = F.pack(k2)
    del k2
    return p


@pytest.mark.parametrize("group", [1, 4])
@pytest.mark.parametrize("tile", [301, 392])
def test_layer_1m_clustered_top_keys(F, orc, layer_1m, group, tile):
    """1,500 top-scoring keys inside one 2048-key tile of the 1M-key layer:
    one scan block finds more candidates than its even share of the row's
    candidate store.  Tile 392 is one the fused threshold samples (the middle
    tiles of 32 equal stretches of 512 tiles are 8 (2j + 1)): the threshold
    stage must leave its cluster out of the estimate; tile 301 is not
    sampled.  The fused call still equals scan then top-k, no
    row is recomputed, and its rows hold the planted keys."""
    w, keys, _, q = layer_1m
    n, G = w.n, w.hq // w.hkv
    head, m = 9, 1500
    print(f"1M clustered, group {group}, tile {tile}", flush=True)
    p = _planted_layer(F, w, keys, q, group, tile, m, head)
    plan = F.plan(q, p.sigma2, w.budget)
    logits = F.scan(p.planes, p.lo, p.hi, n, q, plan)
    idx, vals = F.topk(logits, w.k, group=group)
    ws = torch.empty(F.scan_topk_workspace_bytes([n], w.hkv, w.hq, group, w.k),
                     dtype=torch.uint8, device=dev())
    fidx, fvals = F.scan_topk(p.planes, p.lo, p.hi, n, q, plan, w.k, group, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(fidx, idx) and torch.equal(fvals, vals)
    # the clustered row is answered from its candidates (the blocks' segments
    # and the row's overflow list), not recomputed from full logits: the
    # workspace starts with one threshold word, then one recompute flag per
    # output row
    rows = w.hq // group
    flags = ws[4 * rows:8 * rows].view(torch.int32).cpu().numpy()
    assert not flags.any(), flags
    row = head if group == 1 else head // G
    sel = set(fidx[row].cpu().tolist())
    planted = set(range(tile * 2048, tile * 2048 + m))
    assert planted <= sel
    L = logits.cpu().numpy()
    rows = slice(row, row + 1) if group == 1 else slice(G * row, G * row + G)
    ridx, rvals = orc.topk(L[rows], w.k, group)
    np.testing.assert_array_equal(fidx[row:row + 1].cpu().numpy(), ridx)
    np.testing.assert_array_equal(fvals[row:row + 1].cpu().numpy(), rvals)
