"""GPU parity of fathom_scan_topk: idx and vals bit-identical to fathom_scan
followed by fathom_topk on the same inputs (per query head and per GQA
group; sampled-threshold path, all-candidates path, recompute path for rows
whose candidate count is out of range, and the workspace-logits path for
pinned host planes and other groups), and spot-checked against the oracle."""
import numpy as np
import pytest
import torch

import synth
from parity import assert_topk_tie_tolerant, logit_scale

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


def layer(F, seed, n, hkv, hq, budget=92, fixed_r=None, dtype=torch.float16):
    keys = synth.keys(seed, 0, n, hkv, 128, dtype, 4, device=dev())
    q = synth.queries(seed, 0, hq, 128, device=dev())
    p = F.pack(keys)
    plan = F.plan_fixed(q, fixed_r) if fixed_r is not None else F.plan(q, p.sigma2, budget)
    torch.cuda.synchronize()
    return keys, q, p, plan


def both(F, p, n, q, plan, k, group, meta=None, meta_scale=0.0, planes=None):
    planes = p.planes if planes is None else planes
    logits = F.scan(planes, p.lo, p.hi, n, q, plan, meta, meta_scale)
    ref = F.topk(logits, k, group)
    got = F.scan_topk(planes, p.lo, p.hi, n, q, plan, k, group, meta, meta_scale)
    torch.cuda.synchronize()
    return got, ref, logits


def redo_flags(F, n, hkv, hq, group, k, run):
    """Run `run(ws)` with a workspace of our own and return the per-row redo
    flags the call left there (white-box: the workspace starts with the rows'
    threshold words, then their redo flags)."""
    rows = hq // group
    ws = torch.zeros(F.scan_topk_workspace_bytes([n], hkv, hq, group, k), dtype=torch.uint8,
                     device=dev())
    run(ws)
    torch.cuda.synchronize()
    return ws[4 * rows:8 * rows].view(torch.int32).cpu()


def assert_same(got, ref):
    assert torch.equal(got[0], ref[0]), "idx differ"
    assert torch.equal(got[1], ref[1]), "vals differ"


@pytest.mark.parametrize("n,hkv,hq,k,group", [
    (200000, 8, 32, 1024, 1),     # sampled threshold, per query head
    (200000, 8, 32, 1024, 4),     # per GQA group (group sum in the scan)
    (123457, 8, 32, 2048, 1),     # ragged tail, largest k
    (100000, 4, 8, 1, 2),         # k = 1, groups of 2
    (5000, 8, 32, 64, 1),         # n <= 8192: every key a candidate
    (8192, 2, 8, 512, 4),
    (8193, 2, 8, 512, 1),
    (40000, 2, 16, 256, 1),       # 8 query heads per kv head (two head chunks)
    (40000, 2, 16, 256, 8),       # group 8: logits in the workspace
    (40000, 2, 8, 300, 2),        # group 2 of 4: logits in the workspace
    (30000, 8, 8, 100, 1),        # one query head per kv head
])
def test_scan_topk_equals_scan_then_topk(F, n, hkv, hq, k, group):
    print(f"scan_topk n={n} hkv={hkv} hq={hq} k={k} group={group}", flush=True)
    _, q, p, plan = layer(F, 400 + n % 97, n, hkv, hq)
    got, ref, _ = both(F, p, n, q, plan, k, group)
    assert_same(got, ref)
    if group == 1 or (group == hq // hkv and group <= 4):
        # answered from candidate lists, nothing recomputed
        flags = redo_flags(F, n, hkv, hq, group, k, lambda ws: F.scan_topk(
            p.planes, p.lo, p.hi, n, q, plan, k, group, ws=ws))
        assert torch.all(flags == 0)


@pytest.mark.parametrize("budget", [68, 136, 7])
def test_scan_topk_budgets(F, budget):
    print(f"scan_topk budget={budget}", flush=True)
    _, q, p, plan = layer(F, 500 + budget, 70000, 8, 32, budget)
    got, ref, _ = both(F, p, 70000, q, plan, 512, 1)
    assert_same(got, ref)


def test_scan_topk_fixed_plan_with_side_stream(F):
    n = 90000
    print(f"scan_topk fixed-136 n={n}", flush=True)
    _, q, p, plan = layer(F, 510, n, 8, 32, fixed_r=32)
    meta = synth.side_stream(510, 0, 8, n, device=dev())
    for group in (1, 4):
        got, ref, _ = both(F, p, n, q, plan, 1024, group, meta, 0.01)
        assert_same(got, ref)


def test_scan_topk_all_ties_recomputes(F):
    """B = 0: every logit of a row equals C_h, so every key reaches the
    threshold, the candidate lists overflow and the rows are recomputed from
    full logits; the top k are then the k lowest indices."""
    n = 60000
    print("scan_topk all ties", flush=True)
    _, q, p, plan = layer(F, 520, n, 8, 32, budget=0)
    for group in (1, 4):
        got, ref, _ = both(F, p, n, q, plan, 256, group)
        assert_same(got, ref)
        assert torch.equal(got[0].cpu(), torch.arange(256, dtype=torch.int32).expand_as(got[0]))
        flags = redo_flags(F, n, 8, 32, group, 256, lambda ws: F.scan_topk(
            p.planes, p.lo, p.hi, n, q, plan, 256, group, ws=ws))
        assert torch.all(flags == 1)


def test_scan_topk_sample_misled_recomputes(F):
    """Keys of the sampled tiles made much larger in one channel: the sampled
    threshold is far from the rest of the row, so candidate counts fall
    outside [k, 8192] and rows are recomputed; results still match."""
    n = 256 * 2048
    hkv, hq = 2, 8
    keys = synth.keys(530, 0, n, hkv, 128, torch.float16, 0, device=dev())
    q = synth.queries(530, 0, hq, 128, device=dev())
    ntiles = n // 2048
    # the sampled tiles: the middle tile of each of 32 equal stretches (an
    # eighth of this row)
    for j in range(32):
        t = (2 * j + 1) * ntiles // 64
        keys[t * 2048:(t + 1) * 2048, :, 0] += 60.0
    p = F.pack(keys)
    # kv head 0's query heads weigh the planted channel up, kv head 1's down
    # (thresholds far above / below the rest of the row; group sums too)
    q[:, 0] = torch.where(torch.arange(hq, device=dev()) < hq // 2, 5.0, -5.0)
    plan = F.plan(q, p.sigma2, 92)
    torch.cuda.synchronize()
    print("scan_topk misled sample", flush=True)
    for group in (1, 4):
        got, ref, _ = both(F, p, n, q, plan, 1024, group)
        assert_same(got, ref)
        flags = redo_flags(F, n, hkv, hq, group, 1024, lambda ws: F.scan_topk(
            p.planes, p.lo, p.hi, n, q, plan, 1024, group, ws=ws))
        assert torch.all(flags == 1)


def test_scan_topk_pinned_host_planes(F):
    n = 50000
    print("scan_topk pinned host planes", flush=True)
    _, q, p, plan = layer(F, 540, n, 8, 32)
    host = torch.empty(p.planes.shape, dtype=p.planes.dtype, pin_memory=True)
    host.copy_(p.planes)
    torch.cuda.synchronize()
    got, ref, _ = both(F, p, n, q, plan, 512, 4, planes=host)
    assert_same(got, ref)


def test_scan_topk_batched_sessions(F):
    lengths = [70000, 5000, 0, 123457, 1, 16385]
    budgets = [92, 68, 92, 136, 92, 91]
    hkv, hq, k = 8, 32, 1024
    for group in (1, 4):
        sess, refs = [], []
        for s, (n, B) in enumerate(zip(lengths, budgets)):
            print(f"batched scan_topk session n={n} group={group}", flush=True)
            keys = synth.keys(550, 0, max(n, 1), hkv, 128, torch.float16, 4, device=dev(),
                              session=s)[:n]
            q = synth.queries(550, 0, hq, 128, device=dev(), session=s)
            if n > 0:
                p = F.pack(keys)
                planes, lo, hi, s2 = p.planes, p.lo, p.hi, p.sigma2
            else:
                planes = torch.zeros((hkv, 128, 4, 0), dtype=torch.int32, device=dev())
                lo = torch.zeros((hkv, 128), device=dev())
                hi = torch.ones((hkv, 128), device=dev())
                s2 = torch.ones((hkv, 128), device=dev())
            plan = F.plan(q, s2, B)
            idx = torch.empty((hq // group, k), dtype=torch.int32, device=dev())
            vals = torch.empty((hq // group, k), device=dev())
            sess.append(F.Session(planes, lo, hi, n, q, plan, None, idx, vals))
            if n > 0:
                refs.append(F.topk(F.scan(planes, lo, hi, n, q, plan), k, group))
            else:
                refs.append(None)
        F.scan_topk_batched(sess, k, group)
        torch.cuda.synchronize()
        for s, r in zip(sess, refs):
            if r is None:
                assert torch.all(s.idx == -1) and torch.all(torch.isinf(s.vals))
            else:
                assert torch.equal(s.idx, r[0]) and torch.equal(s.vals, r[1])


@pytest.mark.parametrize("with_empty", [False, True])
def test_scan_topk_batched_recompute_in_some_sessions(F, with_empty):
    """Sessions of one batched call where some rows are recomputed (budget 0:
    every logit of a row ties, so its candidates overflow) beside sessions
    answered from their candidates: each recompute scan block counts into
    its own session's per-kv-head counters and the last one ranks that
    session's rows; every session equals scan then top-k.  Without an empty
    session the final's blocks share the recompute scan's launch; with one,
    the final runs as a launch of its own before it."""
    lengths = [60000, 90000, 40000, 70000]
    budgets = [0, 92, 92, 0]
    if with_empty:
        lengths.insert(2, 0)
        budgets.insert(2, 92)
    hkv, hq, k = 8, 32, 512
    for group in (1, 4):
        sess, refs = [], []
        for s, (n, B) in enumerate(zip(lengths, budgets)):
            print(f"batched recompute session n={n} B={B} group={group} "
                  f"with_empty={with_empty}", flush=True)
            q = synth.queries(560, 0, hq, 128, device=dev(), session=s)
            if n > 0:
                keys = synth.keys(560, 0, n, hkv, 128, torch.float16, 4, device=dev(), session=s)
                p = F.pack(keys)
                planes, lo, hi, s2 = p.planes, p.lo, p.hi, p.sigma2
            else:
                planes = torch.zeros((hkv, 128, 4, 0), dtype=torch.int32, device=dev())
                lo = torch.zeros((hkv, 128), device=dev())
                hi = torch.ones((hkv, 128), device=dev())
                s2 = torch.ones((hkv, 128), device=dev())
            plan = F.plan(q, s2, B)
            idx = torch.empty((hq // group, k), dtype=torch.int32, device=dev())
            vals = torch.empty((hq // group, k), device=dev())
            sess.append(F.Session(planes, lo, hi, n, q, plan, None, idx, vals))
            refs.append(F.topk(F.scan(planes, lo, hi, n, q, plan), k, group) if n > 0 else None)
        for rep in range(2):   # the counters must be back at a clean state for the second call
            for s in sess:
                s.idx.fill_(-7)
            F.scan_topk_batched(sess, k, group)
            torch.cuda.synchronize()
            for s, r in zip(sess, refs):
                if r is None:
                    assert torch.all(s.idx == -1) and torch.all(torch.isinf(s.vals))
                else:
                    assert torch.equal(s.idx, r[0]) and torch.equal(s.vals, r[1])


def test_scan_topk_against_oracle(F, orc):
    """Oracle logits (fp64 from the planes) ranked by the oracle's top-k: the
    fused result agrees up to ties within the logit tolerance."""
    n, hkv, hq, k = 30000, 2, 8, 512
    print("scan_topk vs oracle", flush=True)
    _, q, p, plan = layer(F, 560, n, hkv, hq)
    idx, vals = F.scan_topk(p.planes, p.lo, p.hi, n, q, plan, k, 1)
    torch.cuda.synchronize()
    ref_logits = orc.scan(p.planes.cpu().numpy().view(np.uint32), p.lo.cpu().numpy(),
                          p.hi.cpu().numpy(), n, q.cpu().numpy(), plan.cpu().numpy())
    ridx, _ = orc.topk(ref_logits.astype(np.float32), k, 1)
    A = logit_scale(q.cpu().numpy(), p.lo.cpu().numpy(), p.hi.cpu().numpy(), hq // hkv)
    assert_topk_tie_tolerant(idx.cpu().numpy(), ridx, ref_logits, A, n, k)


def test_scan_topk_threshold_negative_and_outlier_rows(F):
    """The fused threshold's two ways to its key: one histogram of the three
    binades below the largest sampled score (a positive one with enough keys
    there), else two radix digits over every sampled key.  Rows whose scores
    are all negative, and rows whose largest sampled score is one outlier far
    above the rest, take the second way; both still equal scan then top-k."""
    n, hkv, hq = 200000, 2, 8
    keys = synth.keys(540, 0, n, hkv, 128, torch.float16, 0, device=dev())
    keys[:, :, 0] = 8.0                      # a constant channel every head weighs
    ntiles = (n + 2047) // 2048
    t0 = ntiles // 64 * 2048                 # first sampled tile (the middle of stretch 0)
    keys[t0, 1, 1] = 2000.0                  # one key of kv head 1, in the subsample
    p = F.pack(keys)
    q = synth.queries(540, 0, hq, 128, device=dev())
    q[:hq // 2, 0] = -20.0                   # kv head 0: every score negative
    q[hq // 2:, 0] = 0.0
    q[hq // 2:, 1] = 10.0                    # kv head 1: one outlier key on top
    plan = F.plan(q, p.sigma2, 92)
    torch.cuda.synchronize()
    print("scan_topk negative rows and outlier rows", flush=True)
    for group in (1, 4):
        got, ref, logits = both(F, p, n, q, plan, 512, group)
        assert_same(got, ref)
        if group == 1:
            assert float(logits[: hq // 2, :n].max()) < 0.0
            assert int(got[0][hq // 2, 0]) == t0


@pytest.mark.parametrize("n,k", [(150000, 1024), (1 << 20, 2048)])
def test_scan_topk_group_cancelling_heads(F, n, k):
    """Rows per GQA group of four whose heads' weights cancel: in every group
    head 1 is head 0 negated (their plans agree, so the group weight of
    every slot they share is that of heads 2 and 3 alone), and in kv head 0
    heads 2 and 3 cancel as well (every group weight 0, the scores only
    rounding noise around the constant).  The integer pre-check of a key's
    group score against the row's bound must miss no candidate: fused equals
    scan then top-k bit for bit."""
    hkv, hq = 8, 32
    keys = synth.keys(570, 0, n, hkv, 128, torch.float16, 4, device=dev())
    q = synth.queries(570, 0, hq, 128, device=dev()).view(hkv, 4, 128)
    q[:, 1] = -q[:, 0]
    q[0, 3] = -q[0, 2]
    q = q.reshape(hq, 128).contiguous()
    p = F.pack(keys)
    del keys
    plan = F.plan(q, p.sigma2, 92)
    torch.cuda.synchronize()
    print(f"scan_topk cancelling heads n={n} k={k}", flush=True)
    got, ref, _ = both(F, p, n, q, plan, k, 4)
    assert_same(got, ref)


@pytest.mark.parametrize("case", ["rd_two_passes", "group_plan", "side_stream"])
def test_scan_topk_group4_other_paths(F, case):
    """Rows per GQA group of four that keep the general candidate path (more
    than 64 slots, i.e. two matrix-core passes, from a rate-distortion plan
    with a large budget; a side stream) or take the group pre-check with a
    plan shared by the group: fused equals scan then top-k bit for bit."""
    n, hkv, hq, k = 120000, 8, 32, 1024
    keys = synth.keys(580, 0, n, hkv, 128, torch.float16, 4, device=dev())
    q = synth.queries(580, 0, hq, 128, device=dev())
    p = F.pack(keys)
    del keys
    meta, scale = None, 0.0
    if case == "rd_two_passes":
        plan = F.plan_rd(q, p.sigma2, 300)
    elif case == "group_plan":
        plan = F.plan_group(q, p.sigma2, 176)
    else:
        plan = F.plan_fixed(q, 32)
        meta, scale = synth.side_stream(580, 0, hkv, n, device=dev()), 0.25
    torch.cuda.synchronize()
    print(f"scan_topk group 4 other paths case={case}", flush=True)
    got, ref, _ = both(F, p, n, q, plan, k, 4, meta, scale)
    assert_same(got, ref)


def test_scan_topk_recompute_two_head_chunks(F):
    """Eight query heads per kv head (two head chunks of four, two launches of
    the recompute scan) with every logit tied (budget 0): the final's blocks
    in the first launch flag every row, the scan blocks of both chunks
    recompute theirs; equals scan then top-k."""
    n, hkv, hq, k = 60000, 2, 16, 256
    _, q, p, plan = layer(F, 590, n, hkv, hq, budget=0)
    print("scan_topk recompute two head chunks", flush=True)
    flags = redo_flags(F, n, hkv, hq, 1, k, lambda ws: F.scan_topk(
        p.planes, p.lo, p.hi, n, q, plan, k, 1, ws=ws))
    assert int(flags.sum()) == hq
    got, ref, _ = both(F, p, n, q, plan, k, 1)
    assert_same(got, ref)
