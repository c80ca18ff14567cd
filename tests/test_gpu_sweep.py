"""Seeded sweep over the call's configuration space: length, kv heads, GQA
size, top-k group, k, per-head budgets, plan kind, key dtype, planes in HBM or
pinned host memory, with or without the side stream.  Every case: the fused
scan + top-k equals scan followed by top-k bit for bit; for short sessions the
logits also stay within the oracle's tolerance."""
import numpy as np
import pytest
import torch

import synth
from parity import assert_logits_close, logit_scale

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


def make_plan(F, kind, q, p, n, budgets, hkv, rng):
    if kind == "walk":
        return F.plan(q, p.sigma2, budgets)
    if kind == "rd":
        return F.plan_rd(q, p.sigma2, budgets)
    if kind == "group":
        return F.plan_group(q, p.sigma2, rng.integers(0, 513, hkv).tolist())
    if kind == "calibrated":
        return F.plan_calibrated(q, p.lo, p.hi, F.code_hist(p.planes, n), budgets)
    return F.plan_fixed(q, int(rng.integers(0, 129)))


@pytest.mark.parametrize("case", range(32))
def test_sweep_fused_equals_scan_then_topk(F, orc, case):
    rng = np.random.default_rng(7000 + case)
    n = int(rng.choice([1, 17, 2048, 5000, 8193, int(rng.integers(10000, 300000))]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * G
    group = int(rng.choice([g for g in (1, 2, 4, 8) if G % g == 0]))
    k = int(rng.integers(1, 2049))
    kind = str(rng.choice(["walk", "rd", "group", "calibrated", "fixed"]))
    dtype = torch.float16 if rng.random() < 0.7 else torch.float32
    host = bool(rng.random() < 0.3)
    meta = bool(rng.random() < 0.3)
    print(f"sweep case {case}: n={n} hkv={hkv} hq={hq} group={group} k={k} plan={kind} "
          f"dtype={dtype} host={host} meta={meta}", flush=True)
    keys = synth.keys(7000 + case, 0, n, hkv, 128, dtype, 4 if n > 8 else 0, device=dev())
    q = synth.queries(7000 + case, 0, hq, 128, device=dev())
    p = F.pack(keys)
    budgets = rng.integers(0, 513, hq).tolist()
    plan = make_plan(F, kind, q, p, n, budgets, hkv, rng)
    planes = p.planes
    if host:
        planes = torch.empty(p.planes.shape, dtype=p.planes.dtype, pin_memory=True)
        planes.copy_(p.planes)
    side = synth.side_stream(7000 + case, 0, hkv, n, device=dev()) if meta else None
    ms = 0.25 if meta else 0.0
    logits = F.scan(planes, p.lo, p.hi, n, q, plan, side, ms)
    ref = F.topk(logits, k, group)
    got = F.scan_topk(planes, p.lo, p.hi, n, q, plan, k, group, side, ms)
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0]), "idx"
    assert torch.equal(got[1], ref[1]), "vals"
    if n <= 20000:
        oref = orc.scan(p.planes.cpu().numpy().view(np.uint32), p.lo.cpu().numpy(),
                        p.hi.cpu().numpy(), n, q.cpu().numpy(), plan.cpu().numpy(),
                        None if side is None else side.cpu().numpy(), ms)
        A = logit_scale(q.cpu().numpy(), p.lo.cpu().numpy(), p.hi.cpu().numpy(), G, ms)
        assert_logits_close(logits.cpu().numpy(), oref, A)
