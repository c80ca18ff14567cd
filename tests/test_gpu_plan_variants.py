"""GPU parity of the two allocation variants, fathom_plan_rd (rate-distortion
greedy) and fathom_plan_group (one plan per GQA group): bit-exact against the
CPU oracle on identical inputs, including exact ties, zero-importance
channels, tiny values and launches over more than 64 heads; and the scan and
the fused scan + top-k run with these plans (many channels at depths 1..3)."""
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


def T(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def inputs(seed, hq, hkv):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((hq, 128)).astype(np.float32)
    s2 = np.exp(rng.uniform(np.log(0.01), np.log(256), (hkv, 128))).astype(np.float32)
    s2[:, :3] = 0.0
    return rng, q, s2


@pytest.mark.parametrize("hq,hkv", [(32, 8), (1, 1), (96, 8)])
@pytest.mark.parametrize("budget", [0, 1, 3, 5, 18, 91, 92, 136, 300, 511, 512, "random"])
def test_plan_rd_bit_exact(F, orc, hq, hkv, budget):
    print(f"plan_rd hq={hq} hkv={hkv} budget={budget}", flush=True)
    rng, q, s2 = inputs(hq * 7 + (budget if isinstance(budget, int) else 3), hq, hkv)
    B = (rng.integers(0, 513, hq).astype(np.int32) if budget == "random"
         else np.full(hq, budget, np.int32))
    got = F.plan_rd(T(q), T(s2), B.tolist())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), orc.plan_rd(q, s2, B))


def test_plan_rd_exact_ties_and_tiny_values(F, orc):
    hq = 6
    q = np.ones((hq, 128), np.float32)
    # head 1: importances in exact ratios 4^k, so gains tie across channels
    q[1] = np.ldexp(1.0, -(np.arange(128) % 5)).astype(np.float32)
    q[2] = 0.0                                          # every gain zero
    q[3, ::2] = -1.0
    rng = np.random.default_rng(9)
    q[4] = (rng.standard_normal(128) * 1e-20).astype(np.float32)   # subnormal squares
    q[5] = rng.integers(-2, 3, 128).astype(np.float32)
    s2 = np.ones((1, 128), np.float32)
    for B in (1, 7, 92, 129, 383, 512):
        got = F.plan_rd(T(q), T(s2), B)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), orc.plan_rd(q, s2, B), err_msg=str(B))


@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 8), (64, 1), (144, 72), (24, 3)])
@pytest.mark.parametrize("budget", [0, 1, 46, 92, 136, 512, "random"])
def test_plan_group_bit_exact(F, orc, hq, hkv, budget):
    print(f"plan_group hq={hq} hkv={hkv} budget={budget}", flush=True)
    rng, q, s2 = inputs(hq * 11 + hkv + (budget if isinstance(budget, int) else 5), hq, hkv)
    B = (rng.integers(0, 513, hkv).astype(np.int32) if budget == "random"
         else np.full(hkv, budget, np.int32))
    got = F.plan_group(T(q), T(s2), B.tolist())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), orc.plan_group(q, s2, B))


def test_plan_group_ties_and_tiny_values(F, orc):
    G, hkv = 4, 3
    rng = np.random.default_rng(12)
    q = rng.integers(-2, 3, (G * hkv, 128)).astype(np.float32)
    q[G:2 * G] = (rng.standard_normal((G, 128)) * 1e-20).astype(np.float32)
    q[2 * G:] = 0.0
    s2 = np.ones((hkv, 128), np.float32)
    for B in (1, 45, 92, 512):
        got = F.plan_group(T(q), T(s2), B)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), orc.plan_group(q, s2, B),
                                      err_msg=str(B))


def test_plan_variants_are_deterministic(F):
    q = synth.queries(16, 0, 32, 128, device=dev())
    s2 = torch.rand((8, 128), device=dev())
    for fn in (F.plan_rd, F.plan_group):
        a, b = fn(q, s2, 92), fn(q, s2, 92)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


@pytest.mark.parametrize("variant", ["rd", "group"])
def test_scan_and_scan_topk_with_variant_plans(F, orc, variant):
    """The scan reads any depth per (head, channel); these plans put many
    channels at depths 1..3 (rd) or one shared row per group (group)."""
    n, hkv, hq, k = 30000, 2, 8, 512
    print(f"scan with {variant} plan n={n}", flush=True)
    keys = synth.keys(570, 0, n, hkv, 128, torch.float16, 4, device=dev())
    q = synth.queries(570, 0, hq, 128, device=dev())
    p = F.pack(keys)
    plan = F.plan_rd(q, p.sigma2, 92) if variant == "rd" else F.plan_group(q, p.sigma2, 92)
    logits = F.scan(p.planes, p.lo, p.hi, n, q, plan)
    ref_topk = F.topk(logits, k, 1)
    idx, vals = F.scan_topk(p.planes, p.lo, p.hi, n, q, plan, k, 1)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_topk[0]) and torch.equal(vals, ref_topk[1])
    ref = orc.scan(p.planes.cpu().numpy().view(np.uint32), p.lo.cpu().numpy(),
                   p.hi.cpu().numpy(), n, q.cpu().numpy(), plan.cpu().numpy())
    A = logit_scale(q.cpu().numpy(), p.lo.cpu().numpy(), p.hi.cpu().numpy(), hq // hkv)
    assert_logits_close(logits.cpu().numpy(), ref, A)
    ridx, _ = orc.topk(ref.astype(np.float32), k, 1)
    assert_topk_tie_tolerant(idx.cpu().numpy(), ridx, ref, A, n, k)
