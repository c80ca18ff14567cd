"""GPU parity of the calibrated allocation: fathom_code_hist and
fathom_plan_calibrated bit-exact against the CPU oracle (histograms of ragged
and capacity-laid-out planes, plans over many budgets and heads, the
hand-worked point-mass case), and scans of calibrated plans equal to scan
followed by top-k."""
import numpy as np
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


def dev():
    return torch.device("cuda:0")


def u32(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("n,hkv", [(1, 1), (31, 2), (33, 2), (2049, 3), (100000, 8)])
def test_code_hist_bit_exact(F, orc, n, hkv):
    print(f"code_hist n={n} hkv={hkv}", flush=True)
    keys = synth.keys(90 + n % 97, 0, n, hkv, 128, torch.float16, 4, device=dev())
    p = F.pack(keys)
    hist = F.code_hist(p.planes, n)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u32(hist), orc.code_hist(u32(p.planes), n))
    assert int(hist.sum()) == n * hkv * 128


def test_code_hist_ignores_bits_past_n(F, orc):
    n = 5000
    keys = synth.keys(91, 0, n, 2, 128, torch.float16, 4, device=dev())
    p = F.pack(keys)
    cap = torch.randint(-2 ** 31, 2 ** 31 - 1, (2, 128, 4, F.plane_words(20000)),
                        dtype=torch.int32, device=dev())       # garbage everywhere
    W0 = p.planes.shape[-1]
    cap[..., :W0] = p.planes
    # the tail word of n holds garbage above bit n % 32 as well
    tail = n // 32
    cap[..., tail] = cap[..., tail] | torch.tensor(-(1 << (n % 32)), dtype=torch.int32)
    hist = F.code_hist(cap, n)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u32(hist), orc.code_hist(u32(p.planes), n))


def layer(seed, n=60000, hkv=8, hq=32):
    keys = synth.keys(seed, 0, n, hkv, 128, torch.float16, 4, device=dev())
    q = synth.queries(seed, 0, hq, 128, device=dev())
    return keys, q


@pytest.mark.parametrize("hq,hkv", [(32, 8), (96, 8), (1, 1)])
@pytest.mark.parametrize("budget", [0, 1, 5, 68, 92, 136, 300, 511, 512, "random"])
def test_plan_calibrated_bit_exact(F, orc, hq, hkv, budget):
    print(f"plan_calibrated hq={hq} hkv={hkv} budget={budget}", flush=True)
    keys, q = layer(92 + hq, 20000, hkv, hq)
    p = F.pack(keys)
    hist = F.code_hist(p.planes, 20000)
    rng = np.random.default_rng(hq)
    B = (rng.integers(0, 513, hq).astype(np.int32) if budget == "random"
         else np.full(hq, budget, np.int32))
    plan = F.plan_calibrated(q, p.lo, p.hi, hist, B.tolist())
    torch.cuda.synchronize()
    ref = orc.plan_calibrated(q.cpu().numpy(), p.lo.cpu().numpy(), p.hi.cpu().numpy(),
                              u32(hist), B)
    np.testing.assert_array_equal(plan.cpu().numpy(), ref)


def test_plan_calibrated_point_mass_case(F, orc):
    """The oracle's hand-worked case, padded to d = 128 with unread channels."""
    hist = np.zeros((1, 128, 16), np.uint32)
    hist[0, 0, 8] = 16
    hist[0, 1, :] = 1
    hist[0, 2:, 0] = 16                      # constant channels: no error at any depth
    lo = np.zeros((1, 128), np.float32)
    hi = np.full((1, 128), 16.0, np.float32)
    q = np.zeros((1, 128), np.float32)
    q[0, 0], q[0, 1] = np.sqrt(10.0), 1.0
    for B in (1, 3, 4, 5, 6, 7, 8):
        got = F.plan_calibrated(torch.from_numpy(q).to(dev()), torch.from_numpy(lo).to(dev()),
                                torch.from_numpy(hi).to(dev()),
                                torch.from_numpy(hist.view(np.int32)).to(dev()), B)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(),
                                      orc.plan_calibrated(q, lo, hi, hist, B))


def test_scan_topk_with_calibrated_plans(F):
    n = 50000
    keys, q = layer(93, n, 2, 8)
    p = F.pack(keys)
    plan = F.plan_calibrated(q, p.lo, p.hi, F.code_hist(p.planes, n), 92)
    logits = F.scan(p.planes, p.lo, p.hi, n, q, plan)
    ref = F.topk(logits, 512, 1)
    got = F.scan_topk(p.planes, p.lo, p.hi, n, q, plan, 512, 1)
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    assert int(plan.to(torch.int64).sum(1).min()) == 92


@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 8), (64, 1), (144, 72)])
@pytest.mark.parametrize("budget", [0, 3, 92, 176, 512, "random"])
def test_plan_calibrated_group_bit_exact(F, orc, hq, hkv, budget):
    print(f"plan_calibrated_group hq={hq} hkv={hkv} budget={budget}", flush=True)
    keys, q = layer(94 + hq, 8000, hkv, hq)
    p = F.pack(keys)
    hist = F.code_hist(p.planes, 8000)
    rng = np.random.default_rng(hq + hkv)
    B = (rng.integers(0, 513, hkv).astype(np.int32) if budget == "random"
         else np.full(hkv, budget, np.int32))
    plan = F.plan_calibrated_group(q, p.lo, p.hi, hist, B.tolist())
    torch.cuda.synchronize()
    ref = orc.plan_calibrated_group(q.cpu().numpy(), p.lo.cpu().numpy(), p.hi.cpu().numpy(),
                                    u32(hist), B)
    np.testing.assert_array_equal(plan.cpu().numpy(), ref)
