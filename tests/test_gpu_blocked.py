"""GPU parity of per-block ranges (one lo/hi per 2048-key block of a channel,
for long sessions whose key ranges drift):

  * fathom_pack_blocked: planes, lo, hi and sigma2 bit-exact against the
    oracle's pack_blocked, fp16/fp32 keys, aligned (vector kernels) and
    unaligned (scalar kernels) strides, one to many blocks with a ragged tail;
  * fathom_append_blocked: chunks that start blocks, cross them, start exactly
    on a boundary (one new block: the folded range step) or span several new
    blocks (the running-range step), from an empty layer too; planes, lo, hi
    and the clamped counts equal the oracle's step by step;
  * fathom_scan_blocked: logits within 1e-5 * A_h of the oracle's (A_h with
    each channel's largest |lo|, |hi| over blocks), planes in HBM (matrix-core
    kernel) and in pinned host memory (fp32 kernel), per-head and shared
    plans, budgets 0..512; bit-identical to the per-layer scan when every
    block carries the layer's range, and for a layer of one block;
  * fathom_scan_topk_blocked: identical to the blocked scan followed by
    fathom_topk, per head and per GQA group, and its top-k against the
    oracle's own top-k of its own logits (tie-tolerant);
  * the 1M-key, 8-kv-head layer at B = 68: kv head 0's planes and ranges
    bit-exact against the oracle, logits at sampled keys within tolerance,
    and the fused call equal to scan then top-k.
The oracle side always takes the oracle's own pack of the same keys."""
import numpy as np
import pytest
import torch

import synth
from parity import assert_logits_close, assert_topk_tie_tolerant, group_scores, logit_scale

pytestmark = pytest.mark.gpu

RB = 2048


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


def block_scale(q, lo, hi, group):
    """A_h with each channel's largest |lo_b|, |hi_b| over its blocks."""
    m = np.maximum(np.abs(lo), np.abs(hi)).max(1)
    return logit_scale(q, m, m, group)


def keys_np(keys):
    return keys.float().cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("n", [1, 2047, 2049, 3 * RB + 5, 20000])
@pytest.mark.parametrize("aligned", [True, False])
def test_pack_blocked_bit_exact(F, orc, dtype, n, aligned):
    print(f"pack_blocked n={n} dtype={dtype} aligned={aligned}", flush=True)
    full = synth.drifting_keys(11, n % 7, n, 2, 129, dtype, 4, device=dev())
    keys = full[:, :, :128] if not aligned else full[:, :, 1:].contiguous()
    p = F.pack_blocked(keys)
    torch.cuda.synchronize()
    ref = orc.pack_blocked(keys_np(keys))
    np.testing.assert_array_equal(u32(p.planes), ref["planes"])
    np.testing.assert_array_equal(p.lo.cpu().numpy(), ref["lo"])
    np.testing.assert_array_equal(p.hi.cpu().numpy(), ref["hi"])
    np.testing.assert_array_equal(p.sigma2.cpu().numpy(), ref["sigma2"])


def grow(F, orc, keys, n0, chunks, capacity):
    """GPU and oracle layers grown from keys[:n0] (empty when n0 == 0) by the
    chunks in order, compared after every chunk."""
    hkv = keys.shape[1]
    R = orc.range_blocks(capacity)
    W = F.plane_words(capacity)
    planes = torch.zeros((hkv, 128, 4, W), dtype=torch.int32, device=dev())
    lo = torch.zeros((hkv, R, 128), dtype=torch.float32, device=dev())
    hi = torch.zeros_like(lo)
    rp = np.zeros((hkv, 128, 4, W), np.uint32)
    rlo = np.zeros((hkv, R, 128), np.float32)
    rhi = np.zeros_like(rlo)
    kn = keys_np(keys)
    if n0 > 0:
        p = F.pack_blocked(keys[:n0], capacity=capacity)
        planes.copy_(p.planes)
        lo.copy_(p.lo)
        hi.copy_(p.hi)
        r = orc.pack_blocked(kn[:n0], nbc=R)
        rp[..., :r["planes"].shape[-1]] = r["planes"]
        rlo[:] = r["lo"]
        rhi[:] = r["hi"]
    cnt = torch.zeros(1, dtype=torch.int32, device=dev())
    at, total = n0, 0
    for m in chunks:
        F.append_blocked(keys[at:at + m], at, planes, lo, hi, cnt)
        total += orc.append_blocked(kn[at:at + m], at, rp, rlo, rhi)
        at += m
        torch.cuda.synchronize()
        np.testing.assert_array_equal(lo.cpu().numpy(), rlo, err_msg=f"lo after {at}")
        np.testing.assert_array_equal(hi.cpu().numpy(), rhi, err_msg=f"hi after {at}")
        np.testing.assert_array_equal(u32(planes), rp, err_msg=f"planes after {at}")
        assert int(cnt.item()) == total, (at, int(cnt.item()), total)
    return planes, lo, hi, total


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_append_blocked_bit_exact(F, orc, dtype):
    # 1000 old keys; then: inside block 0, up to the boundary, one key that
    # starts block 1 (folded step), across blocks 1..3 (running step), a ragged
    # rest, one more key, and a chunk spanning several new blocks
    n0 = 1000
    chunks = [7, RB - 1007, 1, 3 * RB + 11, 29, 1, 5 * RB + 3]
    n = n0 + sum(chunks)
    print(f"append_blocked chunks {chunks} dtype={dtype}", flush=True)
    keys = synth.drifting_keys(12, 0, n, 2, 128, dtype, 4, drift=4.0, device=dev())
    keys[n0 + 2:n0 + 5] *= 4            # values outside block 0's stored range
    _, _, _, total = grow(F, orc, keys, n0, chunks, n + 2 * RB)
    assert total > 0


def test_append_blocked_from_empty(F, orc):
    chunks = [1, 5, RB - 6, RB, 1, 3 * RB]
    n = sum(chunks)
    keys = synth.drifting_keys(13, 0, n, 2, 128, torch.float16, 4, device=dev())
    print("append_blocked from an empty layer", flush=True)
    grow(F, orc, keys, 0, chunks, n)
    # chunks that only start new blocks take ranges covering their keys
    _, _, _, total = grow(F, orc, keys[:6 * RB], 0, [RB, RB, 3 * RB + 5], 6 * RB)
    assert total == 0


def plans_for(orc, q, s2, budgets):
    return orc.plan(q, s2, budgets)


@pytest.mark.parametrize("pinned", [False, True])
@pytest.mark.parametrize("n,B", [(2049, 68), (20000, 68), (20000, 0), (9000, 512),
                                 (3 * RB + 5, 92)])
def test_scan_blocked_matches_oracle(F, orc, pinned, n, B):
    hkv, hq = 2, 8
    G = hq // hkv
    print(f"scan_blocked n={n} B={B} pinned={pinned}", flush=True)
    keys = synth.drifting_keys(14, B, n, hkv, 128, torch.float16, 4, device=dev())
    q = synth.queries(14, B, hq, 128)
    ref = orc.pack_blocked(keys_np(keys))
    pn = plans_for(orc, q.numpy(), ref["sigma2"], [B] * hq)
    p = F.pack_blocked(keys)
    planes = p.planes
    if pinned:
        planes = torch.empty(p.planes.shape, dtype=torch.int32, pin_memory=True)
        planes.copy_(p.planes)
    qd, pd = q.to(dev()), torch.from_numpy(pn).to(dev())
    L = F.scan_blocked(planes, p.lo, p.hi, n, qd, pd)
    torch.cuda.synchronize()
    R = orc.scan_blocked(ref["planes"], ref["lo"], ref["hi"], n, q.numpy(), pn)
    A = block_scale(q.numpy(), ref["lo"], ref["hi"], G)
    assert_logits_close(L.cpu().numpy(), R, A)


@pytest.mark.parametrize("pinned", [False, True])
def test_scan_blocked_mixed_depths(F, orc, pinned):
    """Random per-head budgets (so the GQA group's heads read different depths
    of the same channels) with a capacity layout of the planes."""
    n, hkv, hq = 13000, 2, 8
    keys = synth.drifting_keys(15, 1, n, hkv, 128, torch.float32, 4, device=dev())
    q = synth.queries(15, 1, hq, 128)
    budgets = synth.random_budgets(15, hq, 0, 300)
    print(f"scan_blocked budgets {budgets} pinned={pinned}", flush=True)
    ref = orc.pack_blocked(keys_np(keys))
    pn = plans_for(orc, q.numpy(), ref["sigma2"], budgets)
    p = F.pack_blocked(keys, capacity=n + 5 * RB)
    planes = p.planes
    if pinned:
        planes = torch.empty(p.planes.shape, dtype=torch.int32, pin_memory=True)
        planes.copy_(p.planes)
    L = F.scan_blocked(planes, p.lo, p.hi, n, q.to(dev()), torch.from_numpy(pn).to(dev()))
    torch.cuda.synchronize()
    R = orc.scan_blocked(ref["planes"], ref["lo"], ref["hi"], n, q.numpy(), pn)
    assert_logits_close(L.cpu().numpy(), R, block_scale(q.numpy(), ref["lo"], ref["hi"], 4))


@pytest.mark.parametrize("pinned", [False, True])
@pytest.mark.parametrize("n", [1500, 100000])
def test_scan_blocked_equals_per_layer_scan(F, pinned, n):
    """A layer whose every block carries the layer's range, and (n <= 2048) a
    layer of one block, score bit for bit as with per-layer ranges."""
    hkv, hq, B = 2, 8, 68
    keys = synth.keys(16, 0, n, hkv, 128, torch.float16, 4, device=dev())
    q = synth.queries(16, 0, hq, 128, device=dev())
    p = F.pack(keys)
    plan = F.plan(q, p.sigma2, B)
    R = F.range_blocks(n)
    lo = p.lo[:, None, :].expand(hkv, R, 128).contiguous()
    hi = p.hi[:, None, :].expand(hkv, R, 128).contiguous()
    planes = p.planes
    if pinned:
        planes = torch.empty(p.planes.shape, dtype=torch.int32, pin_memory=True)
        planes.copy_(p.planes)
    print(f"blocked == per-layer n={n} pinned={pinned}", flush=True)
    a = F.scan(planes, p.lo, p.hi, n, q, plan)
    b = F.scan_blocked(planes, lo, hi, n, q, plan)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    if n <= RB:
        pb = F.pack_blocked(keys)
        assert torch.equal(pb.lo[:, 0], p.lo) and torch.equal(pb.hi[:, 0], p.hi)
        assert torch.equal(pb.sigma2, p.sigma2) and torch.equal(pb.planes, p.planes)


@pytest.mark.parametrize("group", [1, 4])
@pytest.mark.parametrize("n", [9000, 150000])
def test_scan_topk_blocked(F, orc, group, n):
    hkv, hq, k, B = 2, 8, 256, 68
    print(f"scan_topk_blocked n={n} group={group}", flush=True)
    keys = synth.drifting_keys(17, group, n, hkv, 128, torch.float16, 4, device=dev())
    q = synth.queries(17, group, hq, 128)
    ref = orc.pack_blocked(keys_np(keys))
    pn = plans_for(orc, q.numpy(), ref["sigma2"], [B] * hq)
    p = F.pack_blocked(keys)
    qd, pd = q.to(dev()), torch.from_numpy(pn).to(dev())
    L = F.scan_blocked(p.planes, p.lo, p.hi, n, qd, pd)
    idx, vals = F.topk(L, k, group=group)
    fidx, fvals = F.scan_topk_blocked(p.planes, p.lo, p.hi, n, qd, pd, k, group)
    torch.cuda.synchronize()
    assert torch.equal(fidx, idx) and torch.equal(fvals, vals)
    R = orc.scan_blocked(ref["planes"], ref["lo"], ref["hi"], n, q.numpy(), pn)
    A = block_scale(q.numpy(), ref["lo"], ref["hi"], hq // hkv)
    assert_logits_close(L.cpu().numpy(), R, A)
    ridx, _ = orc.topk(R, k, group)
    Rs = R if group == 1 else group_scores(R, group)
    Ar = A if group == 1 else A.reshape(-1, group).sum(1)
    assert_topk_tie_tolerant(fidx.cpu().numpy(), ridx, Rs, Ar, n, k)


def test_layer_1m_blocked(F, orc):
    """The 1M-key layer (8 kv heads, 32 query heads, fp16, B = 68, k = 2048)
    with drifting keys: kv head 0 packed by the oracle (planes, ranges bit for
    bit), logits of its query heads at sampled keys, and the fused call."""
    n, hkv, hq, k, B = 1 << 20, 8, 32, 2048, 68
    print("1M-key blocked layer", flush=True)
    keys = synth.drifting_keys(18, 0, n, hkv, 128, torch.float16, 4, device=dev())
    q = synth.queries(18, 0, hq, 128)
    p = F.pack_blocked(keys)
    torch.cuda.synchronize()
    k0 = keys[:, :1].float().cpu().numpy()
    ref = orc.pack_blocked(k0)
    np.testing.assert_array_equal(u32(p.planes[:1]), ref["planes"])
    np.testing.assert_array_equal(p.lo[:1].cpu().numpy(), ref["lo"])
    np.testing.assert_array_equal(p.hi[:1].cpu().numpy(), ref["hi"])
    np.testing.assert_array_equal(p.sigma2[:1].cpu().numpy(), ref["sigma2"])
    # every kv head planned with kv head 0's oracle sigma2 (any plan is an
    # input of the scan; this one comes from the oracle alone)
    pn = orc.plan(q.numpy(), np.tile(ref["sigma2"], (hkv, 1)), [B] * hq)
    qd, pd = q.to(dev()), torch.from_numpy(pn).to(dev())
    L = F.scan_blocked(p.planes, p.lo, p.hi, n, qd, pd)
    idx, vals = F.topk(L, k)
    fidx, fvals = F.scan_topk_blocked(p.planes, p.lo, p.hi, n, qd, pd, k, 1)
    gidx, gvals = F.topk(L, k, group=4)
    fgidx, fgvals = F.scan_topk_blocked(p.planes, p.lo, p.hi, n, qd, pd, k, 4)
    torch.cuda.synchronize()
    assert torch.equal(fidx, idx) and torch.equal(fvals, vals)
    assert torch.equal(fgidx, gidx) and torch.equal(fgvals, gvals)
    rng = np.random.default_rng(18)
    pick = np.unique(np.concatenate([rng.integers(0, n, 3000), np.arange(n - 20, n),
                                     idx[:4, :3].cpu().numpy().ravel()]))
    R = orc.scan_blocked_at(ref["planes"], ref["lo"], ref["hi"], n, q.numpy()[:4], pn[:4], pick)
    A = block_scale(q.numpy()[:4], ref["lo"], ref["hi"], 4)
    assert_logits_close(L[:4].cpu().numpy()[:, pick], R, A)
