"""GPU parity of fathom_append (decode-time growth of a packed layer):
planes bit-exact against the CPU oracle and the clamped counts equal, for
chunks that cross word and 2048-key block boundaries, fp16/fp32 and strided
keys, device and pinned-host planes; in-range appends equal packing the whole
sequence; and scans of a grown layer whose plane rows have spare capacity
equal scans of the same keys laid out compactly."""
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


def grown(F, keys, n0, chunks, capacity, pinned=False):
    """Pack keys[:n0], copy into capacity planes, append the chunks in order.
    Returns (planes, packed-first, clamped count)."""
    p = F.pack(keys[:n0])
    planes = F.alloc_planes(capacity, keys.shape[1], pin_memory=pinned)
    planes[..., :p.planes.shape[-1]].copy_(p.planes)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev())
    at = n0
    for m in chunks:
        F.append(keys[at:at + m], at, planes, p.lo, p.hi, cnt)
        at += m
    torch.cuda.synchronize()
    return planes, p, int(cnt.item())


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_append_bit_exact_against_oracle(F, orc, dtype):
    n0, chunks = 1000, [1, 7, 31, 32, 33, 2047, 1, 5000, 64]
    n = n0 + sum(chunks)
    print(f"append chunks {chunks} dtype={dtype}", flush=True)
    keys = synth.keys(71, 0, n, 2, 128, dtype, 4, device=dev())
    keys[n0 + 40:n0 + 60] *= 3                       # some values outside the stored range
    planes, p, cnt = grown(F, keys, n0, chunks, n + 3000)
    ref = u32(p.planes)
    ref = np.concatenate([ref, np.zeros(ref.shape[:3] + (planes.shape[-1] - ref.shape[-1],),
                                        np.uint32)], -1)
    expect_cnt = orc.append(keys[n0:].cpu().numpy(), n0, ref, p.lo.cpu().numpy(),
                            p.hi.cpu().numpy())
    np.testing.assert_array_equal(u32(planes), ref)
    assert cnt == expect_cnt and cnt > 0


def test_append_in_range_equals_pack_of_all(F):
    n0, n = 4000, 9000
    k = synth.keys(72, 0, n, 2, 128, torch.float16, 4).numpy()
    for h in range(2):                     # each channel's extremes among the first keys
        for c in range(128):
            i = int(np.argmin(k[:, h, c].astype(np.float32)))
            k[[0, i], h, c] = k[[i, 0], h, c]
            i = 1 + int(np.argmax(k[1:, h, c].astype(np.float32)))
            k[[1, i], h, c] = k[[i, 1], h, c]
    keys = torch.from_numpy(k).to(dev())
    full = F.pack(keys)
    planes, p, cnt = grown(F, keys, n0, [1, 999, 4000], n)
    assert cnt == 0
    assert torch.equal(p.lo, full.lo) and torch.equal(p.hi, full.hi)
    np.testing.assert_array_equal(u32(planes), u32(full.planes))


def test_append_strided_keys_and_pinned_planes(F):
    n0, n = 500, 3000
    big = synth.keys(73, 0, n, 2, 256, torch.float16, 0, device=dev())
    keys = big[:, :, 64:192]                          # stride_tok 512, stride_head 256
    p = F.pack(keys[:n0].contiguous())
    a = F.alloc_planes(4096, 2)
    b = F.alloc_planes(4096, 2, pin_memory=True)
    for t in (a, b):
        t[..., :p.planes.shape[-1]].copy_(p.planes)
    F.append(keys[n0:], n0, a, p.lo, p.hi)
    F.append(keys[n0:].contiguous(), n0, b, p.lo, p.hi)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u32(a), u32(b))


def test_decode_loop_then_scans_of_capacity_planes(F, orc):
    """300 single-token appends across a 2048-key boundary, then scan and
    fused scan + top-k on the capacity layout against the compact layout."""
    n0, n = 1900, 2200
    keys = synth.keys(74, 0, n, 2, 128, torch.float16, 4, device=dev())
    planes, p, _ = grown(F, keys, n0, [1] * (n - n0), 64 * 2048)
    compact = planes[..., :F.plane_words(n)].contiguous()
    q = synth.queries(74, 0, 8, 128, device=dev())
    plan = F.plan(q, p.sigma2, 92)
    a = F.scan(planes, p.lo, p.hi, n, q, plan)
    b = F.scan(compact, p.lo, p.hi, n, q, plan)
    ia, va = F.scan_topk(planes, p.lo, p.hi, n, q, plan, 256, 1)
    ib, vb = F.scan_topk(compact, p.lo, p.hi, n, q, plan, 256, 1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(ia, ib) and torch.equal(va, vb)
    # the grown keys are the oracle's too
    ref = u32(p.planes)
    ref = np.concatenate([ref, np.zeros(ref.shape[:3] + (F.plane_words(n) - ref.shape[-1],),
                                        np.uint32)], -1)
    orc.append(keys[n0:].cpu().numpy(), n0, ref, p.lo.cpu().numpy(), p.hi.cpu().numpy())
    np.testing.assert_array_equal(u32(compact), ref)


def test_batched_sessions_with_capacity_planes(F):
    """Sessions of one batched call with different capacities and lengths."""
    sess, refs = [], []
    for j, (n, cap) in enumerate([(3000, 8192), (5000, 5000), (7000, 20000)]):
        keys = synth.keys(80 + j, 0, n, 2, 128, torch.float16, 4, device=dev())
        p = F.pack(keys)
        planes = F.alloc_planes(cap, 2)
        planes[..., :p.planes.shape[-1]].copy_(p.planes)
        q = synth.queries(80 + j, 0, 8, 128, device=dev())
        plan = F.plan(q, p.sigma2, 92)
        idx = torch.empty((8, 128), dtype=torch.int32, device=dev())
        vals = torch.empty((8, 128), dtype=torch.float32, device=dev())
        sess.append(F.Session(planes, p.lo, p.hi, n, q, plan, idx=idx, vals=vals))
        refs.append(F.scan_topk(p.planes, p.lo, p.hi, n, q, plan, 128, 1))
    F.scan_topk_batched(sess, 128, 1)
    torch.cuda.synchronize()
    for s, (ri, rv) in zip(sess, refs):
        assert torch.equal(s.idx, ri) and torch.equal(s.vals, rv)


def test_pinned_capacity_planes_scan_like_compact(F):
    """Host-resident planes take the host-link kernel: capacity and compact
    layouts of the same keys give identical logits and top-k."""
    n = 9000
    keys = synth.keys(75, 0, n, 2, 128, torch.float16, 4, device=dev())
    p = F.pack(keys)
    cap = F.alloc_planes(3 * 2048 * 2 + 100, 2, pin_memory=True)
    cap[..., :p.planes.shape[-1]].copy_(p.planes)
    compact = torch.empty(p.planes.shape, dtype=p.planes.dtype, pin_memory=True)
    compact.copy_(p.planes)
    q = synth.queries(75, 0, 8, 128, device=dev())
    plan = F.plan(q, p.sigma2, 92)
    a = F.scan(cap, p.lo, p.hi, n, q, plan)
    b = F.scan(compact, p.lo, p.hi, n, q, plan)
    ia, va = F.scan_topk(cap, p.lo, p.hi, n, q, plan, 300, 1)
    ib, vb = F.scan_topk(compact, p.lo, p.hi, n, q, plan, 300, 1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(ia, ib) and torch.equal(va, vb)
