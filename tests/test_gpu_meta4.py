"""GPU parity of the 68-bit fixed-width baseline: the r = 16 plan (the 16
channels with the largest |q_c| at 4 bits) plus the 4-bit per-key side stream
(two keys per byte, even key in the low nibble).  Logits within 1e-5 * A_h of
the oracle (planes in HBM: matrix-core kernel; pinned host memory: fp32
kernel; row lengths that are and are not multiples of 4, and a side stream at
an odd address, which take the per-key loads); the fused call identical to
the scan followed by fathom_topk; and the 1M-key layer with planes and side
stream in pinned host memory, kv head 0 against the oracle's own pack."""
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


def pinned(t):
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


@pytest.mark.parametrize("host", [False, True])
@pytest.mark.parametrize("n,odd_addr", [(12344, False), (4099, False), (20000, True)])
def test_scan_meta4_matches_oracle(F, orc, host, n, odd_addr):
    hkv, hq, scale = 2, 8, 0.37
    print(f"meta4 scan n={n} host={host} odd_addr={odd_addr}", flush=True)
    keys = synth.keys(61, n % 5, n, hkv, 128, torch.float16, 4)
    q = synth.queries(61, n % 5, hq, 128)
    m4 = synth.side_stream4(61, n % 5, hkv, n)
    ref = orc.pack(keys.float().numpy())
    pn = orc.plan_fixed(q.numpy(), 16)
    p = F.pack(keys.to(dev()))
    planes = pinned(p.planes) if host else p.planes
    # the stream in HBM or pinned host memory; odd_addr: the same bytes one
    # byte into a buffer
    if host:
        flat = torch.zeros(m4.numel() + 1, dtype=torch.uint8, pin_memory=True)
    else:
        flat = torch.zeros(m4.numel() + 1, dtype=torch.uint8, device=dev())
    off = 1 if odd_addr else 0
    flat[off:off + m4.numel()].copy_(m4.reshape(-1))
    m = flat[off:off + m4.numel()].view(hkv, m4.shape[1])
    L = F.scan(planes, p.lo, p.hi, n, q.to(dev()), torch.from_numpy(pn).to(dev()), m, scale,
               meta_bits=4)
    torch.cuda.synchronize()
    R = orc.scan(ref["planes"], ref["lo"], ref["hi"], n, q.numpy(), pn, m4.numpy(), scale,
                 meta_bits=4)
    A = logit_scale(q.numpy(), ref["lo"], ref["hi"], hq // hkv, scale)
    assert_logits_close(L.cpu().numpy(), R, A)


@pytest.mark.parametrize("group", [1, 4])
def test_scan_topk_meta4(F, orc, group):
    n, hkv, hq, k, scale = 70000, 2, 8, 512, 0.5
    print(f"meta4 scan_topk group={group}", flush=True)
    keys = synth.keys(62, 0, n, hkv, 128, torch.float16, 4)
    q = synth.queries(62, 0, hq, 128)
    m4 = synth.side_stream4(62, 0, hkv, n)
    ref = orc.pack(keys.float().numpy())
    pn = orc.plan_fixed(q.numpy(), 16)
    p = F.pack(keys.to(dev()))
    qd, pd, md = q.to(dev()), torch.from_numpy(pn).to(dev()), m4.to(dev())
    L = F.scan(p.planes, p.lo, p.hi, n, qd, pd, md, scale, meta_bits=4)
    idx, vals = F.topk(L, k, group=group)
    fidx, fvals = F.scan_topk(p.planes, p.lo, p.hi, n, qd, pd, k, group, md, scale,
                              meta_bits=4)
    torch.cuda.synchronize()
    assert torch.equal(fidx, idx) and torch.equal(fvals, vals)
    R = orc.scan(ref["planes"], ref["lo"], ref["hi"], n, q.numpy(), pn, m4.numpy(), scale,
                 meta_bits=4)
    A = logit_scale(q.numpy(), ref["lo"], ref["hi"], hq // hkv, scale)
    assert_logits_close(L.cpu().numpy(), R, A)
    if group == 1:
        ridx, _ = orc.topk(R, k)
        assert_topk_tie_tolerant(fidx.cpu().numpy(), ridx, R, A, n, k)


def test_layer_1m_meta4_host(F, orc):
    """The 1M-key layer (8 kv heads, 32 query heads), r = 16 with the 4-bit
    stream, planes and stream in pinned host memory, as the benchmark runs it."""
    w = synth.LAYER_1M
    n, scale = w.n, 1.0 / 16
    print("1M-key layer, r = 16 + 4-bit stream, host-resident", flush=True)
    keys = synth.keys(w.seed, 0, n, w.hkv, w.d, w.dtype, w.outliers, device=dev())
    q = synth.queries(w.seed, 0, w.hq, w.d)
    m4 = synth.side_stream4(w.seed, 0, w.hkv, n, device=dev())
    p = F.pack(keys)
    planes, mh = pinned(p.planes), pinned(m4)
    pn = orc.plan_fixed(q.numpy(), 16)
    qd, pd = q.to(dev()), torch.from_numpy(pn).to(dev())
    L = F.scan(planes, p.lo, p.hi, n, qd, pd, mh, scale, meta_bits=4)
    idx, vals = F.topk(L, w.k)
    fidx, fvals = F.scan_topk(planes, p.lo, p.hi, n, qd, pd, w.k, 1, mh, scale, meta_bits=4)
    torch.cuda.synchronize()
    assert torch.equal(fidx, idx) and torch.equal(fvals, vals)
    ref = orc.pack(keys[:, :1].float().cpu().numpy())
    np.testing.assert_array_equal(p.planes[:1].cpu().numpy().view(np.uint32), ref["planes"])
    rng = np.random.default_rng(7)
    pick = np.unique(np.concatenate([rng.integers(0, n, 3000), np.arange(n - 9, n)]))
    G = w.hq // w.hkv
    R = orc.scan_at(ref["planes"], ref["lo"], ref["hi"], n, q.numpy()[:G], pn[:G], pick,
                    m4[:1].cpu().numpy(), scale, meta_bits=4)
    A = logit_scale(q.numpy()[:G], ref["lo"], ref["hi"], G, scale)
    assert_logits_close(L[:G].cpu().numpy()[:, pick], R, A)
