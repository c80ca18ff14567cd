"""GPU parity of fathom_sparse_attention against the CPU oracle (fp64 softmax
over the listed keys): fp16 and fp32 caches, groups 1/2/4/8, ragged and padded
index rows, strided and pinned-host caches, entries out of range, empty rows,
and the decode step's own indices from fathom_scan_topk at the 1M-key size.

Tolerance, derived from the fp32 arithmetic: a score is a sum of d fp32
products along which every term meets at most d + 1 roundings (fused
multiply-adds over runs of channels, a butterfly over the runs, one
scaling), so |s_gpu - s| <= eps_s with
eps_s = scale * (d + 2) * 2^-24 * max_i sum_c |q_c K_ic|.  Score errors move
each softmax weight by a relative 2 eps_s at most (first order), and a
convex combination of V rows then moves by <= 2 eps_s max|V|; the fp32 sums
over <= 64 weights per partial plus the merge add < 1e-5 max|V|.  Hence
|out - ref| <= (2.5 eps_s + 1e-5) max|V| and
|lse - ref| <= 1.5 eps_s + 1e-6 max(1, |lse|)."""
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


def caches(seed, n, hkv, dtype, d=128):
    g = torch.Generator().manual_seed(seed)
    K = (torch.randn((n, hkv, d), generator=g) * 0.8).to(dtype)
    V = torch.randn((n, hkv, d), generator=g).to(dtype)
    return K, V


def check(F, orc, q, K, V, idx, group, scale=None, Kd=None, Vd=None, tag=""):
    """q fp32 CPU [hq][d]; K, V CPU [n][hkv][d]; idx CPU int32 [rows][k]."""
    hq, d = q.shape
    n, hkv, _ = K.shape
    print(f"attention case {tag} n={n} hkv={hkv} hq={hq} k={idx.shape[1]} group={group} "
          f"dtype={K.dtype}", flush=True)
    s = 1.0 / np.sqrt(d) if scale is None else scale
    Kd = K.to(dev()) if Kd is None else Kd
    Vd = V.to(dev()) if Vd is None else Vd
    out, lse = F.sparse_attention(q.to(dev()), Kd, Vd, idx.to(dev()), group, s)
    torch.cuda.synchronize()
    idx_np = idx.numpy()
    clean = np.where((idx_np >= 0) & (idx_np < n), idx_np, -1).astype(np.int32)
    ref_o, ref_l = orc.sparse_attention(q.numpy(), K.numpy(), V.numpy(), clean, group,
                                        float(np.float32(s)))
    got_o, got_l = out.cpu().numpy(), lse.cpu().numpy()
    G = hq // hkv
    Kn = np.abs(K.numpy().astype(np.float64))
    Vn = V.numpy().astype(np.float64)
    for h in range(hq):
        row = clean[h // group]
        sel = row[row >= 0]
        if sel.size == 0:
            assert np.all(got_o[h] == 0) and np.isneginf(got_l[h]), h
            continue
        eps = abs(s) * (d + 2) * 2.0 ** -24 * float(
            (Kn[sel, h // G, :] @ np.abs(q[h].numpy().astype(np.float64))).max())
        vmax = float(np.abs(Vn[sel, h // G, :]).max())
        err_o = float(np.abs(got_o[h].astype(np.float64) - ref_o[h]).max())
        assert err_o <= (2.5 * eps + 1e-5) * vmax, (h, err_o, eps, vmax)
        err_l = abs(float(got_l[h]) - float(ref_l[h]))
        assert err_l <= 1.5 * eps + 1e-6 * max(1.0, abs(float(ref_l[h]))), (h, err_l, eps)
    return out, lse


def rand_idx(seed, rows, k, n, pad=0):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(n, k, replace=False) for _ in range(rows)]).astype(np.int32)
    if pad:
        idx[:, -pad:] = -1
    return torch.from_numpy(idx)


@pytest.mark.parametrize("k", [1, 63, 64, 65, 255, 256, 257, 1000, 2048, 2500])
def test_attention_per_head_fp16(F, orc, k):
    K, V = caches(k, 5000, 2, torch.float16)
    q = torch.randn((8, 128), generator=torch.Generator().manual_seed(k))
    check(F, orc, q, K, V, rand_idx(k, 8, k, 5000), 1)


@pytest.mark.parametrize("k,group,dtype", [(9000, 1, torch.float16), (12345, 2, torch.float32)])
def test_attention_long_rows(F, orc, k, group, dtype):
    """Rows above 8192 entries: 64 entries per wave, more than one batch of
    block partials to merge."""
    n = 20000
    K, V = caches(k, n, 2, dtype)
    q = torch.randn((4, 128), generator=torch.Generator().manual_seed(k))
    check(F, orc, q, K, V, rand_idx(k, 4 // group, k, n, pad=100), group)


@pytest.mark.parametrize("group,hq,hkv", [(2, 8, 2), (4, 8, 2), (8, 16, 2), (4, 32, 8)])
def test_attention_groups(F, orc, group, hq, hkv):
    K, V = caches(group * 10 + hq, 7000, hkv, torch.float16)
    q = torch.randn((hq, 128), generator=torch.Generator().manual_seed(group))
    check(F, orc, q, K, V, rand_idx(group, hq // group, 700, 7000, pad=33), group)


@pytest.mark.parametrize("group", [1, 4])
def test_attention_fp32_caches(F, orc, group):
    K, V = caches(31, 3000, 2, torch.float32)
    q = torch.randn((8, 128), generator=torch.Generator().manual_seed(3))
    check(F, orc, q, K, V, rand_idx(7, 8 // group, 333, 3000, pad=5), group, scale=0.05)


def test_attention_strided_and_pinned_caches(F, orc):
    n, hkv = 4000, 2
    big = torch.randn((n, hkv, 256), generator=torch.Generator().manual_seed(5)).half()
    K, V = big[:, :, :128], big[:, :, 128:]          # stride_tok 512, stride_head 256
    q = torch.randn((8, 128), generator=torch.Generator().manual_seed(6))
    idx = rand_idx(8, 8, 500, n)
    bd = big.to(dev())
    o1, l1 = check(F, orc, q, K.contiguous(), V.contiguous(), idx, 1,
                   Kd=bd[:, :, :128], Vd=bd[:, :, 128:], tag="strided")
    hb = torch.empty(big.shape, dtype=big.dtype, pin_memory=True)
    hb.copy_(big)
    o2, l2 = F.sparse_attention(q.to(dev()), hb[:, :, :128], hb[:, :, 128:], idx.to(dev()), 1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_attention_out_of_range_duplicates_and_empty_rows(F, orc):
    n = 2000
    K, V = caches(9, n, 2, torch.float16)
    q = torch.randn((8, 128), generator=torch.Generator().manual_seed(9))
    idx = rand_idx(9, 8, 300, n)
    idx[0, 10:20] = n + 5                              # skipped like padding
    idx[1, 7] = idx[1, 8]                              # listed twice counts twice
    idx[2, :] = -1                                     # no key at all
    idx[3, 100:] = 2 ** 31 - 1
    check(F, orc, q, K, V, idx, 1)
    out, lse = F.sparse_attention(q.to(dev()), K.to(dev()), V.to(dev()),
                                  torch.zeros((8, 0), dtype=torch.int32, device=dev()), 1)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_attention_is_deterministic(F):
    K, V = caches(11, 3000, 2, torch.float16)
    q = torch.randn((8, 128), generator=torch.Generator().manual_seed(11)).to(dev())
    idx = rand_idx(11, 8, 1024, 3000).to(dev())
    a = F.sparse_attention(q, K.to(dev()), V.to(dev()), idx)
    b = F.sparse_attention(q, K.to(dev()), V.to(dev()), idx)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("group", [1, 4])
def test_attention_after_scan_topk_1m_layer(F, orc, group):
    """The decode step at its full size: the 1M-key layer's keys, its B = 92
    plans, fathom_scan_topk's indices (k = 2048), then attention over them."""
    w = synth.LAYER_1M
    keys = synth.keys(w.seed, 0, w.n, w.hkv, w.d, w.dtype, w.outliers, device=dev())
    vals = synth.keys(w.seed + 1, 0, w.n, w.hkv, w.d, w.dtype, 0, device=dev())
    q = synth.queries(w.seed, 0, w.hq, w.d, device=dev())
    p = F.pack(keys)
    plan = F.plan(q, p.sigma2, w.budget)
    idx, _ = F.scan_topk(p.planes, p.lo, p.hi, w.n, q, plan, w.k, group)
    torch.cuda.synchronize()
    # only the selected rows travel to the oracle: remap them to 0..m-1
    sel = torch.unique(idx[idx >= 0])
    remap = torch.full((w.n,), -1, dtype=torch.int64, device=dev())
    remap[sel] = torch.arange(sel.numel(), device=dev())
    small_idx = remap[idx.long()].to(torch.int32).cpu()
    Ks, Vs = keys[sel].cpu(), vals[sel].cpu()
    out, lse = F.sparse_attention(q, keys, vals, idx, group)
    torch.cuda.synchronize()
    o2, l2 = check(F, orc, q.cpu(), Ks, Vs, small_idx, group, tag="1M layer")
    assert torch.equal(out, o2) and torch.equal(lse, l2)
