"""GPU parity: fathom_pack (planes, lo, hi, sigma2) and fathom_plan /
fathom_plan_fixed, bit-exact against the CPU oracle on identical inputs."""
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


def planes_u32(t):
    return t.cpu().numpy().view(np.uint32)


def check_pack(F, orc, keys):
    print(f"pack case n={keys.shape[0]} hkv={keys.shape[1]} dtype={keys.dtype}", flush=True)
    p = F.pack(keys)
    torch.cuda.synchronize()
    ref = orc.pack(keys.cpu().numpy())
    np.testing.assert_array_equal(p.lo.cpu().numpy(), ref["lo"])
    np.testing.assert_array_equal(p.hi.cpu().numpy(), ref["hi"])
    np.testing.assert_array_equal(planes_u32(p.planes), ref["planes"])
    np.testing.assert_array_equal(p.sigma2.cpu().numpy(), ref["sigma2"])
    return p, ref


@pytest.mark.parametrize("n,hkv,dtype", [
    (4096, 1, torch.float32),     # single-head parity workload
    (1, 1, torch.float16),
    (31, 2, torch.float16),
    (33, 1, torch.float32),
    (64, 1, torch.float16),
    (2048, 1, torch.float16),
    (2049, 3, torch.float16),
    (20000, 8, torch.float16),
])
def test_pack_bit_exact(F, orc, n, hkv, dtype):
    keys = synth.keys(11, n, n, hkv, 128, dtype, 4 if hkv > 1 else 0, device=dev())
    check_pack(F, orc, keys)


def test_pack_qwen_layer_131072(F, orc):
    w = synth.LAYER_128K
    keys = synth.keys(w.seed, 0, w.n, w.hkv, w.d, w.dtype, w.outliers, device=dev())
    check_pack(F, orc, keys)


def test_pack_strided_keys(F, orc):
    # keys as a view into a [n][hkv][256] buffer (token and head strides != dense)
    big = synth.keys(12, 0, 3000, 4, 256, torch.float16, 0, device=dev())
    keys = big[:, :, 64:192]
    assert keys.stride() == (1024, 256, 1)
    p = F.pack(keys)
    torch.cuda.synchronize()
    ref = orc.pack(keys.cpu().numpy())
    np.testing.assert_array_equal(planes_u32(p.planes), ref["planes"])
    np.testing.assert_array_equal(p.sigma2.cpu().numpy(), ref["sigma2"])


def test_pack_unaligned_strides_and_offset(F, orc):
    # rows that are not 16-byte aligned take the scalar kernels
    for dtype in (torch.float16, torch.float32):
        big = synth.keys(15, 0, 2100, 3, 131, dtype, 0, device=dev())
        keys = big[:, :, 1:129]
        assert keys.stride() == (393, 131, 1)
        check_pack(F, orc, keys)


def test_pack_cell_boundaries(F, orc):
    """Keys on and next to the quantiser's cell edges: the codes of values
    whose quotient (x - lo) / delta is an integer, or one ulp away from it,
    are decided by the correctly rounded divide."""
    n = 4096
    keys = synth.keys(16, 0, n, 2, 128, torch.float32, 0, device=dev())
    grid = torch.arange(n, device=dev(), dtype=torch.float32) % 65 * 0.25  # lo 0, hi 16: delta 1
    keys[:, 0, 0] = grid
    keys[:, 0, 1] = torch.nextafter(grid, torch.full_like(grid, 100.0))
    keys[:, 0, 2] = torch.nextafter(grid, torch.full_like(grid, -100.0))
    keys[0, 0, 1:3] = 0.0
    keys[1, 0, 1:3] = 16.0
    keys[:, 1, 3] = torch.arange(n, device=dev(), dtype=torch.float32) % 17 * 0.1 - 0.7
    keys[:, 1, 4] = torch.arange(n, device=dev(), dtype=torch.float32) % 33 * (1.0 / 3.0)
    check_pack(F, orc, keys)


def test_pack_every_fp16_value(F, orc):
    """Each channel holds every finite fp16 value of its own range
    [-lim*(1 + c%3), lim] (lim a power of two that varies with the channel),
    shuffled and repeated; bit-exact against the oracle."""
    bits = torch.arange(65536, dtype=torch.int32)
    vals = bits.to(torch.int16).view(torch.float16)
    vals = vals[torch.isfinite(vals)]
    g = torch.Generator().manual_seed(17)
    cols = []
    for c in range(128):
        lim = float(2.0 ** (c % 17 - 8))
        v = vals[(vals.float() >= -lim * (1 + c % 3)) & (vals.float() <= lim)]
        v = v[torch.randperm(v.numel(), generator=g)]
        reps = -(-vals.numel() // v.numel())
        cols.append(v.repeat(reps)[:vals.numel()])
    keys = torch.stack(cols, dim=1).view(vals.numel(), 1, 128).to(dev())
    check_pack(F, orc, keys)


def test_pack_degenerate_channels(F, orc):
    n = 5000
    keys = synth.keys(13, 0, n, 2, 128, torch.float32, 0, device=dev())
    keys[:, 0, 0] = 3.25                      # constant channel
    keys[:, 0, 1] = 0.0
    keys[::2, 0, 1] = -0.0                    # +-0 only
    keys[:, 1, 5] = -1.0
    keys[1234, 1, 5] = 7.0                    # single outlier: codes 0 and 15
    keys[:, 1, 6] = torch.linspace(-2, 2, n)  # evenly spread
    p, ref = check_pack(F, orc, keys)
    assert ref["sigma2"][0, 0] == 0 and np.signbit(p.lo.cpu().numpy()[0, 1]) == 0


def test_pack_full_size_sampled_channels(F, orc):
    w = synth.LAYER_1M
    keys = synth.keys(w.seed, 0, w.n, w.hkv, w.d, w.dtype, w.outliers, device=dev())
    p = F.pack(keys)
    torch.cuda.synchronize()
    for h, c0 in [(0, 0), (3, 60), (7, 120)]:
        sub = keys[:, h:h + 1, c0:c0 + 8].contiguous().cpu().numpy()
        ref = orc.pack(sub)
        np.testing.assert_array_equal(planes_u32(p.planes[h, c0:c0 + 8]), ref["planes"][0])
        np.testing.assert_array_equal(p.sigma2[h, c0:c0 + 8].cpu().numpy(), ref["sigma2"][0])
        np.testing.assert_array_equal(p.lo[h, c0:c0 + 8].cpu().numpy(), ref["lo"][0])


@pytest.mark.parametrize("hq,hkv", [(32, 8), (1, 1), (8, 1), (96, 8)])
@pytest.mark.parametrize("budget", [0, 1, 3, 18, 68, 91, 92, 136, 511, 512, "random"])
def test_plan_bit_exact(F, orc, hq, hkv, budget):
    rng = np.random.default_rng(hq * 1000 + (budget if isinstance(budget, int) else 7))
    q = rng.standard_normal((hq, 128)).astype(np.float32)
    s2 = np.exp(rng.uniform(np.log(0.01), np.log(256), (hkv, 128))).astype(np.float32)
    s2[:, :3] = 0.0
    B = (rng.integers(0, 513, hq).astype(np.int32) if budget == "random"
         else np.full(hq, budget, np.int32))
    got = F.plan(torch.from_numpy(q).to(dev()), torch.from_numpy(s2).to(dev()), B.tolist())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), orc.plan(q, s2, B))


def test_plan_ties_and_sigma_from_pack(F, orc):
    q = np.ones((4, 128), np.float32)
    q[1, ::3] = -1.0
    q[2, :] = 0.0
    s2 = np.ones((1, 128), np.float32)
    got = F.plan(torch.from_numpy(q).to(dev()), torch.from_numpy(s2).to(dev()), [10, 37, 92, 5])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), orc.plan(q, s2, [10, 37, 92, 5]))
    keys = synth.keys(14, 0, 9000, 8, 128, torch.float16, 4, device=dev())
    p = F.pack(keys)
    qq = synth.queries(14, 0, 32, 128, device=dev())
    got = F.plan(qq, p.sigma2, 92)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(),
                                  orc.plan(qq.cpu().numpy(), p.sigma2.cpu().numpy(), 92))


@pytest.mark.parametrize("r", [0, 1, 16, 32, 127, 128])
def test_plan_fixed_bit_exact(F, orc, r):
    rng = np.random.default_rng(r)
    q = rng.standard_normal((32, 128)).astype(np.float32)
    q[0, :8] = q[0, 8:16]                      # ties in |q|
    q[1, ::2] = -q[1, 1::2]
    got = F.plan_fixed(torch.from_numpy(q).to(dev()), r)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), orc.plan_fixed(q, r))


def test_plan_is_deterministic(F):
    q = synth.queries(15, 0, 32, 128, device=dev())
    s2 = torch.rand((8, 128), device=dev())
    a = F.plan(q, s2, 92)
    b = F.plan(q, s2, 92)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
