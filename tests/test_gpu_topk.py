"""GPU parity of fathom_topk: bit-exact (indices, scores and order) against
the oracle's full sort on the same fp32 scores, per row and per GQA group,
through the sampled-threshold path and through the exact fallback."""
import numpy as np
import pytest
import torch

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


def check(F, orc, S, k, group=1):
    rows, n = S.shape
    print(f"topk case rows={rows} n={n} k={k} group={group}", flush=True)
    St = torch.from_numpy(np.ascontiguousarray(S)).to(dev())
    idx, vals = F.topk(St, k, group=group)
    torch.cuda.synchronize()
    ridx, rvals = orc.topk(S, k, group)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_array_equal(vals.cpu().numpy().view(np.uint32), rvals.view(np.uint32))


@pytest.mark.parametrize("n", [1, 63, 4096, 8192, 8193, 50000, 200001])
@pytest.mark.parametrize("k", [1, 64, 1024, 2048])
def test_topk_rows(F, orc, n, k):
    rng = np.random.default_rng(n + k)
    S = rng.standard_normal((3, n)).astype(np.float32)
    check(F, orc, S, k)


@pytest.mark.parametrize("n,k", [(100000, 1024), (9000, 2048), (3000, 64)])
def test_topk_groups(F, orc, n, k):
    rng = np.random.default_rng(n)
    S = (rng.standard_normal((8, n)) * rng.uniform(0.5, 3, (8, 1))).astype(np.float32)
    check(F, orc, S, k, group=4)


def test_topk_heavy_ties(F, orc):
    rng = np.random.default_rng(1)
    S = np.round(rng.standard_normal((4, 60000)) * 2).astype(np.float32)   # few values
    S[0, ::7] = -0.0
    S[1, :] = 0.0
    check(F, orc, S, 2048)
    check(F, orc, S, 1000)


def test_topk_bucket_overflow_sorts(F, orc):
    """One outlier far above a tight cluster of distinct scores: the binning
    window starts in the exponent bits, the cluster fills one bucket far
    beyond the exact-ranking cap, and the radix select plus sort decides."""
    rng = np.random.default_rng(4)
    S = (1.0 + rng.uniform(0, 1e-3, (3, 6000))).astype(np.float32)
    S[:, 17] = 1e6
    S[1, 100:200] = S[1, 300]                         # ties inside the cluster as well
    check(F, orc, S, 2048)
    check(F, orc, S, 700)


@pytest.mark.parametrize("n", [7000, 300000])
def test_topk_cluster_bucket_above_kth(F, orc, n):
    """1,500 distinct scores in a tiny range far above the rest (top keys
    clustered in one stretch of the row): among the winners they fill one
    bucket beyond the exact-ranking cap, strictly above the k-th word's
    bucket, which is then sorted on its own; with ties inside the cluster,
    per row and per GQA group."""
    rng = np.random.default_rng(n)
    S = rng.standard_normal((4, n)).astype(np.float32)
    at = rng.integers(0, n - 1500, 4)
    for r in range(4):
        S[r, at[r]:at[r] + 1500] = (40.0 + rng.uniform(0, 1e-4, 1500)).astype(np.float32)
    S[2, at[2] + 50:at[2] + 90] = S[2, at[2] + 7]     # ties inside the cluster
    check(F, orc, S, 2048)
    check(F, orc, S, 1800)
    check(F, orc, S, 2048, group=2)


def test_topk_all_equal_takes_lowest_indices(F, orc):
    S = np.full((2, 30000), 1.5, np.float32)            # forces the exact fallback
    check(F, orc, S, 2048)


def test_topk_sample_misses_forces_fallback(F, orc):
    """Large scores placed only where the threshold sample does not look: the
    sampled threshold is far too high or too low, and the exact path decides."""
    n = 300000
    stride = (n * 64 + 16383) // 16384
    stride = (stride + 63) // 64 * 64
    pos = np.arange(n)
    unsampled = (pos % stride) >= 64
    rng = np.random.default_rng(2)
    S = rng.standard_normal((2, n)).astype(np.float32)
    S[0, unsampled] += 50.0          # every big score hides from the sample
    S[1, ~unsampled] += 50.0         # the sample sees only big scores
    check(F, orc, S, 2048)
    check(F, orc, S, 5)


def test_topk_short_rows_pad(F, orc):
    rng = np.random.default_rng(3)
    S = rng.standard_normal((2, 10)).astype(np.float32)
    check(F, orc, S, 64)
    check(F, orc, S[:, :1], 3)


def test_topk_strided_rows(F, orc):
    rng = np.random.default_rng(4)
    big = rng.standard_normal((4, 70001)).astype(np.float32)
    St = torch.from_numpy(big).to(dev())[:, :70000]
    idx, vals = F.topk(St, 512)
    torch.cuda.synchronize()
    ridx, rvals = orc.topk(big[:, :70000], 512)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_array_equal(vals.cpu().numpy(), rvals)


def test_topk_empty_rows(F):
    St = torch.zeros((2, 4), device=dev())
    idx, vals = F.topk(St, 8, n=0)
    torch.cuda.synchronize()
    assert torch.all(idx == -1) and torch.all(torch.isneginf(vals))
