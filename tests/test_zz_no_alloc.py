"""fathom_topk_noalloc (the top-k entry point that allocates nothing: its
workspace is a static device array in the library) against fathom_topk with a
caller workspace, through the C ABI: bit-identical indices and scores on two
calls in a row, the second with a smaller input, then on a group call; and
the host-side rejection of more output rows than the array holds."""
import ctypes

import numpy as np
import pytest
import torch

import sparse_top_key_amd as fathom

pytestmark = pytest.mark.gpu


def _noalloc(scores, rows, n, group, k):
    L = fathom.lib()
    ro = rows // group
    idx = torch.full((ro, k), 7, dtype=torch.int32, device="cuda")
    vals = torch.full((ro, k), 7.0, dtype=torch.float32, device="cuda")
    ld = scores.stride(0)
    rc = L.fathom_topk_noalloc(ctypes.c_void_p(scores.data_ptr()), rows, n, ld, group, k,
                               ctypes.c_void_p(idx.data_ptr()),
                               ctypes.c_void_p(vals.data_ptr()),
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, L.fathom_last_error().decode()
    return idx, vals


def _scores(seed, rows, n):
    g = torch.Generator(device="cuda").manual_seed(seed)
    s = torch.randn((rows, n), generator=g, device="cuda", dtype=torch.float32)
    # ties: a run of equal scores near the top of each row
    s[:, 100:140] = 3.5
    return s


@pytest.mark.parametrize("case", [
    # (rows, n, group, k): the second call is smaller than the first
    [(32, 300_000, 1, 2048), (8, 5_000, 1, 100)],
    [(64, 70_000, 1, 1024), (16, 9_000, 4, 64)],
])
def test_noalloc_equals_workspace_topk(case):
    print("noalloc cases", case, flush=True)
    for seed, (rows, n, group, k) in enumerate(case):
        s = _scores(11 + seed, rows, n)
        ref_idx, ref_vals = fathom.topk(s, k, group=group)
        idx, vals = _noalloc(s, rows, n, group, k)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), (rows, n, group, k)
        assert torch.equal(vals, ref_vals), (rows, n, group, k)
        # a valid top-k: sorted by (score desc, index asc), indices unique
        v = vals.cpu().numpy()
        i = idx.cpu().numpy()
        assert np.all(np.diff(v, axis=1) <= 0)
        for r in range(i.shape[0]):
            assert len(set(i[r].tolist())) == k


def test_noalloc_rejects_too_many_rows():
    L = fathom.lib()
    s = torch.zeros((65, 16), device="cuda")
    idx = torch.empty((65, 4), dtype=torch.int32, device="cuda")
    rc = L.fathom_topk_noalloc(ctypes.c_void_p(s.data_ptr()), 65, 16, 16, 1, 4,
                               ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(idx.data_ptr()),
                               None)
    assert rc == 4
    assert "exceed" in L.fathom_last_error().decode()
