"""GPU checks of the measurement probes: the streaming-read probe and the
scan-traffic probe run on device and pinned-host buffers, and the scan-traffic
probe writes exactly the output rows and keys it covers (its values carry no
meaning), for any depth table, including depths above 4, which it clamps."""
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


@pytest.mark.parametrize("pinned", [False, True])
def test_probe_read_runs(F, pinned):
    n = 1 << 20
    buf = torch.empty(n, dtype=torch.int32, pin_memory=True) if pinned else \
        torch.empty(n, dtype=torch.int32, device=dev())
    buf.fill_(7)
    sink = torch.zeros(1, dtype=torch.int32, device=dev())
    F.probe_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


@pytest.mark.parametrize("n,hkv,rows_out", [(2048, 1, 1), (8192, 2, 4), (6144, 3, 16),
                                            (1 << 16, 8, 4), (4096, 2, 0)])
def test_scan_traffic_probe_writes_its_rows_only(F, n, hkv, rows_out):
    print(f"scan-traffic probe n={n} hkv={hkv} rows_out={rows_out}", flush=True)
    rng = np.random.default_rng(n + hkv)
    W = n // 32
    planes = torch.randint(-2**31, 2**31 - 1, (hkv, 128, 4, W), dtype=torch.int32, device=dev())
    depth = torch.from_numpy(rng.integers(0, 6, (hkv, 128)).astype(np.uint8))
    depth[0, :3] = 255  # clamped to 4
    depth = depth.to(dev())
    ld = n + 64
    out = torch.full((max(hkv * rows_out, 1) + 1, ld), float("nan"), device=dev())
    sink = torch.zeros(1, dtype=torch.int32, device=dev())
    F.probe_scan_traffic(planes, n, depth, rows_out, out if rows_out else None, sink)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    rows = hkv * rows_out
    assert np.isfinite(o[:rows, :n]).all()
    assert np.isnan(o[:rows, n:]).all()
    assert np.isnan(o[rows:]).all()


def test_scan_traffic_probe_rejects_bad_sizes(F):
    planes = torch.zeros((1, 128, 4, 64), dtype=torch.int32, device=dev())
    depth = torch.zeros((1, 128), dtype=torch.uint8, device=dev())
    sink = torch.zeros(1, dtype=torch.int32, device=dev())
    with pytest.raises(F.FathomError):
        F.probe_scan_traffic(planes, 2000, depth, 0, None, sink)
