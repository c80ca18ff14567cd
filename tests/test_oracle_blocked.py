"""Pins of the oracle's per-block ranges (reading R22: one (lo, hi) per
2048-key block of a channel instead of one per layer).  Each pin compares the
oracle with something computed independently here from the raw keys (numpy's
own min/max, quantiser, variance and dot products), or with the per-layer
oracle where the two definitions must agree exactly:

  * a layer of one block is packed and scanned exactly as with per-layer
    ranges (planes, lo, hi, sigma2, logits bit for bit);
  * every block's codes are the 16-cell quantiser of that block's own min and
    max, and its top t planes are that block's t-bit quantiser;
  * sigma2 is the pooled within-block variance of the dequantised values;
  * when every block has the layer's range, the blocked layer equals the
    per-layer one;
  * scores are sum_c q_c (lo_b + (prefix + 1/2) cell_b) of each key's block;
  * append: keys inside an existing block's range equal packing the whole
    sequence; a block the append starts takes the previous block's range
    widened to its new keys (nothing clamps there); keys outside an existing
    block's range clamp and are counted; no other bit changes."""
import numpy as np
import pytest

from test_oracle import t_bit_quantizer, unpack_planes_vectorised

RB = 2048


def np_block_codes(x, lo, hi):
    """Independent fp32 16-cell quantiser of values x with range [lo, hi]."""
    x = np.asarray(x, np.float32)
    lo, hi = np.float32(lo), np.float32(hi)
    delta = np.float32(np.float32(hi - lo) * np.float32(0.0625))
    if delta == 0:
        return np.zeros(x.shape, np.int64)
    y = (x - lo) / delta
    return np.clip(np.floor(y.astype(np.float64)), 0, 15).astype(np.int64)


def keys_for(seed, n, hkv=2, d=8, drift=0.0):
    rng = np.random.default_rng(seed)
    sig = np.exp(rng.uniform(np.log(0.1), np.log(4.0), (hkv, d)))
    z = rng.standard_normal((n, hkv, d))
    # ranges that drift along the sequence, as in a growing session
    ramp = 1.0 + drift * np.arange(n)[:, None, None] / max(n, 1)
    return (z * sig[None] * ramp).astype(np.float16).astype(np.float32)


@pytest.mark.parametrize("n", [1, 5, 300, 2047, 2048])
def test_one_block_is_the_per_layer_pack(orc, n):
    k = keys_for(1, n)
    a = orc.pack(k)
    b = orc.pack_blocked(k)
    np.testing.assert_array_equal(b["planes"], a["planes"])
    np.testing.assert_array_equal(b["lo"][:, 0], a["lo"])
    np.testing.assert_array_equal(b["hi"][:, 0], a["hi"])
    np.testing.assert_array_equal(b["sigma2"], a["sigma2"])


@pytest.mark.parametrize("n", [2049, 5000, 3 * RB + 7])
def test_block_codes_are_the_block_quantiser(orc, n):
    k = keys_for(2, n, drift=3.0)
    b = orc.pack_blocked(k)
    codes = unpack_planes_vectorised(b["planes"], n)
    hkv, d = k.shape[1:]
    for h in range(hkv):
        for c in range(d):
            for blk in range(-(-n // RB)):
                x = k[blk * RB:(blk + 1) * RB, h, c]
                lo, hi = np.float32(x.min() + 0), np.float32(x.max() + 0)
                assert b["lo"][h, blk, c] == lo and b["hi"][h, blk, c] == hi
                np.testing.assert_array_equal(codes[h, c, blk * RB:(blk + 1) * RB],
                                              np_block_codes(x, lo, hi))
    # padding bits stay zero
    W = b["planes"].shape[-1]
    if n < W * 32:
        tail = unpack_planes_vectorised(b["planes"], W * 32)[:, :, n:]
        assert not tail.any()


def test_block_prefix_invariant(orc):
    n = 2 * RB + 100
    k = keys_for(3, n, drift=2.0)
    b = orc.pack_blocked(k)
    codes = unpack_planes_vectorised(b["planes"], n)
    for t in range(5):
        for blk in range(3):
            x = k[blk * RB:(blk + 1) * RB, 0, 3]
            lo, hi = b["lo"][0, blk, 3], b["hi"][0, blk, 3]
            want = t_bit_quantizer(x, lo, hi, t)
            got = codes[0, 3, blk * RB:(blk + 1) * RB] >> (4 - t)
            np.testing.assert_array_equal(got, want)


def test_sigma2_is_pooled_within_block_variance(orc):
    n = 2 * RB + 1000
    k = keys_for(4, n, drift=4.0)
    b = orc.pack_blocked(k)
    codes = unpack_planes_vectorised(b["planes"], n)
    hkv, d = k.shape[1:]
    for h in range(hkv):
        for c in range(d):
            tot = 0.0
            for blk in range(3):
                lo, hi = np.float64(b["lo"][h, blk, c]), np.float64(b["hi"][h, blk, c])
                delta = np.float64(np.float32(np.float32(hi - lo) * np.float32(0.0625)))
                cb = codes[h, c, blk * RB:(blk + 1) * RB].astype(np.float64)
                deq = lo + (cb + 0.5) * delta
                tot += np.var(deq) * (cb.size / n)      # two-pass population variance
            assert abs(b["sigma2"][h, c] - tot) <= 1e-6 * tot + 1e-30


def test_blocks_with_the_layer_range_equal_the_per_layer_layer(orc):
    n = 3 * RB + 17
    k = keys_for(5, n)
    # every block holds the layer's extremes of every channel
    mn, mx = k.min(0), k.max(0)
    for blk in range(4):
        k[blk * RB] = mn
        k[blk * RB + 1] = mx
    a = orc.pack(k)
    b = orc.pack_blocked(k)
    np.testing.assert_array_equal(b["planes"], a["planes"])
    for blk in range(4):
        np.testing.assert_array_equal(b["lo"][:, blk], a["lo"])
        np.testing.assert_array_equal(b["hi"][:, blk], a["hi"])
    rng = np.random.default_rng(6)
    q = rng.standard_normal((4, 8)).astype(np.float32)
    plan = orc.plan(q, a["sigma2"], 14)
    np.testing.assert_array_equal(orc.scan_blocked(b["planes"], b["lo"], b["hi"], n, q, plan),
                                  orc.scan(a["planes"], a["lo"], a["hi"], n, q, plan))


@pytest.mark.parametrize("B", [0, 5, 18, 32])
def test_one_block_scan_is_the_per_layer_scan(orc, B):
    n = 1500
    k = keys_for(7, n)
    a = orc.pack(k)
    b = orc.pack_blocked(k)
    rng = np.random.default_rng(B)
    q = rng.standard_normal((4, 8)).astype(np.float32)
    plan = orc.plan(q, a["sigma2"], B)
    np.testing.assert_array_equal(orc.scan_blocked(b["planes"], b["lo"], b["hi"], n, q, plan),
                                  orc.scan(a["planes"], a["lo"], a["hi"], n, q, plan))


@pytest.mark.parametrize("B", [5, 18, 32])
def test_blocked_scan_is_the_t_bit_reconstruction_of_the_raw_keys(orc, B):
    n = 2 * RB + 333
    k = keys_for(8, n, drift=3.0)
    b = orc.pack_blocked(k)
    rng = np.random.default_rng(100 + B)
    hkv, d = k.shape[1:]
    q = rng.standard_normal((4, d)).astype(np.float32)
    plan = orc.plan(q, b["sigma2"], B)
    got = orc.scan_blocked(b["planes"], b["lo"], b["hi"], n, q, plan)
    want = np.zeros((4, n))
    for h in range(4):
        g = h // 2
        for c in range(d):
            t = int(plan[h, c])
            for blk in range(3):
                sl = slice(blk * RB, min((blk + 1) * RB, n))
                lo, hi = b["lo"][g, blk, c], b["hi"][g, blk, c]
                delta = np.float64(np.float32(np.float32(hi - lo) * np.float32(0.0625)))
                r = t_bit_quantizer(k[sl, g, c], lo, hi, t)     # from the raw keys
                cell = delta * 2.0 ** (4 - t)
                want[h, sl] += np.float64(q[h, c]) * (np.float64(lo) + (r + 0.5) * cell)
    # the oracle rounds an fp64 sum once; the sums differ only in order
    np.testing.assert_allclose(got, want.astype(np.float32), rtol=3e-7, atol=1e-6)
    # scan_at at sampled keys equals the full scan
    pick = np.array([0, 1, RB - 1, RB, 2 * RB + 5, n - 1])
    np.testing.assert_array_equal(
        orc.scan_blocked_at(b["planes"], b["lo"], b["hi"], n, q, plan, pick), got[:, pick])


def fresh(orc, k, n0, n_cap):
    """Blocked pack of the first n0 keys into planes of capacity n_cap keys and
    ranges of capacity ceil(n_cap / 2048) blocks."""
    p = orc.pack_blocked(k[:n0])
    hkv, d = k.shape[1:]
    W = orc.plane_words(n_cap)
    planes = np.zeros((hkv, d, 4, W), np.uint32)
    planes[..., :p["planes"].shape[-1]] = p["planes"]
    nbc = -(-n_cap // RB)
    lo = np.zeros((hkv, nbc, d), np.float32)
    hi = np.zeros((hkv, nbc, d), np.float32)
    lo[:, :p["lo"].shape[1]] = p["lo"]
    hi[:, :p["hi"].shape[1]] = p["hi"]
    return planes, lo, hi


@pytest.mark.parametrize("n0,n", [(1000, 1500), (2100, 4000), (RB + 2, 2 * RB)])
def test_append_inside_the_block_range_equals_the_pack_of_all(orc, n0, n):
    k = keys_for(9, n)
    # the extremes of the last block appear among its first n0 keys
    blk = (n0 - 1) // RB
    b0 = blk * RB
    seg = k[b0:n]
    k[b0] = seg.min(0)
    k[b0 + 1] = seg.max(0)
    planes, lo, hi = fresh(orc, k, n0, n)
    assert orc.append_blocked(k[n0:], n0, planes, lo, hi) == 0
    full = orc.pack_blocked(k)
    np.testing.assert_array_equal(planes, full["planes"])
    np.testing.assert_array_equal(lo, full["lo"])
    np.testing.assert_array_equal(hi, full["hi"])


def test_append_new_blocks_inherit_and_widen_the_previous_range(orc):
    n0, n = 2 * RB - 10, 4 * RB + 50
    k = keys_for(10, n, drift=5.0)          # later keys outgrow earlier ranges
    planes, lo, hi = fresh(orc, k, n0, n)
    lo_before, hi_before = lo.copy(), hi.copy()
    clamped = orc.append_blocked(k[n0:], n0, planes, lo, hi)
    codes = unpack_planes_vectorised(planes, n)
    hkv, d = k.shape[1:]
    want_clamped = 0
    for h in range(hkv):
        for c in range(d):
            # block 1 existed: its range is kept and its new keys clamp
            l1, h1 = lo_before[h, 1, c], hi_before[h, 1, c]
            assert lo[h, 1, c] == l1 and hi[h, 1, c] == h1
            x = k[n0:2 * RB, h, c]
            want_clamped += int(((x < l1) | (x > h1)).sum())
            np.testing.assert_array_equal(codes[h, c, n0:2 * RB], np_block_codes(x, l1, h1))
            # blocks 2.. are new: previous range widened to cover their keys
            pl, ph = l1, h1
            for blk in range(2, 5):
                x = k[blk * RB:min((blk + 1) * RB, n), h, c]
                nl = np.float32(min(pl, x.min()) + 0)
                nh = np.float32(max(ph, x.max()) + 0)
                assert lo[h, blk, c] == nl and hi[h, blk, c] == nh
                np.testing.assert_array_equal(codes[h, c, blk * RB:blk * RB + x.size],
                                              np_block_codes(x, nl, nh))
                pl, ph = nl, nh
    assert clamped == want_clamped


def test_append_block_zero_takes_its_own_range(orc):
    n = 700
    k = keys_for(11, n)
    hkv, d = k.shape[1:]
    planes = np.zeros((hkv, d, 4, orc.plane_words(n)), np.uint32)
    lo = np.zeros((hkv, 1, d), np.float32)
    hi = np.zeros((hkv, 1, d), np.float32)
    assert orc.append_blocked(k, 0, planes, lo, hi) == 0
    full = orc.pack_blocked(k)
    np.testing.assert_array_equal(planes, full["planes"])
    np.testing.assert_array_equal(lo, full["lo"])
    np.testing.assert_array_equal(hi, full["hi"])


def test_append_one_token_at_a_time_equals_one_call_inside_the_range(orc):
    n0, n = 500, 2 * RB + 300
    k = keys_for(12, n)
    # every later key lies inside the first 500 keys' range
    k[n0:] = np.clip(k[n0:], k[:n0].min(0), k[:n0].max(0))
    p1, l1, h1 = fresh(orc, k, n0, n)
    p2, l2, h2 = fresh(orc, k, n0, n)
    assert orc.append_blocked(k[n0:], n0, p1, l1, h1) == 0
    for j in range(n0, n):
        assert orc.append_blocked(k[j:j + 1], j, p2, l2, h2) == 0
    np.testing.assert_array_equal(p1, p2)
    np.testing.assert_array_equal(l1, l2)
    np.testing.assert_array_equal(h1, h2)


def test_append_leaves_every_other_bit_alone(orc):
    n0, m = 3000, 1200
    k = keys_for(13, n0 + m, drift=2.0)
    planes, lo, hi = fresh(orc, k, n0, n0 + m)
    rng = np.random.default_rng(14)
    planes[:] = rng.integers(0, 2 ** 32, planes.shape, dtype=np.uint64).astype(np.uint32)
    before = unpack_planes_vectorised(planes, planes.shape[-1] * 32)
    orc.append_blocked(k[n0:], n0, planes, lo, hi)
    after = unpack_planes_vectorised(planes, planes.shape[-1] * 32)
    np.testing.assert_array_equal(after[:, :, :n0], before[:, :, :n0])
    np.testing.assert_array_equal(after[:, :, n0 + m:], before[:, :, n0 + m:])


def test_blocked_rejects_bad_arguments(orc):
    k = keys_for(15, 3000)
    with pytest.raises(ValueError):
        orc.pack_blocked(k, nbc=1)                  # two blocks need two range slots
    b = orc.pack_blocked(k)
    q = np.ones((2, 8), np.float32)
    plan = np.zeros((2, 8), np.uint8)
    with pytest.raises(ValueError):
        orc.scan_blocked(b["planes"], b["lo"][:, :1], b["hi"][:, :1], 3000, q, plan)
