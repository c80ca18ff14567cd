"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here touches the HIP path.  Each test checks the oracle against an
independent fact: the plane-prefix invariant of the storage side (the top t
planes of a channel are its t-bit quantiser), closed forms, brute force on
tiny inputs, the pages' worked budgets (tests/golden), and library sorts.
"""
import itertools
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# helpers written for the tests (independent of the oracle's code)

def top_planes_value(planes, W, h, c, i, t):
    """Value of the first t plane slots of (h, c) at key i, read MSB first."""
    v = 0
    for s in range(t):
        word = int(planes[h, c, s, i // 32])
        v = (v << 1) | ((word >> (i % 32)) & 1)
    return v


def t_bit_quantizer(x, lo, hi, t):
    """The t-bit min-max quantiser of x over [lo, hi] with 2^t equal cells,
    cell width (hi - lo) / 2^t, in fp32 (independent of the 4-bit code)."""
    x = np.asarray(x, np.float32)
    lo = np.float32(lo)
    hi = np.float32(hi)
    width = np.float32(np.float32(hi - lo) * np.float32(2.0 ** -t))
    if t == 0:
        return np.zeros(x.shape, np.int64)
    if width == 0:
        return np.zeros(x.shape, np.int64)
    y = np.floor((x - lo).astype(np.float32) / width)
    return np.minimum(y, 2 ** t - 1).astype(np.int64)


def all_finite_fp16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    return v[np.isfinite(v)]


def unpack_planes_vectorised(planes, n):
    """codes [hkv][d][n] rebuilt from planes [hkv][d][4][W] (slot 0 = MSB)."""
    hkv, d, _, W = planes.shape
    bits = np.unpackbits(planes.view(np.uint8).reshape(hkv, d, 4, W * 4),
                         axis=-1, bitorder="little")[..., :n]
    return (bits[:, :, 0] * 8 + bits[:, :, 1] * 4 + bits[:, :, 2] * 2
            + bits[:, :, 3]).astype(np.int64)


# --------------------------------------------------------------------------
# pack

def test_plane_prefix_invariant_exhaustive_fp16(orc):
    """Storage side: the first t planes of a channel equal the t-bit
    quantiser of that channel, for every finite fp16 key value."""
    x = all_finite_fp16().astype(np.float32)
    n = x.size
    keys = x.reshape(n, 1, 1)
    p = orc.pack(keys)
    planes = p["planes"]
    lo, hi = p["lo"][0, 0], p["hi"][0, 0]
    assert lo == x.min() and hi == x.max()
    codes = unpack_planes_vectorised(planes, n)[0, 0]
    for t in range(5):
        prefix = codes >> (4 - t) if t else np.zeros_like(codes)
        np.testing.assert_array_equal(prefix, t_bit_quantizer(x, lo, hi, t))


@pytest.mark.parametrize("seed", range(6))
def test_plane_prefix_invariant_random_ranges(orc, seed):
    """Same invariant on random sub-ranges of the fp16 values and on fp32
    samples, per channel, through the bit-by-bit top-plane reader."""
    rng = np.random.default_rng(seed)
    allv = all_finite_fp16().astype(np.float32)
    n, d = 300, 5
    cols = []
    for c in range(d):
        if c < 3:
            a, b = sorted(rng.integers(0, allv.size, 2))
            sub = np.sort(allv)[a:b + 2]
            cols.append(rng.choice(sub, n))
        else:
            cols.append((rng.standard_normal(n) * rng.uniform(0.01, 50))
                        .astype(np.float32))
    keys = np.stack(cols, axis=1).reshape(n, 1, d).astype(np.float32)
    p = orc.pack(keys)
    W = p["planes"].shape[-1]
    for c in range(d):
        lo, hi = p["lo"][0, c], p["hi"][0, c]
        for t in range(5):
            ref = t_bit_quantizer(keys[:, 0, c], lo, hi, t)
            got = [top_planes_value(p["planes"], W, 0, c, i, t) for i in range(n)]
            np.testing.assert_array_equal(got, ref)


def test_quantizer_properties(orc):
    rng = np.random.default_rng(7)
    n, hkv, d = 1000, 2, 16
    keys = (rng.standard_normal((n, hkv, d)) *
            rng.uniform(0.1, 4, (1, hkv, d))).astype(np.float16)
    p = orc.pack(keys)
    x = keys.astype(np.float64).transpose(1, 2, 0)      # [hkv][d][n]
    codes = p["codes"].astype(np.int64)
    assert codes.min() == 0 and codes.max() == 15
    lo = p["lo"].astype(np.float64)[..., None]
    hi = p["hi"].astype(np.float64)[..., None]
    np.testing.assert_array_equal(p["lo"], x.min(-1))
    np.testing.assert_array_equal(p["hi"], x.max(-1))
    delta = (hi - lo) / 16
    # min lands in cell 0, max in cell 15, codes monotone in x
    for h in range(hkv):
        for c in range(d):
            order = np.argsort(x[h, c], kind="stable")
            assert np.all(np.diff(codes[h, c][order]) >= 0)
            assert codes[h, c][order[0]] == 0 and codes[h, c][order[-1]] == 15
    # cell-centre reconstruction is within half a cell (plus fp32 slack)
    deq = lo + (codes + 0.5) * delta
    assert np.all(np.abs(x - deq) <= delta * (0.5 + 1e-5))
    # the planes hold exactly the codes
    np.testing.assert_array_equal(unpack_planes_vectorised(p["planes"], n), codes)
    # padding bits of the last word are zero
    W = p["planes"].shape[-1]
    assert W == 64 * ((n + 2047) // 2048)
    tail = p["planes"][..., n // 32 + 1:]
    assert np.all(tail == 0)
    last = p["planes"][..., n // 32]
    assert np.all((last >> np.uint32(n % 32)) == 0)


def test_constant_channel_and_single_key(orc):
    n = 70
    keys = np.zeros((n, 1, 3), np.float32)
    keys[:, 0, 0] = 2.5                          # constant channel
    keys[:, 0, 1] = np.linspace(-1, 1, n)
    keys[:, 0, 2] = -7.0
    keys[5, 0, 2] = 3.0                          # single distinct value
    p = orc.pack(keys)
    assert np.all(p["codes"][0, 0] == 0) and p["sigma2"][0, 0] == 0
    assert p["lo"][0, 0] == p["hi"][0, 0] == np.float32(2.5)
    assert p["codes"][0, 2, 5] == 15 and np.all(np.delete(p["codes"][0, 2], 5) == 0)
    one = orc.pack(np.array([[[1.25, -3.0]]], np.float32))
    assert np.all(one["codes"] == 0) and np.all(one["sigma2"] == 0)


def test_sigma2_is_variance_of_dequantised_values(orc):
    """sigma_c^2 equals a two-pass fp64 variance of lo + (code + 1/2) delta."""
    rng = np.random.default_rng(11)
    n, hkv, d = 3001, 2, 24
    keys = (rng.standard_normal((n, hkv, d)) * 3).astype(np.float16)
    p = orc.pack(keys)
    lo = p["lo"].astype(np.float64)
    delta = (p["hi"].astype(np.float32) - p["lo"].astype(np.float32)) * np.float32(0.0625)
    deq = lo[..., None] + (p["codes"] + 0.5) * delta.astype(np.float64)[..., None]
    mean = deq.mean(-1, keepdims=True)
    var = ((deq - mean) ** 2).mean(-1)
    np.testing.assert_allclose(p["sigma2"], var, rtol=2e-7, atol=0)
    # and it tracks the raw key variance to within the quantisation noise
    raw = keys.astype(np.float64).var(0)
    assert np.all(np.abs(p["sigma2"] - raw) <= 0.2 * raw + (delta.astype(np.float64) ** 2))


# --------------------------------------------------------------------------
# plan

def w_order(q, sigma2):
    w = (q.astype(np.float32) * q.astype(np.float32)).astype(np.float32) * sigma2
    return w


def test_plan_golden_worked_examples(orc):
    with open(os.path.join(GOLDEN, "plan_worked_examples.json")) as f:
        cases = json.load(f)["cases"]
    rng = np.random.default_rng(3)
    for case in cases:
        d, B = case["d"], case["budget"]
        sigma2 = rng.uniform(0.5, 2.0, (1, d)).astype(np.float32)
        q = rng.standard_normal((1, d)).astype(np.float32)
        w = w_order(q[0], sigma2[0])
        order = np.lexsort((np.arange(d), -w))   # w desc, index asc
        plan = orc.plan(q, sigma2, B)[0]
        assert list(plan[order]) == case["plan_in_w_order"], case["name"]


@pytest.mark.parametrize("B", [0, 1, 3, 4, 17, 18, 68, 91, 92, 136, 511, 512])
def test_plan_invariants(orc, B):
    rng = np.random.default_rng(B)
    hq, hkv, d = 8, 2, 128
    q = rng.standard_normal((hq, d)).astype(np.float32)
    sigma2 = rng.uniform(0.01, 16, (hkv, d)).astype(np.float32)
    plan = orc.plan(q, sigma2, B).astype(np.int64)
    assert np.all(plan.sum(1) == B)
    assert np.all(plan <= 4)
    assert np.all((plan > 0).sum(1) == -(-B // 4))
    # every channel read in full outranks every channel not read at all
    for h in range(hq):
        w = w_order(q[h], sigma2[h // 4])
        read, unread = w[plan[h] == 4], w[plan[h] == 0]
        if read.size and unread.size:
            assert read.min() >= unread.max()


def test_plan_rejects_out_of_range_budget(orc):
    q = np.ones((1, 8), np.float32)
    s = np.ones((1, 8), np.float32)
    for B in (-1, 33):
        with pytest.raises(ValueError):
            orc.plan(q, s, B)


@pytest.mark.parametrize("d", [3, 4, 5, 6])
def test_plan_greedy_is_optimal_brute_force(orc, d):
    """The fill-to-cap walk maximises sum_c w_c t_c over all plans with
    sum t = B and 0 <= t_c <= 4 (the importance-weighted bits read); with
    distinct w the maximiser is unique and equals the walk."""
    rng = np.random.default_rng(100 + d)
    plans = np.array(list(itertools.product(range(5), repeat=d)))
    for trial in range(6):
        q = rng.standard_normal((1, d)).astype(np.float32)
        sigma2 = rng.uniform(0.1, 4, (1, d)).astype(np.float32)
        w = w_order(q[0], sigma2[0]).astype(np.float64)
        for B in range(0, 4 * d + 1):
            feas = plans[plans.sum(1) == B]
            val = feas @ w
            best = feas[val == val.max()]
            got = orc.plan(q, sigma2, B)[0]
            assert len(best) == 1
            np.testing.assert_array_equal(got, best[0])


def test_plan_ties_go_to_lower_channel(orc):
    d = 8
    q = np.ones((1, d), np.float32)
    s = np.ones((1, d), np.float32)
    assert list(orc.plan(q, s, 10)[0]) == [4, 4, 2, 0, 0, 0, 0, 0]
    s2 = s.copy()
    s2[0, 5] = 2.0
    assert list(orc.plan(q, s2, 10)[0]) == [4, 2, 0, 0, 0, 4, 0, 0]


def test_plan_focused_query_spends_budget_on_few_channels(orc):
    """Intuition example 1: a query that depends on one or two channels puts
    its whole budget there."""
    d = 128
    q = np.full((1, d), 1e-3, np.float32)
    q[0, 17], q[0, 90] = 3.0, -2.0
    s = np.ones((1, d), np.float32)
    plan = orc.plan(q, s, 8)[0]
    assert plan[17] == 4 and plan[90] == 4 and plan.sum() == 8


def test_plan_gqa_uses_group_sigma(orc):
    hq, hkv, d = 4, 2, 8
    q = np.ones((hq, d), np.float32)
    s = np.ones((hkv, d), np.float32)
    s[0, 7] = 5.0
    s[1, 2] = 5.0
    plan = orc.plan(q, s, 4)
    assert plan[0, 7] == 4 and plan[1, 7] == 4
    assert plan[2, 2] == 4 and plan[3, 2] == 4


def test_plan_fixed_is_top_r_abs_q_and_matches_equal_sigma(orc):
    rng = np.random.default_rng(5)
    hq, d = 6, 128
    q = rng.standard_normal((hq, d)).astype(np.float32)
    for r in (0, 1, 16, 32, 128):
        fixed = orc.plan_fixed(q, r)
        for h in range(hq):
            order = np.lexsort((np.arange(d), -np.abs(q[h])))
            exp = np.zeros(d, np.uint8)
            exp[order[:r]] = 4
            np.testing.assert_array_equal(fixed[h], exp)
        same = orc.plan(q, np.ones((hq, d), np.float32), 4 * r)
        np.testing.assert_array_equal(fixed, same)


# --------------------------------------------------------------------------
# plan variants: rate-distortion greedy and one plan per GQA group

def distortion(w, plans):
    """sum_c w_c 4^-t_c for each row of plans (exact in fp64 here)."""
    return (w[None, :].astype(np.float64) * np.ldexp(1.0, -2 * plans)).sum(1)


def test_plan_rd_worked_examples(orc):
    one = np.ones((1, 2), np.float32)
    # w = (4, 1): fill-to-cap would give (3, 0), distortion 1/16 + 1; two
    # bits on the first channel and one on the second give 1/4 + 1/4.
    q = np.array([[2.0, 1.0]], np.float32)
    assert list(orc.plan_rd(q, one, 3)[0]) == [2, 1]
    assert list(orc.plan(q, one, 3)[0]) == [3, 0]
    # B = 2 is a tie, (2,0) and (1,1) both cost 5/4: the lower channel wins.
    assert list(orc.plan_rd(q, one, 2)[0]) == [2, 0]
    # equal importances spread the budget evenly, lower channels first
    e = np.ones((1, 4), np.float32)
    for B in range(17):
        exp = [B // 4 + (c < B % 4) for c in range(4)]
        assert list(orc.plan_rd(e, e, B)[0]) == exp


@pytest.mark.parametrize("d", [3, 4, 5])
def test_plan_rd_is_distortion_minimiser_brute_force(orc, d):
    rng = np.random.default_rng(200 + d)
    plans = np.array(list(itertools.product(range(5), repeat=d)))
    for trial in range(6):
        q = rng.standard_normal((1, d)).astype(np.float32)
        sigma2 = rng.uniform(0.1, 4, (1, d)).astype(np.float32)
        w = w_order(q[0], sigma2[0])
        for B in range(0, 4 * d + 1):
            feas = plans[plans.sum(1) == B]
            dist = distortion(w, feas)
            got = orc.plan_rd(q, sigma2, B)[0].astype(np.int64)
            assert got.sum() == B and got.max() <= 4
            best = feas[dist == dist.min()]
            assert len(best) == 1
            np.testing.assert_array_equal(got, best[0])


@pytest.mark.parametrize("B", [0, 1, 5, 64, 92, 136, 300, 511, 512])
def test_plan_rd_no_improving_single_bit_move(orc, B):
    """Moving one bit from any read channel to any channel with room never
    lowers the distortion, and the budget is spent exactly."""
    rng = np.random.default_rng(B + 7)
    hq, hkv, d = 4, 2, 128
    q = rng.standard_normal((hq, d)).astype(np.float32)
    sigma2 = rng.uniform(0.01, 16, (hkv, d)).astype(np.float32)
    plan = orc.plan_rd(q, sigma2, B).astype(np.int64)
    assert np.all(plan.sum(1) == B) and np.all(plan <= 4)
    for h in range(hq):
        w = w_order(q[h], sigma2[h // 2]).astype(np.float64)
        t = plan[h]
        next_gain = np.where(t < 4, w * np.ldexp(1.0, -2 * t), -np.inf)
        last_gain = np.where(t > 0, w * np.ldexp(1.0, -2 * (t - 1)), np.inf)
        assert next_gain.max() <= last_gain.min()


def test_plan_rd_equals_fill_to_cap_when_weights_are_far_apart(orc):
    """When each importance exceeds the next by more than 4^3, every bit of a
    channel is worth more than the first bit of the next: the walk results."""
    d = 12
    rng = np.random.default_rng(11)
    w = np.ldexp(1.0, -7 * np.arange(d)).astype(np.float32)   # ratio 128
    perm = rng.permutation(d)
    sigma2 = w[perm][None, :]
    q = np.ones((1, d), np.float32)
    for B in range(4 * d + 1):
        np.testing.assert_array_equal(orc.plan_rd(q, sigma2, B), orc.plan(q, sigma2, B))


def test_plan_rd_rejects_out_of_range_budget(orc):
    q = np.ones((1, 8), np.float32)
    for B in (-1, 33):
        with pytest.raises(ValueError):
            orc.plan_rd(q, q, B)


def group_weights64(q, sigma2, G):
    hq, d = q.shape
    qq = (q.astype(np.float64) ** 2).reshape(hq // G, G, d).sum(1)
    return qq * sigma2.astype(np.float64)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_plan_group_shares_one_plan_and_spends_group_budget(orc, G):
    rng = np.random.default_rng(G)
    hkv, d = 3, 128
    q = rng.standard_normal((hkv * G, d)).astype(np.float32)
    sigma2 = rng.uniform(0.01, 16, (hkv, d)).astype(np.float32)
    budgets = np.array([0, 92, 512], np.int32)
    plan = orc.plan_group(q, sigma2, budgets).astype(np.int64)
    for g in range(hkv):
        rows = plan[g * G:(g + 1) * G]
        assert np.all(rows == rows[0])
        assert rows[0].sum() == budgets[g] and rows[0].max() <= 4
        # channels read in full outrank unread ones under the summed importance
        W = group_weights64(q, sigma2, G)[g]
        read, unread = W[rows[0] == 4], W[rows[0] == 0]
        if read.size and unread.size:
            assert read.min() >= unread.max()


def test_plan_group_of_one_head_is_the_per_head_plan(orc):
    rng = np.random.default_rng(21)
    q = rng.standard_normal((6, 128)).astype(np.float32)
    sigma2 = rng.uniform(0.01, 16, (6, 128)).astype(np.float32)
    for B in (0, 3, 92, 136, 512):
        np.testing.assert_array_equal(orc.plan_group(q, sigma2, B), orc.plan(q, sigma2, B))


def test_plan_group_of_identical_heads_is_their_plan(orc):
    """Two equal heads: the summed square is exactly twice each, so the order
    (and the plan) is that of either head alone."""
    rng = np.random.default_rng(22)
    q1 = rng.standard_normal((2, 128)).astype(np.float32)
    q = np.repeat(q1, 2, axis=0)
    sigma2 = rng.uniform(0.01, 16, (2, 128)).astype(np.float32)
    for B in (1, 92, 136):
        np.testing.assert_array_equal(orc.plan_group(q, sigma2, B),
                                      orc.plan(q, sigma2, B))


@pytest.mark.parametrize("d", [3, 4, 5])
def test_plan_group_maximises_summed_importance_brute_force(orc, d):
    rng = np.random.default_rng(300 + d)
    plans = np.array(list(itertools.product(range(5), repeat=d)))
    G = 4
    for trial in range(4):
        q = rng.standard_normal((G, d)).astype(np.float32)
        sigma2 = rng.uniform(0.1, 4, (1, d)).astype(np.float32)
        W = group_weights64(q, sigma2, G)[0]
        for B in range(0, 4 * d + 1):
            feas = plans[plans.sum(1) == B]
            val = feas @ W
            best = feas[val == val.max()]
            assert len(best) == 1
            got = orc.plan_group(q, sigma2, B)
            for h in range(G):
                np.testing.assert_array_equal(got[h], best[0])


def test_plan_group_is_invariant_to_head_order_within_group(orc):
    """Integer-valued queries make every sum exact, so reordering the heads of
    a group cannot change the plan."""
    rng = np.random.default_rng(23)
    G, d = 8, 128
    q = rng.integers(-3, 4, (G, d)).astype(np.float32)
    sigma2 = rng.integers(1, 5, (1, d)).astype(np.float32)
    base = orc.plan_group(q, sigma2, 92)
    perm = rng.permutation(G)
    np.testing.assert_array_equal(orc.plan_group(q[perm], sigma2, 92), base)


def test_plan_group_rejects_out_of_range_budget(orc):
    q = np.ones((2, 8), np.float32)
    s = np.ones((1, 8), np.float32)
    for B in (-1, 33):
        with pytest.raises(ValueError):
            orc.plan_group(q, s, B)


# --------------------------------------------------------------------------
# scan

def make_layer(seed, n=300, hkv=2, hq=4, d=16, dtype=np.float16):
    rng = np.random.default_rng(seed)
    sig = np.exp(rng.uniform(np.log(0.1), np.log(4), (hkv, d)))
    keys = (rng.standard_normal((n, hkv, d)) * sig[None]).astype(dtype)
    q = rng.standard_normal((hq, d)).astype(np.float32)
    return keys, q


def test_scan_full_budget_is_full_4bit_dot_product(orc):
    keys, q = make_layer(1)
    n, hkv, d = keys.shape
    hq = q.shape[0]
    p = orc.pack(keys)
    plan = orc.plan(q, p["sigma2"], 4 * d)
    s = orc.scan(p["planes"], p["lo"], p["hi"], n, q, plan)
    lo = p["lo"].astype(np.float64)
    delta = ((p["hi"] - p["lo"]) * np.float32(0.0625)).astype(np.float64)
    G = hq // hkv
    for h in range(hq):
        g = h // G
        deq = lo[g][:, None] + (p["codes"][g] + 0.5) * delta[g][:, None]  # [d][n]
        ref = q[h].astype(np.float64) @ deq
        np.testing.assert_array_equal(s[h], ref.astype(np.float32))


@pytest.mark.parametrize("B", [0, 5, 18, 46, 64])
def test_scan_matches_t_bit_quantiser_from_raw_keys(orc, B):
    """Per key and channel, the scan's value equals the t-bit quantiser of the
    raw key reconstructed at its cell centre, summed against q (computed here
    from the keys, not from the planes)."""
    keys, q = make_layer(2 + B, n=130, hkv=1, hq=2, d=16)
    n, hkv, d = keys.shape
    p = orc.pack(keys)
    plan = orc.plan(q, p["sigma2"], B)
    s = orc.scan(p["planes"], p["lo"], p["hi"], n, q, plan)
    x = keys.astype(np.float32)[:, 0, :]
    for h in range(2):
        acc = np.zeros(n)
        for c in range(d):
            t = int(plan[h, c])
            lo, hi = p["lo"][0, c], p["hi"][0, c]
            qt = t_bit_quantizer(x[:, c], lo, hi, t)
            width = float(np.float32(np.float32(hi - lo) * np.float32(0.0625))) * 2 ** (4 - t)
            acc += float(q[h, c]) * (float(lo) + (qt + 0.5) * width)
        np.testing.assert_array_equal(s[h], acc.astype(np.float32))


def test_scan_zero_budget_is_constant_midpoint(orc):
    keys, q = make_layer(3)
    n = keys.shape[0]
    p = orc.pack(keys)
    plan = orc.plan(q, p["sigma2"], 0)
    s = orc.scan(p["planes"], p["lo"], p["hi"], n, q, plan)
    mid = (p["lo"].astype(np.float64) + p["hi"].astype(np.float64)) / 2
    for h in range(q.shape[0]):
        assert np.all(s[h] == s[h, 0])
        np.testing.assert_allclose(s[h, 0], q[h] @ mid[h // 2], rtol=1e-6)


def test_scan_one_hot_query_ranks_by_code(orc):
    keys, _ = make_layer(4, n=500, hkv=1, hq=1, d=16)
    p = orc.pack(keys)
    c = 9
    q = np.zeros((1, 16), np.float32)
    q[0, c] = 1.0
    plan = orc.plan(q, p["sigma2"], 4)
    assert plan[0, c] == 4
    s = orc.scan(p["planes"], p["lo"], p["hi"], 500, q, plan)[0]
    codes = p["codes"][0, c]
    delta = np.float32(p["hi"][0, c] - p["lo"][0, c]) * np.float32(0.0625)
    np.testing.assert_allclose(s, p["lo"][0, c] + (codes + 0.5) * float(delta),
                               rtol=1e-6)
    assert np.all(np.diff(s[np.argsort(codes, kind="stable")]) >= 0)


def test_scan_ignores_unread_plane_bits(orc):
    """Flipping any bit the plan does not read leaves every logit unchanged."""
    keys, q = make_layer(5, n=200)
    n, hkv, d = keys.shape
    p = orc.pack(keys)
    plan = orc.plan(q, p["sigma2"], 30)
    s0 = orc.scan(p["planes"], p["lo"], p["hi"], n, q, plan)
    G = q.shape[0] // hkv
    depth = np.zeros((hkv, d), np.int64)   # deepest plane any head of the group reads
    for h in range(q.shape[0]):
        depth[h // G] = np.maximum(depth[h // G], plan[h])
    flipped = p["planes"].copy()
    rng = np.random.default_rng(0)
    for g in range(hkv):
        for c in range(d):
            for slot in range(depth[g, c], 4):
                flipped[g, c, slot] ^= rng.integers(0, 2 ** 32, flipped.shape[-1],
                                                   dtype=np.uint64).astype(np.uint32)
    s1 = orc.scan(flipped, p["lo"], p["hi"], n, q, plan)
    np.testing.assert_array_equal(s0, s1)
    # and flipping a read bit does change something
    g, c = np.argwhere(depth > 0)[0]
    flipped2 = p["planes"].copy()
    flipped2[g, c, 0] ^= np.uint32(0xFFFFFFFF)
    s2 = orc.scan(flipped2, p["lo"], p["hi"], n, q, plan)
    assert np.any(s2 != s0)


def test_scan_side_stream_adds_scaled_byte(orc):
    keys, q = make_layer(6, n=100)
    n, hkv, d = keys.shape
    p = orc.pack(keys)
    plan = orc.plan_fixed(q, 4)
    meta = np.random.default_rng(1).integers(0, 256, (hkv, n)).astype(np.uint8)
    s0 = orc.scan(p["planes"], p["lo"], p["hi"], n, q, plan)
    s1 = orc.scan(p["planes"], p["lo"], p["hi"], n, q, plan, meta, 0.25)
    G = q.shape[0] // hkv
    for h in range(q.shape[0]):
        np.testing.assert_allclose(s1[h], s0[h] + 0.25 * meta[h // G], rtol=1e-6,
                                   atol=1e-6)


def np_nibbles(packed, n):
    """Independent unpacking of a 4-bit side stream: key i is the low nibble
    of byte i // 2 when i is even, the high nibble when it is odd."""
    lo = packed & 0x0F
    hi = packed >> 4
    return np.stack([lo, hi], -1).reshape(packed.shape[0], -1)[:, :n]


def test_scan_meta4_nibble_order_worked_example(orc):
    # bytes 0x21, 0x03 hold keys 0, 1, 2 = 1, 2, 3: the same scores as the
    # byte stream [1, 2, 3]
    keys, q = make_layer(21, n=3)
    n, hkv, d = keys.shape
    p = orc.pack(keys)
    plan = orc.plan(q, p["sigma2"], 40)
    packed = np.tile(np.array([[0x21, 0x03]], np.uint8), (hkv, 1))
    bytes_ = np.tile(np.array([[1, 2, 3]], np.uint8), (hkv, 1))
    a = orc.scan(p["planes"], p["lo"], p["hi"], n, q, plan, packed, 0.75, meta_bits=4)
    b = orc.scan(p["planes"], p["lo"], p["hi"], n, q, plan, bytes_, 0.75)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("n", [100, 101, 2049])
def test_scan_meta4_adds_scaled_nibble(orc, n):
    keys, q = make_layer(22, n=n)
    n, hkv, d = keys.shape
    p = orc.pack(keys)
    plan = orc.plan_fixed(q, 16)
    packed = np.random.default_rng(3).integers(0, 256, (hkv, (n + 1) // 2)).astype(np.uint8)
    vals = np_nibbles(packed, n)
    s0 = orc.scan(p["planes"], p["lo"], p["hi"], n, q, plan)
    s1 = orc.scan(p["planes"], p["lo"], p["hi"], n, q, plan, packed, 0.25, meta_bits=4)
    G = q.shape[0] // hkv
    for h in range(q.shape[0]):
        np.testing.assert_allclose(s1[h], s0[h] + 0.25 * vals[h // G], rtol=1e-6, atol=1e-6)
    # the nibbles as a byte stream give the same scores bit for bit
    s8 = orc.scan(p["planes"], p["lo"], p["hi"], n, q, plan, vals.astype(np.uint8), 0.25)
    np.testing.assert_array_equal(s1, s8)
    pick = np.array([0, 1, n - 2, n - 1, n // 2])
    part = orc.scan_at(p["planes"], p["lo"], p["hi"], n, q, plan, pick, packed, 0.25,
                       meta_bits=4)
    np.testing.assert_array_equal(part, s1[:, pick])


def test_read_prefixes_are_shifted_codes(orc):
    keys, q = make_layer(8, n=90)
    n, hkv, d = keys.shape
    p = orc.pack(keys)
    plan = orc.plan(q, p["sigma2"], 23)
    r = orc.read_prefixes(p["planes"], n, plan, hkv)
    G = q.shape[0] // hkv
    for h in range(q.shape[0]):
        for c in range(d):
            t = int(plan[h, c])
            exp = p["codes"][h // G, c] >> (4 - t) if t else 0
            np.testing.assert_array_equal(r[h, :, c], exp)


# --------------------------------------------------------------------------
# top-k

def lexsort_topk(S, k):
    order = np.lexsort((np.arange(S.size), -S.astype(np.float64)))
    return order[:k]


@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (64, 64), (500, 37), (4096, 64),
                                 (50, 80)])
def test_topk_matches_full_sort(orc, n, k):
    rng = np.random.default_rng(n * 31 + k)
    rows = 3
    S = rng.standard_normal((rows, n)).astype(np.float32)
    S[:, ::5] = np.round(S[:, ::5])          # plenty of exact ties
    idx, vals = orc.topk(S, k)
    for r in range(rows):
        exp = lexsort_topk(S[r], k)
        m = min(k, n)
        np.testing.assert_array_equal(idx[r, :m], exp)
        np.testing.assert_array_equal(vals[r, :m], S[r, exp])
        assert np.all(idx[r, m:] == -1) and np.all(np.isneginf(vals[r, m:]))


def test_topk_group_sum_in_fp64(orc):
    rng = np.random.default_rng(9)
    G, n, k = 4, 1000, 25
    S = rng.standard_normal((2 * G, n)).astype(np.float32)
    idx, vals = orc.topk(S, k, group=G)
    for o in range(2):
        tot = S[o * G:(o + 1) * G].astype(np.float64).sum(0).astype(np.float32)
        exp = lexsort_topk(tot, k)
        np.testing.assert_array_equal(idx[o], exp)
        np.testing.assert_array_equal(vals[o], tot[exp])


def test_topk_all_equal_scores_take_lowest_indices(orc):
    S = np.full((1, 100), 2.0, np.float32)
    S[0, 50] = -0.0
    idx, _ = orc.topk(S, 10)
    assert list(idx[0]) == list(range(10))
    S2 = np.zeros((1, 10), np.float32)
    S2[0, 3] = -0.0                 # -0 ties with +0
    idx2, _ = orc.topk(S2, 10)
    assert list(idx2[0]) == list(range(10))


def test_scan_at_equals_full_scan(orc):
    keys, q = make_layer(12, n=700)
    n = keys.shape[0]
    p = orc.pack(keys)
    plan = orc.plan(q, p["sigma2"], [9, 50, 64, 3])
    meta = np.random.default_rng(2).integers(0, 256, (2, n)).astype(np.uint8)
    full = orc.scan(p["planes"], p["lo"], p["hi"], n, q, plan, meta, 0.5)
    pick = np.array([0, 699, 5, 31, 32, 64, 333])
    part = orc.scan_at(p["planes"], p["lo"], p["hi"], n, q, plan, pick, meta, 0.5)
    np.testing.assert_array_equal(part, full[:, pick])


# --------------------------------------------------------------------------
# sparse decode attention over the selected keys

def attn_inputs(seed, n=300, hkv=2, hq=8, d=32):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((hq, d)).astype(np.float32)
    K = rng.standard_normal((n, hkv, d)).astype(np.float16)
    V = rng.standard_normal((n, hkv, d)).astype(np.float16)
    return rng, q, K, V


def sdpa_rows(q, K, V, rows_idx, G, scale):
    """torch's dense scaled-dot-product attention (CPU, fp64) over the listed
    key rows of each head's kv head."""
    import torch
    hq, d = q.shape
    out = np.zeros((hq, d))
    for h in range(hq):
        sel = rows_idx[h]
        k_ = torch.from_numpy(K[sel, h // G, :].astype(np.float64))[None, None]
        v_ = torch.from_numpy(V[sel, h // G, :].astype(np.float64))[None, None]
        q_ = torch.from_numpy(q[h].astype(np.float64))[None, None, None]
        out[h] = torch.nn.functional.scaled_dot_product_attention(
            q_, k_, v_, scale=scale)[0, 0, 0].numpy()
    return out


def test_sparse_attention_all_keys_is_dense_attention(orc):
    _, q, K, V = attn_inputs(1)
    n, hkv, d = K.shape
    G = q.shape[0] // hkv
    idx = np.tile(np.arange(n, dtype=np.int32), (q.shape[0], 1))
    scale = float(np.float32(1 / np.sqrt(d)))
    out, lse = orc.sparse_attention(q, K, V, idx)
    ref = sdpa_rows(q, K, V, [np.arange(n)] * q.shape[0], G, scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-6)


def test_sparse_attention_subset_and_duplicates_match_dense_on_rows(orc):
    rng, q, K, V = attn_inputs(2)
    n, hkv, d = K.shape
    G = q.shape[0] // hkv
    idx = rng.integers(0, n, (q.shape[0], 37)).astype(np.int32)
    idx[:, 5] = idx[:, 6]                              # a key listed twice counts twice
    out, _ = orc.sparse_attention(q, K, V, idx, scale=0.3)
    ref = sdpa_rows(q, K, V, list(idx), G, 0.3)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-6)


def test_sparse_attention_lse_is_logsumexp(orc):
    from scipy.special import logsumexp
    rng, q, K, V = attn_inputs(3)
    n, hkv, d = K.shape
    G = q.shape[0] // hkv
    idx = rng.choice(n, (q.shape[0], 50)).astype(np.int32)
    _, lse = orc.sparse_attention(q, K, V, idx, scale=0.7)
    for h in range(q.shape[0]):
        s = 0.7 * (K[idx[h], h // G, :].astype(np.float64) @ q[h].astype(np.float64))
        assert abs(lse[h] - logsumexp(s)) <= 1e-6 * max(1.0, abs(logsumexp(s)))


def test_sparse_attention_zero_query_averages_values(orc):
    rng, q, K, V = attn_inputs(4)
    q[:] = 0.0
    n, hkv, d = K.shape
    G = q.shape[0] // hkv
    idx = np.stack([rng.choice(n, 20, replace=False) for _ in range(q.shape[0])]).astype(np.int32)
    out, lse = orc.sparse_attention(q, K, V, idx)
    for h in range(q.shape[0]):
        np.testing.assert_allclose(out[h], V[idx[h], h // G, :].astype(np.float64).mean(0),
                                   rtol=0, atol=1e-6)
        assert abs(lse[h] - np.log(20)) < 1e-6


def test_sparse_attention_dominant_key_returns_its_value(orc):
    rng, q, K, V = attn_inputs(5, hq=2, hkv=1)
    q[:] = 0.0
    q[:, 0] = 1.0
    K[:, 0, 0] = 0.0
    K[17, 0, 0] = 8.0                                  # score gap 8 * 50 = 400
    idx = np.array([[3, 17, 40, 99]] * 2, np.int32)
    out, lse = orc.sparse_attention(q, K, V, idx, scale=50.0)
    np.testing.assert_array_equal(out[0], V[17, 0, :].astype(np.float32))
    assert lse[0] == np.float32(400.0)


def test_sparse_attention_permutation_padding_and_group(orc):
    rng, q, K, V = attn_inputs(6)
    n, hkv, d = K.shape
    hq = q.shape[0]
    G = hq // hkv
    idx = np.stack([rng.choice(n, 40, replace=False) for _ in range(hq)]).astype(np.int32)
    out, lse = orc.sparse_attention(q, K, V, idx)
    perm = idx[:, rng.permutation(40)]
    o2, l2 = orc.sparse_attention(q, K, V, perm)
    np.testing.assert_allclose(o2, out, rtol=0, atol=1e-6)
    padded = np.concatenate([idx[:, :13], -np.ones((hq, 9), np.int32), idx[:, 13:]], 1)
    o3, l3 = orc.sparse_attention(q, K, V, padded)
    np.testing.assert_array_equal(o3, out)
    np.testing.assert_array_equal(l3, lse)
    # group mode: one idx row per group of G heads equals that row repeated
    gidx = idx[::G]
    og, lg = orc.sparse_attention(q, K, V, gidx, group=G)
    orep, lrep = orc.sparse_attention(q, K, V, np.repeat(gidx, G, axis=0))
    np.testing.assert_array_equal(og, orep)
    np.testing.assert_array_equal(lg, lrep)
    # groups of 2 inside GQA groups of 4
    o2g, _ = orc.sparse_attention(q, K, V, idx[::2], group=2)
    np.testing.assert_array_equal(o2g, orc.sparse_attention(q, K, V, np.repeat(idx[::2], 2, 0))[0])


def test_sparse_attention_empty_rows_and_rejections(orc):
    _, q, K, V = attn_inputs(7)
    hq = q.shape[0]
    out, lse = orc.sparse_attention(q, K, V, -np.ones((hq, 5), np.int32))
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    out, lse = orc.sparse_attention(q, K, V, np.zeros((hq, 0), np.int32))
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    with pytest.raises(ValueError):
        orc.sparse_attention(q, K, V, np.full((hq, 3), K.shape[0], np.int32))
    with pytest.raises(ValueError):                    # groups must not straddle kv heads
        orc.sparse_attention(q, K, V, np.zeros((1, 3), np.int32), group=8)


# --------------------------------------------------------------------------
# append (decode-time growth of a packed layer with its stored range)

def keys_with_extremes_first(seed, n, hkv, d, n_first):
    """fp16 keys whose per-channel min and max lie among the first n_first."""
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((n, hkv, d)) * rng.uniform(0.2, 3, (1, hkv, d))).astype(np.float16)
    for h in range(hkv):
        for c in range(d):
            lo_i = int(np.argmin(k[:, h, c].astype(np.float32)))
            k[[0, lo_i], h, c] = k[[lo_i, 0], h, c]
            hi_i = 1 + int(np.argmax(k[1:, h, c].astype(np.float32)))
            k[[1, hi_i], h, c] = k[[hi_i, 1], h, c]
    assert n_first >= 2
    return k


def widen(planes, W):
    hkv, d, four, W0 = planes.shape
    out = np.zeros((hkv, d, four, W), np.uint32)
    out[..., :W0] = planes
    return out


@pytest.mark.parametrize("n0,n", [(2, 5), (300, 1000), (2047, 2049), (2048, 4100), (31, 33)])
def test_append_in_range_keys_equals_pack_of_all(orc, n0, n):
    keys = keys_with_extremes_first(n0 + n, n, 2, 16, n0)
    full = orc.pack(keys)
    first = orc.pack(keys[:n0])
    np.testing.assert_array_equal(first["lo"], full["lo"])
    np.testing.assert_array_equal(first["hi"], full["hi"])
    planes = widen(first["planes"], orc.plane_words(n))
    cnt = orc.append(keys[n0:], n0, planes, first["lo"], first["hi"])
    assert cnt == 0
    np.testing.assert_array_equal(planes, full["planes"])


def test_append_one_token_at_a_time_equals_one_call(orc):
    keys = keys_with_extremes_first(8, 700, 2, 16, 100)
    first = orc.pack(keys[:100])
    W = orc.plane_words(700)
    a = widen(first["planes"], W)
    b = a.copy()
    orc.append(keys[100:], 100, a, first["lo"], first["hi"])
    for j in range(100, 700):
        orc.append(keys[j:j + 1], j, b, first["lo"], first["hi"])
    np.testing.assert_array_equal(a, b)


def test_append_clamps_out_of_range_and_counts(orc):
    rng = np.random.default_rng(9)
    base = rng.standard_normal((500, 2, 16)).astype(np.float16)
    p = orc.pack(base)
    new = (rng.standard_normal((300, 2, 16)) * 3).astype(np.float16)   # many outside
    W = orc.plane_words(800)
    planes = widen(p["planes"], W)
    cnt = orc.append(new, 500, planes, p["lo"], p["hi"])
    x = new.astype(np.float32).transpose(1, 2, 0)                      # [hkv][d][m]
    lo, hi = p["lo"][..., None], p["hi"][..., None]
    delta = ((hi - lo) * np.float32(0.0625)).astype(np.float32)
    q = np.floor(((x - lo).astype(np.float32) / delta).astype(np.float32))
    expect = np.clip(q, 0, 15).astype(np.int64)
    got = unpack_planes_vectorised(planes, 800)[:, :, 500:]
    np.testing.assert_array_equal(got, expect)
    assert cnt == int(((x < lo) | (x > hi)).sum()) and cnt > 0
    # keys at the range ends land in codes 0 and 15 without counting
    ends = np.stack([p["lo"], p["hi"]]).astype(np.float16)
    c2 = orc.append(ends, 800, widen(planes, orc.plane_words(802)), p["lo"], p["hi"])
    assert c2 == 0


def test_append_leaves_every_other_bit_alone(orc):
    rng = np.random.default_rng(10)
    hkv, d, W = 2, 8, 128                                   # capacity 4096 keys
    planes = rng.integers(0, 2 ** 32, (hkv, d, 4, W), dtype=np.uint64).astype(np.uint32)
    before = planes.copy()
    lo = np.full((hkv, d), -1, np.float32)
    hi = np.full((hkv, d), 1, np.float32)
    new = rng.uniform(-1, 1, (50, hkv, d)).astype(np.float32)
    orc.append(new, 1000, planes, lo, hi)
    tok = np.arange(W * 32)
    touched = (tok >= 1000) & (tok < 1050)
    b0 = np.unpackbits(before.view(np.uint8), bitorder="little").reshape(hkv, d, 4, W * 32)
    b1 = np.unpackbits(planes.view(np.uint8), bitorder="little").reshape(hkv, d, 4, W * 32)
    np.testing.assert_array_equal(b0[..., ~touched], b1[..., ~touched])
    codes = b1[..., touched]
    val = codes[:, :, 0] * 8 + codes[:, :, 1] * 4 + codes[:, :, 2] * 2 + codes[:, :, 3]
    xs = new.transpose(1, 2, 0)
    exp = np.clip(np.floor(((xs + 1).astype(np.float32) / np.float32(0.125))), 0, 15)
    np.testing.assert_array_equal(val, exp)


def test_append_constant_channel_and_rejections(orc):
    lo = np.zeros((1, 4), np.float32)
    hi = np.zeros((1, 4), np.float32)
    planes = np.full((1, 4, 4, 64), 0xFFFFFFFF, np.uint32)
    new = np.array([[[0, 0, 1, -2]]], np.float32)
    cnt = orc.append(new, 5, planes, lo, hi)
    assert cnt == 2
    assert np.all(unpack_planes_vectorised(planes, 6)[0, :, 5] == 0)
    with pytest.raises(ValueError):                        # rows too short for n_old + m
        orc.append(np.zeros((2, 1, 4), np.float32), 2047, planes, lo, hi)


# --------------------------------------------------------------------------
# calibrated allocation: code histograms, depth errors, exact DP

def test_code_hist_counts_the_quantiser_codes(orc):
    rng = np.random.default_rng(31)
    keys = (rng.standard_normal((3000, 2, 16)) * rng.uniform(0.3, 2, (1, 2, 16))).astype(np.float16)
    p = orc.pack(keys)
    hist = orc.code_hist(p["planes"], 3000)
    for h in range(2):
        for c in range(16):
            codes = t_bit_quantizer(keys[:, h, c].astype(np.float32), p["lo"][h, c],
                                    p["hi"][h, c], 4)
            np.testing.assert_array_equal(hist[h, c], np.bincount(codes, minlength=16))


def test_depth_errors_are_squared_gaps_of_the_raw_keys(orc):
    """E(t) * delta^2 = sum over keys of (4-bit value - t-bit reconstruction)^2,
    both computed here from the raw keys with the independent quantiser."""
    rng = np.random.default_rng(32)
    keys = (rng.standard_normal((2500, 1, 8)) * 1.7).astype(np.float32)
    p = orc.pack(keys)
    E = orc.depth_errors(orc.code_hist(p["planes"], 2500))
    for c in range(8):
        x = keys[:, 0, c]
        lo, hi = p["lo"][0, c], p["hi"][0, c]
        delta = float(np.float32(np.float32(hi - lo) * np.float32(0.0625)))
        x4 = lo + (t_bit_quantizer(x, lo, hi, 4) + 0.5) * delta
        for t in range(5):
            cell = delta * 2 ** (4 - t)
            xt = lo + (t_bit_quantizer(x, lo, hi, t) + 0.5) * cell
            ref = float(((x4 - xt) ** 2).sum()) / delta ** 2
            assert abs(E[0, c, t] - ref) <= 1e-9 * max(1.0, ref), (c, t)
    assert np.all(E[..., 4] == 0)


def test_depth_errors_of_a_point_mass_and_a_uniform_channel(orc):
    """Worked by hand from the cell centres: every key at code 8 leaves
    offsets 0.5, -3.5, -1.5, -0.5, 0 at depths 0..4; one key per code gives
    sum (v + 1/2 - 8)^2 = 340 at depth 0 and 16 (m^2 - 1) / 12 per cell of m
    codes after."""
    hist = np.zeros((1, 2, 16), np.uint32)
    hist[0, 0, 8] = 16
    hist[0, 1, :] = 1
    E = orc.depth_errors(hist)
    np.testing.assert_array_equal(E[0, 0], 16 * np.array([0.25, 12.25, 2.25, 0.25, 0]))
    np.testing.assert_array_equal(E[0, 1], [340, 84, 20, 4, 0])


def test_plan_calibrated_skips_depths_that_add_error(orc):
    """Channel 0: weight 10, every key at code 8; channel 1: weight 1, one key
    per code.  Per-depth costs (weight x E): channel 0 [40, 1960, 360, 40, 0],
    channel 1 [340, 84, 20, 4, 0].  A single bit of channel 0 makes its error
    worse than reading nothing, so with B = 5 the exact minimum is (3, 2)
    (cost 60), where filling channel 1 first and giving channel 0 the rest
    would cost 1960."""
    hist = np.zeros((1, 2, 16), np.uint32)
    hist[0, 0, 8] = 16
    hist[0, 1, :] = 1
    lo = np.zeros((1, 2), np.float32)
    hi = np.full((1, 2), 16.0, np.float32)                       # delta = 1
    q = np.array([[np.sqrt(10.0), 1.0]], np.float32)
    expect = {1: [0, 1], 3: [0, 3], 4: [0, 4], 5: [3, 2], 6: [4, 2], 7: [4, 3], 8: [4, 4]}
    for B, plan in expect.items():
        assert list(orc.plan_calibrated(q, lo, hi, hist, B)[0]) == plan, B


@pytest.mark.parametrize("d", [3, 4, 5])
def test_plan_calibrated_is_the_brute_force_minimum(orc, d):
    rng = np.random.default_rng(400 + d)
    plans = np.array(list(itertools.product(range(5), repeat=d)))
    for trial in range(4):
        q = rng.standard_normal((1, d)).astype(np.float32)
        lo = rng.uniform(-3, -1, (1, d)).astype(np.float32)
        hi = rng.uniform(1, 3, (1, d)).astype(np.float32)
        hist = rng.integers(0, 200, (1, d, 16)).astype(np.uint32)
        E = orc.depth_errors(hist)[0]
        delta = ((hi - lo) * np.float32(0.0625)).astype(np.float32)[0].astype(np.float64)
        w = q[0].astype(np.float64) ** 2 * delta ** 2
        cost = w[:, None] * E                                     # [d][5]
        for B in range(0, 4 * d + 1):
            feas = plans[plans.sum(1) == B]
            tot = np.zeros(len(feas))
            for c in range(d):                                    # channel order, fp64
                tot = tot + cost[c, feas[:, c]]
            best = feas[tot == tot.min()]
            got = orc.plan_calibrated(q, lo, hi, hist, B)[0]
            assert len(best) == 1
            np.testing.assert_array_equal(got, best[0])


def test_plan_calibrated_on_uniform_channels_is_the_rd_plan(orc):
    """With every code equally frequent, reading bit t+1 removes a quarter of
    what bit t removed, so the exact minimum is the rate-distortion greedy on
    the weights q^2 delta^2."""
    rng = np.random.default_rng(41)
    hq, hkv, d = 4, 2, 32
    q = rng.standard_normal((hq, d)).astype(np.float32)
    lo = rng.uniform(-3, -1, (hkv, d)).astype(np.float32)
    hi = rng.uniform(1, 3, (hkv, d)).astype(np.float32)
    hist = np.full((hkv, d, 16), 7, np.uint32)
    delta2 = (((hi - lo) * np.float32(0.0625)).astype(np.float32) ** 2).astype(np.float32)
    for B in (0, 5, 40, 77, 128):
        np.testing.assert_array_equal(orc.plan_calibrated(q, lo, hi, hist, B),
                                      orc.plan_rd(q, delta2, B))


@pytest.mark.parametrize("B", [0, 1, 92, 136, 512])
def test_plan_calibrated_spends_the_budget(orc, B):
    rng = np.random.default_rng(B + 50)
    keys = synth_like = (rng.standard_normal((4000, 2, 128)) *
                         rng.uniform(0.1, 4, (1, 2, 128))).astype(np.float16)
    p = orc.pack(keys)
    hist = orc.code_hist(p["planes"], 4000)
    q = rng.standard_normal((8, 128)).astype(np.float32)
    plan = orc.plan_calibrated(q, p["lo"], p["hi"], hist, B).astype(np.int64)
    assert np.all(plan.sum(1) == B) and np.all(plan <= 4)
    with pytest.raises(ValueError):
        orc.plan_calibrated(q, p["lo"], p["hi"], hist, 513)


def calib_inputs(seed, hq, hkv, d, n=3000):
    rng = np.random.default_rng(seed)
    keys = (rng.standard_normal((n, hkv, d)) * rng.uniform(0.2, 3, (1, hkv, d))).astype(np.float16)
    p = orc_pack_cached(keys)
    q = rng.standard_normal((hq, d)).astype(np.float32)
    return q, p


def orc_pack_cached(keys):
    from oracle import oracle
    p = oracle.pack(keys)
    p["hist"] = oracle.code_hist(p["planes"], keys.shape[0])
    return p


def test_plan_calibrated_group_of_one_head_is_the_per_head_plan(orc):
    q, p = calib_inputs(60, 6, 6, 128)
    for B in (0, 7, 92, 136, 512):
        np.testing.assert_array_equal(
            orc.plan_calibrated_group(q, p["lo"], p["hi"], p["hist"], B),
            orc.plan_calibrated(q, p["lo"], p["hi"], p["hist"], B))


@pytest.mark.parametrize("G", [2, 4])
def test_plan_calibrated_group_of_identical_heads_is_their_plan(orc, G):
    """G equal heads: the summed square is exactly G times each (a power of
    two), so every cost scales exactly and the plan is the single head's."""
    q1, p = calib_inputs(61 + G, 2, 2, 128)
    q = np.repeat(q1, G, axis=0)
    for B in (1, 92, 176):
        grp = orc.plan_calibrated_group(q, p["lo"], p["hi"], p["hist"], B)
        one = orc.plan_calibrated(q1, p["lo"], p["hi"], p["hist"], B)
        np.testing.assert_array_equal(grp, np.repeat(one, G, axis=0))


@pytest.mark.parametrize("d", [3, 4, 5])
def test_plan_calibrated_group_is_the_brute_force_minimum(orc, d):
    rng = np.random.default_rng(600 + d)
    plans = np.array(list(itertools.product(range(5), repeat=d)))
    G = 3
    for trial in range(3):
        q = rng.standard_normal((G, d)).astype(np.float32)
        lo = rng.uniform(-3, -1, (1, d)).astype(np.float32)
        hi = rng.uniform(1, 3, (1, d)).astype(np.float32)
        hist = rng.integers(0, 200, (1, d, 16)).astype(np.uint32)
        E = orc.depth_errors(hist)[0]
        delta = ((hi - lo) * np.float32(0.0625)).astype(np.float32)[0].astype(np.float64)
        S = (q.astype(np.float64) ** 2).sum(0)
        cost = (S * delta ** 2)[:, None] * E
        for B in range(0, 4 * d + 1):
            feas = plans[plans.sum(1) == B]
            tot = np.zeros(len(feas))
            for c in range(d):
                tot = tot + cost[c, feas[:, c]]
            best = feas[tot == tot.min()]
            assert len(best) == 1
            got = orc.plan_calibrated_group(q, lo, hi, hist, B)
            for h in range(G):
                np.testing.assert_array_equal(got[h], best[0])


def test_plan_calibrated_group_spends_each_group_budget(orc):
    q, p = calib_inputs(62, 12, 3, 128)
    budgets = np.array([0, 92, 512], np.int32)
    plan = orc.plan_calibrated_group(q, p["lo"], p["hi"], p["hist"], budgets).astype(np.int64)
    for g in range(3):
        rows = plan[g * 4:(g + 1) * 4]
        assert np.all(rows == rows[0]) and rows[0].sum() == budgets[g]
    with pytest.raises(ValueError):
        orc.plan_calibrated_group(q, p["lo"], p["hi"], p["hist"], [1, 2, 513])
