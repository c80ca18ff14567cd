"""Comparison helpers for the GPU-vs-oracle parity tests."""
import numpy as np

# Logits tolerance: |s_gpu - s_oracle| <= LOGIT_TOL * A_h, with
# A_h = sum_c |q_hc| * max(|lo_c|, |hi_c|) (+ |meta_scale| * 255 with the side
# stream), a bound on |s| and on every term of the sum.  The GPU adds at most
# d + 1 fp32 terms in a fixed order, whose worst-case rounding error is below
# (d + 1) * 2^-24 * 3 * A_h = 2.3e-5 * A_h; for the <= 35 terms of the pages'
# budgets (B <= 136) it is below 6.3e-6 * A_h.  The stated bar is 1e-5.
LOGIT_TOL = 1e-5


def logit_scale(q, lo, hi, group, meta_scale=0.0):
    """A_h per query head: [hq] fp64."""
    q = np.asarray(q, np.float64)
    m = np.maximum(np.abs(np.asarray(lo, np.float64)), np.abs(np.asarray(hi, np.float64)))
    hq = q.shape[0]
    A = np.array([np.abs(q[h]) @ m[h // group] for h in range(hq)])
    return A + abs(meta_scale) * 255.0


def assert_logits_close(got, ref, A, tol=LOGIT_TOL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref) / A[:, None]
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"logit error {worst:.3e} * A_h exceeds {tol:.1e}"
    return worst


def group_scores(logits, group):
    """fp32 group score: rows of a group added in fp64 in row order, rounded once."""
    L = np.asarray(logits, np.float32)
    rows, n = L.shape
    out = np.zeros((rows // group, n), np.float64)
    for o in range(rows // group):
        acc = np.zeros(n, np.float64)
        for j in range(group):
            acc = acc + L[o * group + j].astype(np.float64)
        out[o] = acc
    return out.astype(np.float32)


def assert_topk_tie_tolerant(idx_gpu, idx_ref, ref_scores, A_rows, n, k, tol=LOGIT_TOL):
    """Top-k of GPU logits vs top-k of oracle logits: same size, no duplicate,
    every index < n, and the sets differ only by keys whose oracle score lies
    within 2 * tol * A of the oracle's k-th score."""
    kk = min(k, n)
    for r in range(idx_gpu.shape[0]):
        g = idx_gpu[r, :kk]
        e = idx_ref[r, :kk]
        assert np.all(idx_gpu[r, kk:] == -1)
        assert len(set(g.tolist())) == kk
        assert np.all((g >= 0) & (g < n))
        diff = set(g.tolist()) ^ set(e.tolist())
        if diff:
            kth = ref_scores[r, e[-1]]
            d = np.array(sorted(diff))
            gap = np.abs(ref_scores[r, d].astype(np.float64) - kth)
            assert np.all(gap <= 2 * tol * A_rows[r]), (r, d[gap > 2 * tol * A_rows[r]][:5])
