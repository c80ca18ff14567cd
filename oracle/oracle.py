"""ctypes wrapper of the CPU oracle (``fathom_oracle.c``).

Test infrastructure only: the tests, the bench's CPU-baseline leg and the
smoke check use it.  The product package never imports this module, and this
module imports nothing from the product package.  Arguments are numpy arrays;
fp16 keys are widened to fp32 here (exact).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fathom_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libfathom_oracle.so")
GCC_FLAGS = ["-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off",
             "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libfathom_oracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_int64
        F = ctypes.c_float
        lib.orc_plane_words.restype = L
        lib.orc_plane_words.argtypes = [L]
        lib.orc_pack.argtypes = [P, L, I, I, L, L, P, P, P, P, P]
        lib.orc_plan.argtypes = [P, I, I, I, P, P, P]
        lib.orc_plan_fixed.argtypes = [P, I, I, I, P]
        lib.orc_plan_rd.argtypes = [P, I, I, I, P, P, P]
        lib.orc_plan_group.argtypes = [P, I, I, I, P, P, P]
        lib.orc_scan.argtypes = [P, P, P, L, I, I, P, P, I, P, F, P, L]
        lib.orc_scan_at.argtypes = [P, P, P, L, I, I, P, P, I, P, F, P, L, P]
        lib.orc_scan_meta4.argtypes = [P, P, P, L, I, I, P, P, I, P, F, P, L]
        lib.orc_scan_at_meta4.argtypes = [P, P, P, L, I, I, P, P, I, P, F, P, L, P]
        lib.orc_read_prefixes.argtypes = [P, L, I, I, P, I, P]
        lib.orc_topk.argtypes = [P, I, L, L, I, I, P, P]
        lib.orc_append.argtypes = [P, L, I, I, L, L, L, P, L, P, P, P]
        lib.orc_range_blocks.restype = L
        lib.orc_range_blocks.argtypes = [L]
        lib.orc_pack_blocked.argtypes = [P, L, I, I, L, L, P, P, P, L, P]
        lib.orc_scan_blocked.argtypes = [P, P, P, L, L, I, I, P, P, I, P, L]
        lib.orc_scan_blocked_at.argtypes = [P, P, P, L, L, I, I, P, P, I, P, L, P]
        lib.orc_append_blocked.argtypes = [P, L, I, I, L, L, L, P, L, P, P, L, P]
        lib.orc_code_hist.argtypes = [P, L, I, I, L, P]
        lib.orc_depth_errors.argtypes = [P, I, I, P]
        lib.orc_plan_calibrated.argtypes = [P, I, I, I, P, P, P, P, P]
        lib.orc_plan_calibrated_group.argtypes = [P, I, I, I, P, P, P, P, P]
        lib.orc_sparse_attention.argtypes = [P, I, I, I, P, P, L, L, L, P, I, I, F, P, P]
        for f in ("orc_pack", "orc_plan", "orc_plan_fixed", "orc_plan_rd", "orc_plan_group",
                  "orc_scan", "orc_scan_at", "orc_scan_meta4", "orc_scan_at_meta4",
                  "orc_read_prefixes", "orc_topk", "orc_sparse_attention", "orc_append", "orc_code_hist", "orc_depth_errors",
                  "orc_plan_calibrated", "orc_plan_calibrated_group", "orc_pack_blocked",
                  "orc_scan_blocked", "orc_scan_blocked_at", "orc_append_blocked"):
            getattr(lib, f).restype = I
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name} rejected its arguments")


def plane_words(n: int) -> int:
    return int(_load().orc_plane_words(n))


def pack(keys: np.ndarray):
    """keys [n][hkv][d] (fp16 or fp32) -> dict(codes, planes, lo, hi, sigma2).

    codes [hkv][d][n] uint8, planes [hkv][d][4][W] uint32 (slot 0 = MSB
    plane), lo/hi/sigma2 [hkv][d] fp32.
    """
    k32 = np.ascontiguousarray(keys, dtype=np.float32)
    n, hkv, d = k32.shape
    W = plane_words(n)
    codes = np.empty((hkv, d, n), np.uint8)
    planes = np.empty((hkv, d, 4, W), np.uint32)
    lo = np.empty((hkv, d), np.float32)
    hi = np.empty((hkv, d), np.float32)
    s2 = np.empty((hkv, d), np.float32)
    _check(_load().orc_pack(_ptr(k32), n, hkv, d, hkv * d, d, _ptr(codes),
                            _ptr(planes), _ptr(lo), _ptr(hi), _ptr(s2)), "pack")
    return dict(codes=codes, planes=planes, lo=lo, hi=hi, sigma2=s2)


def plan(q: np.ndarray, sigma2: np.ndarray, budget) -> np.ndarray:
    """q [hq][d] fp32, sigma2 [hkv][d] fp32, budget int or [hq] -> [hq][d] u8."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    sigma2 = np.ascontiguousarray(sigma2, dtype=np.float32)
    hq, d = q.shape
    hkv = sigma2.shape[0]
    b = np.ascontiguousarray(np.broadcast_to(np.asarray(budget, np.int32), (hq,)))
    out = np.empty((hq, d), np.uint8)
    _check(_load().orc_plan(_ptr(q), hq, hkv, d, _ptr(sigma2), _ptr(b),
                            _ptr(out)), "plan")
    return out


def plan_rd(q: np.ndarray, sigma2: np.ndarray, budget) -> np.ndarray:
    """Rate-distortion plan: the B largest gains w_c * 4^-t -> [hq][d] u8."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    sigma2 = np.ascontiguousarray(sigma2, dtype=np.float32)
    hq, d = q.shape
    hkv = sigma2.shape[0]
    b = np.ascontiguousarray(np.broadcast_to(np.asarray(budget, np.int32), (hq,)))
    out = np.empty((hq, d), np.uint8)
    _check(_load().orc_plan_rd(_ptr(q), hq, hkv, d, _ptr(sigma2), _ptr(b),
                               _ptr(out)), "plan_rd")
    return out


def plan_group(q: np.ndarray, sigma2: np.ndarray, budget) -> np.ndarray:
    """One plan per GQA group; budget int or [hkv] -> [hq][d] u8."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    sigma2 = np.ascontiguousarray(sigma2, dtype=np.float32)
    hq, d = q.shape
    hkv = sigma2.shape[0]
    b = np.ascontiguousarray(np.broadcast_to(np.asarray(budget, np.int32), (hkv,)))
    out = np.empty((hq, d), np.uint8)
    _check(_load().orc_plan_group(_ptr(q), hq, hkv, d, _ptr(sigma2), _ptr(b),
                                  _ptr(out)), "plan_group")
    return out


def plan_fixed(q: np.ndarray, r: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float32)
    hq, d = q.shape
    out = np.empty((hq, d), np.uint8)
    _check(_load().orc_plan_fixed(_ptr(q), hq, d, r, _ptr(out)), "plan_fixed")
    return out


def scan(planes, lo, hi, n: int, q, plan_, meta=None, meta_scale: float = 0.0,
         meta_bits: int = 8):
    """-> logits [hq][n] fp32 (computed in fp64, rounded once).  meta: the
    side stream, uint8 [hkv][n] (meta_bits 8) or packed nibbles uint8
    [hkv][ceil(n/2)] (meta_bits 4, even keys in the low nibble)."""
    planes = np.ascontiguousarray(planes, dtype=np.uint32)
    lo = np.ascontiguousarray(lo, dtype=np.float32)
    hi = np.ascontiguousarray(hi, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    plan_ = np.ascontiguousarray(plan_, dtype=np.uint8)
    hkv, d = lo.shape
    hq = q.shape[0]
    if meta is not None:
        meta = np.ascontiguousarray(meta, dtype=np.uint8)
    out = np.empty((hq, max(n, 1)), np.float32)
    fn = _load().orc_scan if meta_bits == 8 else _load().orc_scan_meta4
    _check(fn(_ptr(planes), _ptr(lo), _ptr(hi), n, hkv, d, _ptr(q), _ptr(plan_), hq,
              _ptr(meta), meta_scale, _ptr(out), max(n, 1)), "scan")
    return out[:, :n]


def scan_at(planes, lo, hi, n: int, q, plan_, keys, meta=None, meta_scale: float = 0.0,
            meta_bits: int = 8):
    """Scores of the chosen key indices only -> [hq][len(keys)] fp32."""
    planes = np.ascontiguousarray(planes, dtype=np.uint32)
    lo = np.ascontiguousarray(lo, dtype=np.float32)
    hi = np.ascontiguousarray(hi, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    plan_ = np.ascontiguousarray(plan_, dtype=np.uint8)
    keys = np.ascontiguousarray(keys, dtype=np.int64)
    hkv, d = lo.shape
    hq = q.shape[0]
    if meta is not None:
        meta = np.ascontiguousarray(meta, dtype=np.uint8)
    out = np.empty((hq, keys.size), np.float32)
    fn = _load().orc_scan_at if meta_bits == 8 else _load().orc_scan_at_meta4
    _check(fn(_ptr(planes), _ptr(lo), _ptr(hi), n, hkv, d, _ptr(q), _ptr(plan_), hq,
              _ptr(meta), meta_scale, _ptr(keys), keys.size, _ptr(out)), "scan_at")
    return out


def read_prefixes(planes, n: int, plan_, hkv: int) -> np.ndarray:
    planes = np.ascontiguousarray(planes, dtype=np.uint32)
    plan_ = np.ascontiguousarray(plan_, dtype=np.uint8)
    hq, d = plan_.shape
    out = np.empty((hq, n, d), np.uint8)
    _check(_load().orc_read_prefixes(_ptr(planes), n, hkv, d, _ptr(plan_), hq,
                                     _ptr(out)), "read_prefixes")
    return out


def topk(scores, k: int, group: int = 1):
    """scores [rows][n] fp32 -> (idx [rows/group][k] int32, vals fp32)."""
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    rows, n = scores.shape
    ro = rows // group
    idx = np.empty((ro, k), np.int32)
    vals = np.empty((ro, k), np.float32)
    _check(_load().orc_topk(_ptr(scores), rows, n, max(n, 1), group, k,
                            _ptr(idx), _ptr(vals)), "topk")
    return idx, vals


def sparse_attention(q, K, V, idx, group: int = 1, scale=None):
    """q [hq][d]; K, V [n][hkv][d] (fp16 or fp32); idx [hq/group][k] int32
    -> (out [hq][d] fp32, lse [hq] fp32).  scale defaults to 1/sqrt(d)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    K = np.ascontiguousarray(K, dtype=np.float32)
    V = np.ascontiguousarray(V, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    hq, d = q.shape
    n, hkv, _ = K.shape
    k = idx.shape[1]
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    out = np.empty((hq, d), np.float32)
    lse = np.empty(hq, np.float32)
    _check(_load().orc_sparse_attention(_ptr(q), hq, hkv, d, _ptr(K), _ptr(V), n, hkv * d, d,
                                        _ptr(idx), group, k, scale, _ptr(out), _ptr(lse)),
           "sparse_attention")
    return out, lse


def append(keys_new, n_old: int, planes, lo, hi):
    """Set the bits of keys_new [m][hkv][d] (fp16/fp32) at tokens n_old ..
    n_old+m-1 of planes [hkv][d][4][W] (modified in place, uint32) with the
    stored lo/hi.  Returns the number of values outside [lo, hi]."""
    k32 = np.ascontiguousarray(keys_new, dtype=np.float32)
    m, hkv, d = k32.shape
    assert planes.dtype == np.uint32 and planes.flags["C_CONTIGUOUS"]
    W = planes.shape[-1]
    lo = np.ascontiguousarray(lo, dtype=np.float32)
    hi = np.ascontiguousarray(hi, dtype=np.float32)
    cnt = np.zeros(1, np.int64)
    _check(_load().orc_append(_ptr(k32), m, hkv, d, hkv * d, d, n_old, _ptr(planes), W,
                              _ptr(lo), _ptr(hi), _ptr(cnt)), "append")
    return int(cnt[0])


def code_hist(planes, n: int):
    """planes [hkv][d][4][W] uint32 -> hist [hkv][d][16] uint32 of keys < n."""
    planes = np.ascontiguousarray(planes, dtype=np.uint32)
    hkv, d, _, W = planes.shape
    out = np.empty((hkv, d, 16), np.uint32)
    _check(_load().orc_code_hist(_ptr(planes), n, hkv, d, W, _ptr(out)), "code_hist")
    return out


def depth_errors(hist):
    """hist [hkv][d][16] -> E [hkv][d][5] (fp64, delta^2 units)."""
    hist = np.ascontiguousarray(hist, dtype=np.uint32)
    hkv, d, _ = hist.shape
    out = np.empty((hkv, d, 5), np.float64)
    _check(_load().orc_depth_errors(_ptr(hist), hkv, d, _ptr(out)), "depth_errors")
    return out


def plan_calibrated(q, lo, hi, hist, budget) -> np.ndarray:
    """q [hq][d], lo/hi [hkv][d], hist [hkv][d][16], budget int or [hq] -> plan."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    lo = np.ascontiguousarray(lo, dtype=np.float32)
    hi = np.ascontiguousarray(hi, dtype=np.float32)
    hist = np.ascontiguousarray(hist, dtype=np.uint32)
    hq, d = q.shape
    hkv = lo.shape[0]
    b = np.ascontiguousarray(np.broadcast_to(np.asarray(budget, np.int32), (hq,)))
    out = np.empty((hq, d), np.uint8)
    _check(_load().orc_plan_calibrated(_ptr(q), hq, hkv, d, _ptr(lo), _ptr(hi), _ptr(hist),
                                       _ptr(b), _ptr(out)), "plan_calibrated")
    return out


def plan_calibrated_group(q, lo, hi, hist, budget) -> np.ndarray:
    """One calibrated plan per GQA group; budget int or [hkv] -> plan [hq][d]."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    lo = np.ascontiguousarray(lo, dtype=np.float32)
    hi = np.ascontiguousarray(hi, dtype=np.float32)
    hist = np.ascontiguousarray(hist, dtype=np.uint32)
    hq, d = q.shape
    hkv = lo.shape[0]
    b = np.ascontiguousarray(np.broadcast_to(np.asarray(budget, np.int32), (hkv,)))
    out = np.empty((hq, d), np.uint8)
    _check(_load().orc_plan_calibrated_group(_ptr(q), hq, hkv, d, _ptr(lo), _ptr(hi),
                                             _ptr(hist), _ptr(b), _ptr(out)),
           "plan_calibrated_group")
    return out


# ---- per-block ranges (reading R22) -------------------------------------------
RANGE_BLOCK = 2048


def range_blocks(n: int) -> int:
    return int(_load().orc_range_blocks(n))


def pack_blocked(keys: np.ndarray, nbc=None):
    """keys [n][hkv][d] -> dict(planes [hkv][d][4][W] uint32, lo/hi [hkv][nbc][d]
    fp32 per 2048-key block, sigma2 [hkv][d] fp32 (pooled within-block))."""
    k = np.ascontiguousarray(keys, dtype=np.float32)
    n, hkv, d = k.shape
    nb = range_blocks(n)
    nbc = nb if nbc is None else nbc
    W = plane_words(n)
    planes = np.zeros((hkv, d, 4, W), np.uint32)
    lo = np.zeros((hkv, nbc, d), np.float32)
    hi = np.zeros((hkv, nbc, d), np.float32)
    s2 = np.zeros((hkv, d), np.float32)
    _check(_load().orc_pack_blocked(_ptr(k), n, hkv, d, hkv * d, d, _ptr(planes), _ptr(lo),
                                    _ptr(hi), nbc, _ptr(s2)), "pack_blocked")
    return {"planes": planes, "lo": lo, "hi": hi, "sigma2": s2}


def scan_blocked(planes, lo, hi, n: int, q, plan_):
    """Logits [hq][n] fp32 of a layer packed with per-block ranges lo/hi
    [hkv][nbc][d]."""
    planes = np.ascontiguousarray(planes, dtype=np.uint32)
    lo = np.ascontiguousarray(lo, dtype=np.float32)
    hi = np.ascontiguousarray(hi, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    plan_ = np.ascontiguousarray(plan_, dtype=np.uint8)
    hkv, nbc, d = lo.shape
    hq = q.shape[0]
    out = np.zeros((hq, max(n, 1)), np.float32)
    _check(_load().orc_scan_blocked(_ptr(planes), _ptr(lo), _ptr(hi), nbc, n, hkv, d, _ptr(q),
                                    _ptr(plan_), hq, _ptr(out), out.shape[1]), "scan_blocked")
    return out[:, :n]


def scan_blocked_at(planes, lo, hi, n: int, q, plan_, keys):
    planes = np.ascontiguousarray(planes, dtype=np.uint32)
    lo = np.ascontiguousarray(lo, dtype=np.float32)
    hi = np.ascontiguousarray(hi, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    plan_ = np.ascontiguousarray(plan_, dtype=np.uint8)
    keys = np.ascontiguousarray(keys, dtype=np.int64)
    hkv, nbc, d = lo.shape
    hq = q.shape[0]
    out = np.zeros((hq, keys.size), np.float32)
    _check(_load().orc_scan_blocked_at(_ptr(planes), _ptr(lo), _ptr(hi), nbc, n, hkv, d,
                                       _ptr(q), _ptr(plan_), hq, _ptr(keys), keys.size,
                                       _ptr(out)), "scan_blocked_at")
    return out


def append_blocked(keys_new, n_old: int, planes, lo, hi):
    """Append keys_new [m][hkv][d] as tokens n_old.. in place into planes
    [hkv][d][4][W] and per-block ranges lo/hi [hkv][nbc][d] (reading R22);
    returns the number of clamped values."""
    k = np.ascontiguousarray(keys_new, dtype=np.float32)
    m, hkv, d = k.shape
    assert planes.flags.c_contiguous and planes.dtype == np.uint32
    assert lo.flags.c_contiguous and hi.flags.c_contiguous
    W = planes.shape[-1]
    nbc = lo.shape[1]
    cnt = np.zeros(1, np.int64)
    _check(_load().orc_append_blocked(_ptr(k), m, hkv, d, hkv * d, d, n_old, _ptr(planes), W,
                                      _ptr(lo), _ptr(hi), nbc, _ptr(cnt)), "append_blocked")
    return int(cnt[0])
