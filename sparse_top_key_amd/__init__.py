"""Python binding of libfathom (Fathom's per-query bit-depth top-k key scan on
MI355X).  Argument marshalling only: torch tensors provide device memory and
the current HIP stream; every step of the path runs in the library's HIP
kernels.  There is no CPU fallback: without the built library or a GPU every
call raises.

    planes, lo, hi, sigma2 = pack(keys)            # keys [n][hkv][128] fp16/fp32
    plan_ = plan(q, sigma2, budget=92)              # q [hq][128] fp32
    logits = scan(planes, lo, hi, n, q, plan_)      # [hq][n] fp32
    idx, vals = topk(logits, k=2048)                # [hq][k]
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfathom.so")

D = 128
MAX_K = 2048
MAX_SESSIONS = 64
F16, F32 = 0, 1
_ERRORS = {1: "invalid argument", 2: "unsupported", 3: "HIP error", 4: "workspace"}

_lib = None


class FathomError(RuntimeError):
    pass


class _Session(ctypes.Structure):
    _fields_ = [
        ("planes", ctypes.c_void_p), ("lo", ctypes.c_void_p), ("hi", ctypes.c_void_p),
        ("n", ctypes.c_int64), ("q", ctypes.c_void_p), ("plan", ctypes.c_void_p),
        ("meta", ctypes.c_void_p), ("meta_scale", ctypes.c_float),
        ("logits", ctypes.c_void_p), ("ld_logits", ctypes.c_int64),
        ("idx", ctypes.c_void_p), ("vals", ctypes.c_void_p),
        ("plane_words", ctypes.c_int64),
    ]


def lib():
    """Load libfathom.so (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FathomError(f"{LIB_PATH} is not built; run "
                              "`python -m sparse_top_key_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        sig = {
            "fathom_abi_version": (I32, []),
            "fathom_last_error": (ctypes.c_char_p, []),
            "fathom_plane_words": (I64, [I64]),
            "fathom_planes_bytes": (I64, [I64, I32, I32]),
            "fathom_pack_workspace_bytes": (I64, [I64, I32, I32]),
            "fathom_topk_workspace_bytes": (I64, [I32, I32]),
            "fathom_pack": (I32, [P, I32, I64, I32, I32, I64, I64, P, P, P, P, P, I64, P]),
            "fathom_plan": (I32, [P, I32, I32, I32, P, P, P, P]),
            "fathom_plan_fixed": (I32, [P, I32, I32, I32, P, P]),
            "fathom_plan_rd": (I32, [P, I32, I32, I32, P, P, P, P]),
            "fathom_plan_group": (I32, [P, I32, I32, I32, P, P, P, P]),
            "fathom_code_hist": (I32, [P, I64, I32, I32, I64, P, P]),
            "fathom_plan_calibrated": (I32, [P, I32, I32, I32, P, P, P, P, P, P]),
            "fathom_plan_calibrated_group": (I32, [P, I32, I32, I32, P, P, P, P, P, P]),
            "fathom_attention_workspace_bytes": (I64, [I32, I32]),
            "fathom_append": (I32, [P, I32, I64, I32, I32, I64, I64, I64, P, I64, P, P, P, P]),
            "fathom_sparse_attention": (I32, [P, I32, I32, I32, P, P, I32, I64, I64, I64, P,
                                              I32, I32, F, P, P, P, I64, P]),
            "fathom_scan": (I32, [P, P, P, I64, I32, I32, P, P, I32, P, F, P, I64, P]),
            "fathom_topk": (I32, [P, I32, I64, I64, I32, I32, P, P, P, I64, P]),
            "fathom_topk_noalloc": (I32, [P, I32, I64, I64, I32, I32, P, P, P]),
            "fathom_scan_batched": (I32, [P, I32, I32, I32, I32, P]),
            "fathom_topk_batched": (I32, [P, I32, I32, I32, I32, P, I64, P]),
            "fathom_read_prefixes": (I32, [P, I64, I32, I32, P, I32, P, P]),
            "fathom_plan_stats": (I32, [P, I32, I32, I32, P, P]),
            "fathom_probe_read": (I32, [P, I64, P, I32, P]),
            "fathom_probe_scan_traffic": (I32, [P, I64, I32, P, I32, P, I64, P, P]),
            "fathom_scan_topk_workspace_bytes": (I64, [P, I32, I32, I32, I32, I32]),
            "fathom_scan_topk": (I32, [P, P, P, I64, I32, I32, P, P, I32, P, F, I32, I32, P, P,
                                       P, I64, P]),
            "fathom_scan_topk_batched": (I32, [P, I32, I32, I32, I32, I32, I32, P, I64, P]),
            "fathom_scan_meta4": (I32, [P, P, P, I64, I32, I32, P, P, I32, P, F, P, I64, P]),
            "fathom_scan_topk_meta4": (I32, [P, P, P, I64, I32, I32, P, P, I32, P, F, I32, I32,
                                             P, P, P, I64, P]),
            "fathom_range_blocks": (I64, [I64]),
            "fathom_pack_blocked_workspace_bytes": (I64, [I64, I32, I32]),
            "fathom_pack_blocked": (I32, [P, I32, I64, I32, I32, I64, I64, P, P, P, I64, P, P,
                                          I64, P]),
            "fathom_append_blocked": (I32, [P, I32, I64, I32, I32, I64, I64, I64, P, I64, P, P,
                                            I64, P, P]),
            "fathom_scan_blocked": (I32, [P, P, P, I64, I64, I32, I32, P, P, I32, I64, P, I64,
                                          P]),
            "fathom_scan_topk_blocked": (I32, [P, P, P, I64, I64, I32, I32, P, P, I32, I64, I32,
                                               I32, P, P, P, I64, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


_GPU_SEEN = False


def _require_gpu(*ts: torch.Tensor):
    global _GPU_SEEN
    if not _GPU_SEEN:
        if not torch.cuda.is_available():
            raise FathomError("libfathom needs a ROCm GPU (none visible)")
        _GPU_SEEN = True
    for t in ts:
        if t is not None and not (t.is_cuda or t.is_pinned()):
            raise FathomError("tensor must be on the GPU (or pinned host memory)")


def _check(rc: int, name: str):
    if rc != 0:
        msg = lib().fathom_last_error().decode()
        raise FathomError(f"{name}: {_ERRORS.get(rc, rc)}: {msg}")


# The current stream's raw handle straight from torch's C layer (about 0.1 us
# per call against about 2 us for building a Stream object), where it exists.
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device=None):
    if _RAW_STREAM is None:
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    if device is None or device.index is None:
        index = torch.cuda.current_device()
    else:
        index = device.index
    return ctypes.c_void_p(_RAW_STREAM(index))


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def plane_words(n: int) -> int:
    return int(lib().fathom_plane_words(n))


def pack_workspace_bytes(n: int, hkv: int) -> int:
    return int(lib().fathom_pack_workspace_bytes(n, hkv, D))


def topk_workspace_bytes(out_rows: int, k: int) -> int:
    return int(lib().fathom_topk_workspace_bytes(out_rows, k))


@dataclass
class Packed:
    planes: torch.Tensor   # uint32 [hkv][d][4][W] (stored as int32)
    lo: torch.Tensor       # fp32 [hkv][d]
    hi: torch.Tensor
    sigma2: torch.Tensor
    n: int


def pack(keys: torch.Tensor, planes: Optional[torch.Tensor] = None,
         ws: Optional[torch.Tensor] = None) -> Packed:
    """keys [n][hkv][d] (fp16/fp32, any token/head strides, channel stride 1)."""
    _require_gpu(keys)
    n, hkv, d = keys.shape
    if keys.stride(2) != 1:
        raise FathomError("pack: channel stride must be 1")
    dt = {torch.float16: F16, torch.float32: F32}.get(keys.dtype)
    if dt is None:
        raise FathomError("pack: keys must be fp16 or fp32")
    dev = keys.device
    W = plane_words(n)
    if planes is None:
        planes = torch.empty((hkv, d, 4, W), dtype=torch.int32, device=dev)
    lo = torch.empty((hkv, d), dtype=torch.float32, device=dev)
    hi = torch.empty_like(lo)
    s2 = torch.empty_like(lo)
    need = pack_workspace_bytes(n, hkv) if n > 0 else 0
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib().fathom_pack(_p(keys), dt, n, hkv, d, keys.stride(0), keys.stride(1),
                             _p(planes), _p(lo), _p(hi), _p(s2), _p(ws), ws.numel(),
                             _stream(dev)), "fathom_pack")
    return Packed(planes, lo, hi, s2, n)


def _budgets(budget, count: int):
    vals = [int(budget)] * count if isinstance(budget, int) else [int(x) for x in budget]
    if len(vals) != count:
        raise ValueError(f"expected {count} budgets, got {len(vals)}")
    return (ctypes.c_int32 * count)(*vals)


def _plan_call(fn: str, q, sigma2, budget, n_budgets: int, out):
    _require_gpu(q, sigma2)
    hq, d = q.shape
    hkv = sigma2.shape[0]
    b = _budgets(budget, hq if n_budgets < 0 else n_budgets)
    if out is None:
        out = torch.empty((hq, d), dtype=torch.uint8, device=q.device)
    _check(getattr(lib(), fn)(_p(q.contiguous()), hq, hkv, d, _p(sigma2.contiguous()), b,
                              _p(out), _stream(q.device)), fn)
    return out


def plan(q: torch.Tensor, sigma2: torch.Tensor, budget, out=None) -> torch.Tensor:
    """q [hq][d] fp32, sigma2 [hkv][d] fp32, budget int or sequence of hq ints."""
    return _plan_call("fathom_plan", q, sigma2, budget, -1, out)


def plan_rd(q: torch.Tensor, sigma2: torch.Tensor, budget, out=None) -> torch.Tensor:
    """Rate-distortion allocation; arguments as for plan."""
    return _plan_call("fathom_plan_rd", q, sigma2, budget, -1, out)


def plan_group(q: torch.Tensor, sigma2: torch.Tensor, budget, out=None) -> torch.Tensor:
    """One plan per GQA group; budget int or sequence of hkv ints."""
    return _plan_call("fathom_plan_group", q, sigma2, budget, sigma2.shape[0], out)


def code_hist(planes: torch.Tensor, n: int, out=None) -> torch.Tensor:
    """Histogram of the 4-bit codes per (kv head, channel) -> int32 [hkv][d][16]
    (counts, stored as int32)."""
    _require_gpu(planes)
    hkv, d = planes.shape[0], planes.shape[1]
    if out is None:
        out = torch.empty((hkv, d, 16), dtype=torch.int32, device=planes.device
                          if planes.is_cuda else "cuda")
    _check(lib().fathom_code_hist(_p(planes), n, hkv, d, planes.shape[-1], _p(out),
                                  _stream(out.device)), "fathom_code_hist")
    return out


def plan_calibrated(q: torch.Tensor, lo: torch.Tensor, hi: torch.Tensor, hist: torch.Tensor,
                    budget, out=None) -> torch.Tensor:
    """Calibrated allocation (exact DP on measured per-depth errors); budget int
    or sequence of hq ints."""
    _require_gpu(q, lo, hist)
    hq, d = q.shape
    hkv = lo.shape[0]
    b = _budgets(budget, hq)
    if out is None:
        out = torch.empty((hq, d), dtype=torch.uint8, device=q.device)
    _check(lib().fathom_plan_calibrated(_p(q.contiguous()), hq, hkv, d, _p(lo.contiguous()),
                                        _p(hi.contiguous()), _p(hist.contiguous()), b, _p(out),
                                        _stream(q.device)), "fathom_plan_calibrated")
    return out


def plan_calibrated_group(q: torch.Tensor, lo: torch.Tensor, hi: torch.Tensor,
                          hist: torch.Tensor, budget, out=None) -> torch.Tensor:
    """One calibrated plan per GQA group; budget int or sequence of hkv ints."""
    _require_gpu(q, lo, hist)
    hq, d = q.shape
    hkv = lo.shape[0]
    b = _budgets(budget, hkv)
    if out is None:
        out = torch.empty((hq, d), dtype=torch.uint8, device=q.device)
    _check(lib().fathom_plan_calibrated_group(_p(q.contiguous()), hq, hkv, d,
                                              _p(lo.contiguous()), _p(hi.contiguous()),
                                              _p(hist.contiguous()), b, _p(out),
                                              _stream(q.device)),
           "fathom_plan_calibrated_group")
    return out


def plan_fixed(q: torch.Tensor, r: int, out=None) -> torch.Tensor:
    _require_gpu(q)
    hq, d = q.shape
    if out is None:
        out = torch.empty((hq, d), dtype=torch.uint8, device=q.device)
    _check(lib().fathom_plan_fixed(_p(q.contiguous()), hq, d, r, _p(out),
                                   _stream(q.device)), "fathom_plan_fixed")
    return out


def _has_capacity(planes: torch.Tensor, n: int) -> bool:
    """Planes laid out for more keys than n (rows longer than plane_words(n))."""
    return planes.dim() == 4 and planes.shape[-1] != plane_words(n)


def scan(planes: torch.Tensor, lo: torch.Tensor, hi: torch.Tensor, n: int,
         q: torch.Tensor, plan_: torch.Tensor, meta: Optional[torch.Tensor] = None,
         meta_scale: float = 0.0, out: Optional[torch.Tensor] = None,
         meta_bits: int = 8) -> torch.Tensor:
    """-> logits [hq][n] fp32.  planes may live in pinned host memory.  meta:
    uint8 [hkv][n] (meta_bits 8) or packed nibbles [hkv][ceil(n/2)] (4)."""
    _require_gpu(planes, lo, q, plan_)
    hkv, d = lo.shape
    hq = q.shape[0]
    if out is None:
        out = torch.empty((hq, max(n, 1)), dtype=torch.float32, device=q.device)
    if meta_bits == 4:
        if _has_capacity(planes, n):
            raise FathomError("scan: the 4-bit side stream takes compact planes")
        _check(lib().fathom_scan_meta4(_p(planes), _p(lo), _p(hi), n, hkv, d, _p(q), _p(plan_),
                                       hq, _p(meta), meta_scale, _p(out), out.stride(0),
                                       _stream(q.device)), "fathom_scan_meta4")
        return out[:, :n]
    if _has_capacity(planes, n):
        scan_batched([Session(planes, lo, hi, n, q, plan_, logits=out, meta=meta,
                              meta_scale=meta_scale)])
        return out[:, :n]
    _check(lib().fathom_scan(_p(planes), _p(lo), _p(hi), n, hkv, d, _p(q), _p(plan_), hq,
                             _p(meta), meta_scale, _p(out), out.stride(0),
                             _stream(q.device)), "fathom_scan")
    return out[:, :n]


def topk(scores: torch.Tensor, k: int, group: int = 1, n: Optional[int] = None,
         ws: Optional[torch.Tensor] = None, idx=None, vals=None):
    """scores [rows][>=n] fp32 (row stride = scores.stride(0)) ->
    (idx int32 [rows/group][k], vals fp32 [rows/group][k])."""
    _require_gpu(scores)
    rows = scores.shape[0]
    n = scores.shape[1] if n is None else n
    ro = rows // group
    dev = scores.device
    if idx is None:
        idx = torch.empty((ro, k), dtype=torch.int32, device=dev)
    if vals is None:
        vals = torch.empty((ro, k), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(max(topk_workspace_bytes(ro, k), 1), dtype=torch.uint8, device=dev)
    ld = max(scores.stride(0), n) if rows > 1 else max(scores.shape[1], n, 1)
    _check(lib().fathom_topk(_p(scores), rows, n, ld, group, k, _p(idx), _p(vals), _p(ws),
                             ws.numel(), _stream(dev)), "fathom_topk")
    return idx, vals


@dataclass
class Session:
    """One decode session of the batched calls (tensors on the GPU unless noted)."""
    planes: torch.Tensor           # device or pinned host
    lo: torch.Tensor
    hi: torch.Tensor
    n: int
    q: torch.Tensor
    plan: torch.Tensor
    logits: Optional[torch.Tensor] = None   # [hq][ld] (not used by scan_topk_batched)
    idx: Optional[torch.Tensor] = None
    vals: Optional[torch.Tensor] = None
    meta: Optional[torch.Tensor] = None
    meta_scale: float = 0.0


def _sessions(sess: Sequence[Session]):
    arr = (_Session * len(sess))()
    for i, s in enumerate(sess):
        arr[i] = _Session(s.planes.data_ptr(), s.lo.data_ptr(), s.hi.data_ptr(), s.n,
                          s.q.data_ptr(), s.plan.data_ptr(),
                          s.meta.data_ptr() if s.meta is not None else None, s.meta_scale,
                          s.logits.data_ptr() if s.logits is not None else None,
                          s.logits.stride(0) if s.logits is not None else 0,
                          s.idx.data_ptr() if s.idx is not None else None,
                          s.vals.data_ptr() if s.vals is not None else None,
                          s.planes.shape[-1])
    return arr


def scan_batched(sess: Sequence[Session]):
    s0 = sess[0]
    hkv, d = s0.lo.shape
    hq = s0.q.shape[0]
    _check(lib().fathom_scan_batched(_sessions(sess), len(sess), hkv, d, hq,
                                     _stream(s0.q.device)), "fathom_scan_batched")


def topk_batched(sess: Sequence[Session], k: int, group: int = 1,
                 ws: Optional[torch.Tensor] = None):
    s0 = sess[0]
    hq = s0.q.shape[0]
    ro = hq // group
    if ws is None:
        ws = torch.empty(max(topk_workspace_bytes(ro * len(sess), k), 1), dtype=torch.uint8,
                         device=s0.q.device)
    _check(lib().fathom_topk_batched(_sessions(sess), len(sess), hq, group, k, _p(ws),
                                     ws.numel(), _stream(s0.q.device)), "fathom_topk_batched")


def scan_topk_workspace_bytes(ns: Sequence[int], hkv: int, hq: int, group: int, k: int) -> int:
    arr = (ctypes.c_int64 * len(ns))(*[int(x) for x in ns])
    return int(lib().fathom_scan_topk_workspace_bytes(arr, len(ns), hkv, hq, group, k))


def scan_topk(planes: torch.Tensor, lo: torch.Tensor, hi: torch.Tensor, n: int,
              q: torch.Tensor, plan_: torch.Tensor, k: int, group: int = 1,
              meta: Optional[torch.Tensor] = None, meta_scale: float = 0.0,
              ws: Optional[torch.Tensor] = None, idx=None, vals=None, meta_bits: int = 8):
    """Scan + top-k in one call -> (idx int32 [hq/group][k], vals fp32 [hq/group][k]),
    the result of scan() followed by topk()."""
    _require_gpu(planes, lo, q, plan_)
    hkv, d = lo.shape
    hq = q.shape[0]
    ro = hq // group
    dev = q.device
    if idx is None:
        idx = torch.empty((ro, k), dtype=torch.int32, device=dev)
    if vals is None:
        vals = torch.empty((ro, k), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(max(scan_topk_workspace_bytes([n], hkv, hq, group, k), 1),
                         dtype=torch.uint8, device=dev)
    if meta_bits == 4:
        if _has_capacity(planes, n):
            raise FathomError("scan_topk: the 4-bit side stream takes compact planes")
        _check(lib().fathom_scan_topk_meta4(_p(planes), _p(lo), _p(hi), n, hkv, d, _p(q),
                                            _p(plan_), hq, _p(meta), meta_scale, group, k,
                                            _p(idx), _p(vals), _p(ws), ws.numel(),
                                            _stream(dev)), "fathom_scan_topk_meta4")
        return idx, vals
    if _has_capacity(planes, n):
        scan_topk_batched([Session(planes, lo, hi, n, q, plan_, idx=idx, vals=vals, meta=meta,
                                   meta_scale=meta_scale)], k, group, ws)
        return idx, vals
    _check(lib().fathom_scan_topk(_p(planes), _p(lo), _p(hi), n, hkv, d, _p(q), _p(plan_), hq,
                                  _p(meta), meta_scale, group, k, _p(idx), _p(vals), _p(ws),
                                  ws.numel(), _stream(dev)), "fathom_scan_topk")
    return idx, vals


def scan_topk_batched(sess: Sequence[Session], k: int, group: int = 1,
                      ws: Optional[torch.Tensor] = None):
    """Scan + top-k of every session into its idx/vals."""
    s0 = sess[0]
    hkv, d = s0.lo.shape
    hq = s0.q.shape[0]
    if ws is None:
        ws = torch.empty(max(scan_topk_workspace_bytes([s.n for s in sess], hkv, hq, group, k),
                             1), dtype=torch.uint8, device=s0.q.device)
    _check(lib().fathom_scan_topk_batched(_sessions(sess), len(sess), hkv, d, hq, group, k,
                                          _p(ws), ws.numel(), _stream(s0.q.device)),
           "fathom_scan_topk_batched")


def append(keys: torch.Tensor, n_old: int, planes: torch.Tensor, lo: torch.Tensor,
           hi: torch.Tensor, clamped: Optional[torch.Tensor] = None) -> None:
    """Write keys [m][hkv][d] (fp16/fp32, channel stride 1) as tokens n_old ..
    n_old+m-1 of planes [hkv][d][4][W] (W a capacity, see alloc_planes), with
    the stored lo/hi.  clamped: optional 1-element int32 device tensor that
    receives the count of values outside [lo, hi] (added to)."""
    _require_gpu(keys, planes, lo)
    m, hkv, d = keys.shape
    if keys.stride(2) != 1:
        raise FathomError("channel stride of keys must be 1")
    dtype = {torch.float16: F16, torch.float32: F32}.get(keys.dtype)
    if dtype is None:
        raise FathomError("keys must be float16 or float32")
    _check(lib().fathom_append(_p(keys), dtype, m, hkv, d, keys.stride(0), keys.stride(1),
                               n_old, _p(planes), planes.shape[-1], _p(lo), _p(hi),
                               _p(clamped), _stream(lo.device)), "fathom_append")


# ---- per-block ranges (one lo/hi per 2048-key block of a channel) ----------

def range_blocks(n: int) -> int:
    return int(lib().fathom_range_blocks(n))


def pack_blocked(keys: torch.Tensor, capacity: Optional[int] = None,
                 ws: Optional[torch.Tensor] = None) -> Packed:
    """keys [n][hkv][d] -> Packed with lo, hi fp32 [hkv][R][d] (R = the range
    blocks of `capacity` keys, default n) and planes [hkv][d][4][W] with room
    for `capacity` keys (zeroed past n)."""
    _require_gpu(keys)
    n, hkv, d = keys.shape
    if keys.stride(2) != 1:
        raise FathomError("pack_blocked: channel stride must be 1")
    dt = {torch.float16: F16, torch.float32: F32}.get(keys.dtype)
    if dt is None:
        raise FathomError("pack_blocked: keys must be fp16 or fp32")
    dev = keys.device
    cap = n if capacity is None else max(int(capacity), n)
    R = max(range_blocks(cap), 1)
    if cap == n:
        planes = torch.empty((hkv, d, 4, plane_words(n)), dtype=torch.int32, device=dev)
    else:
        planes = torch.zeros((hkv, d, 4, plane_words(cap)), dtype=torch.int32, device=dev)
    lo = torch.zeros((hkv, R, d), dtype=torch.float32, device=dev)
    hi = torch.zeros_like(lo)
    s2 = torch.empty((hkv, d), dtype=torch.float32, device=dev)
    need = int(lib().fathom_pack_blocked_workspace_bytes(n, hkv, d)) if n > 0 else 0
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if cap == n:
        _check(lib().fathom_pack_blocked(_p(keys), dt, n, hkv, d, keys.stride(0), keys.stride(1),
                                         _p(planes), _p(lo), _p(hi), R, _p(s2), _p(ws),
                                         ws.numel(), _stream(dev)), "fathom_pack_blocked")
    else:
        # pack into rows of plane_words(n), then place them in the capacity rows
        tmp = torch.empty((hkv, d, 4, plane_words(n)), dtype=torch.int32, device=dev)
        _check(lib().fathom_pack_blocked(_p(keys), dt, n, hkv, d, keys.stride(0), keys.stride(1),
                                         _p(tmp), _p(lo), _p(hi), R, _p(s2), _p(ws),
                                         ws.numel(), _stream(dev)), "fathom_pack_blocked")
        planes[..., :tmp.shape[-1]] = tmp
    return Packed(planes, lo, hi, s2, n)


def append_blocked(keys: torch.Tensor, n_old: int, planes: torch.Tensor, lo: torch.Tensor,
                   hi: torch.Tensor, clamped: Optional[torch.Tensor] = None) -> None:
    """append() for per-block ranges: lo, hi [hkv][R][d] are read and written
    (the blocks the call starts get their ranges first)."""
    _require_gpu(keys, planes, lo)
    m, hkv, d = keys.shape
    if keys.stride(2) != 1:
        raise FathomError("channel stride of keys must be 1")
    dtype = {torch.float16: F16, torch.float32: F32}.get(keys.dtype)
    if dtype is None:
        raise FathomError("keys must be float16 or float32")
    _check(lib().fathom_append_blocked(_p(keys), dtype, m, hkv, d, keys.stride(0),
                                       keys.stride(1), n_old, _p(planes), planes.shape[-1],
                                       _p(lo), _p(hi), lo.shape[1], _p(clamped),
                                       _stream(lo.device)), "fathom_append_blocked")


def scan_blocked(planes: torch.Tensor, lo: torch.Tensor, hi: torch.Tensor, n: int,
                 q: torch.Tensor, plan_: torch.Tensor,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """scan() with per-block ranges lo, hi [hkv][R][d] -> logits [hq][n]."""
    _require_gpu(planes, lo, q, plan_)
    hkv, R, d = lo.shape
    hq = q.shape[0]
    if out is None:
        out = torch.empty((hq, max(n, 1)), dtype=torch.float32, device=q.device)
    _check(lib().fathom_scan_blocked(_p(planes), _p(lo), _p(hi), R, n, hkv, d, _p(q),
                                     _p(plan_), hq, planes.shape[-1], _p(out), out.stride(0),
                                     _stream(q.device)), "fathom_scan_blocked")
    return out[:, :n]


def scan_topk_blocked(planes: torch.Tensor, lo: torch.Tensor, hi: torch.Tensor, n: int,
                      q: torch.Tensor, plan_: torch.Tensor, k: int, group: int = 1,
                      ws: Optional[torch.Tensor] = None, idx=None, vals=None):
    """scan_topk() with per-block ranges lo, hi [hkv][R][d]."""
    _require_gpu(planes, lo, q, plan_)
    hkv, R, d = lo.shape
    hq = q.shape[0]
    ro = hq // group
    dev = q.device
    if idx is None:
        idx = torch.empty((ro, k), dtype=torch.int32, device=dev)
    if vals is None:
        vals = torch.empty((ro, k), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(max(scan_topk_workspace_bytes([n], hkv, hq, group, k), 1),
                         dtype=torch.uint8, device=dev)
    _check(lib().fathom_scan_topk_blocked(_p(planes), _p(lo), _p(hi), R, n, hkv, d, _p(q),
                                          _p(plan_), hq, planes.shape[-1], group, k, _p(idx),
                                          _p(vals), _p(ws), ws.numel(), _stream(dev)),
           "fathom_scan_topk_blocked")
    return idx, vals


def alloc_planes(capacity: int, hkv: int, d: int = D, device="cuda", pin_memory=False):
    """Zeroed planes [hkv][d][4][W] with room for `capacity` keys."""
    W = plane_words(capacity)
    if pin_memory:
        t = torch.zeros((hkv, d, 4, W), dtype=torch.int32, pin_memory=True)
    else:
        t = torch.zeros((hkv, d, 4, W), dtype=torch.int32, device=device)
    return t


def attention_workspace_bytes(hq: int, k: int) -> int:
    return int(lib().fathom_attention_workspace_bytes(hq, k))


def sparse_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     idx: torch.Tensor, group: int = 1, scale: Optional[float] = None,
                     out=None, lse=None, ws=None):
    """Attention of each query head over its selected keys.

    q fp32 [hq][d]; k_cache, v_cache [n][hkv][d] fp16 or fp32 (device or
    pinned host, same strides, channel stride 1); idx int32 [hq/group][k]
    (entries < 0 or >= n skipped).  -> (out fp32 [hq][d], lse fp32 [hq])."""
    _require_gpu(q, k_cache, v_cache, idx)
    hq, d = q.shape
    n, hkv, _ = k_cache.shape
    if k_cache.stride() != v_cache.stride() or k_cache.dtype != v_cache.dtype:
        raise FathomError("k_cache and v_cache must share dtype and strides")
    if k_cache.stride(2) != 1:
        raise FathomError("channel stride of the caches must be 1")
    dtype = {torch.float16: F16, torch.float32: F32}.get(k_cache.dtype)
    if dtype is None:
        raise FathomError("caches must be float16 or float32")
    k = idx.shape[1]
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    dev = q.device
    if out is None:
        out = torch.empty((hq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((hq,), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(max(attention_workspace_bytes(hq, k), 1), dtype=torch.uint8, device=dev)
    _check(lib().fathom_sparse_attention(_p(q.contiguous()), hq, hkv, d, _p(k_cache), _p(v_cache),
                                         dtype, n, k_cache.stride(0), k_cache.stride(1),
                                         _p(idx.contiguous()), group, k, float(scale), _p(out),
                                         _p(lse), _p(ws), ws.numel(), _stream(dev)),
           "fathom_sparse_attention")
    return out, lse


def read_prefixes(planes: torch.Tensor, n: int, plan_: torch.Tensor, hkv: int) -> torch.Tensor:
    _require_gpu(plan_)
    hq, d = plan_.shape
    out = torch.empty((hq, n, d), dtype=torch.uint8, device=plan_.device)
    _check(lib().fathom_read_prefixes(_p(planes), n, hkv, d, _p(plan_), hq, _p(out),
                                      _stream(plan_.device)), "fathom_read_prefixes")
    return out


def plan_stats(plan_host: torch.Tensor, group: int):
    """Host-side: (hist[5] of depths, union bits per group) of a CPU plan copy."""
    p = plan_host.contiguous().cpu()
    hq, d = p.shape
    hist = (ctypes.c_uint32 * 5)()
    ub = (ctypes.c_uint32 * (hq // group))()
    _check(lib().fathom_plan_stats(ctypes.c_void_p(p.data_ptr()), hq, d, group, hist, ub),
           "fathom_plan_stats")
    return list(hist), list(ub)


def probe_read(buf: torch.Tensor, out: torch.Tensor, blocks: int = 0):
    """Stream-read `buf` (device or pinned host) once; out = 1-word device tensor."""
    _check(lib().fathom_probe_read(_p(buf), buf.numel() * buf.element_size(), _p(out),
                                   blocks, _stream(out.device)), "fathom_probe_read")


def probe_scan_traffic(planes: torch.Tensor, n: int, depth: torch.Tensor, rows_out: int,
                       out: Optional[torch.Tensor], sink: torch.Tensor):
    """Move the bytes of an HBM logits scan with no arithmetic: planes [hkv][128][4][n/32]
    on the GPU, depth uint8 [hkv][128] (plane slots read per channel), out fp32 rows
    [hkv*rows_out][>= n] (values meaningless), sink a 1-word device tensor."""
    _require_gpu(planes, depth, sink)
    hkv = planes.shape[0]
    ld = out.stride(0) if out is not None else 0
    _check(lib().fathom_probe_scan_traffic(_p(planes), n, hkv, _p(depth.contiguous()), rows_out,
                                           _p(out), ld, _p(sink), _stream(sink.device)),
           "fathom_probe_scan_traffic")
