"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, computes sizes, and rejects bad arguments on the host before any
launch.  fathom_plan_stats is host-only and is checked against plans from the
oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fathom.h")


@pytest.fixture(scope="module")
def L():
    import sparse_top_key_amd as fathom
    if not os.path.exists(fathom.LIB_PATH):
        from sparse_top_key_amd import build
        build.build()
    return fathom.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int32_t|int64_t|const char \*)\s*(fathom_\w+)\(",
                                 text, re.M)))


def test_header_declares_the_path():
    names = declared_functions()
    for f in ("fathom_pack", "fathom_plan", "fathom_plan_fixed", "fathom_plan_rd",
              "fathom_plan_group", "fathom_sparse_attention", "fathom_append",
              "fathom_code_hist", "fathom_plan_calibrated", "fathom_plan_calibrated_group",
              "fathom_scan",
              "fathom_topk", "fathom_scan_batched", "fathom_topk_batched",
              "fathom_read_prefixes", "fathom_plan_stats", "fathom_probe_read",
              "fathom_probe_scan_traffic", "fathom_topk_noalloc"):
        assert f in names


def test_library_exports_every_declared_symbol(L):
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_top_key_amd", "libfathom.so"))
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_sizes(L):
    assert L.fathom_abi_version() == 2
    for n in (1, 31, 32, 2047, 2048, 2049, 1 << 20):
        W = 64 * ((n + 2047) // 2048)
        assert L.fathom_plane_words(n) == W
        assert L.fathom_planes_bytes(n, 8, 128) == 8 * 128 * 4 * W * 4
    assert L.fathom_pack_workspace_bytes(1 << 20, 8, 128) > 0
    assert L.fathom_pack_workspace_bytes(0, 8, 128) == 0
    assert L.fathom_pack_workspace_bytes(10, 8, 64) == 0
    assert L.fathom_topk_workspace_bytes(32, 2048) >= 32 * 8192 * 8
    assert L.fathom_topk_workspace_bytes(32, 2049) == 0
    assert L.fathom_topk_workspace_bytes(0, 16) == 0


DUMMY = ctypes.c_void_p(0x1000)


def err(L):
    return L.fathom_last_error().decode()


def test_plan_validation(L):
    b = (ctypes.c_int32 * 4)(92, 92, 92, 92)
    assert L.fathom_plan(None, 4, 1, 128, DUMMY, b, DUMMY, None) == 1
    assert L.fathom_plan(DUMMY, 4, 3, 128, DUMMY, b, DUMMY, None) == 1
    assert "multiple" in err(L)
    assert L.fathom_plan(DUMMY, 4, 1, 64, DUMMY, b, DUMMY, None) == 2
    bad = (ctypes.c_int32 * 4)(92, 513, 92, 92)
    assert L.fathom_plan(DUMMY, 4, 1, 128, DUMMY, bad, DUMMY, None) == 1
    assert "budget_bits[1] = 513" in err(L)
    neg = (ctypes.c_int32 * 4)(92, 0, -1, 92)
    assert L.fathom_plan(DUMMY, 4, 1, 128, DUMMY, neg, DUMMY, None) == 1
    assert L.fathom_plan_fixed(DUMMY, 4, 128, 129, DUMMY, None) == 1
    assert L.fathom_plan_fixed(DUMMY, 4, 128, -1, DUMMY, None) == 1


def test_plan_variant_validation(L):
    b = (ctypes.c_int32 * 4)(92, 92, 92, 92)
    assert L.fathom_plan_rd(None, 4, 1, 128, DUMMY, b, DUMMY, None) == 1
    assert L.fathom_plan_rd(DUMMY, 4, 3, 128, DUMMY, b, DUMMY, None) == 1
    assert L.fathom_plan_rd(DUMMY, 4, 1, 64, DUMMY, b, DUMMY, None) == 2
    bad = (ctypes.c_int32 * 4)(92, 92, 92, 513)
    assert L.fathom_plan_rd(DUMMY, 4, 1, 128, DUMMY, bad, DUMMY, None) == 1
    assert "fathom_plan_rd: budget_bits[3] = 513" in err(L)
    # the group plan reads one budget per kv head: hkv = 2 checks entries 0, 1
    g = (ctypes.c_int32 * 2)(92, -1)
    assert L.fathom_plan_group(DUMMY, 4, 2, 128, DUMMY, g, DUMMY, None) == 1
    assert "fathom_plan_group: budget_bits[1] = -1" in err(L)
    assert L.fathom_plan_group(DUMMY, 4, 1, 128, DUMMY, None, DUMMY, None) == 1
    assert L.fathom_plan_group(DUMMY, 6, 4, 128, DUMMY, b, DUMMY, None) == 1
    assert L.fathom_plan_group(DUMMY, 4, 1, 96, DUMMY, b, DUMMY, None) == 2


def test_pack_validation(L):
    args = [DUMMY, 0, 100, 8, 128, 1024, 128, DUMMY, DUMMY, DUMMY, DUMMY]
    ws_need = L.fathom_pack_workspace_bytes(100, 8, 128)
    assert L.fathom_pack(None, *args[1:], DUMMY, ws_need, None) == 1
    assert L.fathom_pack(DUMMY, 7, *args[2:], DUMMY, ws_need, None) == 1
    a0 = list(args)
    a0[2] = 0
    assert L.fathom_pack(*a0, DUMMY, ws_need, None) == 1
    a1 = list(args)
    a1[4] = 96
    assert L.fathom_pack(*a1, DUMMY, ws_need, None) == 2
    assert L.fathom_pack(*args, DUMMY, ws_need - 1, None) == 4
    assert L.fathom_pack(*args, None, ws_need, None) == 4


def test_scan_validation(L):
    base = [DUMMY, DUMMY, DUMMY, 100, 8, 128, DUMMY, DUMMY, 32, None, 0.0, DUMMY, 100, None]
    a = list(base)
    a[8] = 30                                     # hq not a multiple of hkv
    assert L.fathom_scan(*a) == 1
    a = list(base)
    a[12] = 99                                    # ld < n
    assert L.fathom_scan(*a) == 1
    a = list(base)
    a[0] = None
    assert L.fathom_scan(*a) == 1
    a = list(base)
    a[5] = 256
    assert L.fathom_scan(*a) == 2
    a = list(base)
    a[3] = -1
    assert L.fathom_scan(*a) == 1


def test_topk_validation(L):
    ws = L.fathom_topk_workspace_bytes(32, 64)
    base = [DUMMY, 32, 1000, 1000, 1, 64, DUMMY, DUMMY, DUMMY, ws, None]
    a = list(base)
    a[5] = 0
    assert L.fathom_topk(*a) == 1
    a[5] = 2049
    assert L.fathom_topk(*a) == 1
    a = list(base)
    a[4] = 3                                      # 32 rows not a multiple of 3
    assert L.fathom_topk(*a) == 1
    a = list(base)
    a[3] = 999                                    # ld < n
    assert L.fathom_topk(*a) == 1
    a = list(base)
    a[9] = ws - 1
    assert L.fathom_topk(*a) == 4
    a = list(base)
    a[6] = None
    assert L.fathom_topk(*a) == 1


def test_topk_noalloc_validation(L):
    # every rejection happens on the host, before the scratch array is looked up
    base = [DUMMY, 32, 1000, 1000, 1, 64, DUMMY, DUMMY, None]
    a = list(base)
    a[5] = 2049
    assert L.fathom_topk_noalloc(*a) == 1
    a = list(base)
    a[4] = 3
    assert L.fathom_topk_noalloc(*a) == 1
    a = list(base)
    a[3] = 999
    assert L.fathom_topk_noalloc(*a) == 1
    a = list(base)
    a[6] = None
    assert L.fathom_topk_noalloc(*a) == 1
    a = list(base)
    a[1] = 65                                     # 65 output rows > 64 held
    assert L.fathom_topk_noalloc(*a) == 4
    assert "exceed" in err(L)


def test_batched_validation(L):
    import sparse_top_key_amd as fathom
    arr = (fathom._Session * 2)()
    assert L.fathom_scan_batched(arr, 0, 8, 128, 32, None) == 1
    assert L.fathom_scan_batched(arr, 65, 8, 128, 32, None) == 1
    arr[0].n = 10                                 # n > 0 with null pointers
    assert L.fathom_scan_batched(arr, 2, 8, 128, 32, None) == 1
    assert L.fathom_topk_batched(arr, 2, 32, 4, 0, DUMMY, 1 << 30, None) == 1


def test_scan_topk_validation(L):
    import sparse_top_key_amd as fathom
    ns = (ctypes.c_int64 * 1)(1000)
    ws = L.fathom_scan_topk_workspace_bytes(ns, 1, 8, 32, 1, 64)
    # candidate lists of 32 rows + full logits of the 32 rows (fallback)
    assert ws >= 32 * 8192 * 8 + 32 * 1000 * 4
    assert L.fathom_scan_topk_workspace_bytes(ns, 1, 8, 30, 1, 64) == 0   # hq % hkv
    assert L.fathom_scan_topk_workspace_bytes(ns, 1, 8, 32, 3, 64) == 0   # hq % group
    assert L.fathom_scan_topk_workspace_bytes(ns, 1, 8, 32, 1, 2049) == 0
    assert L.fathom_scan_topk_workspace_bytes(None, 1, 8, 32, 1, 64) == 0
    assert L.fathom_scan_topk_workspace_bytes(ns, 0, 8, 32, 1, 64) == 0
    neg = (ctypes.c_int64 * 1)(-5)
    assert L.fathom_scan_topk_workspace_bytes(neg, 1, 8, 32, 1, 64) == 0
    base = [DUMMY, DUMMY, DUMMY, 1000, 8, 128, DUMMY, DUMMY, 32, None, 0.0, 1, 64,
            DUMMY, DUMMY, DUMMY, ws, None]
    for pos, val, code in ((12, 0, 1), (12, 2049, 1), (11, 3, 1), (16, ws - 1, 4),
                           (0, None, 1), (13, None, 1), (14, None, 1), (5, 64, 2),
                           (8, 30, 1), (3, -1, 1), (15, None, 4)):
        a = list(base)
        a[pos] = val
        assert L.fathom_scan_topk(*a) == code, (pos, val)
    arr = (fathom._Session * 2)()
    assert L.fathom_scan_topk_batched(arr, 0, 8, 128, 32, 1, 64, DUMMY, 1 << 40, None) == 1
    assert L.fathom_scan_topk_batched(arr, 65, 8, 128, 32, 1, 64, DUMMY, 1 << 40, None) == 1
    assert L.fathom_scan_topk_batched(None, 1, 8, 128, 32, 1, 64, DUMMY, 1 << 40, None) == 1
    arr[0].n = 10                                 # n > 0 with null pointers
    assert L.fathom_scan_topk_batched(arr, 2, 8, 128, 32, 1, 64, DUMMY, 1 << 40, None) == 1


def test_probe_validation(L):
    assert L.fathom_probe_read(None, 16, DUMMY, 0, None) == 1
    assert L.fathom_probe_read(DUMMY, 17, DUMMY, 0, None) == 1
    assert L.fathom_probe_read(ctypes.c_void_p(0x1008), 16, DUMMY, 0, None) == 1
    # scan-traffic probe: every argument is checked before anything is launched
    st = L.fathom_probe_scan_traffic
    assert st(None, 4096, 2, DUMMY, 4, DUMMY, 4096, DUMMY, None) == 1
    assert st(DUMMY, 4096, 2, None, 4, DUMMY, 4096, DUMMY, None) == 1
    assert st(DUMMY, 4096, 2, DUMMY, 4, DUMMY, 4096, None, None) == 1
    assert st(DUMMY, 0, 2, DUMMY, 4, DUMMY, 4096, DUMMY, None) == 1
    assert st(DUMMY, 4095, 2, DUMMY, 4, DUMMY, 4096, DUMMY, None) == 1
    assert st(DUMMY, 4096, 0, DUMMY, 4, DUMMY, 4096, DUMMY, None) == 1
    assert st(DUMMY, 4096, 65, DUMMY, 4, DUMMY, 4096, DUMMY, None) == 1
    assert st(DUMMY, 4096, 2, DUMMY, 17, DUMMY, 4096, DUMMY, None) == 1
    assert st(DUMMY, 4096, 2, DUMMY, -1, DUMMY, 4096, DUMMY, None) == 1
    assert st(DUMMY, 4096, 2, DUMMY, 4, None, 4096, DUMMY, None) == 1
    assert st(DUMMY, 4096, 2, DUMMY, 4, DUMMY, 4095, DUMMY, None) == 1
    assert st(DUMMY, 4096, 2, DUMMY, 4, DUMMY, 4098, DUMMY, None) == 1
    assert st(ctypes.c_void_p(0x1008), 4096, 2, DUMMY, 4, DUMMY, 4096, DUMMY, None) == 1
    assert st(DUMMY, 4096, 2, DUMMY, 4, ctypes.c_void_p(0x1004), 4096, DUMMY, None) == 1


@pytest.mark.parametrize("group", [1, 2, 4])
def test_plan_stats_matches_oracle_plans(L, orc, group):
    rng = np.random.default_rng(group)
    hq, hkv, d = 8, 8 // group, 128
    q = rng.standard_normal((hq, d)).astype(np.float32)
    s2 = rng.uniform(0.1, 4, (hkv, d)).astype(np.float32)
    budgets = rng.integers(0, 4 * d + 1, hq).astype(np.int32)
    plan = orc.plan(q, s2, budgets)
    hist = (ctypes.c_uint32 * 5)()
    ub = (ctypes.c_uint32 * (hq // group))()
    assert L.fathom_plan_stats(plan.ctypes.data_as(ctypes.c_void_p), hq, d, group, hist, ub) == 0
    exp_hist = [int((plan == t).sum()) for t in range(5)]
    assert list(hist) == exp_hist
    exp_ub = [int(plan[g * group:(g + 1) * group].max(0).sum()) for g in range(hq // group)]
    assert list(ub) == exp_ub
    bad = plan.copy()
    bad[0, 0] = 5
    assert L.fathom_plan_stats(bad.ctypes.data_as(ctypes.c_void_p), hq, d, group, hist, ub) == 1


def test_product_path_refuses_to_run_without_gpu():
    import torch

    import sparse_top_key_amd as fathom
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    with pytest.raises(fathom.FathomError):
        fathom.pack(torch.zeros((64, 1, 128), dtype=torch.float16))


def test_attention_validation(L):
    A = ctypes.c_void_p(0x10000)                  # 16-byte aligned dummy
    U = ctypes.c_void_p(0x10008)                  # 8-byte aligned only
    ws = L.fathom_attention_workspace_bytes(8, 2048)
    assert ws == 8 * 32 * 130 * 4                 # 32 partials of 64 entries per head
    assert L.fathom_attention_workspace_bytes(8, 9000) == 8 * 36 * 130 * 4  # 256 per partial
    assert L.fathom_attention_workspace_bytes(8, -1) == 0
    base = [A, 8, 2, 128, A, A, 0, 1000, 256, 128, A, 1, 2048, ctypes.c_float(0.1), A, A, A,
            ws, None]

    def call(**kw):
        # every case below fails validation, so nothing is ever enqueued
        a = list(base)
        pos = dict(q=0, hq=1, hkv=2, d=3, kc=4, vc=5, dtype=6, n=7, st=8, sh=9, idx=10,
                   group=11, k=12, scale=13, ws=16, wsb=17)
        for key, v in kw.items():
            a[pos[key]] = v
        return L.fathom_sparse_attention(*a)
    assert call(q=None) == 1
    assert call(hkv=3) == 1
    assert call(d=64) == 2
    assert call(dtype=5) == 1
    assert call(kc=None) == 1
    assert call(group=3) == 1                     # does not divide hq / hkv = 4
    assert call(group=8) == 1
    assert call(kc=U) == 2 and "16-byte" in err(L)
    assert call(st=260) == 2
    assert call(k=-1) == 1
    assert call(wsb=ws - 1) == 4
    assert call(scale=ctypes.c_float(float("inf"))) == 1
    assert call(n=-1) == 1


def test_append_validation(L):
    A = ctypes.c_void_p(0x10000)
    # every case below fails validation, so nothing is ever enqueued
    base = [A, 0, 10, 8, 128, 1024, 128, 4090, A, 128, A, A, None, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return L.fathom_append(*a)
    assert call(0, None) == 1                    # keys
    assert call(1, 3) == 1                       # dtype
    assert call(3, 0) == 1                       # hkv
    assert call(4, 64) == 2                      # d
    assert call(2, -1) == 1                      # m
    assert call(9, 64) == 1 and "plane_words" in err(L)   # 4100 keys need 192 words
    assert call(9, 200) == 1                     # not a multiple of 64
    assert call(8, None) == 1                    # planes
    assert call(7, -5) == 1                      # n_old


def test_session_plane_words_validation(L):
    from sparse_top_key_amd import _Session
    A = 0x10000
    s = (_Session * 1)()
    s[0] = _Session(A, A, A, 5000, A, A, None, 0.0, A, 5000, None, None, 64)
    assert L.fathom_scan_batched(s, 1, 8, 128, 32, None) == 1   # 5000 keys need 192 words
    assert "plane_words" in err(L)
    s[0] = _Session(A, A, A, 5000, A, A, None, 0.0, A, 5000, None, None, 200)
    assert L.fathom_scan_batched(s, 1, 8, 128, 32, None) == 1   # not a multiple of 64


def test_calibrated_validation(L):
    A = ctypes.c_void_p(0x10000)
    U = ctypes.c_void_p(0x10004)
    # every case below fails validation, so nothing is ever enqueued
    assert L.fathom_code_hist(None, 100, 8, 128, 0, A, None) == 1
    assert L.fathom_code_hist(A, 100, 8, 64, 0, A, None) == 2
    assert L.fathom_code_hist(A, -1, 8, 128, 0, A, None) == 1
    assert L.fathom_code_hist(A, 5000, 8, 128, 64, A, None) == 1    # 5000 keys need 192 words
    assert L.fathom_code_hist(U, 100, 8, 128, 0, A, None) == 2 and "16-byte" in err(L)
    b = (ctypes.c_int32 * 4)(92, 92, 600, 92)
    assert L.fathom_plan_calibrated(A, 4, 1, 128, A, A, A, b, A, None) == 1
    assert "budget_bits[2] = 600" in err(L)
    assert L.fathom_plan_calibrated(A, 4, 3, 128, A, A, A, b, A, None) == 1
    assert L.fathom_plan_calibrated(A, 4, 1, 128, A, A, None, b, A, None) == 1
    g = (ctypes.c_int32 * 2)(92, 513)            # one budget per kv head
    assert L.fathom_plan_calibrated_group(A, 4, 2, 128, A, A, A, g, A, None) == 1
    assert "budget_bits[1] = 513" in err(L)
    assert L.fathom_plan_calibrated_group(A, 4, 3, 128, A, A, A, g, A, None) == 1


def test_blocked_sizes(L):
    for n, nb in ((0, 0), (1, 1), (2047, 1), (2048, 1), (2049, 2), (1 << 31, 1 << 20)):
        assert L.fathom_range_blocks(n) == nb
    assert L.fathom_pack_blocked_workspace_bytes(5000, 8, 128) == 3 * 8 * 128 * 8
    assert L.fathom_pack_blocked_workspace_bytes(0, 8, 128) == 0
    assert L.fathom_pack_blocked_workspace_bytes(10, 8, 64) == 0


def test_pack_blocked_validation(L):
    A = ctypes.c_void_p(0x10000)
    ws = L.fathom_pack_blocked_workspace_bytes(5000, 8, 128)
    # every case below fails validation, so nothing is ever enqueued
    base = [A, 0, 5000, 8, 128, 1024, 128, A, A, A, 3, A, A, ws, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return L.fathom_pack_blocked(*a)
    assert call(0, None) == 1                    # keys
    assert call(8, None) == 1                    # lo
    assert call(1, 5) == 1                       # dtype
    assert call(2, 0) == 1                       # n
    assert call(4, 96) == 2                      # d
    assert call(10, 2) == 1 and "range_stride" in err(L)   # 5000 keys span 3 blocks
    assert call(10, (1 << 20) + 1) == 1          # above 2^20
    assert call(13, ws - 1) == 4                 # workspace
    assert call(12, None) == 4


def test_append_blocked_validation(L):
    A = ctypes.c_void_p(0x10000)
    base = [A, 0, 10, 8, 128, 1024, 128, 4090, A, 192, A, A, 3, None, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return L.fathom_append_blocked(*a)
    assert call(0, None) == 1                    # keys
    assert call(10, None) == 1                   # lo
    assert call(4, 64) == 2                      # d
    assert call(9, 64) == 1 and "plane_words" in err(L)
    assert call(12, 1) == 1 and "range_stride" in err(L)   # 4100 keys span 3 blocks
    assert call(12, 0) == 1
    assert call(7, -1) == 1                      # n_old


def test_scan_blocked_validation(L):
    A = ctypes.c_void_p(0x10000)
    base = [A, A, A, 3, 5000, 8, 128, A, A, 32, 0, A, 5000, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return L.fathom_scan_blocked(*a)
    assert call(3, 2) == 1 and "range_stride" in err(L)
    assert call(3, (1 << 20) + 1) == 1
    assert call(9, 30) == 1                      # hq not a multiple of hkv
    assert call(6, 256) == 2                     # d
    assert call(12, 4999) == 1                   # ld < n
    assert call(10, 100) == 1                    # plane_words
    assert call(0, None) == 1


def test_scan_topk_blocked_validation(L):
    A = ctypes.c_void_p(0x10000)
    ws = L.fathom_scan_topk_workspace_bytes((ctypes.c_int64 * 1)(5000), 1, 8, 32, 1, 64)
    base = [A, A, A, 3, 5000, 8, 128, A, A, 32, 0, 1, 64, A, A, A, ws, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return L.fathom_scan_topk_blocked(*a)
    assert call(3, 2) == 1 and "range_stride" in err(L)
    assert call(12, 0) == 1                      # k
    assert call(12, 4096) == 1
    assert call(11, 3) == 1                      # group does not divide hq
    assert call(16, ws - 1) == 4                 # workspace
    assert call(13, None) == 1                   # idx


def test_meta4_validation(L):
    A = ctypes.c_void_p(0x10000)
    base = [A, A, A, 5000, 8, 128, A, A, 32, A, 0.5, A, 5000, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return L.fathom_scan_meta4(*a)
    assert call(9, None) == 1 and "side stream" in err(L)   # meta4 required
    assert call(8, 30) == 1                      # hq not a multiple of hkv
    assert call(5, 64) == 2                      # d
    assert call(12, 4999) == 1                   # ld < n
    ws = L.fathom_scan_topk_workspace_bytes((ctypes.c_int64 * 1)(5000), 1, 8, 32, 1, 64)
    tbase = [A, A, A, 5000, 8, 128, A, A, 32, A, 0.5, 1, 64, A, A, A, ws, None]

    def tcall(i, v):
        a = list(tbase)
        a[i] = v
        return L.fathom_scan_topk_meta4(*a)
    assert tcall(9, None) == 1
    assert tcall(12, 0) == 1                     # k
    assert tcall(16, ws - 1) == 4                # workspace

