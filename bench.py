"""Throughput of Fathom's read path on one MI355X.

One step = one decode step of one layer: fathom_plan (32 query heads, B = 92)
-> fathom_scan (1,048,576 keys x 8 kv heads, union planes of each GQA group)
-> fathom_topk (k = 2048 per query head), on the Qwen3-8B-shaped 1M-token
layer with the K planes in pinned host memory read zero-copy (the offloaded
case), and again with the planes in HBM.  Inputs (keys, queries) are seeded
synthetic data already resident when timing starts; several layers rotate so
that no step re-reads planes still held in the 256 MB last-level cache.

Prints ONE JSON line.  value = key vectors (token x kv head) scored and
selected per second, host-resident.  Also reported: the HBM-resident step,
the in-library fixed 136-bit scan (top-32 |q| channels x 4 bits + an 8-bit
per-key side stream) on identical inputs, streaming-read probes, and the CPU
oracle on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sparse_top_key_amd as fathom  # noqa: E402
import synth  # noqa: E402

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, published
PCIE_PEAK_GBPS = 64.0         # PCIe Gen5 x16, published, one direction
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_traffic.json")
SCAN_SOURCE = os.path.join(ROOT, "sparse_top_key_amd", "csrc", "scan.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Layer:
    """One layer's K cache (planes in HBM and in pinned host memory), its
    queries, plans and output buffers."""

    def __init__(self, w, layer, dev, host, fixed_r):
        keys = synth.keys(w.seed, layer, w.n, w.hkv, w.d, w.dtype, w.outliers, device=dev)
        p = fathom.pack(keys)
        del keys
        self.n = w.n
        self.planes = p.planes
        self.lo, self.hi, self.sigma2 = p.lo, p.hi, p.sigma2
        self.host = None
        if host:
            self.host = torch.empty(p.planes.shape, dtype=p.planes.dtype, pin_memory=True)
            self.host.copy_(p.planes)
        self.q = synth.queries(w.seed, layer, w.hq, w.d, device=dev)
        self.meta = synth.side_stream(w.seed, layer, w.hkv, w.n, device=dev)
        self.meta_host = None
        if host:
            self.meta_host = torch.empty(self.meta.shape, dtype=torch.uint8, pin_memory=True)
            self.meta_host.copy_(self.meta)
        # the r = 16 baseline's 4-bit stream (two keys per byte)
        self.meta4 = synth.side_stream4(w.seed, layer, w.hkv, w.n, device=dev)
        self.meta4_host = None
        if host:
            self.meta4_host = torch.empty(self.meta4.shape, dtype=torch.uint8, pin_memory=True)
            self.meta4_host.copy_(self.meta4)
        self.budget = [w.budget] * w.hq
        self.group_budget = [w.budget] * w.hkv
        self.group_budget176 = [176] * w.hkv     # about the per-head plans' union bits
        self.hist = fathom.code_hist(p.planes, w.n)     # per-layer statistic, like sigma2
        self.plan = torch.empty((w.hq, w.d), dtype=torch.uint8, device=dev)
        self.plan_fixed = fathom.plan_fixed(self.q, fixed_r)
        self.logits = torch.empty((w.hq, w.n), dtype=torch.float32, device=dev)
        self.idx = torch.empty((w.hq, w.k), dtype=torch.int32, device=dev)
        self.vals = torch.empty((w.hq, w.k), dtype=torch.float32, device=dev)


def union_plane_bytes(plan, hkv, n):
    """Plane bytes one scan reads: per kv head, sum_c max_{h in group} t_hc
    bits per key (the planes of a GQA group are read once for the group)."""
    p = plan.cpu()
    hq = p.shape[0]
    hist, ub = fathom.plan_stats(p, hq // hkv)
    return sum(ub) * n // 8, ub, hist


def run_steps(layers, w, ws, steps, mode, fixed=False, fused=False, per_call=True,
              variant=None, with_meta=True, meta_bits=8):
    """mode: 'host' or 'hbm'.  fused: fathom_scan_topk in place of fathom_scan
    then fathom_topk (ws must then be its workspace).  fixed: True (r = 32,
    the 136-bit baseline) or the baseline's channel count r.  variant: None (the
    fill-to-cap walk), 'rd' (rate-distortion plan) or 'group' (one plan per
    GQA group, budget B per kv head).  with_meta: the fixed baselines read
    their side stream (8-bit: fixed-136, or the r = 16 form at 72 bits; 4-bit,
    meta_bits 4: the r = 16 form at 68 bits); without it, r = 32 is
    fixed-128.  per_call: events around
    every call (for the per-call times); otherwise none, since an event
    recorded between two calls stalls the stream for a few microseconds.
    Returns the per-step event lists (empty lists when per_call is off)."""
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] if per_call else []
          for _ in range(steps)]
    for s in range(steps):
        L = layers[s % len(layers)]
        planes = L.host if mode == "host" else L.planes
        meta = None
        if fixed and with_meta and meta_bits == 4:
            meta = L.meta4_host if mode == "host" else L.meta4
        elif fixed and with_meta:
            meta = L.meta_host if mode == "host" else L.meta
        e = ev[s]
        if per_call:
            e[0].record()
        if fixed:                                     # query-only plan of the baselines
            plan = fathom.plan_fixed(L.q, 32 if fixed is True else int(fixed), out=L.plan)
        elif variant == "rd":
            plan = fathom.plan_rd(L.q, L.sigma2, L.budget, out=L.plan)
        elif variant == "group":
            plan = fathom.plan_group(L.q, L.sigma2, L.group_budget, out=L.plan)
        elif variant == "calibrated":
            plan = fathom.plan_calibrated(L.q, L.lo, L.hi, L.hist, L.budget, out=L.plan)
        elif variant == "group_calibrated":
            plan = fathom.plan_calibrated_group(L.q, L.lo, L.hi, L.hist, L.group_budget176,
                                                out=L.plan)
        else:
            plan = fathom.plan(L.q, L.sigma2, L.budget, out=L.plan)
        if per_call:
            e[1].record()
        if fused:
            fathom.scan_topk(planes, L.lo, L.hi, L.n, L.q, plan, w.k, 1, meta, 0.0, ws=ws,
                             idx=L.idx, vals=L.vals, meta_bits=meta_bits)
            if per_call:
                e[2].record()
        else:
            fathom.scan(planes, L.lo, L.hi, L.n, L.q, plan, meta, 0.0, out=L.logits,
                        meta_bits=meta_bits)
            if per_call:
                e[2].record()
            fathom.topk(L.logits, w.k, ws=ws, idx=L.idx, vals=L.vals)
        if per_call:
            e[3].record()
    return ev


def summarize(ev):
    tot = [a[0].elapsed_time(a[3]) for a in ev]
    plan = [a[0].elapsed_time(a[1]) for a in ev]
    scan = [a[1].elapsed_time(a[2]) for a in ev]
    topk = [a[2].elapsed_time(a[3]) for a in ev]
    return dict(call_step_ms=float(np.mean(tot)), plan_ms=float(np.mean(plan)),
                scan_ms=float(np.mean(scan)), topk_ms=float(np.mean(topk)),
                scan_ms_p10=float(np.percentile(scan, 10)),
                scan_ms_p90=float(np.percentile(scan, 90)))


def timed(layers, w, ws, steps, warmup, mode, fixed=False, fused=False, variant=None,
          with_meta=True, meta_bits=8):
    """Throughput: K steps between one pair of events (and synchronisations);
    then the same K steps again with events around every call, for the
    per-call times (the scan's is the one the rooflines use)."""
    kw = dict(variant=variant, with_meta=with_meta, meta_bits=meta_bits)
    run_steps(layers, w, ws, warmup, mode, fixed, fused, per_call=False, **kw)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    run_steps(layers, w, ws, steps, mode, fixed, fused, per_call=False, **kw)
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    r = {"step_ms": a.elapsed_time(b) / steps, "wall_ms_per_step": wall * 1e3 / steps}
    ev = run_steps(layers, w, ws, steps, mode, fixed, fused, per_call=True, **kw)
    torch.cuda.synchronize()
    r.update(summarize(ev))
    return r


def timed_graph(layers, w, ws, steps, warmup):
    """The HBM fused step (plan + fathom_scan_topk) captured once per layer
    into a HIP graph and replayed: the same kernels without the host's launch
    gaps (the library enqueues only kernels, with no copy, memset, allocation
    or synchronisation, so a step can be captured as it is)."""
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):            # warm-up outside the capture
        for L in layers:
            fathom.plan(L.q, L.sigma2, L.budget, out=L.plan)
            fathom.scan_topk(L.planes, L.lo, L.hi, L.n, L.q, L.plan, w.k, 1, ws=ws,
                             idx=L.idx, vals=L.vals)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for L in layers:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fathom.plan(L.q, L.sigma2, L.budget, out=L.plan)
            fathom.scan_topk(L.planes, L.lo, L.hi, L.n, L.q, L.plan, w.k, 1, ws=ws,
                             idx=L.idx, vals=L.vals)
        graphs.append(g)
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    del graphs
    return {"step_ms": round(ms, 4), "keys_per_s": round(w.n * w.hkv / (ms * 1e-3), 1)}


def scan_traffic_probe(layers, w, steps, warmup, dense=False, rows_out=None):
    """The HBM logits scan's own bytes moved with none of its arithmetic: per
    layer, the plane rows its union plan reads and all its logits rows, rotating
    layers like the scan.  dense: the same number of plane rows per kv head, as
    whole channels (every load instruction full).  rows_out: logits rows written
    per kv head (default all of its query heads; 0 = reads only, as the fused
    call's candidate scan).  -> mean ms per launch."""
    g = w.hq // w.hkv
    rows_out = g if rows_out is None else rows_out
    depths = [L.plan.view(w.hkv, g, w.d).amax(1).contiguous() for L in layers]
    if dense:
        packed = []
        for dp in depths:
            rows = dp.to(torch.int64).sum(1).tolist()
            t = torch.zeros((w.hkv, w.d), dtype=torch.uint8)
            for kv, u in enumerate(rows):
                t[kv, :u // 4] = 4
                if u % 4:
                    t[kv, u // 4] = u % 4
            packed.append(t.to(dp.device))
        depths = packed
    sink = torch.zeros(1, dtype=torch.int32, device=layers[0].q.device)

    def launch(i):
        L = layers[i % len(layers)]
        fathom.probe_scan_traffic(L.planes, L.n, depths[i % len(layers)], rows_out,
                                  L.logits if rows_out else None, sink)

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        launch(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def probes(dev):
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    res = {}
    dbuf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    hbuf = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    hbuf.fill_(1)
    dbuf.fill_(1)
    for name, buf, reps in (("hbm_read", dbuf, 10), ("host_read_zero_copy", hbuf, 3)):
        best = 0.0
        for blocks in (0, 1024, 4096):
            fathom.probe_read(buf, out, blocks)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fathom.probe_read(buf, out, blocks)
            b.record()
            torch.cuda.synchronize()
            gbps = buf.numel() * reps / (a.elapsed_time(b) * 1e-3) / 1e9
            best = max(best, gbps)
        res[name + "_GBps"] = round(best, 2)
    d2 = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    d2.copy_(hbuf, non_blocking=True)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(3):
        d2.copy_(hbuf, non_blocking=True)
    b.record()
    torch.cuda.synchronize()
    res["h2d_copy_GBps"] = round(3 * d2.numel() / (a.elapsed_time(b) * 1e-3) / 1e9, 2)
    del dbuf, hbuf, d2
    torch.cuda.empty_cache()
    return res


def cpu_baseline(layer0, w, n_sample, n_sample_mt):
    """The CPU oracle, as it stands, on the first keys of one layer: plan,
    scan (fp64) and top-k for all 32 query heads.  Timed on one thread over
    n_sample keys, and on all the host cores this process may use (at most
    16) over n_sample_mt keys: the oracle's own calls run unchanged on
    disjoint (kv head, key range) pieces from a thread pool (its C calls
    release the GIL), then its top-k runs per kv head on the joined rows."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import oracle
    hkv, hq = w.hkv, w.hq
    g = hq // hkv
    n_big = max(n_sample, n_sample_mt)
    W = oracle.plane_words(n_big)
    planes = layer0.planes[..., :W].contiguous().cpu().numpy().view(np.uint32)
    lo, hi = layer0.lo.cpu().numpy(), layer0.hi.cpu().numpy()
    q, s2 = layer0.q.cpu().numpy(), layer0.sigma2.cpu().numpy()

    # one thread
    Ws = oracle.plane_words(n_sample)
    p1 = np.ascontiguousarray(planes[..., :Ws])
    t0 = time.perf_counter()
    plan = oracle.plan(q, s2, w.budget)
    logits = oracle.scan(p1, lo, hi, n_sample, q, plan)
    oracle.topk(logits, w.k)
    dt1 = time.perf_counter() - t0
    del logits, p1

    # all the cores this process may use, up to the 16 host cores that go with
    # one GPU on this kind of box: pieces of whole 2048-key tiles
    visible = len(os.sched_getaffinity(0))
    cores = max(1, min(16, visible))
    chunks = max(1, -(-cores // hkv))
    tiles = -(-n_sample_mt // 2048)
    bounds = [min(n_sample_mt, (tiles * j // chunks) * 2048) for j in range(chunks + 1)]
    pieces = []
    for h in range(hkv):
        for j in range(chunks):
            a, b = bounds[j], bounds[j + 1]
            if b > a:
                pieces.append((h, a, b, np.ascontiguousarray(
                    planes[h:h + 1, ..., a // 32:(b + 2047) // 2048 * 64])))
    logits = np.empty((hq, n_sample_mt), np.float32)

    def scan_piece(pc):
        h, a, b, pl = pc
        logits[h * g:(h + 1) * g, a:b] = oracle.scan(
            pl, lo[h:h + 1], hi[h:h + 1], b - a, q[h * g:(h + 1) * g], plan[h * g:(h + 1) * g])

    def topk_head(h):
        return oracle.topk(logits[h * g:(h + 1) * g], w.k)

    with ThreadPoolExecutor(cores) as ex:
        t0 = time.perf_counter()
        plan = oracle.plan(q, s2, w.budget)
        list(ex.map(scan_piece, pieces))
        list(ex.map(topk_head, range(hkv)))
        dtm = time.perf_counter() - t0
    cpu_model = None
    try:
        fields = {}
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ":" in ln:
                    k_, v_ = ln.split(":", 1)
                    fields.setdefault(k_.strip(), v_.strip())
        cpu_model = (f"{fields.get('model name', '?')} (vendor {fields.get('vendor_id', '?')}, "
                     f"family {fields.get('cpu family', '?')}, model {fields.get('model', '?')}, "
                     f"stepping {fields.get('stepping', '?')}, {fields.get('cpu MHz', '?')} MHz)")
    except OSError:
        pass
    plane_bytes_mt = n_sample_mt * hkv * 176 // 8   # about 176 union bits per (kv head, key)
    return dict(value=round(n_sample_mt * hkv / dtm, 1), unit="keys/s", cores=cores,
                kind="oracle", cpu_model=cpu_model, cpus_visible=visible,
                cores_note=("threads used: every CPU this process may use "
                            f"({visible}), at most the 16 host cores that go with one GPU"),
                plane_bytes_per_s_approx=round(plane_bytes_mt / dtm, 1),
                sample=(f"first {n_sample_mt} keys of the 1M-key layer, all {hkv} kv heads / "
                        f"{hq} query heads: plan + fp64 scan + top-{w.k} (full sort), "
                        f"{dtm:.1f} s on {cores} threads ({len(pieces)} scan pieces of "
                        f"(kv head, key range), then top-k per kv head)"),
                single_thread=dict(
                    value=round(n_sample * hkv / dt1, 1), unit="keys/s", cores=1,
                    sample=(f"first {n_sample} keys, same work, {dt1:.1f} s on 1 thread")))


def _event_pair():
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def bench_pack(dev, reps=5):
    """fathom_pack of one 1M-key layer (storage side, off the per-token path)."""
    w = synth.LAYER_1M
    keys = synth.keys(w.seed, 99, w.n, w.hkv, w.d, w.dtype, w.outliers, device=dev)
    planes = torch.empty((w.hkv, w.d, 4, fathom.plane_words(w.n)), dtype=torch.int32, device=dev)
    ws = torch.empty(fathom.pack_workspace_bytes(w.n, w.hkv), dtype=torch.uint8, device=dev)
    fathom.pack(keys, planes=planes, ws=ws)
    torch.cuda.synchronize()
    a, b = _event_pair()
    a.record()
    for _ in range(reps):
        fathom.pack(keys, planes=planes, ws=ws)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    # keys read once and planes written; the range over all n keys must be
    # known before the first code, so a second read of the keys is inherent
    alg = keys.numel() * keys.element_size() + planes.numel() * 4
    two_pass = alg + keys.numel() * keys.element_size()
    return {"workload": "pack one 1M-key layer (fp16 keys -> planes, lo, hi, sigma2)",
            "ms": round(ms, 3), "keys_per_s": round(w.n * w.hkv / (ms * 1e-3), 1),
            "algorithmic_bytes": alg, "achieved_GBps": round(alg / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "two_pass_bytes": two_pass,
            "two_pass_GBps": round(two_pass / (ms * 1e-3) / 1e9, 1)}


def bench_layer_128k(dev, steps, warmup):
    """131072-key layer, planes in HBM, B in {68, 92, 136}, k = 1024."""
    w = synth.LAYER_128K
    layers = []
    for l in range(8):                      # 8 x 64 MiB of planes rotate past the MALL
        keys = synth.keys(w.seed, l, w.n, w.hkv, w.d, w.dtype, w.outliers, device=dev)
        p = fathom.pack(keys)
        del keys
        q = synth.queries(w.seed, l, w.hq, w.d, device=dev)
        layers.append((p, q, torch.empty((w.hq, w.d), dtype=torch.uint8, device=dev),
                       torch.empty((w.hq, w.n), device=dev)))
    ws = torch.empty(fathom.topk_workspace_bytes(w.hq, w.k), dtype=torch.uint8, device=dev)
    idx = torch.empty((w.hq, w.k), dtype=torch.int32, device=dev)
    vals = torch.empty((w.hq, w.k), device=dev)
    out = {"workload": "qwen3-8b layer n=131072, planes in HBM, k=1024"}
    for B in (68, 92, 136):
        def step(i):
            p, q, plan, logits = layers[i % len(layers)]
            fathom.plan(q, p.sigma2, B, out=plan)
            fathom.scan(p.planes, p.lo, p.hi, w.n, q, plan, out=logits)
            fathom.topk(logits, w.k, ws=ws, idx=idx, vals=vals)
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        a, b = _event_pair()
        a.record()
        for i in range(steps):
            step(i)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        ub = [union_plane_bytes(L[2], w.hkv, w.n)[0] for L in layers]
        # the same step through the fused call (plan -> scan_topk, planes in HBM)
        fws = torch.empty(fathom.scan_topk_workspace_bytes([w.n], w.hkv, w.hq, 1, w.k),
                          dtype=torch.uint8, device=dev)

        def fstep(i):
            p, q, plan, _ = layers[i % len(layers)]
            fathom.plan(q, p.sigma2, B, out=plan)
            fathom.scan_topk(p.planes, p.lo, p.hi, w.n, q, plan, w.k, 1, ws=fws, idx=idx,
                             vals=vals)
        for i in range(warmup):
            fstep(i)
        torch.cuda.synchronize()
        a, b = _event_pair()
        a.record()
        for i in range(steps):
            fstep(i)
        b.record()
        torch.cuda.synchronize()
        fms = a.elapsed_time(b) / steps
        ubm = int(np.mean(ub))
        gbps = ubm / (fms * 1e-3) / 1e9
        out[f"B{B}"] = {"step_ms": round(ms, 4),
                        "keys_per_s": round(w.n * w.hkv / (ms * 1e-3), 1),
                        "union_plane_bytes": ubm,
                        "fused_step_ms": round(fms, 4),
                        "fused_keys_per_s": round(w.n * w.hkv / (fms * 1e-3), 1),
                        "fused_roofline": {"bound": "hbm", "achieved": round(gbps, 1),
                                           "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                           "frac": round(gbps / HBM_PEAK_GBPS, 4),
                                           "algorithmic_bytes": ubm}}
        del fws
    return out


def bench_clustered(dev, steps, warmup, iid_step_ms):
    """The 1M-key layer with 1,500 top-scoring keys planted inside one
    2048-key tile of one query head's kv head (a different head and tile per
    layer): one scan block finds more candidates than its share of the row's
    candidate store.  Fused HBM step time against the i.i.d. layers', and the
    rows recomputed from full logits."""
    w = synth.LAYER_1M
    G = w.hq // w.hkv
    layers = []
    for l in range(4):
        keys = synth.keys(w.seed, l, w.n, w.hkv, w.d, w.dtype, w.outliers, device=dev)
        q = synth.queries(w.seed, l, w.hq, w.d, device=dev)
        head, tile, m = 5 + 7 * l, 101 + 97 * l, 1500
        g = head // G
        sd = keys[:, g, :].float().std(0)
        v = (3.0 * sd * torch.sign(q[head])).to(keys.dtype)
        t0 = tile * 2048
        keys[t0:t0 + m, g, :] = v
        keys[t0:t0 + m, g, 0] = (v[0].float() + 0.01 * sd[0] * torch.arange(
            m, device=dev, dtype=torch.float32) / m).to(keys.dtype)
        p = fathom.pack(keys)
        del keys
        layers.append((p, q, torch.empty((w.hq, w.d), dtype=torch.uint8, device=dev)))
    fws = torch.empty(fathom.scan_topk_workspace_bytes([w.n], w.hkv, w.hq, 1, w.k),
                      dtype=torch.uint8, device=dev)
    idx = torch.empty((w.hq, w.k), dtype=torch.int32, device=dev)
    vals = torch.empty((w.hq, w.k), device=dev)

    def step(i):
        p, q, plan = layers[i % len(layers)]
        fathom.plan(q, p.sigma2, w.budget, out=plan)
        fathom.scan_topk(p.planes, p.lo, p.hi, w.n, q, plan, w.k, 1, ws=fws, idx=idx, vals=vals)
    flagged = 0
    for i in range(len(layers)):
        step(i)
        torch.cuda.synchronize()
        # the workspace starts with one threshold word, then one recompute
        # flag per output row
        flagged += int(fws[4 * w.hq:8 * w.hq].view(torch.int32).ne(0).sum())
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    a, b = _event_pair()
    a.record()
    for i in range(steps):
        step(i)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    return {"workload": ("1M-key layer, planes in HBM, B=92, k=2048: 1500 top keys of one "
                         "query head inside one 2048-key tile"),
            "fused_step_ms": round(ms, 4), "iid_fused_step_ms": round(iid_step_ms, 4),
            "ratio_to_iid": round(ms / iid_step_ms, 3),
            "rows_recomputed": flagged, "rows_total": len(layers) * w.hq}


def bench_blocked(dev, steps, warmup, n_layers=4):
    """Per-block ranges (one lo/hi per 2048-key block of a channel) against
    per-layer ranges on the same keys: 1M-key layers whose key ranges drift
    along the sequence (synth.drifting_keys, drift 3), B = 92, k = 2048.  Fused
    plan + scan + top-k step times with planes in HBM and in pinned host
    memory, their ratios, the cost of pack and of a one-token append, and the
    recall@2048 of each against the exact top-k of the fp64 logits q . k of
    the fp16 keys (torch's matmul on the GPU, as in plan_quality)."""
    w = synth.LAYER_1M
    G = w.hq // w.hkv
    layers = []
    recall = {"per_layer": [], "per_block": []}
    fws = torch.empty(fathom.scan_topk_workspace_bytes([w.n], w.hkv, w.hq, 1, w.k),
                      dtype=torch.uint8, device=dev)
    idx = torch.empty((w.hq, w.k), dtype=torch.int32, device=dev)
    vals = torch.empty((w.hq, w.k), device=dev)
    pack_ms = {"per_layer": [], "per_block": []}
    for l in range(n_layers):
        keys = synth.drifting_keys(w.seed, l, w.n, w.hkv, w.d, w.dtype, w.outliers, device=dev)
        q = synth.queries(w.seed, l, w.hq, w.d, device=dev)
        for name, fn in (("per_layer", fathom.pack), ("per_block", fathom.pack_blocked)):
            fn(keys)
            torch.cuda.synchronize()
            a, b = _event_pair()
            a.record()
            p = fn(keys)
            b.record()
            torch.cuda.synchronize()
            pack_ms[name].append(a.elapsed_time(b))
            host = torch.empty(p.planes.shape, dtype=p.planes.dtype, pin_memory=True)
            host.copy_(p.planes)
            plan = torch.empty((w.hq, w.d), dtype=torch.uint8, device=dev)
            layers.append((name, p, host, q, plan))
        if l == 0:
            exact = []
            for g in range(w.hkv):
                K = keys[:, g, :].double()
                s = q[g * G:(g + 1) * G].double() @ K.T
                exact.append(torch.topk(s, w.k, dim=1).indices)
                del K, s
            exact = torch.cat(exact).cpu().numpy()
            for name, p, host, q_, plan in layers:
                fathom.plan(q_, p.sigma2, w.budget, out=plan)
                if name == "per_layer":
                    fathom.scan_topk(p.planes, p.lo, p.hi, w.n, q_, plan, w.k, 1, ws=fws,
                                     idx=idx, vals=vals)
                else:
                    fathom.scan_topk_blocked(p.planes, p.lo, p.hi, w.n, q_, plan, w.k, 1,
                                             ws=fws, idx=idx, vals=vals)
                got = idx.cpu().numpy()
                recall[name] = float(np.mean([len(np.intersect1d(got[h], exact[h])) / w.k
                                              for h in range(w.hq)]))
        del keys
    out = {"workload": ("1M-key layers (8 kv heads, fp16) with drifting key ranges, B=92, "
                        "k=2048: per-block ranges against per-layer ranges on the same keys")}
    for mode in ("hbm", "host"):
        for kind in ("per_layer", "per_block"):
            sel = [L for L in layers if L[0] == kind]

            def step(i):
                _, p, host, q, plan = sel[i % len(sel)]
                planes = host if mode == "host" else p.planes
                fathom.plan(q, p.sigma2, w.budget, out=plan)
                if kind == "per_layer":
                    fathom.scan_topk(planes, p.lo, p.hi, w.n, q, plan, w.k, 1, ws=fws,
                                     idx=idx, vals=vals)
                else:
                    fathom.scan_topk_blocked(planes, p.lo, p.hi, w.n, q, plan, w.k, 1,
                                             ws=fws, idx=idx, vals=vals)
            for i in range(warmup):
                step(i)
            torch.cuda.synchronize()
            a, b = _event_pair()
            a.record()
            for i in range(steps):
                step(i)
            b.record()
            torch.cuda.synchronize()
            out[f"{mode}_{kind}_fused_step_ms"] = round(a.elapsed_time(b) / steps, 4)
        out[f"{mode}_time_ratio_block_to_layer"] = round(
            out[f"{mode}_per_block_fused_step_ms"] / out[f"{mode}_per_layer_fused_step_ms"], 4)
    out["pack_ms"] = {k: round(float(np.mean(v)), 3) for k, v in pack_ms.items()}
    # one decode token appended to each layout (block 511 already holds keys)
    _, pb, _, _, _ = [L for L in layers if L[0] == "per_block"][0]
    _, pl, _, _, _ = [L for L in layers if L[0] == "per_layer"][0]
    tok = synth.drifting_keys(w.seed, 99, 1, w.hkv, w.d, w.dtype, w.outliers, device=dev)
    for kind, fn in (("per_layer", lambda: fathom.append(tok, w.n - 1, pl.planes, pl.lo, pl.hi)),
                     ("per_block", lambda: fathom.append_blocked(tok, w.n - 1, pb.planes, pb.lo,
                                                                 pb.hi))):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = _event_pair()
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        out[f"append_1_token_{kind}_us"] = round(a.elapsed_time(b) / steps * 1e3, 2)
    out["recall_at_2048"] = {k: round(v, 4) for k, v in recall.items()}
    del layers
    return out


def plan_quality(dev, layers_q=2):
    """Recall of each plan's top-k against the exact top-k of the fp64 logits
    q . k of the fp16 keys (not timed; torch's matmul on the GPU is the
    reference here, never part of the path).  1M-key layers, k = 2048 per
    query head, mean over heads and layers."""
    w = synth.LAYER_1M
    G = w.hq // w.hkv
    kinds = [("fathom_B92", lambda p, q: fathom.plan(q, p.sigma2, 92)),
             ("rd_B92", lambda p, q: fathom.plan_rd(q, p.sigma2, 92)),
             ("calibrated_B92", lambda p, q: fathom.plan_calibrated(
                 q, p.lo, p.hi, fathom.code_hist(p.planes, p.n), 92)),
             ("calibrated_B68", lambda p, q: fathom.plan_calibrated(
                 q, p.lo, p.hi, fathom.code_hist(p.planes, p.n), 68)),
             ("calibrated_B136", lambda p, q: fathom.plan_calibrated(
                 q, p.lo, p.hi, fathom.code_hist(p.planes, p.n), 136)),
             ("group_B92_per_kv_head", lambda p, q: fathom.plan_group(q, p.sigma2, 92)),
             ("group_B368_per_kv_head", lambda p, q: fathom.plan_group(q, p.sigma2, 4 * 92)),
             ("fathom_B68", lambda p, q: fathom.plan(q, p.sigma2, 68)),
             ("rd_B68", lambda p, q: fathom.plan_rd(q, p.sigma2, 68)),
             ("fathom_B136", lambda p, q: fathom.plan(q, p.sigma2, 136)),
             ("rd_B136", lambda p, q: fathom.plan_rd(q, p.sigma2, 136)),
             ("group_B176_per_kv_head", lambda p, q: fathom.plan_group(q, p.sigma2, 176)),
             ("group_calibrated_B176_per_kv_head", lambda p, q: fathom.plan_calibrated_group(
                 q, p.lo, p.hi, fathom.code_hist(p.planes, p.n), 176)),
             ("group_calibrated_B92_per_kv_head", lambda p, q: fathom.plan_calibrated_group(
                 q, p.lo, p.hi, fathom.code_hist(p.planes, p.n), 92)),
             ("fixed136", None),
             ("fixed_r16", 16),
             ("full_4bit_B512", lambda p, q: fathom.plan(q, p.sigma2, 512))]
    rec = {name: [] for name, _ in kinds}
    bits = {name: [] for name, _ in kinds}
    ws = torch.empty(fathom.scan_topk_workspace_bytes([w.n], w.hkv, w.hq, 1, w.k),
                     dtype=torch.uint8, device=dev)
    for l in range(layers_q):
        keys = synth.keys(w.seed, l, w.n, w.hkv, w.d, w.dtype, w.outliers, device=dev)
        q = synth.queries(w.seed, l, w.hq, w.d, device=dev)
        p = fathom.pack(keys)
        exact = []
        for g in range(w.hkv):
            K = keys[:, g, :].double()
            s = q[g * G:(g + 1) * G].double() @ K.T
            exact.append(torch.topk(s, w.k, dim=1).indices)
            del K, s
        exact = torch.cat(exact).cpu().numpy()
        del keys
        for name, fn in kinds:
            if fn is None or isinstance(fn, int):
                plan = fathom.plan_fixed(q, 32 if fn is None else fn)
            else:
                plan = fn(p, q)
            idx, _ = fathom.scan_topk(p.planes, p.lo, p.hi, w.n, q, plan, w.k, 1, ws=ws)
            got = idx.cpu().numpy()
            rec[name].append(np.mean([len(np.intersect1d(got[h], exact[h])) / w.k
                                      for h in range(w.hq)]))
            bits[name].append(np.mean(union_plane_bytes(plan, w.hkv, w.n)[1]))
        del p
        torch.cuda.empty_cache()
    return {"workload": f"{layers_q} x 1M-key layers, recall@2048 vs exact fp64 logits "
                        "(fixed plans scored without the side stream's term)",
            **{name: {"recall": round(float(np.mean(rec[name])), 4),
                      "union_bits_per_kv_head": round(float(np.mean(bits[name])), 1)}
               for name, _ in kinds}}


def bench_attention(dev, steps, warmup):
    """Sparse attention over the k = 2048 keys fathom_scan_topk selects on the
    1M-key layer (fp16 K and V, token-major), alone and as the last call of
    the decode step plan -> scan_topk -> attention; K/V and planes in HBM and
    in pinned host memory."""
    w = synth.LAYER_1M
    keys = synth.keys(w.seed, 0, w.n, w.hkv, w.d, w.dtype, w.outliers, device=dev)
    vals = synth.keys(w.seed + 1, 0, w.n, w.hkv, w.d, w.dtype, 0, device=dev)
    q = synth.queries(w.seed, 0, w.hq, w.d, device=dev)
    p = fathom.pack(keys)
    host = {}
    for name, t in (("planes", p.planes), ("k", keys), ("v", vals)):
        host[name] = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
        host[name].copy_(t)
    plan = fathom.plan(q, p.sigma2, w.budget)
    out = {"workload": "1M-key layer, fp16 K/V [n][8][128], 32 query heads, k=2048 selected keys"}
    for group in (1, 4):
        rows = w.hq // group
        fws = torch.empty(fathom.scan_topk_workspace_bytes([w.n], w.hkv, w.hq, group, w.k),
                          dtype=torch.uint8, device=dev)
        idx = torch.empty((rows, w.k), dtype=torch.int32, device=dev)
        vls = torch.empty((rows, w.k), dtype=torch.float32, device=dev)
        fathom.scan_topk(p.planes, p.lo, p.hi, w.n, q, plan, w.k, group, ws=fws, idx=idx,
                         vals=vls)
        aws = torch.empty(fathom.attention_workspace_bytes(w.hq, w.k), dtype=torch.uint8,
                          device=dev)
        o = torch.empty((w.hq, w.d), dtype=torch.float32, device=dev)
        lse = torch.empty((w.hq,), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        nvalid = int((idx >= 0).sum())
        alg = nvalid * 2 * w.d * 2 + idx.numel() * 4   # K and V rows + the indices
        for res in ("hbm", "host"):
            Kc, Vc = (keys, vals) if res == "hbm" else (host["k"], host["v"])
            planes = p.planes if res == "hbm" else host["planes"]

            def attn():
                fathom.sparse_attention(q, Kc, Vc, idx, group, out=o, lse=lse, ws=aws)

            def step():
                fathom.plan(q, p.sigma2, w.budget, out=plan)
                fathom.scan_topk(planes, p.lo, p.hi, w.n, q, plan, w.k, group, ws=fws,
                                 idx=idx, vals=vls)
                attn()
            for fn, label in ((attn, "attention"), (step, "decode_step")):
                for _ in range(warmup):
                    fn()
                torch.cuda.synchronize()
                a, b = _event_pair()
                a.record()
                for _ in range(steps):
                    fn()
                b.record()
                torch.cuda.synchronize()
                ms = a.elapsed_time(b) / steps
                rec = {"ms": round(ms, 4)}
                if label == "attention":
                    gbps = alg / (ms * 1e-3) / 1e9
                    peak = HBM_PEAK_GBPS if res == "hbm" else PCIE_PEAK_GBPS
                    rec.update({"algorithmic_bytes": alg, "GBps": round(gbps, 1),
                                "frac_of_peak": round(gbps / peak, 4)})
                out[f"group{group}_{res}_{label}"] = rec
    del keys, vals, host
    return out


def bench_append(dev, steps, warmup):
    """fathom_append on the 1M-key layer's planes (capacity for 2^20 + 8192
    keys): one decode token (8 kv heads x 128 channels) and a 4096-key chunk."""
    w = synth.LAYER_1M
    n0 = w.n - 4096
    keys = synth.keys(w.seed, 0, w.n, w.hkv, w.d, w.dtype, w.outliers, device=dev)
    p = fathom.pack(keys[:n0])
    planes = fathom.alloc_planes(w.n + 8192, w.hkv)
    planes[..., :p.planes.shape[-1]].copy_(p.planes)
    del p.planes
    out = {"workload": "append to the 1M-key layer (fp16 keys, 8 kv heads, capacity 2^20+8192)"}
    for m in (1, 4096):
        def call():
            fathom.append(keys[n0:n0 + m], n0, planes, p.lo, p.hi)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        a, b = _event_pair()
        a.record()
        for _ in range(steps):
            call()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        # the same calls replayed from a HIP graph: the device time without
        # the per-call host cost (the call rewrites the same bits every time)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            call()
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=side):
                for _ in range(steps):
                    call()
        torch.cuda.synchronize()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        gms = a.elapsed_time(b) / steps
        del g
        words = -(-(n0 % 32 + m) // 32)
        alg = m * w.hkv * w.d * 2 + 2 * words * w.hkv * w.d * 4 * 4   # keys + plane words read and written
        out[f"m{m}"] = {"us": round(ms * 1e3, 2), "graph_us": round(gms * 1e3, 2),
                        "algorithmic_bytes": alg, "GBps": round(alg / (ms * 1e-3) / 1e9, 1)}
    del keys, planes
    return out


def bench_sessions(dev, steps, warmup):
    """16 ragged sessions (64K..512K keys), per-session B, planes in pinned host
    memory, one batched scan and one batched top-k (k = 1024 per query head)."""
    w = synth.SESSIONS_16
    lengths = synth.session_lengths(w)
    budgets = synth.session_budgets(w)
    sess, sig = [], []
    for s_, (n, B) in enumerate(zip(lengths, budgets)):
        keys = synth.keys(w.seed, 0, n, w.hkv, w.d, w.dtype, w.outliers, device=dev, session=s_)
        p = fathom.pack(keys)
        del keys
        host = torch.empty(p.planes.shape, dtype=p.planes.dtype, pin_memory=True)
        host.copy_(p.planes)
        p.planes = None
        q = synth.queries(w.seed, 0, w.hq, w.d, device=dev, session=s_)
        plan = torch.empty((w.hq, w.d), dtype=torch.uint8, device=dev)
        sess.append(fathom.Session(host, p.lo, p.hi, n, q, plan,
                                   torch.empty((w.hq, n), device=dev),
                                   torch.empty((w.hq, w.k), dtype=torch.int32, device=dev),
                                   torch.empty((w.hq, w.k), device=dev)))
        sig.append((p.sigma2, B))
    ws = torch.empty(fathom.topk_workspace_bytes(w.hq * len(sess), w.k), dtype=torch.uint8,
                     device=dev)
    torch.cuda.empty_cache()

    def step():
        for S, (s2, B) in zip(sess, sig):
            fathom.plan(S.q, s2, B, out=S.plan)
        fathom.scan_batched(sess)
        fathom.topk_batched(sess, w.k, group=1, ws=ws)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a, b = _event_pair()
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    total = sum(lengths) * w.hkv
    plane_b = sum(union_plane_bytes(S.plan, w.hkv, S.n)[0] for S in sess)
    return {"workload": "16 sessions, n uniform in [64K, 512K] (sum %d keys), B per session "
                        "from {68, 92, 136}, planes in pinned host memory, k=1024" % sum(lengths),
            "step_ms": round(ms, 3), "keys_per_s": round(total / (ms * 1e-3), 1),
            "union_plane_bytes": plane_b,
            "link_GBps": round(plane_b / (ms * 1e-3) / 1e9, 2)}


def bench_step36(dev, steps, warmup):
    """Full decode step at 1M tokens: 36 layers x (plan, scan, top-k), B = 92
    and the fixed-136 scan, planes in HBM and in pinned host memory."""
    w = synth.STEP_36L_1M
    layers = []
    for l in range(w.layers):
        keys = synth.keys(w.seed, l, w.n, w.hkv, w.d, w.dtype, w.outliers, device=dev)
        p = fathom.pack(keys)
        del keys
        host = torch.empty(p.planes.shape, dtype=p.planes.dtype, pin_memory=True)
        host.copy_(p.planes)
        q = synth.queries(w.seed, l, w.hq, w.d, device=dev)
        meta = synth.side_stream(w.seed, l, w.hkv, w.n, device=dev)
        layers.append((p, host, q, meta))
    plan = torch.empty((w.hq, w.d), dtype=torch.uint8, device=dev)
    logits = torch.empty((w.hq, w.n), device=dev)
    idx = torch.empty((w.hq, w.k), dtype=torch.int32, device=dev)
    vals = torch.empty((w.hq, w.k), device=dev)
    ws = torch.empty(fathom.topk_workspace_bytes(w.hq, w.k), dtype=torch.uint8, device=dev)
    fws = torch.empty(fathom.scan_topk_workspace_bytes([w.n], w.hkv, w.hq, 1, w.k),
                      dtype=torch.uint8, device=dev)
    out = {"workload": "36 layers x 1M keys (18 GiB of planes), 32 query heads, k=2048"}
    for mode in ("hbm", "host", "hbm_fused"):
        for fixed in (False, True):
            def step():
                for p, host, q, meta in layers:
                    if fixed:
                        fathom.plan_fixed(q, 32, out=plan)
                    else:
                        fathom.plan(q, p.sigma2, w.budget, out=plan)
                    if mode == "hbm_fused":
                        fathom.scan_topk(p.planes, p.lo, p.hi, w.n, q, plan, w.k, 1,
                                         meta if fixed else None, 0.0, ws=fws, idx=idx,
                                         vals=vals)
                        continue
                    fathom.scan(host if mode == "host" else p.planes, p.lo, p.hi, w.n, q, plan,
                                meta if fixed else None, 0.0, out=logits)
                    fathom.topk(logits, w.k, ws=ws, idx=idx, vals=vals)
            for _ in range(warmup):
                step()
            torch.cuda.synchronize()
            a, b = _event_pair()
            a.record()
            for _ in range(steps):
                step()
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / steps
            out[f"{mode}{'_fixed136' if fixed else ''}"] = {
                "step_ms": round(ms, 3),
                "keys_per_s": round(w.layers * w.n * w.hkv / (ms * 1e-3), 1)}
        out[f"{mode}_speedup_vs_fixed136"] = round(
            out[f"{mode}_fixed136"]["step_ms"] / out[mode]["step_ms"], 3)
    return out


def scan_traffic_from_profiles():
    """HBM bytes per scan launch from committed rocprofv3 counter runs, valid
    only for the scan source they were taken on."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    h = hashlib.sha256(open(SCAN_SOURCE, "rb").read()).hexdigest()
    if rec.get("scan_source_sha256") != h:
        return None
    return rec


CAND_FILE = os.path.join(ROOT, "profiles", "scan_topk_1m_layer_candidate_scan.json")


def candidate_scan_from_profiles():
    """The fused call's candidate-scan kernel time from the committed kernel
    trace (valid only for the scan source it was taken on)."""
    if not os.path.exists(CAND_FILE):
        return None
    with open(CAND_FILE) as f:
        rec = json.load(f)
    h = hashlib.sha256(open(SCAN_SOURCE, "rb").read()).hexdigest()
    if rec.get("scan_source_sha256") != h:
        return None
    rec["file"] = os.path.relpath(CAND_FILE, ROOT)
    return rec


def res_modes(args):
    return ["host", "hbm"] if args.only == "all" else [args.only]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=4, help="rotating layers (cache defeat)")
    ap.add_argument("--cpu-sample", type=int, default=131072,
                    help="keys of the single-thread oracle sample")
    ap.add_argument("--cpu-sample-mt", type=int, default=524288,
                    help="keys of the all-core oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--only", choices=["all", "hbm", "host"], default="all",
                    help="profiling runs: restrict to one residency")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads (pack, 128K layer, 16 sessions, 36 layers)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="counter runs: first copy 256 MiB device-to-device so the "
                         "HBM byte counters can be scaled by a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path "
              "shards by kv head or token range, see DESIGN.md", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    w = synth.LAYER_1M
    fathom.lib()

    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    probe = {} if args.no_probe else probes(dev)
    log(f"probes: {probe}")

    host = args.only in ("all", "host")
    layers = [Layer(w, l, dev, host, 32) for l in range(args.layers)]
    ws = torch.empty(fathom.topk_workspace_bytes(w.hq, w.k), dtype=torch.uint8, device=dev)
    fws = torch.empty(fathom.scan_topk_workspace_bytes([w.n], w.hkv, w.hq, 1, w.k),
                      dtype=torch.uint8, device=dev)
    # plans once, for the byte accounting (the timed steps recompute them)
    for L in layers:
        fathom.plan(L.q, L.sigma2, L.budget, out=L.plan)
    torch.cuda.synchronize()
    # algorithmic plane bytes: mean over the rotating layers
    per = [union_plane_bytes(L.plan, w.hkv, w.n) for L in layers]
    plane_b = int(np.mean([x[0] for x in per]))
    ub, hist = per[0][1], per[0][2]
    fper = [union_plane_bytes(L.plan_fixed, w.hkv, w.n) for L in layers]
    fixed_plan_b = int(np.mean([x[0] for x in fper]))
    fub = fper[0][1]
    meta_b = w.hkv * w.n
    logits_b = w.hq * w.n * 4
    log(f"union bits per kv head {ub}, depth histogram {hist}; fixed-136 union {fub}")
    traffic_probe_ms = dense_probe_ms = reads_probe_ms = None
    if probe and "hbm" in res_modes(args):
        traffic_probe_ms = scan_traffic_probe(layers, w, args.steps, args.warmup)
        dense_probe_ms = scan_traffic_probe(layers, w, args.steps, args.warmup, dense=True)
        reads_probe_ms = scan_traffic_probe(layers, w, args.steps, args.warmup, rows_out=0)
        log(f"scan-traffic probe: {traffic_probe_ms * 1e3:.1f} us per launch "
            f"(as whole channels: {dense_probe_ms * 1e3:.1f} us; "
            f"plane reads only: {reads_probe_ms * 1e3:.1f} us)")

    res = {}
    for mode in res_modes(args):
        res[mode] = timed(layers, w, ws, args.steps, args.warmup, mode)
        res[mode + "_fixed"] = timed(layers, w, ws, args.steps, args.warmup, mode, fixed=True)
        res[mode + "_fused"] = timed(layers, w, fws, args.steps, args.warmup, mode, fused=True)
        res[mode + "_fixed_fused"] = timed(layers, w, fws, args.steps, args.warmup, mode,
                                           fixed=True, fused=True)
        for key in (mode, mode + "_fixed", mode + "_fused", mode + "_fixed_fused"):
            log(f"{key}: {res[key]}")
    graph = None
    if "hbm" in res_modes(args):
        graph = timed_graph(layers, w, fws, args.steps, args.warmup)
        log(f"hbm_fused, HIP graph per step: {graph}")

    variants = {}
    if not args.no_extra:
        for var, fn, bud in (("rd", fathom.plan_rd, "budget"),
                             ("group", fathom.plan_group, "group_budget"),
                             ("calibrated", None, "budget"),
                             ("group_calibrated", None, "group_budget176")):
            if var == "calibrated":
                vper = [union_plane_bytes(fathom.plan_calibrated(L.q, L.lo, L.hi, L.hist,
                                                                 L.budget), w.hkv, w.n)
                        for L in layers]
            elif var == "group_calibrated":
                vper = [union_plane_bytes(fathom.plan_calibrated_group(
                    L.q, L.lo, L.hi, L.hist, L.group_budget176), w.hkv, w.n) for L in layers]
            else:
                vper = [union_plane_bytes(fn(L.q, L.sigma2, getattr(L, bud)), w.hkv, w.n)
                        for L in layers]
            v = {"union_plane_bytes": int(np.mean([x[0] for x in vper])),
                 "union_bits_per_kv_head": vper[0][1], "depth_histogram": vper[0][2]}
            for mode in res_modes(args):
                t = timed(layers, w, fws, args.steps, args.warmup, mode, fused=True,
                          variant=var)
                v[mode + "_fused"] = {"keys_per_s": round(w.n * w.hkv / (t["step_ms"] * 1e-3), 1),
                                      **{k: round(x, 4) for k, x in t.items()}}
                log(f"{var} {mode}_fused: {t}")
            variants[var] = v
        # the r = 16 analogue of the baseline: 64 plane bits per query head and
        # a side stream of r/4 = 4 bits per key (68 bits, the pages' figure)
        # or of 8 bits (72 bits); the pages compare Fathom with it
        fper16 = [union_plane_bytes(fathom.plan_fixed(L.q, 16), w.hkv, w.n) for L in layers]
        for name, mbits in (("fixed_r16", 8), ("fixed_r16_68bit", 4)):
            v = {"union_plane_bytes": int(np.mean([x[0] for x in fper16])),
                 "meta_bytes": w.hkv * w.n * mbits // 8, "meta_bits_per_key": mbits,
                 "bits_per_key": 64 + mbits, "union_bits_per_kv_head": fper16[0][1]}
            for mode in res_modes(args):
                t = timed(layers, w, fws, args.steps, args.warmup, mode, fixed=16, fused=True,
                          meta_bits=mbits)
                v[mode + "_fused"] = {"keys_per_s": round(w.n * w.hkv / (t["step_ms"] * 1e-3), 1),
                                      **{k: round(x, 4) for k, x in t.items()}}
                log(f"{name} {mode}_fused: {t}")
            variants[name] = v
        # fixed-128: the r = 32 plan without the side stream
        v = {"union_plane_bytes": fixed_plan_b}
        for mode in res_modes(args):
            t = timed(layers, w, fws, args.steps, args.warmup, mode, fixed=True, fused=True,
                      with_meta=False)
            v[mode + "_fused"] = {"keys_per_s": round(w.n * w.hkv / (t["step_ms"] * 1e-3), 1),
                                  **{k: round(x, 4) for k, x in t.items()}}
            v[mode + "_speedup_of_fathom"] = round(t["step_ms"] / res[mode + "_fused"]["step_ms"], 3)
            log(f"fixed-128 {mode}_fused: {t}")
        variants["fixed128"] = v

    keys_per_step = w.n * w.hkv
    main_mode = "host" if "host" in res else "hbm"
    r = res[main_mode]
    value = keys_per_step / (r["step_ms"] * 1e-3)
    traffic = scan_traffic_from_profiles()
    if main_mode == "host":
        achieved = plane_b / (r["scan_ms"] * 1e-3) / 1e9
        roofline = {"bound": "host_link", "achieved": round(achieved, 2),
                    "peak": PCIE_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / PCIE_PEAK_GBPS, 4),
                    "traffic": (traffic or {}).get("host_scan_fetch_bytes"),
                    "kernel": "scan_kernel<4, 2, false> (planes in pinned host memory, fp32 FMA form)",
                    "algorithmic_bytes": plane_b,
                    "frac_of_measured_link_peak": (round(achieved / probe["host_read_zero_copy_GBps"], 4)
                                                   if probe else None),
                    "end_to_end_frac": round(plane_b / (r["step_ms"] * 1e-3) / 1e9 /
                                             PCIE_PEAK_GBPS, 4)}
    out = {
        "metric": "keys scanned/s (1M-token layer, B=92, k=2048, planes zero-copy from pinned host)",
        "value": round(value, 1),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["step_ms"], 4),
        "query_keys_per_s": round(value * w.hq / w.hkv, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded Qwen3-8B-shaped keys, log-uniform channel scales + 4 outlier channels, fp16)",
        "config": {"workload": ("qwen3-8b layer: n=1048576 keys fp16, 8 kv heads x d128, "
                                "32 query heads (GQA 4), B=92 bits/key, k=2048 per query head, "
                                f"K planes {'in pinned host memory (zero-copy)' if main_mode == 'host' else 'in HBM'}"),
                   "steps_rotate_layers": args.layers},
    }
    if main_mode == "host":
        out["roofline"] = roofline
    if "hbm" in res:
        h = res["hbm"]
        # algorithmic bytes: the union plane bytes alone; the fp32 logits the
        # unfused scan writes (and top-k reads back) are not the method's
        ach = plane_b / (h["scan_ms"] * 1e-3) / 1e9
        out["roofline_hbm"] = {
            "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBPS, 4),
            "traffic": (traffic or {}).get("hbm_scan_bytes"),
            "kernel": "scan_mfma_kernel<4, 0, false, false> (planes in HBM, all logits written)",
            "algorithmic_bytes": plane_b,
            "non_algorithmic_bytes": logits_b,
            "achieved_with_logits_GBps": round((plane_b + logits_b) / (h["scan_ms"] * 1e-3) / 1e9, 1),
            "end_to_end_plane_GBps": round(plane_b / (h["step_ms"] * 1e-3) / 1e9, 1)}
        hf = res["hbm_fused"]
        e2e = plane_b / (hf["step_ms"] * 1e-3) / 1e9
        out["roofline_hbm_fused_step"] = {
            "bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBPS,
            "what": "union plane bytes over the whole plan + scan_topk step (event-timed)",
            "achieved": round(e2e, 1), "frac": round(e2e / HBM_PEAK_GBPS, 4),
            "algorithmic_bytes": plane_b, "step_ms": round(hf["step_ms"], 4)}
        if graph:
            ge = plane_b / (graph["step_ms"] * 1e-3) / 1e9
            out["roofline_hbm_fused_step"]["hip_graph"] = {
                "what": ("the same step replayed from a HIP graph captured per layer (eager "
                         "launches already run back to back: no host gaps to remove)"),
                "step_ms": graph["step_ms"], "keys_per_s": graph["keys_per_s"],
                "achieved": round(ge, 1), "frac": round(ge / HBM_PEAK_GBPS, 4)}
        cand = candidate_scan_from_profiles()
        if cand:
            ca = plane_b / (cand["candidate_scan_us"] * 1e-6) / 1e9
            out["roofline_hbm_fused_step"]["candidate_scan"] = {
                "kernel": cand["kernel"], "avg_us_kernel_trace": cand["candidate_scan_us"],
                "achieved": round(ca, 1), "frac": round(ca / HBM_PEAK_GBPS, 4),
                "source": cand["file"]}
        if traffic_probe_ms:
            # the same bytes moved by fathom_probe_scan_traffic, with no arithmetic
            pat = (plane_b + logits_b) / (traffic_probe_ms * 1e-3) / 1e9
            out["roofline_hbm"]["scan_traffic_probe_GBps"] = round(pat, 1)
            out["roofline_hbm"]["frac_of_scan_traffic_probe"] = round(
                (plane_b + logits_b) / (h["scan_ms"] * 1e-3) / 1e9 / pat, 4)
            # the same number of plane rows per kv head read as whole channels
            out["roofline_hbm"]["scan_traffic_probe_whole_channels_GBps"] = round(
                (plane_b + logits_b) / (dense_probe_ms * 1e-3) / 1e9, 1)
            # the plane reads alone (the fused call's candidate scan writes no logits)
            out["roofline_hbm"]["scan_traffic_probe_reads_only_GBps"] = round(
                plane_b / (reads_probe_ms * 1e-3) / 1e9, 1)
        if main_mode == "host":
            out["hbm_resident"] = {"keys_per_s": round(keys_per_step / (h["step_ms"] * 1e-3), 1),
                                   **{k: round(v, 4) for k, v in h.items()}}
            hf = res["hbm_fused"]
            out["hbm_resident_fused"] = {
                "keys_per_s": round(keys_per_step / (hf["step_ms"] * 1e-3), 1),
                "step_ms": round(hf["step_ms"], 4),
                "scan_topk_ms": round(hf["scan_ms"], 4),
                "plane_GBps": round(plane_b / (hf["scan_ms"] * 1e-3) / 1e9, 1)}
        else:
            out["roofline"] = out.pop("roofline_hbm")
    out["timings_ms"] = {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in res.items()}
    out["timings_note"] = ("*_fused rows call fathom_scan_topk; with planes in pinned host memory "
                           "('host_fused', 'host_fixed_fused') that call scans the logits into "
                           "its workspace and runs the plain top-k on them (the sampled "
                           "candidate scan needs device-resident planes), so those rows time "
                           "scan then top-k inside one call")
    for mode in ("host", "hbm"):
        if mode in res:
            out.setdefault("fixed136_speedup", {})[mode] = round(
                res[mode + "_fixed"]["step_ms"] / res[mode]["step_ms"], 3)
            out["fixed136_speedup"][mode + "_fused"] = round(
                res[mode + "_fixed_fused"]["step_ms"] / res[mode + "_fused"]["step_ms"], 3)
            out.setdefault("fixed136_scan_speedup", {})[mode] = round(
                res[mode + "_fixed"]["scan_ms"] / res[mode]["scan_ms"], 3)
    out["bytes"] = {"fathom_union_plane_bytes": plane_b, "fixed136_plane_bytes": fixed_plan_b,
                    "fixed136_meta_bytes": meta_b, "logits_bytes": logits_b,
                    "union_bits_per_kv_head": ub, "fixed136_union_bits": fub,
                    "depth_histogram": hist}
    if variants:
        variants["note"] = ("B=92 per query head (rd, calibrated) or per kv head (group: the "
                            "whole GQA group reads 92 plane bits per key; group_calibrated: 176, "
                            "about the per-head plans' union); fixed_r16: top-16 |q| channels x 4 "
                            "bits + the 8-bit side stream; fused scan + top-k steps")
        fb = plane_b
        for name, key in (("fathom_vs_fixed_r16", "fixed_r16"),
                          ("fathom_vs_fixed_r16_68bit", "fixed_r16_68bit")):
            f16 = variants[key]
            variants[name] = {
                "baseline_bits_per_key": f16["bits_per_key"],
                "byte_ratio": round(fb / (f16["union_plane_bytes"] + f16["meta_bytes"]), 4),
                **{m + "_time_ratio": round(res[m + "_fused"]["step_ms"] /
                                            f16[m + "_fused"]["step_ms"], 4)
                   for m in res_modes(args)}}
        out["plan_variants"] = variants
    out["probe"] = probe
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(layers[0], w, args.cpu_sample, args.cpu_sample_mt)
    if not args.no_extra:
        del layers
        torch.cuda.empty_cache()
        extra = {}
        if "hbm_fused" in res:
            extra["clustered_1m_hbm"] = bench_clustered(dev, 30, 5, res["hbm_fused"]["step_ms"])
            log(f"clustered: {extra['clustered_1m_hbm']}")
            torch.cuda.empty_cache()
        extra["blocked_ranges_1m"] = bench_blocked(dev, 30, 5)
        log(f"blocked ranges: {extra['blocked_ranges_1m']}")
        torch.cuda.empty_cache()
        extra["pack"] = bench_pack(dev)
        log(f"pack: {extra['pack']}")
        torch.cuda.empty_cache()
        extra["layer_131072_hbm"] = bench_layer_128k(dev, 50, 5)
        log(f"128K layer: {extra['layer_131072_hbm']}")
        torch.cuda.empty_cache()
        extra["sessions_16_host"] = bench_sessions(dev, 5, 2)
        log(f"16 sessions: {extra['sessions_16_host']}")
        torch.cuda.empty_cache()
        extra["step_36_layers"] = bench_step36(dev, 3, 1)
        log(f"36-layer step: {extra['step_36_layers']}")
        torch.cuda.empty_cache()
        extra["append_1m"] = bench_append(dev, 50, 5)
        log(f"append: {extra['append_1m']}")
        torch.cuda.empty_cache()
        extra["attention_1m"] = bench_attention(dev, 20, 3)
        log(f"attention: {extra['attention_1m']}")
        torch.cuda.empty_cache()
        extra["plan_quality"] = plan_quality(dev)
        log(f"plan quality: {extra['plan_quality']}")
        out["other_workloads"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
