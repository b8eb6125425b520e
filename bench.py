"""Benchmark: one decode layer-step of top-p sparse attention with an INT4 K estimate, on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload all|C1..C5] [--layers L] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch: Quest-style page selection (or, for the
hierarchical layer, cluster-level top-p) -> INT4 weight estimate -> per-head top-p (bisection) -> GQA
union -> split-K sparse attention -> merge.  Steps rotate over L layer caches of identical shape, enough
that the rotation exceeds 4 GiB and its INT4 codes and page bounds alone exceed 1 GiB, so every step
reads cold HBM rather than the 256 MB Infinity Cache, as a many-layer model does (up to 1 GiB of
layers are drawn independently, the rest are device copies of them at their own addresses).  Inputs
are resident in HBM before timing starts.

By default (``--workload all``) the line covers the metric's whole context range: the headline is the
256K-token hierarchical layer (C5, the largest single-GPU configuration), and the 32K Llama-shaped
layer (C2), the 16-sequence 32K layer (C3) and the 4-sequence 128K layer (C4) follow under
``workloads`` in the same JSON line, each measured the same way.

Per workload: K timed steps between synchronisations (``value`` = microseconds per layer-step, lower is
better); then a pass with timing events around every stage kernel (events created without the
system-scope fence, which would otherwise write back and invalidate caches at every event and
distort the kernels it brackets); ``roofline`` describes the split-K attention kernel (the stage that
moves most bytes): its algorithmic bytes per launch (512 B of K/V rows + 4 B index per kept token,
plus the group's q) over its event-timed duration.  ``cpu_baseline`` times the numpy oracle on a
bounded sample of the headline workload on the host cores.

With ``--estimator-bits`` it instead reports the estimator's precision ablation (2-, 4- and 8-bit K
codes on the Llama-layer workload at its p = 0.85): the event-timed estimate kernel per layer-step and
the true attention mass (exact bf16 q.k softmax) of every head's selected set, one JSON line.

With ``--offload`` it runs the offloading scenario of the pages (paperlayer §E): the bf16 K/V of the
Llama-layer workload stay in pinned host memory and the kernels read the selected rows over PCIe,
while the INT4 codes and page bounds sit in HBM; it times the decode step with top-p (p = 0.85) and
with the base selector alone (p = 1: every selected page is loaded, Quest's budget), one JSON line.

With ``--baselines`` it compares, on one layer-step, top-p against the top-k baseline at the same mean
budget (top-k on the estimated weights, and top-k on the exact weights as an oracle reference), each
with group-union and head-wise attention: K/V rows read, per-head set sizes, output error against
attention over all the base selector's candidates (what the pruning approximates) and against dense
attention, and decode time, one JSON line.

With ``--cluster-approx`` (hierarchical workload) it measures the optional approximation of the
clusters no head keeps: the time of that step and each head's output error against dense attention
with and without it, one JSON line.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse decode attention µs/layer-step + HBM GB/s fraction, 32K–256K ctx"
HBM_PEAK = 8.0e12  # MI355X HBM3E, bytes/s
DESCR = {
    "C1": "single MHA head, n=4096, no selector, p=0.9",
    "C2": "Llama-3-8B-shaped decode layer: B=1, 32/8 GQA heads, n=32768, 4 K outlier channels, keep 1/4 pages, p=0.85",
    "C3": "head heterogeneity: B=16, 32/8 heads, n=32768, per-head temperature, keep 1/4, p=0.85",
    "C4": "long context: B=4, 32/8 heads, n=131072, 64 planted keys per head, keep 1/4, p=0.9",
    "C5": "Double-P hierarchical: B=1, 32/8 heads, n=262144, 4096 Zipf(1.1) clusters, cluster p1=0.95 "
          "then token p=0.9",
}
HEADLINE = "C5"
LINE = ["C2", "C3", "C4", "C5"]  # the metric's 32K-256K range, headline last
STAGES_CLUSTER = ["cluster_scores_topp", "cluster_pages", "estimate", "topp_union", "attention", "merge"]
EVENT_NO_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all", choices=sorted(DESCR) + ["all"])
    ap.add_argument("--layers", type=int, default=0, help="layer caches rotated (0: see above)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-units", type=int, default=0, help="oracle sample size in units (0: auto)")
    ap.add_argument("--estimator-bits", action="store_true",
                    help="report the 2/4/8-bit estimator ablation instead of the step benchmark")
    ap.add_argument("--baselines", action="store_true",
                    help="compare top-p with the equal-budget top-k baseline, union vs head-wise")
    ap.add_argument("--cluster-approx", action="store_true",
                    help="measure the optional approximation of the unkept clusters (C5)")
    ap.add_argument("--offload", action="store_true",
                    help="time the decode with K/V in pinned host memory (top-p vs the base selector alone)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 5 plain 512 MiB device copies (reference for HBM byte counters)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    cdir = os.path.join(ROOT, "top_sparse_attention_int4_amd", "csrc")
    for f in sorted(os.listdir(cdir)):
        with open(os.path.join(cdir, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


class FenceFreeEvents:
    """Raw HIP timing events created with hipEventDisableSystemFence (the runtime's own flag for
    events used only to time work: no cache write-back and invalidation at each event)."""

    def __init__(self, n: int):
        import top_sparse_attention_int4_amd as twl
        self.L = twl.lib()
        self.L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.L.hipEventCreateWithFlags.restype = ctypes.c_int
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventElapsedTime.restype = ctypes.c_int
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventRecord.restype = ctypes.c_int
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.L.hipEventDestroy.restype = ctypes.c_int
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.L.hipEventCreateWithFlags(ctypes.byref(e), EVENT_NO_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e.value)

    def handles(self, i0: int, n: int) -> list:
        return self.ev[i0:i0 + n]

    def record(self, i: int, stream) -> None:
        if self.L.hipEventRecord(ctypes.c_void_p(self.ev[i]), ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, i: int, j: int) -> float:
        out = ctypes.c_float()
        if self.L.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(self.ev[i]), ctypes.c_void_p(self.ev[j])) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self) -> None:
        for e in self.ev:
            self.L.hipEventDestroy(ctypes.c_void_p(e))
        self.ev = []


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only (the path would shard over (batch, kv-head) units with no "
              "exchange). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import top_sparse_attention_int4_amd as twl

    twl.lib()  # raises if the library is missing or stale: build it before running
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.estimator_bits:
        estimator_bits_report(args, dev)
        return
    if args.offload:
        offload_report(args, dev)
        return
    if args.baselines:
        baselines_report(args, dev)
        return
    if args.cluster_approx:
        cluster_approx_report(args, dev)
        return
    if args.copy_calibration:
        # a plain device copy of known size: 512 MiB read + 512 MiB written per launch
        src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    names = LINE if args.workload == "all" else [args.workload]
    head = HEADLINE if args.workload == "all" else args.workload
    copy_gbps = plain_copy_gbps(dev)
    floor_us = launch_floor_us(dev)
    recs, wl = {}, {}
    for name in names:
        recs[name], wl[name] = measure_workload(name, args, dev, copy_gbps)
        torch.cuda.empty_cache()
    r = recs[head]
    line = {
        "metric": METRIC,
        "value": r["us_per_layer_step"],
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {**r["config"], "parallelism": "single GPU",
                   "also_in_line": [n for n in names if n != head]},
        "hbm": r["hbm"],
        "step_us_with_events": r["step_us_with_events"],
        "budgets": r["budgets"],
        "stages_us": r["stages_us"],
        "event_gap_us": r["event_gap_us"],
        "six_empty_kernels_us": floor_us,
        "roofline": r["roofline"],
        "workloads": {n: {k: recs[n][k] for k in ("config", "us_per_layer_step", "hbm", "stages_us", "event_gap_us",
                                                  "roofline", "budgets")}
                      for n in names if n != head},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl[head], args.cpu_units)
    print(json.dumps(line), flush=True)


def launch_floor_us(dev) -> float:
    """Six back-to-back one-element kernels queued behind a long copy (so they run as fast as the
    GPU dispatches them), between fence-free events: the floor of a six-kernel dependent chain."""
    import torch
    src = torch.empty(64 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    tiny = torch.empty(1, dtype=torch.float32, device=dev)
    ev = FenceFreeEvents(2)
    stream = torch.cuda.current_stream()
    out = []
    for _ in range(5):
        torch.cuda.synchronize()
        dst.copy_(src)
        ev.record(0, stream)
        for _ in range(6):
            tiny.zero_()
        ev.record(1, stream)
        torch.cuda.synchronize()
        out.append(ev.ms(0, 1) * 1e3)
    ev.close()
    del src, dst
    return round(float(np.median(out)), 3)


def plain_copy_gbps(dev) -> float:
    """A plain 512 MiB device copy on this GPU (read + written bytes over time)."""
    import torch
    src = torch.empty(128 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(5):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    s = a.elapsed_time(b) / 5 * 1e-3
    del src, dst
    return 2 * (128 << 20) * 4 / s / 1e9


def head_budgets(w, cache, t, dev):
    """Every query head's top-p budget on one layer, read through the split entry points outside the
    timed region: the candidates the base selector (or the cluster stage) hands the head and the tokens
    its own top-p keeps.  The budget adapting per head and per step is the point of top-p over a fixed
    budget (Paper-Notes 核心问题; paperlayer §3.2), and C3 is built to spread it."""
    import torch
    import top_sparse_attention_int4_amd as twl
    B, Hq, Hkv, G = w.batch, w.num_q_heads, w.num_kv_heads, w.group
    U = B * Hkv
    sm = twl.DEFAULT_SM_SCALE
    i32 = dict(dtype=torch.int32, device=dev)
    if w.csize is not None:
        C = w.num_clusters
        maxcand = w.max_seq_len
        ws = torch.empty(twl.workspace_bytes(cache, maxcand), dtype=torch.uint8, device=dev)
        rg = torch.empty((U, C, 2), **i32)
        ct = torch.empty((U,), **i32)
        twl.select_clusters_topp(cache, t["q"], sm, w.p1, 32, t["centroids"], t["csize"], t["coff"], C, rg, ct, ws)
        cand = dict(ranges=rg, count=ct, max_items=C)
    elif w.keep_frac < 1.0:
        mk = twl.keep_count(w.max_pages, w.keep_frac)
        maxcand = 16 * mk
        ws = torch.empty(twl.workspace_bytes(cache, maxcand), dtype=torch.uint8, device=dev)
        ids = torch.full((U, mk), -1, **i32)
        cnt = torch.zeros((U,), **i32)
        twl.select_pages(cache, t["q"], w.keep_frac, mk, ids, cnt, ws)
        cand = dict(page_ids=ids, count=cnt, max_items=mk)
    else:
        return None
    mw = -(-maxcand // 32)
    thr = torch.empty((B, Hq), device=dev)
    hm = torch.zeros((B, Hq, mw), **i32)
    indptr = torch.empty(U + 1, **i32)
    toks = torch.empty(U * maxcand, **i32)
    twl.estimate_topp(cache, t["q"], sm, w.p, 32, **cand, threshold=thr, head_mask=hm, mask_words=mw,
                      sel_indptr=indptr, sel_tokens=toks, ws=ws)
    torch.cuda.synchronize()
    kept = np.unpackbits(hm.cpu().numpy().view(np.uint8), axis=-1).sum(axis=-1).reshape(B * Hq)
    # candidates per unit: the valid slots of the listed pages, or the lengths of the kept ranges
    ncand = np.zeros(U, np.int64)
    if "ranges" in cand:
        r, c_ = rg.cpu().numpy(), ct.cpu().numpy()
        for u in range(U):
            ncand[u] = int(np.maximum(r[u, :c_[u], 1], 0).sum())
    else:
        pg, c_ = ids.cpu().numpy(), cnt.cpu().numpy()
        for u in range(U):
            n = int(w.seq_lens[u // Hkv])
            ncand[u] = int(np.clip(n - 16 * pg[u, :c_[u]].astype(np.int64), 0, 16).sum())
    frac = kept / np.maximum(np.repeat(ncand, G), 1)
    union = np.diff(indptr.cpu().numpy()) / np.maximum(ncand, 1)
    pct = lambda x, qs: {f"p{q}": round(float(np.percentile(x, q)), 4) for q in qs}
    return {"heads": int(B * Hq), "candidates_per_unit_median": int(np.median(ncand)),
            "kept_tokens_per_head": {"min": int(kept.min()), **pct(kept, (10, 50, 90)), "max": int(kept.max())},
            "kept_fraction_of_candidates": {"min": round(float(frac.min()), 4), **pct(frac, (10, 50, 90)),
                                            "max": round(float(frac.max()), 4)},
            "group_union_fraction_of_candidates_mean": round(float(union.mean()), 4)}


def measure_workload(name, args, dev, copy_gbps):
    """One workload's record (and its layer-0 workload object, for the CPU baseline)."""
    import torch
    import top_sparse_attention_int4_amd as twl
    from gen import make_config
    from gen.device import upload

    # ---- layers ----------------------------------------------------------------------------------
    w0 = make_config(name, layer=0)
    # per (page, kv-head): K and V 4 KiB each; INT4 codes 1 KiB, scale/zero 256 B, page bounds 512 B
    small = 0.4375 * w0.k_pages.nbytes
    per_layer = 2 * w0.k_pages.nbytes + small
    # enough layers that the whole rotation exceeds 4 GiB and its codes and bounds alone exceed 1 GiB
    # (four times the 256 MB Infinity Cache), as in a many-layer model
    L = args.layers or max(math.ceil((4 << 30) / per_layer), math.ceil((1 << 30) / small))
    n_drawn = min(L, max(1, math.ceil((1 << 30) / per_layer)))
    print(f"[bench] {name}: {L} layer(s) ({n_drawn} drawn, the rest device copies), "
          f"{per_layer / 1e6:.0f} MB each", file=sys.stderr, flush=True)
    layers = []
    for li in range(L):
        if li < n_drawn:
            w = w0 if li == 0 else make_config(name, layer=li)
            t = upload(w, dev)
        else:
            # a copy at its own addresses: the same values (so the same work), cold in every cache
            w, t0 = layers[li % n_drawn][0], layers[li % n_drawn][2]
            t = dict(t0)
            t["k_pages"], t["v_pages"] = t0["k_pages"].clone(), t0["v_pages"].clone()
        cache = twl.PagedCache(t["k_pages"], t["v_pages"], t["page_table"], t["seq_lens"], w.num_q_heads,
                               max_seq_len=w.max_seq_len)
        twl.quantize_k(cache, torch.zeros(w.batch, dtype=torch.int32, device=dev), t["seq_lens"], w.max_seq_len)
        layers.append((w, cache, t))
    torch.cuda.synchronize()
    w = w0
    B, Hq, Hkv = w.batch, w.num_q_heads, w.num_kv_heads
    U = B * Hkv
    kf, p = w.keep_frac, w.p
    clusters = w.csize is not None
    selector = kf < 1.0 and not clusters
    maxcand = 16 * twl.keep_count(w.max_pages, kf) if selector else w.max_seq_len
    ws = torch.empty(twl.workspace_bytes(layers[0][1], maxcand), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, 128), device=dev)
    lse = torch.empty((B, Hq), device=dev)
    thr = torch.empty((B, Hq), device=dev)
    indptrs = [torch.zeros(U + 1, dtype=torch.int32, device=dev) for _ in range(L)]
    toks = torch.empty(U * maxcand, dtype=torch.int32, device=dev)

    def step(i, events=None, lists=False):
        # the timed step returns out, lse and the thresholds; the compacted kept-token list is an
        # optional output, requested once per layer outside the timed region for the byte count
        _, cache, t = layers[i % L]
        ip, tk = (indptrs[i % L], toks) if lists else (None, None)
        if clusters:
            twl.decode_clusters(cache, t["q"], p=p, p1=w.p1, centroids=t["centroids"], csize=t["csize"],
                                coff=t["coff"], out=out, lse=lse, threshold=thr, sel_indptr=ip, sel_tokens=tk,
                                ws=ws, events=events)
        elif events is not None:
            twl.decode_profiled(cache, t["q"], events, p=p, keep_frac=kf, out=out, lse=lse, threshold=thr,
                                sel_indptr=ip, sel_tokens=tk, ws=ws)
        else:
            twl.decode(cache, t["q"], p=p, keep_frac=kf, out=out, lse=lse, threshold=thr, sel_indptr=ip,
                       sel_tokens=tk, ws=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # ---- timed region: K plain steps -------------------------------------------------------------
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # ---- second timed pass: fence-free events around every stage kernel --------------------------
    nev = 2 * twl.NUM_STAGES
    K2 = args.steps
    fe = FenceFreeEvents(nev * K2)
    torch.cuda.synchronize()
    for i in range(K2):
        step(i, fe.handles(i * nev, nev))
    torch.cuda.synchronize()
    stage_ms = np.zeros(twl.NUM_STAGES)
    gap_ms = []
    for i in range(K2):
        b0 = i * nev
        for s_ in range(twl.NUM_STAGES):
            stage_ms[s_] += fe.ms(b0 + 2 * s_, b0 + 2 * s_ + 1)
        # between one stage's closing event and the next stage's opening one nothing is enqueued:
        # those gaps are the cost of an event record inside a busy stream
        gap_ms += [fe.ms(b0 + 2 * s_ + 1, b0 + 2 * s_ + 2) for s_ in range(twl.NUM_STAGES - 1)]
    stage_ms /= K2
    fe.close()
    gap_us = float(np.median(gap_ms)) * 1e3
    for li in range(L):
        step(li, lists=True)
    torch.cuda.synchronize()
    kept = [indptrs[li].cpu().numpy() for li in range(L)]
    budgets = head_budgets(w0, layers[0][1], layers[0][2], dev)

    # ---- per-step spread: a third pass with one event pair around each step -----------------------
    fp = FenceFreeEvents(2 * args.steps)
    stream = torch.cuda.current_stream()
    for i in range(args.steps):
        fp.record(2 * i, stream)
        step(i)
        fp.record(2 * i + 1, stream)
    torch.cuda.synchronize()
    st_us = np.array([fp.ms(2 * i, 2 * i + 1) for i in range(args.steps)]) * 1e3
    fp.close()
    step_spread = {k: round(float(np.percentile(st_us, q)), 3) for k, q in (("p10", 10), ("p50", 50), ("p90", 90))}

    # ---- the INT4 append (a0), timed alone ---------------------------------------------------------
    _, cache0, t0 = layers[0]
    zeros_b = torch.zeros(B, dtype=torch.int32, device=dev)
    ntok = int(w.seq_lens.astype(np.int64).sum())
    for _ in range(2):
        twl.quantize_k(cache0, zeros_b, t0["seq_lens"], w.max_seq_len)
    a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a_.record()
    for _ in range(5):
        twl.quantize_k(cache0, zeros_b, t0["seq_lens"], w.max_seq_len)
    b_.record()
    torch.cuda.synchronize()
    # per (token, kv-head): 256 B of K read, 64 B of codes and 16 B of scale/zero written;
    # per (page, kv-head): 512 B of bounds written
    append_bytes = Hkv * (ntok * (256 + 80) + int((-(-w.seq_lens.astype(np.int64) // 16)).sum()) * 512)
    append_gbps = append_bytes / (a_.elapsed_time(b_) / 5 * 1e-3) / 1e9

    # ---- algorithmic bytes (per layer-step, averaged over the layers) ----------------------------
    seq = w.seq_lens.astype(np.int64)
    pages = -(-seq // 16)
    sel_tokens_total = float(np.mean([ip[-1] for ip in kept]))
    q_bytes = 2 * Hq * 128
    if clusters:
        # candidates = tokens of the kept clusters, read back from one extra cluster selection per layer
        C = w.num_clusters
        ncand = []
        for _, cache, t in layers:
            rg = torch.empty((U, C, 2), dtype=torch.int32, device=dev)
            ct = torch.empty((U,), dtype=torch.int32, device=dev)
            twl.select_clusters_topp(cache, t["q"], twl.DEFAULT_SM_SCALE, w.p1, 32, t["centroids"], t["csize"],
                                     t["coff"], C, rg, ct, ws)
            rg, ct = rg.cpu().numpy(), ct.cpu().numpy()
            ncand.append(sum(int(rg[u, :ct[u], 1].sum()) for u in range(U)))
        cand_units_total = float(np.mean(ncand))
        bytes_sel = U * C * (256 + 8)  # centroid rows + size and offset
    else:
        cand = np.array([min(16 * twl.keep_count(int(P), kf), int(n)) if selector else int(n)
                         for P, n in zip(pages, seq)])  # valid candidates per sequence (upper bound)
        cand_units_total = float(cand.sum() * Hkv)
        bytes_sel = (512 * pages.sum() * Hkv) if selector else 0
    bytes_est = 80 * cand_units_total
    bytes_attn = 516 * sel_tokens_total + q_bytes
    bytes_step = bytes_sel + bytes_est + bytes_attn + 4 * Hq * 128 + q_bytes
    attn_ms = stage_ms[4]
    achieved = bytes_attn / (attn_ms * 1e-3)

    traffic = None
    prof = os.path.join(ROOT, "profiles", f"traffic_attn_splitk_{name}.json")
    if os.path.exists(prof):
        with open(prof) as fh:
            tr = json.load(fh)
        if tr.get("kernel_source_hash") == kernel_source_hash():
            traffic = tr.get("hbm_bytes_per_launch")
    # bytes the whole step touches (counter passes over every kernel of the step, committed under
    # profiles/), while the kernel sources still hash to the recorded value
    touched = None
    prof = os.path.join(ROOT, "profiles", f"traffic_step_{name}.json")
    if os.path.exists(prof):
        with open(prof) as fh:
            tr = json.load(fh)
        if tr.get("kernel_source_hash") == kernel_source_hash():
            touched = tr.get("hbm_bytes_per_step")
    step_s = ms_per_step * 1e-3
    rec = {
        "us_per_layer_step": round(ms_per_step * 1e3, 3),
        "ms_per_step": round(ms_per_step, 6),
        "config": {"workload": f"{name}: {DESCR[name]}", "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "context": int(seq.max()), "p": p, "keep_frac": kf, "layers_rotated": L,
                   **({"p1": w.p1, "num_clusters": w.num_clusters} if clusters else {})},
        "hbm": {"algorithmic_bytes_per_step": int(bytes_step), "gbps": round(bytes_step / step_s / 1e9, 1),
                "frac_of_8TBps": round(bytes_step / step_s / HBM_PEAK, 4),
                "touched_bytes_per_step": touched,
                "touched_frac_of_8TBps": (round(touched / step_s / HBM_PEAK, 4) if touched else None),
                "copy_gbps": round(copy_gbps, 1),
                "frac_of_copy": round(bytes_step / step_s / 1e9 / copy_gbps, 4),
                "append_gbps": round(append_gbps, 1),
                "candidates_per_step": cand_units_total, "kept_tokens_per_step": sel_tokens_total},
        "step_us_with_events": step_spread,
        "budgets": budgets,
        "stages_us": {n: round(float(x) * 1e3, 3)
                      for n, x in zip(STAGES_CLUSTER if clusters else twl.STAGE_NAMES, stage_ms)},
        "event_gap_us": round(gap_us, 3),
        "roofline": {"kernel": "k_attn (split-K sparse attention)", "bound": "hbm",
                     "achieved": round(achieved / 1e9, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(bytes_attn), "avg_launch_us": round(attn_ms * 1e3, 3),
                     "frac_of_copy": round(achieved / 1e9 / copy_gbps, 4)},
    }
    del layers, ws, toks, indptrs
    return rec, w0


def estimator_bits_report(args, dev):
    """The pages' precision ablation (paperlayer §4.2, Fig. 6): top-p at p = 0.85 on weights estimated
    from 2-, 4- and 8-bit K codes.  Per width: the estimate kernel's event-timed duration (decode
    steps rotating over enough code copies that they come from HBM), and per query head the exact
    attention mass of its selected set -- over the base selector's candidates (top-p's domain) and
    over the whole context -- from a float32 softmax of the bf16 q.k logits."""
    import torch
    import top_sparse_attention_int4_amd as twl
    from gen import make_config
    from gen.device import upload

    name = "C2" if args.workload == "C2" else args.workload
    w = make_config(name)
    if w.csize is not None or w.keep_frac >= 1.0:
        raise SystemExit("--estimator-bits needs a page-selector workload (C2, C3 or C4)")
    t = upload(w, dev)
    B, Hq, Hkv, G = w.batch, w.num_q_heads, w.num_kv_heads, w.group
    U = B * Hkv
    sm = float(np.float32(1.0 / math.sqrt(128)))
    mk = twl.keep_count(w.max_pages, w.keep_frac)
    maxcand = 16 * mk
    mw = maxcand // 32
    # exact logits of every (b, q-head) over its sequence, float32 from bf16
    kf = t["k_pages"].view(torch.bfloat16).float() if t["k_pages"].dtype != torch.bfloat16 else t["k_pages"].float()
    qf = t["q"].view(torch.bfloat16).float() if t["q"].dtype != torch.bfloat16 else t["q"].float()
    exact = {}
    for b in range(B):
        n = int(w.seq_lens[b])
        npg = -(-n // 16)
        pt = t["page_table"][b, :npg].long()
        kseq = kf[pt].permute(1, 0, 2, 3).reshape(Hkv, npg * 16, 128)[:, :n]      # [Hkv][n][128]
        for h in range(Hkv):
            lg = (kseq[h] @ qf[b, h * G:(h + 1) * G].T).T * sm                       # [G][n]
            exact[(b, h)] = lg
    rows = []
    L = 32  # code copies rotated in the timing (4-bit codes of one copy: 17 MB)
    for bits in (2, 4, 8):
        caches = []
        for li in range(L):
            c = twl.PagedCache(t["k_pages"], t["v_pages"], t["page_table"], t["seq_lens"], Hq,
                               max_seq_len=w.max_seq_len, key_bits=bits)
            twl.quantize_k(c, torch.zeros(B, dtype=torch.int32, device=dev), t["seq_lens"], w.max_seq_len)
            caches.append(c)
        ws = torch.empty(twl.workspace_bytes(caches[0], maxcand), dtype=torch.uint8, device=dev)
        out = torch.empty((B, Hq, 128), device=dev)
        K = max(args.steps, 20)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * twl.NUM_STAGES)] for _ in range(K)]
        for i in range(5):
            twl.decode(caches[i % L], t["q"], p=w.p, keep_frac=w.keep_frac, out=out, ws=ws)
        torch.cuda.synchronize()
        for i in range(K):
            twl.decode_profiled(caches[i % L], t["q"], evs[i], p=w.p, keep_frac=w.keep_frac, out=out, ws=ws)
        torch.cuda.synchronize()
        est_us = 1e3 * float(np.mean([evs[i][4].elapsed_time(evs[i][5]) for i in range(K)]))
        # the selection of one step, split into its stages to read every head's kept set
        ids = torch.full((U, mk), -1, dtype=torch.int32, device=dev)
        cnt = torch.zeros(U, dtype=torch.int32, device=dev)
        twl.select_pages(caches[0], t["q"], w.keep_frac, mk, ids, cnt, ws)
        thr = torch.empty((B, Hq), device=dev)
        mass = torch.empty((B, Hq), device=dev)
        hm = torch.zeros((B, Hq, mw), dtype=torch.int32, device=dev)
        indptr = torch.empty(U + 1, dtype=torch.int32, device=dev)
        toks = torch.empty(U * maxcand, dtype=torch.int32, device=dev)
        twl.estimate_topp(caches[0], t["q"], sm, w.p, 32, page_ids=ids, count=cnt, max_items=mk, threshold=thr,
                          mass=mass, head_mask=hm, mask_words=mw, sel_indptr=indptr, sel_tokens=toks, ws=ws)
        torch.cuda.synchronize()
        ids_h, cnt_h = ids.cpu().numpy(), cnt.cpu().numpy()
        bits_m = np.unpackbits(hm.cpu().numpy().view(np.uint8), axis=-1, bitorder="little")
        m_cand, m_full, frac = [], [], []
        for b in range(B):
            n = int(w.seq_lens[b])
            for h in range(Hkv):
                u = b * Hkv + h
                pages = ids_h[u, :cnt_h[u]].astype(np.int64)
                cand = (pages[:, None] * 16 + np.arange(16)[None, :]).reshape(-1)
                ok = cand < n
                lg = exact[(b, h)]
                cidx = torch.from_numpy(cand[ok]).to(dev)
                for j in range(G):
                    sel = np.nonzero(bits_m[b, h * G + j, :cand.size][ok])[0]
                    wc = torch.softmax(lg[j, cidx], 0)
                    wf = torch.softmax(lg[j], 0)
                    s_idx = torch.from_numpy(sel).to(dev)
                    m_cand.append(float(wc[s_idx].sum()))
                    m_full.append(float(wf[cidx[s_idx]].sum()))
                    frac.append(sel.size / max(1, int(ok.sum())))
        rows.append({"bits": bits, "estimate_us": round(est_us, 3),
                     "true_mass_over_candidates": {"mean": round(float(np.mean(m_cand)), 5),
                                                   "min": round(float(np.min(m_cand)), 5)},
                     "true_mass_over_context": {"mean": round(float(np.mean(m_full)), 5),
                                                "min": round(float(np.min(m_full)), 5)},
                     "kept_fraction_of_candidates": round(float(np.mean(frac)), 5),
                     "code_bytes_per_candidate_head": 16 * bits + 16})
        del caches
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "estimator precision ablation (top-p at p, true selected mass vs code bits)",
                      "workload": name, "p": w.p, "heads": B * Hq, "steps": K, "data": "synthetic",
                      "rows": rows}))


def baselines_report(args, dev):
    """Top-p against the fixed-budget top-k baseline (paperlayer §3, Fig. 2-3) and group-union against
    head-wise attention for GQA (paperlayer §B.2; Paper-Notes "局限与展望").  k = the mean size of the
    heads' top-p sets, so both spend the same total budget.  Errors are relative L2 distances of each
    head's output from attention over every candidate of the base selector (the decode at p = 1) --
    the quantity top-p bounds -- and from dense attention over the whole context (float32 torch)."""
    import torch
    import top_sparse_attention_int4_amd as twl
    from gen import make_config
    from gen.device import upload

    name = args.workload
    w = make_config(name)
    if w.csize is not None or w.keep_frac >= 1.0:
        raise SystemExit("--baselines runs the page-selector workloads (C2, C3, C4)")
    t = upload(w, dev)
    B, Hq, Hkv, G = w.batch, w.num_q_heads, w.num_kv_heads, w.group
    U = B * Hkv
    sm = float(np.float32(1.0 / math.sqrt(128)))
    mk = twl.keep_count(w.max_pages, w.keep_frac)
    maxcand = 16 * mk
    mw = maxcand // 32
    cache = twl.PagedCache(t["k_pages"], t["v_pages"], t["page_table"], t["seq_lens"], Hq, max_seq_len=w.max_seq_len)
    twl.quantize_k(cache, torch.zeros(B, dtype=torch.int32, device=dev), t["seq_lens"], w.max_seq_len)
    ws = torch.empty(twl.workspace_bytes(cache, maxcand), dtype=torch.uint8, device=dev)
    # dense references and the per-unit logical K/V, float32
    kf, vf, qf = t["k_pages"].float(), t["v_pages"].float(), t["q"].float()
    dense, kv = {}, {}
    for b in range(B):
        n = int(w.seq_lens[b])
        npg = -(-n // 16)
        pt = t["page_table"][b, :npg].long()
        ks = kf[pt].permute(1, 0, 2, 3).reshape(Hkv, npg * 16, 128)[:, :n]
        vs = vf[pt].permute(1, 0, 2, 3).reshape(Hkv, npg * 16, 128)[:, :n]
        for h in range(Hkv):
            lg = (ks[h] @ qf[b, h * G:(h + 1) * G].T).T * sm                  # [G][n]
            dense[(b, h)] = (torch.softmax(lg, -1) @ vs[h], lg)
            kv[(b, h)] = vs[h]
    # the heads' top-p sets (split entry points: page ids, then head bitmaps over the candidates)
    ids = torch.full((U, mk), -1, dtype=torch.int32, device=dev)
    cnt = torch.zeros(U, dtype=torch.int32, device=dev)
    twl.select_pages(cache, t["q"], w.keep_frac, mk, ids, cnt, ws)
    thr = torch.empty((B, Hq), device=dev)
    hm = torch.zeros((B, Hq, mw), dtype=torch.int32, device=dev)
    indptr = torch.empty(U + 1, dtype=torch.int32, device=dev)
    toks = torch.empty(U * maxcand, dtype=torch.int32, device=dev)
    twl.estimate_topp(cache, t["q"], sm, w.p, 32, page_ids=ids, count=cnt, max_items=mk, threshold=thr,
                      head_mask=hm, mask_words=mw, sel_indptr=indptr, sel_tokens=toks, ws=ws)
    torch.cuda.synchronize()
    bits_m = np.unpackbits(hm.cpu().numpy().view(np.uint8), axis=-1, bitorder="little")
    k_eq = max(1, int(round(float(np.mean(bits_m[..., :maxcand].sum(-1))))))
    ids_h, cnt_h = ids.cpu().numpy(), cnt.cpu().numpy()
    out = torch.empty((B, Hq, 128), device=dev)
    K = max(10, min(args.steps, 50))

    o_cand = torch.empty((B, Hq, 128), device=dev)
    twl.decode(cache, t["q"], p=1.0, keep_frac=w.keep_frac, out=o_cand, ws=ws)
    torch.cuda.synchronize()

    def err_of(o, ref=None):
        e = []
        for (b, h), (od, _) in dense.items():
            r = od if ref is None else ref[b, h * G:(h + 1) * G]
            x = o[b, h * G:(h + 1) * G]
            e.append((torch.linalg.norm(x - r, dim=-1) / torch.linalg.norm(r, dim=-1)).cpu().numpy())
        e = np.concatenate(e)
        return {"mean": round(float(e.mean()), 6), "max": round(float(e.max()), 6)}

    rows = []
    for label, topk in (("top-p", 0), (f"top-k (estimated weights, k={k_eq})", k_eq)):
        for headwise in (False, True):
            for _ in range(3):
                twl.decode(cache, t["q"], p=w.p, keep_frac=w.keep_frac, out=out, ws=ws, topk=topk, headwise=headwise)
            a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for _ in range(K):
                twl.decode(cache, t["q"], p=w.p, keep_frac=w.keep_frac, out=out, ws=ws, topk=topk, headwise=headwise)
            b_.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b_) / K * 1e3
            twl.decode(cache, t["q"], p=w.p, keep_frac=w.keep_frac, out=out, ws=ws, topk=topk, headwise=headwise,
                       sel_indptr=indptr, sel_tokens=toks)
            torch.cuda.synchronize()
            rows.append({"selection": label, "attention": "head-wise" if headwise else "group union",
                         "kv_rows_read": int(indptr[-1].item()), "us_per_layer_step": round(us, 1),
                         "error_vs_candidates": err_of(out, o_cand), "error_vs_dense": err_of(out)})
    # oracle reference: top-k on the exact weights over the same candidates, head-wise
    o_ref = torch.zeros((B, Hq, 128), device=dev)
    rows_ref = 0
    for (b, h), (od, lg) in dense.items():
        u = b * Hkv + h
        n = int(w.seq_lens[b])
        pages = ids_h[u, :cnt_h[u]].astype(np.int64)
        cand = (pages[:, None] * 16 + np.arange(16)[None, :]).reshape(-1)
        cidx = torch.from_numpy(cand[cand < n]).to(dev)
        union = set()
        for j in range(G):
            top = cidx[torch.topk(lg[j, cidx], min(k_eq, cidx.numel())).indices]
            union |= set(top.tolist())
            o_ref[b, h * G + j] = torch.softmax(lg[j, top], 0) @ kv[(b, h)][top]
        rows_ref += len(union)
    rows.append({"selection": f"top-k (exact weights, k={k_eq}; torch reference)", "attention": "head-wise",
                 "kv_rows_read": rows_ref, "us_per_layer_step": None,
                 "error_vs_candidates": err_of(o_ref, o_cand), "error_vs_dense": err_of(o_ref)})
    print(json.dumps({"metric": "top-p vs equal-budget top-k; group union vs head-wise attention",
                      "workload": name, "p": w.p, "heads": B * Hq, "steps": K, "data": "synthetic",
                      "top_p_set_size": {"mean": round(float(np.mean(bits_m[..., :maxcand].sum(-1))), 1),
                                         "min": int(bits_m[..., :maxcand].sum(-1).min()),
                                         "max": int(bits_m[..., :maxcand].sum(-1).max())},
                      "rows": rows}))


def cluster_approx_report(args, dev):
    """The optional merge of the unkept clusters (as centroid key and mean value, times their size)
    into the hierarchical decode's output: its event-timed duration, and every head's relative L2
    error against dense attention over the whole context (float32 torch) with and without it."""
    import torch
    import top_sparse_attention_int4_amd as twl
    from gen import make_config
    from gen.device import upload

    name = args.workload if args.workload == "C5" else "C5"
    w = make_config(name)
    t = upload(w, dev)
    B, Hq, Hkv, G = w.batch, w.num_q_heads, w.num_kv_heads, w.group
    C = w.csize.shape[-1]
    sm = float(np.float32(1.0 / math.sqrt(128)))
    cache = twl.PagedCache(t["k_pages"], t["v_pages"], t["page_table"], t["seq_lens"], Hq, max_seq_len=w.max_seq_len)
    twl.quantize_k(cache, torch.zeros(B, dtype=torch.int32, device=dev), t["seq_lens"], w.max_seq_len)
    ws = torch.empty(twl.workspace_bytes(cache, max(C, w.max_seq_len)), dtype=torch.uint8, device=dev)
    vm = torch.empty((B, Hkv, C, 128), device=dev)
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    twl.cluster_value_means(cache, t["csize"], t["coff"], vm)
    a1.record()
    out = torch.empty((B, Hq, 128), device=dev)
    lse = torch.empty((B, Hq), device=dev)
    K = max(10, min(args.steps, 50))
    dec_us, apx_us = [], []
    for i in range(K + 3):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        twl.decode_clusters(cache, t["q"], p=w.p, p1=w.p1, centroids=t["centroids"], csize=t["csize"],
                            coff=t["coff"], out=out, lse=lse, ws=ws)
        e[1].record()
        if i == K + 2:
            base = out.clone()
        twl.cluster_approx_unkept(cache, t["q"], p1=w.p1, centroids=t["centroids"], csize=t["csize"], vmean=vm,
                                  out=out, lse=lse, ws=ws)
        e[2].record()
        torch.cuda.synchronize()
        if i >= 3:
            dec_us.append(e[0].elapsed_time(e[1]) * 1e3)
            apx_us.append(e[1].elapsed_time(e[2]) * 1e3)
    approx = out.clone()
    kf, vf, qf = t["k_pages"].float(), t["v_pages"].float(), t["q"].float()
    errs = {"decode": [], "decode + unkept clusters": []}
    for b in range(B):
        n = int(w.seq_lens[b])
        npg = -(-n // 16)
        pt = t["page_table"][b, :npg].long()
        ks = kf[pt].permute(1, 0, 2, 3).reshape(Hkv, npg * 16, 128)[:, :n]
        vs = vf[pt].permute(1, 0, 2, 3).reshape(Hkv, npg * 16, 128)[:, :n]
        for h in range(Hkv):
            od = torch.softmax((ks[h] @ qf[b, h * G:(h + 1) * G].T).T * sm, -1) @ vs[h]
            for key, o in (("decode", base), ("decode + unkept clusters", approx)):
                x = o[b, h * G:(h + 1) * G]
                errs[key].append((torch.linalg.norm(x - od, dim=-1) / torch.linalg.norm(od, dim=-1)).cpu().numpy())
    rows = {k: {"mean": round(float(np.concatenate(v).mean()), 5), "max": round(float(np.concatenate(v).max()), 5)}
            for k, v in errs.items()}
    torch.cuda.synchronize()
    print(json.dumps({"metric": "unkept-cluster approximation: time and error against dense attention",
                      "workload": name, "clusters": C, "p1": w.p1, "p": w.p, "steps": K, "data": "synthetic",
                      "decode_us": round(float(np.mean(dec_us)), 1), "approx_us": round(float(np.mean(apx_us)), 1),
                      "value_means_us_once": round(a0.elapsed_time(a1) * 1e3, 1),
                      "error_vs_dense": rows}))


def offload_report(args, dev):
    """K/V in pinned host memory (paperlayer §E): decode µs per layer-step with top-p at the workload's
    p and with p = 1 (the base selector's pages all loaded, as Quest alone would), plus the K/V rows
    each loads; the same decode with K/V in HBM for reference."""
    import torch
    import top_sparse_attention_int4_amd as twl
    from gen import make_config
    from gen.device import upload

    name = args.workload
    w = make_config(name)
    if w.csize is not None:
        raise SystemExit("--offload runs the page-selector workloads (C1-C4)")
    t = upload(w, dev)
    B, Hq, Hkv = w.batch, w.num_q_heads, w.num_kv_heads
    U = B * Hkv
    maxcand = 16 * twl.keep_count(w.max_pages, w.keep_frac) if w.keep_frac < 1.0 else w.max_seq_len
    zeros = torch.zeros(B, dtype=torch.int32, device=dev)
    kh = t["k_pages"].cpu().pin_memory()
    vh = t["v_pages"].cpu().pin_memory()
    placements = {}
    for where, (kk, vv) in (("host", (kh, vh)), ("device", (t["k_pages"], t["v_pages"]))):
        c = twl.PagedCache(kk, vv, t["page_table"], t["seq_lens"], Hq, max_seq_len=w.max_seq_len)
        twl.quantize_k(c, zeros, t["seq_lens"], w.max_seq_len)
        placements[where] = c
    torch.cuda.synchronize()
    ws = torch.empty(twl.workspace_bytes(placements["host"], maxcand), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, 128), device=dev)
    indptr = torch.zeros(U + 1, dtype=torch.int32, device=dev)
    toks = torch.empty(U * maxcand, dtype=torch.int32, device=dev)
    K = max(10, min(args.steps, 50))
    rows = []
    for where, c in placements.items():
        for mode, p in (("top-p", w.p), ("base selector only (p = 1)" if w.keep_frac < 1.0 else "dense (p = 1)", 1.0)):
            for _ in range(3):
                twl.decode(c, t["q"], p=p, keep_frac=w.keep_frac, out=out, ws=ws)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for _ in range(K):
                twl.decode(c, t["q"], p=p, keep_frac=w.keep_frac, out=out, ws=ws)
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / K * 1e3
            twl.decode(c, t["q"], p=p, keep_frac=w.keep_frac, out=out, ws=ws, sel_indptr=indptr, sel_tokens=toks)
            torch.cuda.synchronize()
            loaded = int(indptr[-1].item())
            rows.append({"kv": where, "mode": mode, "p": p, "us_per_layer_step": round(us, 1),
                         "kv_rows_loaded": loaded, "kv_bytes_loaded": loaded * 512,
                         "kv_gb_per_s": round(loaded * 512 / (us * 1e-6) / 1e9, 1)})
    host = [r["us_per_layer_step"] for r in rows if r["kv"] == "host"]
    print(json.dumps({"metric": "offloaded-KV decode µs/layer-step (top-p vs base selector alone)",
                      "workload": name, "steps": K, "data": "synthetic", "rows": rows,
                      "host_speedup_of_top_p": round(host[1] / host[0], 2)}))


def cpu_baseline(w, units: int):
    """The numpy oracle (as it stands, single-threaded) on a bounded sample of the workload: whole
    (sequence, kv-head) units of the layer-step, repeated until about 10 s of CPU work has been done
    (capped at about 30 s), scaled to microseconds per whole layer-step."""
    from threadpoolctl import threadpool_limits

    from oracle import pipeline
    U = w.batch * w.num_kv_heads
    sample = [(u // w.num_kv_heads, u % w.num_kv_heads) for u in range(U)]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        pipeline.decode(w, units=sample[:1])
        one = time.perf_counter() - t0
        n = units or max(1, min(U, int(10.0 / max(one, 1e-3))))
        reps, dt = 0, 0.0
        while dt < 10.0 and (reps == 0 or dt + dt / reps < 30.0):
            t0 = time.perf_counter()
            pipeline.decode(w, units=sample[:n])
            dt += time.perf_counter() - t0
            reps += 1
    per_step = dt / (reps * n) * U
    return {"value": round(per_step * 1e6, 1), "unit": "us/layer-step", "cores": 1, "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "blas_threads": 1,
            "sample": f"{n} of {U} (sequence, kv-head) units of one layer-step x {reps} repetitions, numpy "
                      f"float64 oracle on 1 thread, {dt:.1f} s in total, scaled to {U} units"}


if __name__ == "__main__":
    main()
