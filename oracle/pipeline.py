"""The whole select-then-prune decode step, composed from O1-O11 (Paper-Notes "整体框架";
paperlayer §4.1, Fig. 5): existing selector with a generous budget -> INT4 weight estimate ->
per-head top-p -> group union -> sparse attention over the survivors.

``decode_unit`` runs one (sequence b, kv-head h) unit; ``decode`` runs them all.  Inputs are plain
arrays (bf16 as uint16 bits) in the logical per-sequence order:

  q        uint16 [G][128]      the group's query heads
  kseq     uint16 [n][128]      this kv-head's keys, token order
  vseq     uint16 [n][128]
  keep_frac  selector budget as a fraction of pages (>= 1: every page is a candidate)
  ranges   optional (begin, length) candidate ranges (the cluster path) instead of pages

``band`` (optional) states the precision of an implementation the result will be compared with: a
callable ``band(qbits_h, codes, scale16, zero16, logits) -> (err, tau_p_extra)`` giving, per
candidate, a bound on that implementation's logit error (which bounds its relative weight error) and
its mass-sum resolution.  It only widens the ambiguity sets of ``topp.topp_sort``; the sets
themselves are always those of the float64 definition.
"""

from __future__ import annotations

import math

import numpy as np

from . import attention, doublep, estimate, quantize, select, topp


def decode_unit(q: np.ndarray, kseq: np.ndarray, vseq: np.ndarray, *, p: float, keep_frac: float,
                sm: float, ranges=None, bits: int = 4, topk: int = 0, headwise: bool = False,
                band=None) -> dict:
    """``topk`` > 0 replaces each head's top-p set by its top-k set (the fixed-budget baseline);
    ``headwise`` makes each query head attend over its own set instead of the group's union."""
    n = kseq.shape[0]
    G = q.shape[0]
    out: dict = {}
    # ---- base selector -------------------------------------------------------------------------
    if ranges is not None:
        cand = select.candidates_from_ranges(ranges)
        out["pages"] = None
    elif keep_frac >= 1.0:
        npg = -(-n // 16)
        out["pages"] = np.arange(npg, dtype=np.int32)
        cand = select.candidates_from_pages(out["pages"], n)
    else:
        kmin, kmax = quantize.page_bounds(kseq[:, None, :])
        kmin, kmax = kmin[:, 0, :], kmax[:, 0, :]
        gs = select.group_scores(q, kmin, kmax)
        out["group_scores"] = gs
        out["pages"] = select.top_pages(gs, select.keep_count(kmin.shape[0], keep_frac))
        cand = select.candidates_from_pages(out["pages"], n)
    out["candidates"] = cand
    # ---- INT4 estimate, softmax, top-p per query head ------------------------------------------
    qz = quantize.quantize_rows(kseq[cand], bits) if cand.size else None
    heads = []
    for h in range(G):
        err, extra = None, 0.0
        if cand.size:
            lg = estimate.logits_f64(q[h], qz["codes"], qz["scale"], qz["zero"], sm)
            W = estimate.softmax_f64(lg)
            if band is not None:
                err, extra = band(q[h], qz["codes"], qz["scale"], qz["zero"], lg)
        else:
            lg = np.zeros(0)
            W = np.zeros(0)
        res = topp.topk_sort(W, topk, err) if topk > 0 else topp.topp_sort(W, p, err, extra)
        hd = {"logits": lg, "W": W, "topp": res, "tokens": cand[res["sel"]], "err": err}
        heads.append(hd)
    out["heads"] = heads
    # ---- union and attention -------------------------------------------------------------------
    U = attention.union([hd["tokens"] for hd in heads])
    out["union"] = U
    o = np.zeros((G, 128))
    lse = np.zeros(G)
    for h in range(G):
        o[h], lse[h] = attention.sparse_attention(q[h], kseq, vseq, heads[h]["tokens"] if headwise else U, sm)
    out["out"], out["lse"] = o, lse
    return out


def decode(w, *, p=None, keep_frac=None, sm=None, units=None, bits=4, topk=0, headwise=False,
           approx_unkept=False, band=None, ranges=None) -> dict:
    """Run the oracle on a workload-like object (fields of ``gen.Workload``).

    ``units`` optionally restricts the work to a list of (b, kv-head) pairs; the cluster path is
    taken when the workload carries clusters (``w.csize`` is not None); ``bits`` is the code width
    of the estimator's key copy; ``topk`` / ``headwise`` select the baselines; ``approx_unkept`` adds
    the unkept clusters' centroid contributions on the cluster path; ``band`` is passed to
    ``decode_unit``.  On the cluster path ``ranges`` may map (b, h) to given kept ranges (int
    [m][2] of (first token, length)): the token stage then runs on those instead of the oracle's own
    cluster selection (which is still computed and returned), so a second implementation's token
    stage can be checked on its own cluster choice.
    Returns ``{(b, h): decode_unit result}``.
    """
    p = w.p if p is None else p
    keep_frac = w.keep_frac if keep_frac is None else keep_frac
    sm = float(np.float32(1.0 / math.sqrt(128))) if sm is None else sm
    G = w.num_q_heads // w.num_kv_heads
    if units is None:
        units = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    res = {}
    logical_k = {}
    logical_v = {}
    for b, h in units:
        if b not in logical_k:
            logical_k[b] = w.logical("k", b)
            logical_v[b] = w.logical("v", b)
        q = w.q[b, h * G:(h + 1) * G]
        kseq, vseq = logical_k[b][:, h, :], logical_v[b][:, h, :]
        if getattr(w, "csize", None) is not None:
            cs = doublep.select_clusters(q, w.centroids[b, h], w.csize[b, h], w.p1, sm)
            own = doublep.ranges_of(cs["kept"], w.coff[b, h])
            rg = own if ranges is None or (b, h) not in ranges else np.asarray(ranges[(b, h)], np.int64)
            r = decode_unit(q, kseq, vseq, p=p, keep_frac=1.0, sm=sm, ranges=rg, bits=bits, band=band)
            r["clusters"] = cs
            r["ranges"] = rg
            r["own_ranges"] = own
            if approx_unkept:
                # the clusters the token stage ran on (the given ranges, when there are any)
                first = {int(w.coff[b, h][c]): c for c in range(len(w.csize[b, h])) if w.csize[b, h][c] > 0}
                kept = np.array(sorted(first[int(x)] for x in rg[:, 0]), np.int64) if len(rg) else np.zeros(0, np.int64)
                vm = doublep.value_means(vseq, w.csize[b, h], w.coff[b, h])
                for j in range(G):
                    lam = cs["per_head"][j]["lam"]
                    r["out"][j], r["lse"][j] = doublep.approx_unkept(r["out"][j], r["lse"][j], lam, w.csize[b, h],
                                                                     kept, vm)
        else:
            r = decode_unit(q, kseq, vseq, p=p, keep_frac=keep_frac, sm=sm, bits=bits, topk=topk,
                            headwise=headwise, band=band)
        res[(b, h)] = r
    return res
