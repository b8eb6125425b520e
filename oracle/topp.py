"""O7 minimal top-p token set (sort-based), its ambiguity sets, and a model of the bisection search.

Definition (Paper-Notes "关键设计 / Oracle Top-p"; paperlayer §3.2): given weights W and a threshold
p, choose the smallest index set I with sum_{i in I} W_i >= p.  Taking the candidates in decreasing
weight (ties by increasing index) and stopping at the first prefix whose mass reaches p gives a set of
minimal size, and among minimal sets the one of largest mass.  p >= 1 selects every candidate.

Several sets can be correct (any minimal set that reaches p; and equal weights at the cut), and a
float32 implementation can move the cut by one rank when a prefix mass lies within rounding of p.
The comparison therefore names the tokens whose membership is not decided to that precision:

* clause (i):  |W_i - w*| <= TAU_W * w*   (w* = weight of the last token of the canonical set;
  ties included), TAU_W = 1e-6;
* clause (ii): the token at sorted rank r when |S_{r-1} - p| <= TAU_P (S = prefix masses),
  TAU_P = 1e-5.

``topp_bisect`` models the search the pages use instead of a sort (Paper-Notes "关键设计 / 高效Top-p":
binary search for the threshold m with sum_{W_i >= m} W_i >= p, O(log(max W / eps)) rounds): midpoints
are taken on the order-preserving uint32 image of the non-negative float32 weights, keeping the
invariant f(lo) >= p > f(hi) and returning lo, so the returned set always reaches p and, once the
search has converged (at most 31 steps), equals the sort-based set up to ties.
"""

from __future__ import annotations

import math

import numpy as np

from .numerics import f32_from_key, f32_key

TAU_W = 1e-6
TAU_P = 1e-5


def _prefix_sums(ws: np.ndarray) -> np.ndarray:
    if ws.size <= 256:
        return np.array([math.fsum(ws[:r + 1]) for r in range(ws.size)], dtype=np.float64)
    return np.cumsum(ws, dtype=np.float64)


def topp_sort(W: np.ndarray, p: float) -> dict:
    """Canonical minimal top-p set of ``W`` (float64 weights summing to ~1).

    Returns a dict with ``sel`` (sorted indices), ``k`` (its size), ``w_star`` (weight of its last
    token in decreasing order), ``mass`` (its prefix mass), and the ambiguity index arrays
    ``amb_i`` and ``amb_ii``.
    """
    W = np.asarray(W, dtype=np.float64)
    N = W.size
    if N == 0:
        e = np.zeros(0, np.int64)
        return {"sel": e, "k": 0, "w_star": math.nan, "mass": 0.0, "amb_i": e, "amb_ii": e,
                "order": e, "S": np.zeros(0)}
    order = np.lexsort((np.arange(N), -W))
    ws = W[order]
    S = _prefix_sums(ws)
    if p >= 1.0:
        k = N
    else:
        k = int(np.searchsorted(S, p, side="left")) + 1
        k = min(k, N)
    sel = np.sort(order[:k])
    w_star = float(ws[k - 1])
    amb_i = np.nonzero(np.abs(W - w_star) <= TAU_W * w_star)[0]
    s_prev = np.concatenate([[0.0], S[:-1]])
    amb_ii = np.sort(order[np.abs(s_prev - p) <= TAU_P]) if p < 1.0 else np.zeros(0, np.int64)
    return {"sel": sel, "k": k, "w_star": w_star, "mass": float(S[k - 1]), "amb_i": amb_i,
            "amb_ii": amb_ii, "order": order, "S": S}


def set_matches(gpu_sel: np.ndarray, res: dict, W: np.ndarray, p: float) -> tuple[bool, str]:
    """Parity rule: the symmetric difference lies inside the ambiguity sets and the GPU set's mass
    (under ``W``) reaches p - TAU_P."""
    g = np.unique(np.asarray(gpu_sel, np.int64))
    if np.asarray(W).size == 0:  # no candidates: the empty set is the only subset
        return (g.size == 0), "empty candidate list"
    o = res["sel"]
    diff = np.setxor1d(g, o)
    allowed = np.union1d(res["amb_i"], res["amb_ii"])
    bad = np.setdiff1d(diff, allowed)
    mass = math.fsum(np.asarray(W, np.float64)[g]) if g.size else 0.0
    if bad.size:
        return False, f"{bad.size} unambiguous tokens differ (e.g. {bad[:8].tolist()})"
    if p < 1.0 and mass < p - TAU_P:
        return False, f"selected mass {mass:.8f} < p - tau ({p - TAU_P:.8f})"
    if p >= 1.0 and g.size != W.size:
        return False, "p = 1 must select every candidate"
    return True, f"ok (|diff|={diff.size}, amb_i={res['amb_i'].size}, amb_ii={res['amb_ii'].size})"


FLOOR = 2.0**-40  # weights below this fraction of the largest carry no mass in the search


def topk_sort(W: np.ndarray, k: int) -> dict:
    """Top-k baseline at a fixed budget (the comparison the pages draw against top-p: paperlayer §3,
    Fig. 2-3, and Paper-Notes "研究背景"): the k largest weights, every weight tied with the k-th kept.

    Reading for the tail: weights below FLOOR times the largest count as one tie at zero, so a budget
    that reaches them keeps every candidate (the search in the kernels resolves keys from that floor
    up).  Returns ``sel`` (sorted indices), ``w_star`` (the k-th largest weight, 0 when all are kept)
    and ``amb_i`` (indices within TAU_W relative of w_star: their membership is decided by rounding).
    """
    W = np.asarray(W, dtype=np.float64)
    N = W.size
    e = np.zeros(0, np.int64)
    if N == 0 or k <= 0:
        return {"sel": e, "w_star": math.nan, "amb_i": e, "amb_ii": e}
    above = int(np.count_nonzero(W >= FLOOR * W.max()))
    if k > above:
        return {"sel": np.arange(N), "w_star": 0.0, "amb_i": e, "amb_ii": e}
    ws = np.sort(W)[::-1]
    w_star = float(ws[k - 1])
    sel = np.nonzero(W >= w_star)[0]
    amb_i = np.nonzero(np.abs(W - w_star) <= TAU_W * w_star)[0]
    return {"sel": sel, "w_star": w_star, "amb_i": amb_i, "amb_ii": e}  # (no prefix-mass clause)


def topk_matches(gpu_sel: np.ndarray, res: dict) -> tuple[bool, str]:
    """Parity rule for top-k: the symmetric difference lies inside the near-ties of the k-th weight."""
    g = np.unique(np.asarray(gpu_sel, np.int64))
    diff = np.setxor1d(g, res["sel"])
    bad = np.setdiff1d(diff, res["amb_i"])
    if bad.size:
        return False, f"{bad.size} unambiguous tokens differ (e.g. {bad[:8].tolist()})"
    return True, f"ok (|diff|={diff.size})"


def topp_bisect(w: np.ndarray, p: float, iters: int = 32) -> dict:
    """Bisection on the uint32 image of float32 weights ``w`` (not necessarily normalised).

    Mass sums are exact-ish float64 sums of the float32 weights, so this models the search logic,
    not a particular rounding order.  Returns ``threshold`` (float32), ``sel`` (indices with
    w >= threshold), ``steps`` and whether the bracket ``converged``.
    """
    w = np.asarray(w, dtype=np.float32)
    N = w.size
    if N == 0:
        return {"threshold": np.float32(0), "sel": np.zeros(0, np.int64), "steps": 0, "converged": True}
    if p >= 1.0:
        return {"threshold": np.float32(0), "sel": np.arange(N), "steps": 0, "converged": True}
    keys = f32_key(w).astype(np.int64)
    Z = math.fsum(w.astype(np.float64))
    target = p * Z
    lo, hi = 0, int(keys.max()) + 1
    steps = 0
    while steps < iters and hi - lo > 1:
        mid = (lo + hi) // 2
        f = math.fsum(w[keys >= mid].astype(np.float64))
        if f >= target:
            lo = mid
        else:
            hi = mid
        steps += 1
    thr = f32_from_key(lo)
    return {"threshold": thr, "sel": np.nonzero(keys >= lo)[0], "steps": steps,
            "converged": hi - lo <= 1}
