"""O7 minimal top-p token set (sort-based), its ambiguity sets, the top-k baseline, and a model of the
bisection search.

Definition (Paper-Notes "关键设计 / Oracle Top-p"; paperlayer §3.2): given weights W and a threshold
p, choose the smallest index set I with sum_{i in I} W_i >= p.  Taking the candidates in decreasing
weight (ties by increasing index) and stopping at the first prefix whose mass reaches p gives a set of
minimal size, and among minimal sets the one of largest mass.  p >= 1 selects every candidate.

Several sets can be correct (any minimal set that reaches p; equal weights at the cut), and an
implementation that holds the weights to finite precision can move the cut when a token's weight or
a prefix mass lies within that precision of the decision.  The comparison therefore names the tokens
whose membership the stated precision does not decide:

* clause (i):  |W_i - w*| <= (TAU_W + e_i + e_*) w*   (w* = weight of the last token of the canonical
  set, e_* its error; ties included).  TAU_W = 1e-6 is the parity band of the method's statement; e is
  an optional per-token bound on the implementation's relative weight error beyond it (the error of
  its logits: a logit off by d moves the weight ratio of two tokens by at most d_i + d_*);
* clause (ii): the token at sorted rank r when |S_{r-1} - p| <= tau_p (S = prefix masses), with
  tau_p = TAU_P + 2 sum_j W_j e_j + tau_p_extra: relative weight errors e_j move a prefix mass by at
  most twice their W-weighted mean (the normaliser moves with them); tau_p_extra covers a stated
  resolution of the implementation's mass sums.  TAU_P = 1e-6.

``topk_sort`` is the fixed-budget baseline the pages contrast with top-p (paperlayer §3.1): the k
largest weights, every weight tied with the k-th kept.

``topp_bisect`` models the search the pages use instead of a sort (Paper-Notes "关键设计 / 高效Top-p":
binary search for the threshold m with sum_{W_i >= m} W_i >= p, O(log(max W / eps)) rounds).  Reading
of "32 iterations in fp32": the threshold is a float32 value and each step halves an interval of its
uint32 bit pattern (order-preserving for non-negative floats), from [0, 2^31) -- so step s decides bit
30 - s of the threshold's pattern, top bit first, and 31 steps resolve it exactly.  The weights are
searched on the scale where the largest is 1 (the max-subtracted exponentials of the softmax, before
division by their sum Z), against the target p * Z; converged, this keeps the same set as comparing
W_i with p, and a shorter search stops at a superset that still reaches p.
"""

from __future__ import annotations

import math

import numpy as np

from .numerics import f32_from_key

TAU_W = 1e-6
TAU_P = 1e-6


def _prefix_sums(ws: np.ndarray) -> np.ndarray:
    if ws.size <= 256:
        return np.array([math.fsum(ws[:r + 1]) for r in range(ws.size)], dtype=np.float64)
    return np.cumsum(ws, dtype=np.float64)


def _errs(err, N: int) -> np.ndarray:
    if err is None:
        return np.zeros(N)
    e = np.asarray(err, np.float64)
    return np.broadcast_to(e, (N,)).astype(np.float64)


def topp_sort(W: np.ndarray, p: float, err=None, tau_p_extra: float = 0.0) -> dict:
    """Canonical minimal top-p set of ``W`` (float64 weights summing to ~1).

    ``err`` (optional, scalar or per token): bound on the relative weight error of the implementation
    under comparison, beyond TAU_W; ``tau_p_extra``: its mass-sum resolution (see module docstring).
    Returns ``sel`` (sorted indices), ``k`` (its size), ``w_star`` (weight of its last token in
    decreasing order), ``mass`` (its prefix mass), the ambiguity index arrays ``amb_i`` and ``amb_ii``,
    ``amb_i_base`` (clause (i) at TAU_W alone) and ``tau_p``.
    """
    W = np.asarray(W, dtype=np.float64)
    N = W.size
    if N == 0:
        e = np.zeros(0, np.int64)
        return {"sel": e, "k": 0, "w_star": math.nan, "mass": 0.0, "amb_i": e, "amb_ii": e, "amb_i_base": e,
                "order": e, "S": np.zeros(0), "tau_p": TAU_P}
    er = _errs(err, N)
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
    e_star = float(er[order[k - 1]])
    dist = np.abs(W - w_star)
    amb_i = np.nonzero(dist <= (TAU_W + er + e_star) * w_star)[0]
    amb_i_base = np.nonzero(dist <= TAU_W * w_star)[0]
    tau_p = TAU_P + 2.0 * float(np.dot(W, er)) + float(tau_p_extra)
    s_prev = np.concatenate([[0.0], S[:-1]])
    amb_ii = np.sort(order[np.abs(s_prev - p) <= tau_p]) if p < 1.0 else np.zeros(0, np.int64)
    return {"sel": sel, "k": k, "w_star": w_star, "mass": float(S[k - 1]), "amb_i": amb_i,
            "amb_ii": amb_ii, "amb_i_base": amb_i_base, "order": order, "S": S, "tau_p": tau_p}


def diff_counts(gpu_sel: np.ndarray, res: dict) -> dict:
    """How many tokens the two sets differ in, and which clause excuses them: ``base`` (clause (i) at
    TAU_W alone), ``band`` (clause (i) only through the implementation's stated error), ``cut``
    (clause (ii) only), ``bad`` (none)."""
    g = np.unique(np.asarray(gpu_sel, np.int64))
    diff = np.setxor1d(g, res["sel"])
    base = np.intersect1d(diff, res["amb_i_base"])
    rest = np.setdiff1d(diff, base)
    band = np.intersect1d(rest, res["amb_i"])
    rest = np.setdiff1d(rest, band)
    cut = np.intersect1d(rest, res["amb_ii"])
    bad = np.setdiff1d(rest, cut)
    return {"diff": int(diff.size), "base": int(base.size), "band": int(band.size), "cut": int(cut.size),
            "bad": int(bad.size), "bad_idx": bad}


def set_matches(gpu_sel: np.ndarray, res: dict, W: np.ndarray, p: float) -> tuple[bool, str]:
    """Parity rule: the symmetric difference lies inside the ambiguity sets and the GPU set's mass
    (under ``W``) reaches p - tau_p."""
    g = np.unique(np.asarray(gpu_sel, np.int64))
    if np.asarray(W).size == 0:  # no candidates: the empty set is the only subset
        return (g.size == 0), "empty candidate list"
    c = diff_counts(g, res)
    mass = math.fsum(np.asarray(W, np.float64)[g]) if g.size else 0.0
    if c["bad"]:
        return False, f"{c['bad']} unambiguous tokens differ (e.g. {c['bad_idx'][:8].tolist()})"
    if p < 1.0 and mass < p - res["tau_p"]:
        return False, f"selected mass {mass:.9f} < p - tau_p ({p - res['tau_p']:.9f})"
    if p >= 1.0 and g.size != np.asarray(W).size:
        return False, "p = 1 must select every candidate"
    return True, f"ok (|diff|={c['diff']}: base {c['base']}, band {c['band']}, cut {c['cut']})"


def topk_sort(W: np.ndarray, k: int, err=None) -> dict:
    """Top-k baseline at a fixed budget (the comparison the pages draw against top-p: paperlayer §3.1,
    Fig. 2-3, and Paper-Notes "研究背景"): the k largest weights, every weight tied with the k-th kept;
    k >= the candidate count keeps all.  Returns ``sel`` (sorted indices), ``w_star`` (the k-th
    largest weight), ``amb_i`` (indices whose weight lies within TAU_W + e_i + e_* relative of w_star:
    their membership is decided by rounding) and ``amb_i_base`` (the same at TAU_W alone)."""
    W = np.asarray(W, dtype=np.float64)
    N = W.size
    e = np.zeros(0, np.int64)
    if N == 0 or k <= 0:
        return {"sel": e, "w_star": math.nan, "amb_i": e, "amb_ii": e, "amb_i_base": e}
    if k >= N:
        return {"sel": np.arange(N), "w_star": float(W.min()), "amb_i": e, "amb_ii": e, "amb_i_base": e}
    er = _errs(err, N)
    order = np.lexsort((np.arange(N), -W))
    kth = order[k - 1]
    w_star = float(W[kth])
    sel = np.nonzero(W >= w_star)[0]
    dist = np.abs(W - w_star)
    amb_i = np.nonzero(dist <= (TAU_W + er + er[kth]) * w_star)[0]
    amb_i_base = np.nonzero(dist <= TAU_W * w_star)[0]
    return {"sel": sel, "w_star": w_star, "amb_i": amb_i, "amb_ii": e, "amb_i_base": amb_i_base}


def topk_matches(gpu_sel: np.ndarray, res: dict, extra_amb=None) -> tuple[bool, str]:
    """Parity rule for top-k: the symmetric difference lies inside the near-ties of the k-th weight
    (and inside ``extra_amb``, indices a caller declares undecided)."""
    g = np.unique(np.asarray(gpu_sel, np.int64))
    diff = np.setxor1d(g, res["sel"])
    allowed = res["amb_i"] if extra_amb is None else np.union1d(res["amb_i"], np.asarray(extra_amb, np.int64))
    bad = np.setdiff1d(diff, allowed)
    if bad.size:
        return False, f"{bad.size} unambiguous tokens differ (e.g. {bad[:8].tolist()})"
    return True, f"ok (|diff|={diff.size})"


def topp_bisect(W: np.ndarray, p: float, iters: int = 32, tau: float = 0.0, err=None,
                max_branches: int = 16) -> dict:
    """Bisection of the threshold's float32 bit pattern over [0, 2^31), ``iters`` steps (see the module
    docstring).  ``W`` are non-negative weights of any scale (searched as e = W / max W); masses are
    float64 sums.

    For comparison with an implementation of stated precision: ``err`` (scalar or per token) bounds
    its relative weight error beyond TAU_W, so its test e_i >= v may go either way when
    |e_i / v - 1| <= band_i = TAU_W + err_i + err_max (err_max: the largest weight's error, which sets
    the scale); ``tau`` bounds its relative mass error.  A step whose decision those bounds leave open
    is followed both ways.

    Returns ``threshold`` (the float32 threshold on the max-1 scale), ``key`` (its bit pattern),
    ``sel`` (indices with e >= threshold), ``steps``, ``converged``, ``band`` (per token, zero without
    ``err``) and ``keys``: the bit patterns reachable when open steps may go either way (the exactly
    decided one first; at most ``max_branches``).
    """
    W = np.asarray(W, dtype=np.float64)
    N = W.size
    if N == 0 or p >= 1.0 or W.max() <= 0:
        sel = np.zeros(0, np.int64) if N == 0 else np.arange(N)
        return {"threshold": np.float32(0), "key": 0, "sel": sel, "steps": 0, "converged": True, "keys": [0],
                "band": np.zeros(N)}
    e = W / W.max()
    if err is None:
        band = np.zeros(N)
    else:
        er = _errs(err, N)
        band = TAU_W + er + er[int(np.argmax(W))]
    Z = math.fsum(e)
    target = p * Z

    def masses(key: int) -> tuple[float, float, float]:
        v = float(f32_from_key(key))
        exact = e[e >= v].sum()
        sure = e[e >= v * (1 + band)].sum() - tau * Z
        maybe = e[e >= v * (1 - band)].sum() + tau * Z
        return exact, sure, maybe

    states = [(0, 1 << 31)]  # (lo, hi); the first is the exactly decided path
    steps = 0
    while steps < iters and states[0][1] - states[0][0] > 1:
        nxt = []
        for lo, hi in states:
            if hi - lo <= 1:
                nxt.append((lo, hi))
                continue
            mid = (lo + hi) // 2
            f, f_sure, f_maybe = masses(mid)
            take = (mid, hi) if f >= target else (lo, mid)
            nxt.append(take)
            if f_sure < target <= f_maybe and len(states) + len(nxt) < max_branches:
                nxt.append((lo, mid) if f >= target else (mid, hi))
        states = nxt
        steps += 1
    key = states[0][0]
    thr = f32_from_key(key)
    keys = [key] + sorted({s[0] for s in states} - {key})
    return {"threshold": thr, "key": key, "sel": np.nonzero(e >= float(thr))[0], "steps": steps,
            "converged": states[0][1] - states[0][0] <= 1, "keys": keys, "band": band}


def bisect_matches(gpu_sel: np.ndarray, b: dict, W: np.ndarray) -> tuple[bool, str]:
    """An implementation's stopped-early set against ``topp_bisect``'s result ``b``: equal, for one of
    the reachable threshold patterns, to {e >= threshold} up to tokens within their band of it."""
    g = np.unique(np.asarray(gpu_sel, np.int64))
    W = np.asarray(W, np.float64)
    if W.size == 0:
        return g.size == 0, "empty candidate list"
    e = W / W.max()
    for key in b["keys"]:
        v = float(f32_from_key(key))
        want = np.nonzero(e >= v)[0]
        diff = np.setxor1d(g, want)
        if v > 0 and diff.size:
            near = np.abs(e[diff] / v - 1.0) <= b["band"][diff]
        else:
            near = np.ones(diff.size, bool) if diff.size == 0 else np.zeros(diff.size, bool)
        if np.all(near):
            return True, f"ok (threshold pattern {key:#x}, |diff|={diff.size}, {len(b['keys'])} reachable)"
    return False, f"no reachable threshold pattern matches ({len(b['keys'])} tried)"
