"""O8 GQA union, O9 sparse attention over a token set, O10 dense attention and the top-p error bound.

* O8 -- for GQA the query heads of a group attend over the union of the tokens that each head's
  top-p pruning keeps, so the group's tokens are read once (paperlayer §B.2, Fig. 13: group-wise
  variable-length attention over a flattened paged cache).  For MHA the union is the head's own set.
* O9 -- softmax attention of one query head over an index set, in float64 from bf16 K and V:
  o = sum_i softmax_i(sm q.k_i) v_i and lse = ln sum_i exp(sm q.k_i) (natural log).  An empty set
  gives o = 0 and lse = -inf.
* O10 -- dense attention over every token, the exact top-p set of the true weights, and the bound of
  Paper-Notes "关键设计" (output error at most (1-p)*||V||_F, independent of the token count), checked
  in three forms:
    (a) masked, not renormalised:  || o - W_I^T V ||          <= (1 - s) ||V||_F
    (b) renormalised top-p output: || o - o_I ||              <= sqrt(2) (1 - s) ||V||_2
    (c) renormalised, as printed:  || o - o_I ||              <= (1 - p) ||V||_F   (when V has stable
        rank >= 2, which (b) then implies)
  with s = W(I) >= p the mass of the exact top-p set I.
"""

from __future__ import annotations

import math

import numpy as np

from .numerics import bf16_to_f32
from .topp import topp_sort


def union(sets) -> np.ndarray:
    sets = [np.asarray(s, np.int64) for s in sets]
    if not sets:
        return np.zeros(0, np.int64)
    return np.unique(np.concatenate(sets))


def sparse_attention(qbits_h: np.ndarray, kbits: np.ndarray, vbits: np.ndarray, idx: np.ndarray,
                     sm: float) -> tuple[np.ndarray, float]:
    """``kbits``/``vbits`` uint16 [n][128] (one kv-head, logical order); ``idx`` token ids."""
    idx = np.asarray(idx, np.int64)
    if idx.size == 0:
        return np.zeros(128), -math.inf
    q = bf16_to_f32(qbits_h).astype(np.float64)
    K = bf16_to_f32(kbits[idx]).astype(np.float64)
    V = bf16_to_f32(vbits[idx]).astype(np.float64)
    s = float(np.float32(sm)) * (K @ q)
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    return (e @ V) / z, float(m + math.log(z))


def dense_weights(qbits_h: np.ndarray, kbits: np.ndarray, sm: float) -> np.ndarray:
    q = bf16_to_f32(qbits_h).astype(np.float64)
    K = bf16_to_f32(kbits).astype(np.float64)
    s = float(np.float32(sm)) * (K @ q)
    e = np.exp(s - s.max())
    return e / e.sum()


def topp_bound_check(qbits_h: np.ndarray, kbits: np.ndarray, vbits: np.ndarray, p: float,
                     sm: float) -> dict:
    """O10 for one head: exact top-p of the true weights and the three bound forms."""
    W = dense_weights(qbits_h, kbits, sm)
    V = bf16_to_f32(vbits).astype(np.float64)
    o = W @ V
    res = topp_sort(W, p)
    I = res["sel"]
    s = math.fsum(W[I])
    masked = W[I] @ V[I]
    renorm = masked / s
    fro = float(np.linalg.norm(V))
    spec = float(np.linalg.norm(V, 2))
    err_masked = float(np.linalg.norm(o - masked))
    err_renorm = float(np.linalg.norm(o - renorm))
    return {
        "k": res["k"], "s": s, "fro": fro, "spec": spec, "stable_rank": (fro / spec) ** 2,
        "err_masked": err_masked, "err_renorm": err_renorm,
        "bound_a": (1 - s) * fro, "bound_b": math.sqrt(2) * (1 - s) * spec, "bound_c": (1 - p) * fro,
    }
