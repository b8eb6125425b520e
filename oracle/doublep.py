"""O11 Double-P: cluster-level top-p on size-weighted centroids, then token-level top-p.

Source: "Double-P: Hierarchical Top-P Sparse Attention for Long-Context LLMs", sections "方法详解"
and "关键设计": a coarse top-p at cluster level scores each cluster by its size-weighted centroid;
a second, token-level top-p runs inside the kept clusters; only the surviving tokens enter the
attention.  The page gives no formulas; readings taken:

* clusters are contiguous token ranges of one (sequence, kv-head) (keys stored sorted by cluster);
  centroid mu_c and size n_c are inputs;
* cluster logit  lambda_c = fl(sm * fold_{c'=0..127}(acc + q_c' * mu_c,c'))  -- a float32 fold from +0
  (bf16 x bf16 products are exact), the float32 order being the specification because a set is
  decided from it;
* cluster weight u_c = n_c exp(lambda_c - M) / sum_c' n_c' exp(lambda_c' - M), M the largest
  logit of a non-empty cluster, in float64 -- the softmax mass the cluster would carry if all its
  keys sat at the centroid;
* top-p (p1) per query head over the clusters (O7), union over the GQA group, kept clusters listed
  in ascending order as (begin, length) ranges (empty clusters never listed);
* token level: the INT4 estimate, one softmax and one top-p (p2) per query head over all tokens of
  the kept ranges (O5-O7), the group union (O8) and sparse attention (O9).  Unkept clusters are
  dropped.
"""

from __future__ import annotations

import numpy as np

from .numerics import F32, bf16_to_f32
from .topp import topp_sort


def cluster_logits_spec(qbits_h: np.ndarray, centroid_bits: np.ndarray, sm: float) -> np.ndarray:
    q = bf16_to_f32(qbits_h)
    mu = bf16_to_f32(centroid_bits)
    acc = np.zeros(mu.shape[0], F32)
    for c in range(128):
        acc = (acc + (q[c] * mu[:, c]).astype(F32)).astype(F32)
    return (F32(sm) * acc).astype(F32)


def cluster_weights(lam: np.ndarray, csize: np.ndarray) -> np.ndarray:
    lam = np.asarray(lam, np.float64)
    n = np.asarray(csize, np.float64)
    live = n > 0
    w = np.zeros_like(lam)
    if not np.any(live):
        return w
    M = lam[live].max()
    w[live] = n[live] * np.exp(lam[live] - M)
    return w / w.sum()


def select_clusters(qbits_group: np.ndarray, centroid_bits: np.ndarray, csize: np.ndarray,
                    p1: float, sm: float) -> dict:
    """Per (sequence, kv-head): per-head cluster top-p, union, and the kept ranges."""
    per_head = []
    for h in range(qbits_group.shape[0]):
        lam = cluster_logits_spec(qbits_group[h], centroid_bits, sm)
        W = cluster_weights(lam, csize)
        live = np.nonzero(np.asarray(csize) > 0)[0]
        res = topp_sort(W[live], p1)
        per_head.append({"lam": lam, "W": W, "live": live, "res": res, "kept": live[res["sel"]]})
    kept = np.unique(np.concatenate([ph["kept"] for ph in per_head])) if per_head else np.zeros(0, np.int64)
    return {"per_head": per_head, "kept": kept}


def ranges_of(kept: np.ndarray, coff: np.ndarray) -> np.ndarray:
    kept = np.asarray(kept, np.int64)
    return np.stack([coff[kept], coff[kept + 1] - coff[kept]], axis=1).astype(np.int64) \
        if kept.size else np.zeros((0, 2), np.int64)
