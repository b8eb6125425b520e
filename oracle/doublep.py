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
* optional cluster-level approximation of the unkept clusters (the abstract's refinement to token
  level only where needed; the method summary has only selected tokens in the attention, so this is
  an option, off by default): a cluster that no head of the group keeps enters the softmax as its
  n_c members collapsed onto (mu_c, vbar_c), vbar_c the mean of its value rows -- n_c exp(lambda_c)
  joins the normaliser and n_c exp(lambda_c) vbar_c the numerator, combined with the attention's
  (out, lse) in log-sum-exp form.  Exact when every member's key is mu_c and value is vbar_c.
"""

from __future__ import annotations

import math

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


def value_means(vbits_seq: np.ndarray, csize: np.ndarray, coff: np.ndarray) -> np.ndarray:
    """Mean value row of each cluster (float64 [C][128]; zeros for an empty cluster).  ``vbits_seq``
    uint16 [n][128] of one (sequence, kv-head) in token order."""
    v = bf16_to_f32(vbits_seq).astype(np.float64)
    C = len(csize)
    out = np.zeros((C, 128))
    for c in range(C):
        n = int(csize[c])
        if n > 0:
            out[c] = v[int(coff[c]):int(coff[c]) + n].mean(axis=0)
    return out


def approx_unkept(out_h: np.ndarray, lse_h: float, lam: np.ndarray, csize: np.ndarray, kept: np.ndarray,
                  vmean: np.ndarray) -> tuple[np.ndarray, float]:
    """Combine one head's attention output (``out_h``, natural-log ``lse_h``) with the clusters not in
    ``kept`` (the group's kept cluster ids): each non-empty one adds n_c exp(lambda_c) to the
    normaliser and n_c exp(lambda_c) vbar_c to the numerator."""
    C = len(csize)
    unk = np.setdiff1d(np.nonzero(np.asarray(csize) > 0)[0], np.asarray(kept, np.int64))
    if unk.size == 0:
        return np.asarray(out_h, np.float64), float(lse_h)
    s = np.asarray(lam, np.float64)[unk] + np.log(np.asarray(csize, np.float64)[unk])
    M = max(float(s.max()), float(lse_h))
    wa = math.exp(lse_h - M) if np.isfinite(lse_h) else 0.0
    wc = np.exp(s - M)
    den = wa + wc.sum()
    num = wa * np.asarray(out_h, np.float64) + wc @ vmean[unk]
    return num / den, M + math.log(den)
