"""O3 Quest-style page scores and top-K page selection; O4 candidate token lists.

The Twilight pages take an existing token selector unchanged and give it a generous budget
(Paper-Notes "整体框架": e.g. 1/4 of the tokens; paperlayer §4.1, Fig. 5); they name Quest among the
selectors but do not define Quest's score.  Readings taken here:

* page score of query head h:  sigma_h(page) = sum_c max(q_c * kmin_c, q_c * kmax_c), the tightest
  per-channel upper bound of q.k over keys inside the page's min/max box;
* it is evaluated as a float32 left-to-right fold over c = 0..127 starting from +0 (the products of
  two bf16 values are exact in float32, so only the additions round);
* a GQA group shares one candidate set per (sequence, kv-head), ranked by the group score, the
  float32 fold over the group's query heads in order starting from +0;
* the kept count is K = ceil(fp32(keep_frac) * fp32(P)) clamped to [1, P] (0 for an empty sequence);
  ties in score go to the lower page id; the kept pages are listed in ascending order.

The float32 fold order is the specification (a set of integers is decided from it), so it is written
as one IEEE float32 operation at a time.
"""

from __future__ import annotations

import numpy as np

from .numerics import F32, bf16_to_f32

PAGE = 16


def page_scores_head(qbits: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """sigma_h for every page: ``qbits`` uint16 [128]; ``kmin``/``kmax`` float32 [P][128]."""
    q = bf16_to_f32(qbits)
    P = kmin.shape[0]
    acc = np.zeros(P, F32)
    for c in range(128):
        qc = q[c]
        term = np.maximum((qc * kmin[:, c]).astype(F32), (qc * kmax[:, c]).astype(F32))
        acc = (acc + term).astype(F32)
    return acc


def group_scores(qbits_group: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """Group score: float32 fold over the group's query heads (``qbits_group`` uint16 [G][128])."""
    gs = np.zeros(kmin.shape[0], F32)
    for h in range(qbits_group.shape[0]):
        gs = (gs + page_scores_head(qbits_group[h], kmin, kmax)).astype(F32)
    return gs


def keep_count(num_pages: int, keep_frac: float) -> int:
    if num_pages <= 0:
        return 0
    k = int(np.ceil(F32(keep_frac) * F32(num_pages)))
    return max(1, min(num_pages, k))


def top_pages(scores: np.ndarray, k: int) -> np.ndarray:
    """The k pages with the largest score (ties to the lower id), returned in ascending order."""
    ids = np.arange(scores.shape[0])
    order = np.lexsort((ids, -scores.astype(np.float64)))
    return np.sort(order[:k]).astype(np.int32)


def candidates_from_pages(pages: np.ndarray, seq_len: int) -> np.ndarray:
    """O4: valid token ids of the listed pages, ascending (pages ascending)."""
    if len(pages) == 0:
        return np.zeros(0, np.int64)
    t = (np.asarray(pages, np.int64)[:, None] * PAGE + np.arange(PAGE)[None, :]).reshape(-1)
    return t[t < seq_len]


def candidates_from_ranges(ranges: np.ndarray) -> np.ndarray:
    """Concatenation of (begin, length) token ranges in list order."""
    parts = [np.arange(int(b), int(b) + int(n), dtype=np.int64) for b, n in ranges if n > 0]
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)
