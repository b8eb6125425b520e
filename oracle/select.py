"""O3 Quest-style page scores and top-K page selection; O4 candidate token lists.

The Twilight pages take an existing token selector unchanged and give it a generous budget
(Paper-Notes "整体框架": e.g. 1/4 of the tokens; paperlayer §4.1, Fig. 5); they name Quest among the
selectors but do not define Quest's score.  Readings taken here:

* page score of query head h:  sigma_h(page) = sum_c max(q_c * kmin_c, q_c * kmax_c), the tightest
  per-channel upper bound of q.k over keys inside the page's min/max box;
* it is evaluated as a float32 left-to-right fold over c = 0..127 starting from +0 (the products of
  two bf16 values are exact in float32, so only the additions round);
* a GQA group shares one candidate set per (sequence, kv-head), ranked by the group score, the sum
  over the group's query heads of sigma_h.  Since kmin_c <= kmax_c, max(q_c kmin_c, q_c kmax_c) =
  q+_c kmax_c + q-_c kmin_c (q+ = max(q, 0), q- = min(q, 0)), so the group score is
  sum_c (P_c kmax_c + N_c kmin_c) with P_c, N_c the sums of the group's q+_c and q-_c: it is evaluated
  that way, P_c and N_c as float32 sums over the heads in order from +0, then one float32 fold over
  c = 0..127 from +0 that adds P_c kmax_c and then N_c kmin_c, each with one rounding (a fused
  multiply-add: P_c kmax_c need not be exact in float32 once several heads are summed);
* the kept count is K = ceil(fp32(keep_frac) * fp32(P)) clamped to [1, P] (0 for an empty sequence);
  ties in score go to the lower page id; the kept pages are listed in ascending order.

The float32 fold order is the specification (a set of integers is decided from it), so it is written
as one IEEE float32 operation at a time.
"""

from __future__ import annotations

import numpy as np

from .numerics import F32, bf16_to_f32, f32_fma

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


def group_query_parts(qbits_group: np.ndarray):
    """P_c and N_c: float32 sums over the group's heads, in order from +0, of q+_c and q-_c."""
    q = bf16_to_f32(qbits_group)
    P = np.zeros(q.shape[1], F32)
    N = np.zeros(q.shape[1], F32)
    for h in range(q.shape[0]):
        P = (P + np.where(q[h] > 0, q[h], F32(0.0))).astype(F32)
        N = (N + np.where(q[h] < 0, q[h], F32(0.0))).astype(F32)
    return P, N


def group_scores(qbits_group: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """Group score of every page (``qbits_group`` uint16 [G][128]; ``kmin``/``kmax`` float32 [P][128]):
    the fold over channels of P_c kmax_c then N_c kmin_c, each added with one float32 rounding."""
    P, N = group_query_parts(qbits_group)
    acc = np.zeros(kmin.shape[0], F32)
    for c in range(128):
        acc = f32_fma(P[c], kmax[:, c], acc)
        acc = f32_fma(N[c], kmin[:, c], acc)
    return acc


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
