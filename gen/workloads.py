"""Seeded synthetic decode workloads (inputs only; none of the method's arithmetic lives here).

Every array is drawn from numpy's PCG64 (``np.random.default_rng(seed)``) in float32 and rounded to
bfloat16 (round-to-nearest-even) before it is stored.  Draw order is fixed: K, then V, then q, then the
structure that the workload plants (outlier channels, temperatures, planted keys, clusters), then the
permutation of physical pages.  Changing this order changes every derived value, so it is part of the
recipe.

Layouts (all little-endian, bf16 stored as uint16 bit patterns):

* ``q``          uint16 [B][Hq][128]
* ``k_pages``    uint16 [num_phys_pages][Hkv][16][128]   paged K cache, 16 tokens per page
* ``v_pages``    uint16 [num_phys_pages][Hkv][16][128]   paged V cache
* ``page_table`` int32  [B][max_pages]                   logical page -> physical page (0 when unused)
* ``seq_lens``   int32  [B]

Token ``t`` of sequence ``b`` lives in physical page ``page_table[b][t // 16]``, slot ``t % 16``.
Slots past the end of a sequence hold the constant bf16 value 5.0, so a consumer that reads them by
mistake changes its result.

The hierarchical (cluster) workload additionally carries, per (b, kv-head), clusters that are contiguous
token ranges: ``csize`` int32 [B][Hkv][C], ``coff`` int32 [B][Hkv][C+1] and bf16 centroids
``centroids`` uint16 [B][Hkv][C][128] (the bf16 rounding of the fp32 mean of the member keys; a
cluster with no member has size 0 and a zero centroid).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

HEAD_DIM = 128
PAGE_SIZE = 16
FILL_VALUE = 5.0  # content of unused slots in a sequence's last page


# --------------------------------------------------------------------------------------------------
# bf16 bit helpers (input preparation only)
# --------------------------------------------------------------------------------------------------
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); return the uint16 bit patterns.
    (For a finite value the rounding increment never carries out of 32 bits.)"""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _round_bf16(x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bf16_bits_from_f32(x))


# --------------------------------------------------------------------------------------------------
# Workload container
# --------------------------------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    seq_lens: np.ndarray
    page_table: np.ndarray
    k_pages: np.ndarray
    v_pages: np.ndarray
    q: np.ndarray
    p: float
    keep_frac: float
    iters: int = 32
    centroids: Optional[np.ndarray] = None
    csize: Optional[np.ndarray] = None
    coff: Optional[np.ndarray] = None
    p1: Optional[float] = None
    meta: dict = field(default_factory=dict)

    head_dim: int = HEAD_DIM
    page_size: int = PAGE_SIZE

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def num_phys_pages(self) -> int:
        return int(self.k_pages.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    @property
    def num_clusters(self) -> int:
        return 0 if self.csize is None else int(self.csize.shape[2])

    def logical(self, which: str, b: int) -> np.ndarray:
        """Gather sequence ``b`` of K or V back into logical order: uint16 [n_b][Hkv][128]."""
        pages = self.k_pages if which == "k" else self.v_pages
        n = int(self.seq_lens[b])
        npg = -(-n // PAGE_SIZE)
        phys = self.page_table[b, :npg]
        x = pages[phys]  # [npg][Hkv][16][128]
        x = x.transpose(0, 2, 1, 3).reshape(npg * PAGE_SIZE, self.num_kv_heads, HEAD_DIM)
        return x[:n]

    def nbytes(self) -> int:
        return int(self.k_pages.nbytes + self.v_pages.nbytes)


# --------------------------------------------------------------------------------------------------
# Configurations (shapes and structure of the pages' decode workloads)
# --------------------------------------------------------------------------------------------------
CONFIGS = {
    # single MHA head, no base selector, peaked by 8 planted keys
    "C1": dict(batch=1, num_q_heads=1, num_kv_heads=1, seq_len=4096, kind="peaked",
               seed=0, p=0.9, keep_frac=1.0),
    # Llama-3-8B shaped decode layer, 4 K outlier channels
    "C2": dict(batch=1, num_q_heads=32, num_kv_heads=8, seq_len=32768, kind="outlier",
               seed=1, p=0.85, keep_frac=0.25),
    # head heterogeneity: per-head softmax temperature, log-uniform
    "C3": dict(batch=16, num_q_heads=32, num_kv_heads=8, seq_len=32768, kind="temperature",
               seed=2, p=0.85, keep_frac=0.25),
    # long context, 64 planted keys (cos 0.6) per query head
    "C4": dict(batch=4, num_q_heads=32, num_kv_heads=8, seq_len=131072, kind="planted",
               seed=3, p=0.9, keep_frac=0.25),
    # hierarchical: 4096-cluster Gaussian mixture, Zipf(1.1) sizes; cluster top-p 0.95, token 0.9
    "C5": dict(batch=1, num_q_heads=32, num_kv_heads=8, seq_len=262144, kind="cluster",
               seed=4, p=0.9, keep_frac=1.0, p1=0.95, num_clusters=4096),
}


def make_config(name: str, layer: int = 0, seq_len: Optional[int] = None,
                batch: Optional[int] = None) -> Workload:
    """Build a named configuration.  ``layer`` selects an independent draw of the same shape
    (seed + 1000*layer) so that timing can rotate over distinct caches.  ``seq_len``/``batch``
    override the size (used for reduced-size rehearsals; the named sizes are the defaults)."""
    c = dict(CONFIGS[name])
    n = int(seq_len if seq_len is not None else c.pop("seq_len"))
    c.pop("seq_len", None)
    B = int(batch if batch is not None else c.pop("batch"))
    c.pop("batch", None)
    seed = int(c.pop("seed")) + 1000 * int(layer)
    return make_custom(batch=B, seq_lens=[n] * B, seed=seed, name=f"{name}/L{layer}", **c)


def make_custom(*, batch: int, num_q_heads: int, num_kv_heads: int, seq_lens, kind: str = "normal",
                seed: int = 0, p: float = 0.85, keep_frac: float = 0.25, iters: int = 32,
                p1: Optional[float] = None, num_clusters: Optional[int] = None,
                planted_per_head: int = 64, n_peaks: int = 8, name: str = "custom") -> Workload:
    """Build a workload of any shape.

    kind:
      * ``normal``      K, V, q ~ N(0, 1)
      * ``outlier``     as normal, then 4 K channels (shared by all heads) scaled by 8
      * ``temperature`` as normal, then q of each (b, q-head) scaled by beta = exp(U[ln .05, ln 3.5])
      * ``planted``     as normal, then per (b, q-head) ``planted_per_head`` positions (distinct within
                        the GQA group) get k = sqrt(128) * (0.6 qhat + 0.8 u), u a unit vector orthogonal
                        to qhat, so cos(q, k) = 0.6 before rounding
      * ``peaked``      as normal, then ``n_peaks`` positions per (b, kv-head) get k = 3 qhat + N(0, 0.1^2)
                        (qhat of the group's first query head)
      * ``cluster``     keys from a ``num_clusters``-component Gaussian mixture per (b, kv-head):
                        means ~ N(0, 0.5 I), labels with P(c) ~ (c+1)^-1.1, k = mean + N(0, 0.5 I),
                        tokens stored sorted by cluster so clusters are contiguous ranges
    """
    B, Hq, Hkv, d = int(batch), int(num_q_heads), int(num_kv_heads), HEAD_DIM
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    seq_lens = np.asarray(seq_lens, dtype=np.int32).reshape(B)
    rng = np.random.default_rng(seed)
    meta: dict = {"kind": kind}

    # ---- K, V, q in that order --------------------------------------------------------------
    kscale = np.float32(np.sqrt(0.5)) if kind == "cluster" else np.float32(1.0)
    K = [rng.standard_normal((int(n), Hkv, d), dtype=np.float32) * kscale for n in seq_lens]
    V = [bf16_bits_from_f32(rng.standard_normal((int(n), Hkv, d), dtype=np.float32)) for n in seq_lens]
    qf = rng.standard_normal((B, Hq, d), dtype=np.float32)

    centroids = csize = coff = None
    # ---- structure ----------------------------------------------------------------------------
    if kind == "normal":
        pass
    elif kind == "outlier":
        ids = np.sort(rng.choice(d, size=4, replace=False))
        meta["outlier_channels"] = ids.tolist()
        for b in range(B):
            K[b][:, :, ids] *= np.float32(8.0)
    elif kind == "temperature":
        beta = np.exp(rng.uniform(np.log(0.05), np.log(3.5), size=(B, Hq))).astype(np.float32)
        meta["beta"] = beta
        qf = qf * beta[:, :, None]
    elif kind in ("planted", "peaked"):
        qr = _round_bf16(qf).astype(np.float64)
        qhat = qr / np.linalg.norm(qr, axis=-1, keepdims=True)
        positions = {}
        for b in range(B):
            n = int(seq_lens[b])
            for h in range(Hkv):
                if kind == "planted":
                    m = min(planted_per_head * G, n)
                    pos = rng.choice(n, size=m, replace=False) if m else np.zeros(0, np.int64)
                    for j in range(G):
                        hq = h * G + j
                        pj = pos[j * planted_per_head:(j + 1) * planted_per_head]
                        if pj.size == 0:
                            continue
                        g = rng.standard_normal((pj.size, d))
                        u = g - (g @ qhat[b, hq])[:, None] * qhat[b, hq][None, :]
                        u /= np.linalg.norm(u, axis=-1, keepdims=True)
                        K[b][pj, h, :] = (np.sqrt(d) * (0.6 * qhat[b, hq][None, :] + 0.8 * u)).astype(np.float32)
                        positions[(b, hq)] = pj
                else:
                    m = min(n_peaks, n)
                    pos = rng.choice(n, size=m, replace=False) if m else np.zeros(0, np.int64)
                    noise = rng.standard_normal((m, d)) * 0.1
                    K[b][pos, h, :] = (3.0 * qhat[b, h * G][None, :] + noise).astype(np.float32)
                    positions[(b, h)] = pos
        meta["planted_positions"] = positions
    elif kind == "cluster":
        C = int(num_clusters or 64)
        probs = (np.arange(1, C + 1, dtype=np.float64) ** -1.1)
        probs /= probs.sum()
        centroids = np.zeros((B, Hkv, C, d), np.uint16)
        csize = np.zeros((B, Hkv, C), np.int32)
        coff = np.zeros((B, Hkv, C + 1), np.int32)
        for b in range(B):
            n = int(seq_lens[b])
            for h in range(Hkv):
                mu = rng.standard_normal((C, d)).astype(np.float32) * np.float32(np.sqrt(0.5))
                labels = np.sort(rng.choice(C, size=n, p=probs))
                K[b][:, h, :] = K[b][:, h, :] + mu[labels]
                kr = _round_bf16(K[b][:, h, :]).astype(np.float64)
                cnt = np.bincount(labels, minlength=C)
                csize[b, h] = cnt
                coff[b, h, 1:] = np.cumsum(cnt)
                sums = np.zeros((C, d))
                np.add.at(sums, labels, kr)
                mean = np.where(cnt[:, None] > 0, sums / np.maximum(cnt, 1)[:, None], 0.0)
                centroids[b, h] = bf16_bits_from_f32(mean.astype(np.float32))
    else:
        raise ValueError(f"unknown workload kind {kind!r}")

    q = bf16_bits_from_f32(qf)
    Kb = [bf16_bits_from_f32(k) for k in K]
    del K

    # ---- paging: physical pages are a seeded permutation of the logical ones --------------------
    npages = [-(-int(n) // PAGE_SIZE) for n in seq_lens]
    total = int(sum(npages))
    max_pages = max(1, max(npages) if npages else 1)
    perm = rng.permutation(total).astype(np.int32)
    page_table = np.zeros((B, max_pages), np.int32)
    nphys = max(total, 1)
    fill = bf16_bits_from_f32(np.array([FILL_VALUE], np.float32))[0]
    k_pages = np.full((nphys, Hkv, PAGE_SIZE, d), fill, np.uint16)
    v_pages = np.full((nphys, Hkv, PAGE_SIZE, d), fill, np.uint16)
    off = 0
    for b in range(B):
        n, npg = int(seq_lens[b]), npages[b]
        phys = perm[off:off + npg]
        off += npg
        page_table[b, :npg] = phys
        if npg == 0:
            continue
        pad = npg * PAGE_SIZE - n
        for src, dst in ((Kb[b], k_pages), (V[b], v_pages)):
            x = np.concatenate([src, np.full((pad, Hkv, d), fill, np.uint16)], axis=0) if pad else src
            dst[phys] = x.reshape(npg, PAGE_SIZE, Hkv, d).transpose(0, 2, 1, 3)

    return Workload(name=name, seed=int(seed), batch=B, num_q_heads=Hq, num_kv_heads=Hkv,
                    seq_lens=seq_lens, page_table=page_table, k_pages=k_pages, v_pages=v_pages,
                    q=q, p=float(p), keep_frac=float(keep_frac), iters=int(iters),
                    centroids=centroids, csize=csize, coff=coff,
                    p1=None if p1 is None else float(p1), meta=meta)
