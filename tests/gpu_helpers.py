"""Helpers for the GPU parity tests: upload a workload, build the INT4 shadow with the library, and
run the oracle on the same seeded inputs.  The oracle only ever receives generator outputs."""

from __future__ import annotations

import math

import numpy as np
import torch

import top_sparse_attention_int4_amd as twl
from gen.device import upload

SM = twl.DEFAULT_SM_SCALE


def device_cache(w, device="cuda", key_bits=4):
    t = upload(w, device)
    cache = twl.PagedCache(t["k_pages"], t["v_pages"], t["page_table"], t["seq_lens"], w.num_q_heads,
                           max_seq_len=max(w.max_seq_len, 0), key_bits=key_bits)
    tb = torch.zeros(w.batch, dtype=torch.int32, device=device)
    twl.quantize_k(cache, tb, t["seq_lens"], max(w.max_seq_len, 0))
    return cache, t


def max_keep(w, keep_frac):
    return twl.keep_count(w.max_pages, keep_frac)


def workspace(cache, maxcand, device="cuda"):
    n = twl.workspace_bytes(cache, maxcand)
    return torch.empty(n, dtype=torch.uint8, device=device)


def run_decode(w, cache, t, *, p=None, keep_frac=None, iters=32, device="cuda", with_lists=True, topk=0,
               headwise=False):
    p = w.p if p is None else p
    keep_frac = w.keep_frac if keep_frac is None else keep_frac
    B, Hq, U = w.batch, w.num_q_heads, w.batch * w.num_kv_heads
    maxcand = 16 * max_keep(w, keep_frac) if keep_frac < 1 else max(w.max_seq_len, 0)
    ws = workspace(cache, maxcand, device)
    out = torch.full((B, Hq, 128), float("nan"), device=device)
    lse = torch.full((B, Hq), float("nan"), device=device)
    thr = torch.full((B, Hq), float("nan"), device=device)
    indptr = torch.full((U + 1,), -7, dtype=torch.int32, device=device)
    toks = torch.full((max(U * maxcand, 1),), -7, dtype=torch.int32, device=device)
    twl.decode(cache, t["q"], p=p, keep_frac=keep_frac, iters=iters, out=out, lse=lse, threshold=thr,
               sel_indptr=indptr if with_lists else None, sel_tokens=toks if with_lists else None, ws=ws,
               topk=topk, headwise=headwise)
    torch.cuda.synchronize()
    return {"out": out.cpu().numpy(), "lse": lse.cpu().numpy(), "thr": thr.cpu().numpy(),
            "indptr": indptr.cpu().numpy(), "tokens": toks.cpu().numpy()}


def unit_tokens(res, u):
    a, b = int(res["indptr"][u]), int(res["indptr"][u + 1])
    return res["tokens"][a:b]


def check_union(gpu_tokens, r, p):
    """GPU union vs oracle union: differences only in tokens some head finds ambiguous, and each
    head's kept set (restricted to its candidates) must still reach p - tau under oracle weights."""
    cand = r["candidates"]
    amb = set()
    for hd in r["heads"]:
        res = hd["topp"]
        amb |= set(cand[np.union1d(res["amb_i"], res["amb_ii"]).astype(np.int64)].tolist())
    g = set(np.asarray(gpu_tokens).tolist())
    o = set(r["union"].tolist())
    bad = (g ^ o) - amb
    return bad, g ^ o


def attn_tolerance(qg, kseq, vseq, oracle_union, gpu_tokens):
    """2e-3 plus the largest output change the differing tokens can cause: under the true softmax over
    the union of both sets, moving tokens of total weight a in or out shifts the output by at most
    2 a max|v| (``qg`` uint16 [G][128]; ``kseq``/``vseq`` uint16 [n][128] of the unit's kv-head)."""
    from oracle.attention import dense_weights
    from oracle.numerics import bf16_to_f32
    diff = np.setxor1d(np.asarray(oracle_union, np.int64), np.asarray(gpu_tokens, np.int64))
    if diff.size == 0:
        return 2e-3
    both = np.union1d(np.asarray(oracle_union, np.int64), np.asarray(gpu_tokens, np.int64))
    pos = np.searchsorted(both, diff)
    vmax = float(np.abs(bf16_to_f32(vseq[both])).max())
    extra = 0.0
    for h in range(qg.shape[0]):
        a = dense_weights(qg[h], kseq[both], SM)
        extra = max(extra, 2 * float(a[pos].sum()) * vmax)
    return 2e-3 + extra
