"""GPU parity of the Double-P cluster stage and of the top-p above 65536 candidates per head.

Bars as for the token path: the kept clusters of a unit must contain every cluster some head keeps
unambiguously and only clusters some head keeps or finds ambiguous (oracle.topp rule on the size-
weighted cluster weights); ranges are the kept clusters' exact (first token, length) in ascending
order.  The token stage (sets, union, attention) is then checked as in test_gpu_parity, with the
oracle run on the GPU's own kept ranges, so a unit whose kept clusters differ in ambiguous ones is
still compared.
"""

import math

import numpy as np
import pytest
import torch

import top_sparse_attention_int4_amd as twl
from gen import make_config, make_custom
from oracle import doublep
from oracle.topp import set_matches
from tests.gpu_helpers import (SM, SetStats, attn_tolerance, check_bisect, check_union, device_cache, oracle_decode,
                               unit_tokens, workspace)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    twl.lib()


def _print_case(name):
    print(f"[case] {name}", flush=True)


CLUSTER = [
    dict(batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=[3000, 1777], kind="cluster", seed=11, p=0.9, p1=0.95,
         num_clusters=96),
    dict(batch=1, num_q_heads=8, num_kv_heads=1, seq_lens=[5000], kind="cluster", seed=12, p=0.9, p1=0.9,
         num_clusters=1500),
    dict(batch=3, num_q_heads=2, num_kv_heads=2, seq_lens=[40, 0, 700], kind="cluster", seed=13, p=0.85, p1=0.95,
         num_clusters=64),
    dict(batch=1, num_q_heads=4, num_kv_heads=2, seq_lens=[2500], kind="cluster", seed=14, p=0.9, p1=1.0,
         num_clusters=200),
    # more than 4096 kept clusters (4614 non-empty of 6000, all kept at p1 = 1): the range prefix sums
    # no longer fit the union kernel's LDS and the block starts are searched in global memory
    dict(batch=1, num_q_heads=4, num_kv_heads=1, seq_lens=[60000], kind="cluster", seed=15, p=0.9, p1=1.0,
         num_clusters=6000),
]
CLUSTER_IDS = ["g4_two_seqs", "g8_1500_clusters", "g1_empty_seq", "p1_one", "over_4096_kept"]


def _cluster_gpu(w, cache, t, p1, iters=32):
    U, C = w.batch * w.num_kv_heads, w.num_clusters
    ranges = torch.full((U, C, 2), -7, dtype=torch.int32, device="cuda")
    count = torch.full((U,), -7, dtype=torch.int32, device="cuda")
    ws = workspace(cache, max(C, w.max_seq_len))
    twl.select_clusters_topp(cache, t["q"], SM, p1, iters, t["centroids"], t["csize"], t["coff"], C, ranges, count, ws)
    torch.cuda.synchronize()
    return ranges.cpu().numpy(), count.cpu().numpy()


def _check_clusters(w, ranges, count, p1, b, h):
    """Kept clusters of unit (b, h) against the oracle's per-head cluster top-p."""
    G = w.group
    u = b * w.num_kv_heads + h
    cs = doublep.select_clusters(w.q[b, h * G:(h + 1) * G], w.centroids[b, h], w.csize[b, h], p1, SM)
    coff, csize = w.coff[b, h], w.csize[b, h]
    n = int(count[u])
    rg = ranges[u, :n]
    # every listed range is one non-empty cluster, exactly, in ascending order
    first = {int(coff[c]): c for c in range(w.num_clusters) if csize[c] > 0}
    got = []
    for beg, ln in rg:
        assert int(beg) in first, (b, h, beg)
        c = first[int(beg)]
        assert int(ln) == int(csize[c]), (b, h, c, ln)
        got.append(c)
    assert np.all(np.diff(got) > 0)
    sure, possible = set(), set()
    for ph in cs["per_head"]:
        res, live = ph["res"], ph["live"]
        amb = set(live[np.union1d(res["amb_i"], res["amb_ii"]).astype(np.int64)].tolist())
        kept = set(ph["kept"].tolist())
        sure |= kept - amb
        possible |= kept | amb
    g = set(got)
    assert sure <= g, (b, h, sorted(sure - g)[:8])
    assert g <= possible, (b, h, sorted(g - possible)[:8])
    return got, sorted(cs["kept"].tolist())


@pytest.mark.parametrize("cfg", CLUSTER, ids=CLUSTER_IDS)
def test_cluster_select_parity(cfg):
    w = make_custom(**cfg)
    _print_case(w.name)
    cache, t = device_cache(w)
    ranges, count = _cluster_gpu(w, cache, t, w.p1)
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            _check_clusters(w, ranges, count, w.p1, b, h)


def _decode_clusters(w, cache, t, p=None, iters=32, events=None, lists=True):
    B, Hq, U = w.batch, w.num_q_heads, w.batch * w.num_kv_heads
    ws = workspace(cache, w.max_seq_len)
    out = torch.full((B, Hq, 128), float("nan"), device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    thr = torch.full((B, Hq), float("nan"), device="cuda")
    indptr = torch.full((U + 1,), -7, dtype=torch.int32, device="cuda")
    toks = torch.full((max(U * w.max_seq_len, 1),), -7, dtype=torch.int32, device="cuda")
    twl.decode_clusters(cache, t["q"], p=w.p if p is None else p, p1=w.p1, centroids=t["centroids"],
                        csize=t["csize"], coff=t["coff"], iters=iters, out=out, lse=lse, threshold=thr,
                        sel_indptr=indptr if lists else None, sel_tokens=toks if lists else None, ws=ws,
                        events=events)
    torch.cuda.synchronize()
    return {"out": out.cpu().numpy(), "lse": lse.cpu().numpy(), "thr": thr.cpu().numpy(),
            "indptr": indptr.cpu().numpy(), "tokens": toks.cpu().numpy()}


def _gpu_ranges(ranges, count, u):
    return np.asarray(ranges[u, :int(count[u])], np.int64).reshape(-1, 2)


def _oracle_on_gpu_ranges(w, ranges, count, units, **kw):
    """The oracle's decode of ``units`` with its token stage on the GPU's kept ranges (after checking
    the GPU's kept clusters against the oracle's cluster top-p)."""
    given = {}
    for b, h in units:
        _check_clusters(w, ranges, count, w.p1, b, h)
        given[(b, h)] = _gpu_ranges(ranges, count, b * w.num_kv_heads + h)
    return oracle_decode(w, units=units, ranges=given, **kw)


def _check_token_stage(w, g, res):
    """Token-level union and attention of every unit in ``res``."""
    G = w.group
    for (b, h), r in res.items():
        u = b * w.num_kv_heads + h
        gt = unit_tokens(g, u)
        bad, diff = check_union(gt, r, w.p)
        assert not bad, (b, h, sorted(bad)[:8])
        assert np.all(np.diff(gt) > 0)
        k, v = w.logical("k", b)[:, h], w.logical("v", b)[:, h]
        tol = attn_tolerance(w.q[b, h * G:(h + 1) * G], k, v, r["union"], gt)
        for j in range(G):
            if len(r["union"]) == 0:
                assert np.all(g["out"][b, h * G + j] == 0)
                continue
            err = np.max(np.abs(g["out"][b, h * G + j] - r["out"][j]))
            assert err <= tol, (b, h * G + j, err, tol, len(diff))


def _all_units(w):
    return [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]


@pytest.mark.parametrize("cfg", CLUSTER, ids=CLUSTER_IDS)
def test_decode_clusters_end_to_end(cfg):
    w = make_custom(**cfg)
    _print_case(w.name)
    cache, t = device_cache(w)
    g = _decode_clusters(w, cache, t)
    ranges, count = _cluster_gpu(w, cache, t, w.p1)
    _check_token_stage(w, g, _oracle_on_gpu_ranges(w, ranges, count, _all_units(w)))


@pytest.mark.parametrize("cfg", CLUSTER[:3], ids=CLUSTER_IDS[:3])
def test_cluster_value_means_parity(cfg):
    w = make_custom(**cfg)
    _print_case(w.name + " value means")
    cache, t = device_cache(w)
    C = w.csize.shape[-1]
    vm = torch.full((w.batch, w.num_kv_heads, C, 128), float("nan"), device="cuda")
    twl.cluster_value_means(cache, t["csize"], t["coff"], vm)
    torch.cuda.synchronize()
    vm = vm.cpu().numpy()
    for b in range(w.batch):
        v = w.logical("v", b)
        for h in range(w.num_kv_heads):
            want = doublep.value_means(v[:, h], w.csize[b, h], w.coff[b, h])
            assert np.allclose(vm[b, h], want, rtol=0, atol=1e-5), (b, h)


@pytest.mark.parametrize("cfg", CLUSTER[:4], ids=CLUSTER_IDS[:4])
def test_decode_clusters_approx_unkept(cfg):
    # the decode, then the unkept clusters merged in as (centroid, mean value) with their sizes
    w = make_custom(**cfg)
    _print_case(w.name + " approx unkept")
    cache, t = device_cache(w)
    g = _decode_clusters(w, cache, t)
    B, Hq, C = w.batch, w.num_q_heads, w.csize.shape[-1]
    out = torch.from_numpy(g["out"]).cuda()
    lse = torch.from_numpy(g["lse"]).cuda()
    vm = torch.empty((B, w.num_kv_heads, C, 128), device="cuda")
    twl.cluster_value_means(cache, t["csize"], t["coff"], vm)
    ws = workspace(cache, max(C, w.max_seq_len))
    twl.cluster_approx_unkept(cache, t["q"], p1=w.p1, centroids=t["centroids"], csize=t["csize"], vmean=vm,
                              out=out, lse=lse, ws=ws)
    torch.cuda.synchronize()
    go, gl = out.cpu().numpy(), lse.cpu().numpy()
    ranges, count = _cluster_gpu(w, cache, t, w.p1)
    res = _oracle_on_gpu_ranges(w, ranges, count, _all_units(w), approx_unkept=True)
    G = w.group
    for (b, h), r in res.items():
        u = b * w.num_kv_heads + h
        gt = unit_tokens(g, u)
        k, v = w.logical("k", b)[:, h], w.logical("v", b)[:, h]
        tol = attn_tolerance(w.q[b, h * G:(h + 1) * G], k, v, r["union"], gt) if len(r["union"]) else 2e-3
        for j in range(G):
            if int(w.seq_lens[b]) == 0:
                continue
            assert np.max(np.abs(go[b, h * G + j] - r["out"][j])) <= tol, (b, h * G + j)
            assert abs(gl[b, h * G + j] - r["lse"][j]) <= 1e-3, (b, h * G + j)
        if int(count[u]) == int((w.csize[b, h] > 0).sum()):  # every cluster kept: the outputs are unchanged
            assert np.array_equal(go[b, h * G:(h + 1) * G], g["out"][b, h * G:(h + 1) * G])


def test_decode_clusters_fused_equals_split():
    w = make_custom(**CLUSTER[0])
    _print_case(w.name)
    cache, t = device_cache(w)
    a = _decode_clusters(w, cache, t)
    b = _decode_clusters(w, cache, t)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    ranges, count = _cluster_gpu(w, cache, t, w.p1)
    U, C = w.batch * w.num_kv_heads, w.num_clusters
    rg = torch.from_numpy(ranges).cuda()
    ct = torch.from_numpy(count).cuda()
    ws = workspace(cache, w.max_seq_len)
    thr = torch.empty((w.batch, w.num_q_heads), device="cuda")
    indptr = torch.empty((U + 1,), dtype=torch.int32, device="cuda")
    toks = torch.empty((U * w.max_seq_len,), dtype=torch.int32, device="cuda")
    twl.estimate_topp(cache, t["q"], SM, w.p, 32, ranges=rg, count=ct, max_items=C, threshold=thr,
                      sel_indptr=indptr, sel_tokens=toks, ws=ws)
    out = torch.empty((w.batch, w.num_q_heads, 128), device="cuda")
    lse = torch.empty((w.batch, w.num_q_heads), device="cuda")
    twl.sparse_attn(cache, t["q"], SM, indptr, toks, w.max_seq_len, out, lse, ws)
    torch.cuda.synchronize()
    assert np.array_equal(indptr.cpu().numpy(), a["indptr"])
    n = int(a["indptr"][-1])
    assert np.array_equal(toks.cpu().numpy()[:n], a["tokens"][:n])
    assert np.array_equal(thr.cpu().numpy(), a["thr"])
    # same kept sets, attention partitioned differently: float32 sums agree to rounding
    assert np.allclose(out.cpu().numpy(), a["out"], rtol=1e-5, atol=1e-5)
    assert np.allclose(lse.cpu().numpy(), a["lse"], rtol=1e-5, atol=1e-5)


# ---- top-p above 65536 candidates per head ------------------------------------------------------------
WIDE = dict(batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=[100000, 70001], kind="temperature", seed=21,
            keep_frac=1.0, p=0.9)


def _estimate_all(w, cache, t, p, iters=32):
    U, Hq = w.batch * w.num_kv_heads, w.num_q_heads
    maxcand = w.max_seq_len
    mw = (maxcand + 31) // 32
    thr = torch.empty((w.batch, Hq), device="cuda")
    mass = torch.empty((w.batch, Hq), device="cuda")
    hm = torch.zeros((w.batch, Hq, mw), dtype=torch.int32, device="cuda")
    indptr = torch.empty((U + 1,), dtype=torch.int32, device="cuda")
    toks = torch.empty((U * maxcand,), dtype=torch.int32, device="cuda")
    ws = workspace(cache, maxcand)
    twl.estimate_topp(cache, t["q"], SM, p, iters, threshold=thr, mass=mass, head_mask=hm, mask_words=mw,
                      sel_indptr=indptr, sel_tokens=toks, ws=ws)
    torch.cuda.synchronize()
    return {"thr": thr.cpu().numpy(), "mass": mass.cpu().numpy(), "mask": hm.cpu().numpy().view(np.uint32),
            "indptr": indptr.cpu().numpy(), "tokens": toks.cpu().numpy()}


def _mask_indices(words, ncand):
    bits = np.unpackbits(words.view(np.uint8), bitorder="little")
    return np.nonzero(bits[:ncand])[0]


@pytest.fixture(scope="module")
def wide_case():
    w = make_custom(**WIDE)
    cache, t = device_cache(w)
    return w, cache, t, oracle_decode(w)


def _check_wide_sets(w, g, res, st, units=None):
    G = w.group
    for (b, h), r in res.items():
        if units is not None and (b, h) not in units:
            continue
        u = b * w.num_kv_heads + h
        ncand = len(r["candidates"])
        for j, hd in enumerate(r["heads"]):
            hq = h * G + j
            sel = _mask_indices(g["mask"][b, hq], ncand)
            ok, msg = set_matches(sel, hd["topp"], hd["W"], w.p)
            assert ok, (b, hq, msg)
            st.add(sel, hd["topp"])
            assert abs(g["mass"][b, hq] - math.fsum(hd["W"][sel])) < 1e-5
        bad, _ = check_union(unit_tokens(g, u), r, w.p)
        assert not bad, (b, h, sorted(bad)[:8])
        assert np.all(np.diff(unit_tokens(g, u)) > 0)


def test_wide_topp_parity(wide_case):
    w, cache, t, res = wide_case
    _print_case(w.name + " wide top-p")
    g = _estimate_all(w, cache, t, w.p)
    for (b, h), r in res.items():
        assert len(r["candidates"]) > 65536 or b == 1
    st = SetStats(w.name + " wide")
    _check_wide_sets(w, g, res, st)
    st.report()


def test_wide_topp_p_one_and_few_iterations(wide_case):
    w, cache, t, res = wide_case
    _print_case(w.name + " wide top-p, p=1 and few steps")
    g1 = _estimate_all(w, cache, t, 1.0)
    full = _estimate_all(w, cache, t, 0.9)
    for b in range(w.batch):
        n = int(w.seq_lens[b])
        for hq in range(w.num_q_heads):
            assert len(_mask_indices(g1["mask"][b, hq], n)) == n
    for it in (4, 11, 20, 27):
        few = _estimate_all(w, cache, t, 0.9, iters=it)
        for (b, h), r in res.items():
            n = len(r["candidates"])
            for j in range(w.group):
                hq = h * w.group + j
                s_few = _mask_indices(few["mask"][b, hq], n)
                s_full = _mask_indices(full["mask"][b, hq], n)
                assert set(s_full.tolist()) <= set(s_few.tolist())
                hd = r["heads"][j]
                ok, msg = check_bisect(s_few, hd, 0.9, it)
                assert ok, (it, b, hq, msg)
                assert math.fsum(hd["W"][s_few]) >= 0.9 - hd["topp"]["tau_p"]


def test_wide_decode_end_to_end(wide_case):
    w, cache, t, res = wide_case
    _print_case(w.name + " wide decode")
    from tests.gpu_helpers import run_decode
    g = run_decode(w, cache, t)
    for (b, h), r in res.items():
        u = b * w.num_kv_heads + h
        gt = unit_tokens(g, u)
        bad, diff = check_union(gt, r, w.p)
        assert not bad, (b, h, sorted(bad)[:8])
        G = w.group
        k, v = w.logical("k", b)[:, h], w.logical("v", b)[:, h]
        tol = attn_tolerance(w.q[b, h * G:(h + 1) * G], k, v, r["union"], gt)
        for j in range(G):
            err = np.max(np.abs(g["out"][b, h * G + j] - r["out"][j]))
            assert err <= tol, (b, h * G + j, err, tol)


@pytest.mark.parametrize("iters", [32, 20, 11, 4])
def test_wide_decode_without_lists_is_bitwise_the_same(wide_case, iters):
    # The timed form of the decode (no token list requested) sorts most candidates by logit bounds
    # and weighs only those near the first level's bin; the listed run weighs every candidate.  Both
    # give bitwise the same outputs, with the bin's threshold still open (32, 20 steps) and fixed by
    # the first level (11, 4 steps).
    w, cache, t, res = wide_case
    _print_case(w.name + f" wide decode, no lists, {iters} steps")
    from tests.gpu_helpers import run_decode
    a = run_decode(w, cache, t, iters=iters)
    b = run_decode(w, cache, t, iters=iters, with_lists=False)
    for k in ("out", "lse", "thr"):
        assert np.array_equal(a[k], b[k], equal_nan=True), k


# ---- full-size hierarchical layer (262144 tokens, 4096 clusters) ----------------------------------------
def test_c5_full_size_sampled_units():
    w = make_config("C5")
    _print_case(w.name)
    cache, t = device_cache(w)
    g = _decode_clusters(w, cache, t)
    ranges, count = _cluster_gpu(w, cache, t, w.p1)
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            _check_clusters(w, ranges, count, w.p1, b, h)
    units = [(0, 0), (0, 2), (0, 5), (0, 7)]
    res = _oracle_on_gpu_ranges(w, ranges, count, units)
    _check_token_stage(w, g, res)
    # per-head token sets on the GPU's kept ranges (the multi-block top-p: ~250K candidates per head)
    U, C = w.batch * w.num_kv_heads, w.num_clusters
    maxcand = w.max_seq_len
    mw = (maxcand + 31) // 32
    thr = torch.empty((w.batch, w.num_q_heads), device="cuda")
    mass = torch.empty((w.batch, w.num_q_heads), device="cuda")
    hm = torch.zeros((w.batch, w.num_q_heads, mw), dtype=torch.int32, device="cuda")
    indptr = torch.empty((U + 1,), dtype=torch.int32, device="cuda")
    toks = torch.empty((U * maxcand,), dtype=torch.int32, device="cuda")
    ws = workspace(cache, maxcand)
    twl.estimate_topp(cache, t["q"], SM, w.p, 32, ranges=torch.from_numpy(ranges).cuda(),
                      count=torch.from_numpy(count).cuda(), max_items=C, threshold=thr, mass=mass, head_mask=hm,
                      mask_words=mw, sel_indptr=indptr, sel_tokens=toks, ws=ws)
    torch.cuda.synchronize()
    e = {"mask": hm.cpu().numpy().view(np.uint32), "mass": mass.cpu().numpy(), "indptr": indptr.cpu().numpy(),
         "tokens": toks.cpu().numpy()}
    st = SetStats(w.name)
    _check_wide_sets(w, e, res, st)
    st.report()
    assert np.all(np.isfinite(g["out"]))
    # the timed form (no token list requested) is bitwise the same
    g2 = _decode_clusters(w, cache, t, lists=False)
    for k in ("out", "lse", "thr"):
        assert np.array_equal(g[k], g2[k], equal_nan=True), k
