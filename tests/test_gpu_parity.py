"""GPU parity: every stage of the HIP path against the CPU oracle on the same seeded inputs.

Bars (the parity rules that go with the oracle):
* INT4 codes, fp16 scale/zero, page bounds and page selections: bit-exact;
* top-p sets: the oracle's sets come from the float64 definition of the estimate (bf16 query times
  the exactly dequantised codes).  They must equal the GPU's except for tokens the oracle marks
  ambiguous -- within 1e-6 relative of the threshold weight, widened per token by the estimate
  kernel's stated logit error (tests/kernel_model.py), or at a rank whose preceding prefix mass is
  within tau_p of p (1e-6 plus that error's weighted mean and the kernel's fixed-point mass
  resolution) -- and the kept mass (oracle weights) must reach p - tau_p.  Each test prints how many
  tokens each clause excused;
* stopped-early searches: the oracle's bisection model at the same number of steps;
* attention output and lse: within 2e-3 max-abs (plus, when the sets differ in ambiguous tokens,
  the output change those tokens can cause).
"""

import math

import numpy as np
import pytest
import torch

import top_sparse_attention_int4_amd as twl
from gen import make_config, make_custom
from oracle import numerics, quantize, select
from oracle.topp import set_matches
from tests.gpu_helpers import (SM, SetStats, attn_tolerance, bounds_rows, check_bisect, check_union, device_cache,
                               max_keep, oracle_decode, run_decode, shadow_by_phys, unit_tokens, workspace)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    twl.lib()


TINY = [
    dict(batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=[777, 300], kind="outlier", seed=4, keep_frac=0.25, p=0.85),
    dict(batch=3, num_q_heads=4, num_kv_heads=4, seq_lens=[17, 1, 1000], kind="normal", seed=5, keep_frac=0.25, p=0.9),
    dict(batch=1, num_q_heads=16, num_kv_heads=2, seq_lens=[2047], kind="temperature", seed=6, keep_frac=0.3, p=0.85),
    dict(batch=2, num_q_heads=8, num_kv_heads=4, seq_lens=[4100, 64], kind="planted", seed=7, keep_frac=0.25, p=0.9,
         planted_per_head=16),
    dict(batch=1, num_q_heads=1, num_kv_heads=1, seq_lens=[1500], kind="peaked", seed=8, keep_frac=1.0, p=0.9),
    dict(batch=2, num_q_heads=4, num_kv_heads=1, seq_lens=[0, 33], kind="normal", seed=9, keep_frac=0.25, p=0.85),
]
TINY_IDS = ["outlier_g4", "mha_edge_lens", "temp_g8", "planted_g2", "peaked_all", "empty_seq"]


def _print_case(name):
    print(f"[case] {name}", flush=True)


# ---- a0: quantisation ------------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", TINY + [None], ids=TINY_IDS + ["C1"])
def test_quantize_bitexact(cfg):
    w = make_config("C1") if cfg is None else make_custom(**cfg)
    _print_case(w.name)
    cache, t = device_cache(w)
    torch.cuda.synchronize()
    exp = quantize.expected_paged(w.k_pages, w.page_table, w.seq_lens)
    # the library stores the shadow by logical page; compare it in the oracle's physical order
    k4 = shadow_by_phys(w, cache.k4.cpu().numpy())
    meta = shadow_by_phys(w, cache.k4_meta.cpu().numpy().view(np.uint16))
    kb = shadow_by_phys(w, bounds_rows(cache.kbound.cpu().numpy().view(np.uint16)))
    m3 = np.broadcast_to(exp["tok_mask"][:, None, :], k4.shape[:3])
    assert np.array_equal(k4[m3], exp["k4"][m3])
    assert np.array_equal(meta[m3], exp["k4_meta"][m3])
    pm = exp["page_mask"]
    # bounds compared as values (the sign of a zero bound is not specified)
    assert np.array_equal(numerics.bf16_to_f32(kb[pm]), numerics.bf16_to_f32(exp["kbound"][pm]))


@pytest.mark.parametrize("bits", [2, 8])
@pytest.mark.parametrize("cfg", [TINY[0], TINY[3]], ids=[TINY_IDS[0], TINY_IDS[3]])
def test_quantize_bitexact_other_widths(cfg, bits):
    w = make_custom(**cfg)
    _print_case(f"{w.name} bits={bits}")
    cache, t = device_cache(w, key_bits=bits)
    torch.cuda.synchronize()
    exp = quantize.expected_paged(w.k_pages, w.page_table, w.seq_lens, bits=bits)
    k4 = shadow_by_phys(w, cache.k4.cpu().numpy())
    meta = shadow_by_phys(w, cache.k4_meta.cpu().numpy().view(np.uint16))
    assert k4.shape[-1] == 16 * bits
    m3 = np.broadcast_to(exp["tok_mask"][:, None, :], k4.shape[:3])
    assert np.array_equal(k4[m3], exp["k4"][m3])
    assert np.array_equal(meta[m3], exp["k4_meta"][m3])


def test_quantize_incremental_equals_bulk():
    w = make_custom(batch=2, num_q_heads=4, num_kv_heads=2, seq_lens=[70, 45], seed=12)
    _print_case(w.name)
    bulk, t = device_cache(w)
    inc = twl.PagedCache(t["k_pages"], t["v_pages"], t["page_table"], t["seq_lens"], w.num_q_heads,
                         max_seq_len=w.max_seq_len)
    steps = [(0, 5), (5, 16), (16, 17), (17, 40), (40, 70)]
    for a, b in steps:
        tb = torch.tensor([min(a, 70), min(a, 45)], dtype=torch.int32, device="cuda")
        te = torch.tensor([min(b, 70), min(b, 45)], dtype=torch.int32, device="cuda")
        twl.quantize_k(inc, tb, te, b - a)
    torch.cuda.synchronize()
    for name in ("k4", "k4_meta"):
        x, y = getattr(bulk, name).cpu().numpy(), getattr(inc, name).cpu().numpy()
        for b_ in range(2):
            n = int(w.seq_lens[b_])
            for tok in range(n):
                assert np.array_equal(x[b_, tok // 16, :, tok % 16], y[b_, tok // 16, :, tok % 16])
    kb_bulk, kb_inc = bulk.kbound.cpu().numpy(), inc.kbound.cpu().numpy()
    for b_ in range(2):
        npg = -(-int(w.seq_lens[b_]) // 16)
        assert np.array_equal(kb_bulk[b_, :npg], kb_inc[b_, :npg])


# ---- a1: page selection ----------------------------------------------------------------------------
def _select_pages_gpu(w, cache, t, keep_frac):
    mk = max_keep(w, keep_frac)
    U = w.batch * w.num_kv_heads
    ids = torch.full((U, mk), -1, dtype=torch.int32, device="cuda")
    cnt = torch.full((U,), -1, dtype=torch.int32, device="cuda")
    ws = workspace(cache, 16 * mk)
    twl.select_pages(cache, t["q"], keep_frac, mk, ids, cnt, ws)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("cfg", TINY[:4] + [TINY[5]], ids=TINY_IDS[:4] + [TINY_IDS[5]])
def test_select_pages_bitexact(cfg):
    w = make_custom(**cfg)
    _print_case(w.name)
    cache, t = device_cache(w)
    ids, cnt = _select_pages_gpu(w, cache, t, w.keep_frac)
    G = w.group
    for b in range(w.batch):
        k = w.logical("k", b)
        for h in range(w.num_kv_heads):
            u = b * w.num_kv_heads + h
            n = int(w.seq_lens[b])
            if n == 0:
                assert cnt[u] == 0
                continue
            kmin, kmax = quantize.page_bounds(k[:, h:h + 1, :])
            gs = select.group_scores(w.q[b, h * G:(h + 1) * G], kmin[:, 0], kmax[:, 0])
            want = select.top_pages(gs, select.keep_count(kmin.shape[0], w.keep_frac))
            assert cnt[u] == len(want)
            assert np.array_equal(ids[u, :cnt[u]], want), (b, h)


def test_select_pages_full_size_llama_layer():
    w = make_config("C2")
    _print_case(w.name)
    cache, t = device_cache(w)
    ids, cnt = _select_pages_gpu(w, cache, t, w.keep_frac)
    k = w.logical("k", 0)
    for h in range(w.num_kv_heads):
        kmin, kmax = quantize.page_bounds(k[:, h:h + 1, :])
        gs = select.group_scores(w.q[0, h * 4:(h + 1) * 4], kmin[:, 0], kmax[:, 0])
        want = select.top_pages(gs, 512)
        assert cnt[h] == 512 and np.array_equal(ids[h, :512], want)


def _check_select_against_oracle(w, ids, cnt):
    G = w.group
    for b in range(w.batch):
        k = w.logical("k", b)
        for h in range(w.num_kv_heads):
            u = b * w.num_kv_heads + h
            kmin, kmax = quantize.page_bounds(k[:, h:h + 1, :])
            gs = select.group_scores(w.q[b, h * G:(h + 1) * G], kmin[:, 0], kmax[:, 0])
            want = select.top_pages(gs, select.keep_count(kmin.shape[0], w.keep_frac))
            assert cnt[u] == len(want), (b, h)
            assert np.array_equal(ids[u, :cnt[u]], want), (b, h)


@pytest.mark.parametrize("G", [1, 4, 8])
def test_select_pages_large_grid_ragged(G):
    # more than 512 64-page blocks, so the page scores run as 4-wave blocks of 256 pages; 1400 pages
    # per sequence is not a multiple of 256 (the last block of each unit reaches past the allocated
    # pages) and the sequences end mid-page, mid-block and after one token
    kv = 8 if G < 8 else 4
    w = make_custom(batch=3 if G < 8 else 6, num_q_heads=G * kv, num_kv_heads=kv,
                    seq_lens=([22400, 17001, 1] if G < 8 else [22400, 17001, 1, 300, 16 * 1400 - 7, 4100]),
                    kind="outlier", seed=90 + G, keep_frac=0.25, p=0.85, name=f"select_large_grid_g{G}")
    assert w.batch * kv * -(-w.max_seq_len // 16 // 64) > 512
    _print_case(w.name)
    cache, t = device_cache(w)
    ids, cnt = _select_pages_gpu(w, cache, t, w.keep_frac)
    _check_select_against_oracle(w, ids, cnt)


def test_select_pages_tied_scores():
    # every sequence repeats 5 page contents, so each score value is shared by many pages and the
    # K-th key falls inside a run of ties, which go to the lowest page ids
    w = make_custom(batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=[16 * 700, 16 * 2048], kind="normal",
                    seed=21, keep_frac=0.25, p=0.9, name="tied_pages")
    _print_case(w.name)
    for b in range(w.batch):
        npg = int(w.seq_lens[b]) // 16
        phys = w.page_table[b, :npg]
        w.k_pages[phys] = w.k_pages[phys[np.arange(npg) % 5]]
    cache, t = device_cache(w)
    ids, cnt = _select_pages_gpu(w, cache, t, w.keep_frac)
    k = w.logical("k", 0)
    kmin, kmax = quantize.page_bounds(k[:, 0:1, :])
    gs_b0 = select.group_scores(w.q[0, 0:4], kmin[:, 0], kmax[:, 0])
    assert len(np.unique(gs_b0)) <= 5  # the case really has ties
    _check_select_against_oracle(w, ids, cnt)


def test_select_pages_beyond_register_keys():
    # 8750 pages in one unit (more than the 8192 scores one block holds in registers)
    w = make_custom(batch=1, num_q_heads=4, num_kv_heads=1, seq_lens=[140000], kind="outlier", seed=22,
                    keep_frac=0.25, p=0.9, name="long_unit_select")
    _print_case(w.name)
    cache, t = device_cache(w)
    ids, cnt = _select_pages_gpu(w, cache, t, w.keep_frac)
    _check_select_against_oracle(w, ids, cnt)


# ---- a2-a5: estimate, top-p, union on oracle-given candidates ---------------------------------------
def _estimate_on_pages(w, cache, t, pages_per_unit, p, iters=32):
    U, Hq = w.batch * w.num_kv_heads, w.num_q_heads
    mk = max(1, max(len(x) for x in pages_per_unit))
    ids = torch.zeros((U, mk), dtype=torch.int32)
    cnt = torch.zeros((U,), dtype=torch.int32)
    for u, pg in enumerate(pages_per_unit):
        ids[u, :len(pg)] = torch.from_numpy(np.asarray(pg, np.int32))
        cnt[u] = len(pg)
    ids, cnt = ids.cuda(), cnt.cuda()
    maxcand = 16 * mk
    mw = (maxcand + 31) // 32
    thr = torch.empty((w.batch, Hq), device="cuda")
    mass = torch.empty((w.batch, Hq), device="cuda")
    hm = torch.zeros((w.batch, Hq, mw), dtype=torch.int32, device="cuda")
    indptr = torch.empty((U + 1,), dtype=torch.int32, device="cuda")
    toks = torch.empty((U * maxcand,), dtype=torch.int32, device="cuda")
    ws = workspace(cache, maxcand)
    twl.estimate_topp(cache, t["q"], SM, p, iters, page_ids=ids, count=cnt, max_items=mk, threshold=thr,
                      mass=mass, head_mask=hm, mask_words=mw, sel_indptr=indptr, sel_tokens=toks, ws=ws)
    torch.cuda.synchronize()
    return {"thr": thr.cpu().numpy(), "mass": mass.cpu().numpy(), "mask": hm.cpu().numpy().view(np.uint32),
            "indptr": indptr.cpu().numpy(), "tokens": toks.cpu().numpy()}


def _mask_indices(words, ncand):
    bits = np.unpackbits(words.view(np.uint8), bitorder="little")
    return np.nonzero(bits[:ncand])[0]


def _check_head_sets(w, g, res, p, stats, units=None):
    """Every head's GPU bitmap against the oracle's top-p set, the reported kept mass, and the union."""
    G = w.group
    for (b, h), r in res.items():
        if units is not None and (b, h) not in units:
            continue
        u = b * w.num_kv_heads + h
        ncand = len(r["candidates"])
        for j, hd in enumerate(r["heads"]):
            hq = h * G + j
            sel = _mask_indices(g["mask"][b, hq], ncand)
            ok, msg = set_matches(sel, hd["topp"], hd["W"], p)
            assert ok, (b, hq, msg)
            stats.add(sel, hd["topp"])
            if ncand:
                assert abs(g["mass"][b, hq] - math.fsum(hd["W"][sel])) < 1e-5
        bad, _ = check_union(unit_tokens(g, u), r, p)
        assert not bad, (b, h, sorted(bad)[:8])
        assert np.all(np.diff(unit_tokens(g, u)) > 0)


@pytest.mark.parametrize("cfg", TINY, ids=TINY_IDS)
def test_estimate_topp_parity(cfg):
    w = make_custom(**cfg)
    _print_case(w.name)
    cache, t = device_cache(w)
    res = oracle_decode(w)
    pages = [res[(b, h)]["pages"] for b in range(w.batch) for h in range(w.num_kv_heads)]
    g = _estimate_on_pages(w, cache, t, pages, w.p)
    st = SetStats(w.name)
    _check_head_sets(w, g, res, w.p, st)
    st.report()


@pytest.mark.parametrize("bits", [2, 8])
@pytest.mark.parametrize("cfg", [TINY[0], TINY[2], TINY[3]], ids=[TINY_IDS[0], TINY_IDS[2], TINY_IDS[3]])
def test_estimate_topp_parity_other_widths(cfg, bits):
    w = make_custom(**cfg)
    _print_case(f"{w.name} bits={bits}")
    cache, t = device_cache(w, key_bits=bits)
    res = oracle_decode(w, bits=bits)
    pages = [res[(b, h)]["pages"] for b in range(w.batch) for h in range(w.num_kv_heads)]
    g = _estimate_on_pages(w, cache, t, pages, w.p)
    st = SetStats(f"{w.name} bits={bits}")
    _check_head_sets(w, g, res, w.p, st)
    st.report()


@pytest.mark.parametrize("name", ["C2", "C3", "C4"])
def test_topp_sets_match_the_definition_full_size(name):
    # every head of the Llama-shaped layer, and 8 sampled (sequence, kv-head) units of the two large
    # layers, against the float64 definition of the estimate
    w = make_config(name)
    _print_case(w.name)
    cache, t = device_cache(w)
    U = w.batch * w.num_kv_heads
    ids, cnt = _select_pages_gpu(w, cache, t, w.keep_frac)
    if U <= 8:
        units = [(u // w.num_kv_heads, u % w.num_kv_heads) for u in range(U)]
    else:
        rng = np.random.default_rng(1)
        units = [(int(u) // w.num_kv_heads, int(u) % w.num_kv_heads) for u in rng.choice(U, size=8, replace=False)]
    res = oracle_decode(w, units=units)
    for (b, h), r in res.items():
        u = b * w.num_kv_heads + h
        assert np.array_equal(ids[u, :cnt[u]], r["pages"]), (b, h)
    g = _estimate_on_pages(w, cache, t, [ids[u, :cnt[u]] for u in range(U)], w.p)
    st = SetStats(w.name)
    _check_head_sets(w, g, res, w.p, st)
    st.report()


def test_topp_p_one_and_few_iterations():
    w = make_custom(batch=1, num_q_heads=4, num_kv_heads=1, seq_lens=[900], seed=3, keep_frac=0.5)
    _print_case(w.name)
    cache, t = device_cache(w)
    res = oracle_decode(w, p=0.9)
    r = res[(0, 0)]
    pages = [r["pages"]]
    ncand = len(r["candidates"])
    g1 = _estimate_on_pages(w, cache, t, pages, 1.0)
    for hq in range(4):
        assert len(_mask_indices(g1["mask"][0, hq], ncand)) == ncand
    full = _estimate_on_pages(w, cache, t, pages, 0.9, iters=32)
    for it in (1, 3, 8, 13, 20, 25, 30):
        few = _estimate_on_pages(w, cache, t, pages, 0.9, iters=it)
        for hq in range(4):
            s_few = _mask_indices(few["mask"][0, hq], ncand)
            s_full = _mask_indices(full["mask"][0, hq], ncand)
            assert set(s_full.tolist()) <= set(s_few.tolist())
            hd = r["heads"][hq]
            ok, msg = check_bisect(s_few, hd, 0.9, it)
            assert ok, (it, hq, msg)
            assert math.fsum(hd["W"][s_few]) >= 0.9 - hd["topp"]["tau_p"]


# ---- a6-a7: attention on oracle-given token sets --------------------------------------------------
@pytest.mark.parametrize("cfg", TINY, ids=TINY_IDS)
def test_sparse_attn_on_oracle_sets(cfg):
    w = make_custom(**cfg)
    _print_case(w.name)
    cache, t = device_cache(w)
    res = oracle_decode(w)
    U = w.batch * w.num_kv_heads
    lists = [res[(b, h)]["union"] for b in range(w.batch) for h in range(w.num_kv_heads)]
    # add a few random extra sets: everything, a strided subset
    indptr = np.zeros(U + 1, np.int32)
    for u, l in enumerate(lists):
        indptr[u + 1] = indptr[u] + len(l)
    toks = np.concatenate(lists).astype(np.int32) if indptr[-1] else np.zeros(1, np.int32)
    out = torch.full((w.batch, w.num_q_heads, 128), float("nan"), device="cuda")
    lse = torch.full((w.batch, w.num_q_heads), float("nan"), device="cuda")
    maxsel = int(max(len(l) for l in lists))
    ws = workspace(cache, max(maxsel, 1))
    twl.sparse_attn(cache, t["q"], SM, torch.from_numpy(indptr).cuda(), torch.from_numpy(toks).cuda(), maxsel,
                    out, lse, ws)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    G = w.group
    for (b, h), r in res.items():
        for j in range(G):
            hq = h * G + j
            if len(r["union"]) == 0:
                assert np.all(o[b, hq] == 0) and l[b, hq] == -np.inf
                continue
            assert np.max(np.abs(o[b, hq] - r["out"][j])) <= 2e-3, (b, hq)
            assert abs(l[b, hq] - r["lse"][j]) <= 2e-3


def test_sparse_attn_all_tokens_and_single_token():
    w = make_custom(batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=[3000, 5], seed=21)
    _print_case(w.name)
    cache, t = device_cache(w)
    from oracle.attention import sparse_attention
    U = 4
    lists = [np.arange(3000), np.array([1234]), np.arange(5), np.array([], np.int64)]
    indptr = np.zeros(U + 1, np.int32)
    for u, l in enumerate(lists):
        indptr[u + 1] = indptr[u] + len(l)
    toks = np.concatenate(lists).astype(np.int32)
    out = torch.empty((2, 8, 128), device="cuda")
    lse = torch.empty((2, 8), device="cuda")
    ws = workspace(cache, 3000)
    twl.sparse_attn(cache, t["q"], SM, torch.from_numpy(indptr).cuda(), torch.from_numpy(toks).cuda(), 3000,
                    out, lse, ws)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    for b in range(2):
        k, v = w.logical("k", b), w.logical("v", b)
        for h in range(2):
            idx = lists[b * 2 + h]
            for j in range(4):
                hq = h * 4 + j
                if len(idx) == 0:
                    assert np.all(o[b, hq] == 0)
                    continue
                ref, _ = sparse_attention(w.q[b, hq], k[:, h], v[:, h], idx, SM)
                assert np.max(np.abs(o[b, hq] - ref)) <= 2e-3
    # a single token returns its value row (bf16 exactly representable in fp32)
    assert np.array_equal(o[0, 4], numerics.bf16_to_f32(w.logical("v", 0)[1234, 1]))


# ---- whole decode step ---------------------------------------------------------------------------
def _check_decode(w, g, res, units=None, topk=False):
    G = w.group
    for (b, h), r in res.items():
        if units is not None and (b, h) not in units:
            continue
        u = b * w.num_kv_heads + h
        gt = unit_tokens(g, u)
        bad, diff = check_union(gt, r, w.p, topk=topk)
        assert not bad, (b, h, sorted(bad)[:8])
        k, v = w.logical("k", b)[:, h], w.logical("v", b)[:, h]
        tol = attn_tolerance(w.q[b, h * G:(h + 1) * G], k, v, r["union"], gt)
        for j in range(G):
            hq = h * G + j
            if len(r["union"]) == 0:
                assert np.all(g["out"][b, hq] == 0)
                continue
            err = np.max(np.abs(g["out"][b, hq] - r["out"][j]))
            assert err <= tol, (b, hq, err, tol, len(diff))
            if len(diff) == 0:
                assert abs(g["lse"][b, hq] - r["lse"][j]) <= 2e-3, (b, hq)


@pytest.mark.parametrize("cfg", TINY, ids=TINY_IDS)
def test_decode_end_to_end(cfg):
    w = make_custom(**cfg)
    _print_case(w.name)
    cache, t = device_cache(w)
    g = run_decode(w, cache, t)
    _check_decode(w, g, oracle_decode(w))


@pytest.mark.parametrize("bits", [2, 8])
def test_decode_end_to_end_other_widths(bits):
    w = make_custom(**TINY[0])
    _print_case(f"{w.name} bits={bits}")
    cache, t = device_cache(w, key_bits=bits)
    g = run_decode(w, cache, t)
    _check_decode(w, g, oracle_decode(w, bits=bits))


def test_decode_with_kv_in_pinned_host_memory():
    # the offloading scenario: K/V stay in pinned host memory, read over PCIe by the same kernels;
    # the outputs match the oracle, and every output is bitwise the device-resident run's
    w = make_custom(**TINY[3])
    _print_case(w.name + " host K/V")
    cache, t = device_cache(w)
    g_dev = run_decode(w, cache, t)
    kh = t["k_pages"].cpu().pin_memory()
    vh = t["v_pages"].cpu().pin_memory()
    cache_h = twl.PagedCache(kh, vh, t["page_table"], t["seq_lens"], w.num_q_heads, max_seq_len=w.max_seq_len)
    twl.quantize_k(cache_h, torch.zeros(w.batch, dtype=torch.int32, device="cuda"), t["seq_lens"], w.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(cache_h.k4, cache.k4) and torch.equal(cache_h.kbound, cache.kbound)
    g_host = run_decode(w, cache_h, t)
    _check_decode(w, g_host, oracle_decode(w))
    for k in ("out", "lse", "thr", "indptr"):
        assert np.array_equal(np.asarray(g_host[k]), np.asarray(g_dev[k]), equal_nan=True), k
    n = int(g_dev["indptr"][-1])
    assert np.array_equal(g_host["tokens"][:n], g_dev["tokens"][:n])


@pytest.mark.parametrize("cfg", [TINY[0], TINY[2], TINY[3]], ids=[TINY_IDS[0], TINY_IDS[2], TINY_IDS[3]])
def test_decode_topk_baseline(cfg):
    # the fixed-budget baseline: every head keeps its 40 largest estimated weights
    w = make_custom(**cfg)
    _print_case(w.name + " top-40")
    cache, t = device_cache(w)
    g = run_decode(w, cache, t, topk=40)
    _check_decode(w, g, oracle_decode(w, topk=40), topk=True)


@pytest.mark.parametrize("cfg", [TINY[0], TINY[2], TINY[3], TINY[5]],
                         ids=[TINY_IDS[0], TINY_IDS[2], TINY_IDS[3], TINY_IDS[5]])
def test_decode_headwise(cfg):
    # each query head attends over its own top-p set instead of the group's union
    w = make_custom(**cfg)
    _print_case(w.name + " head-wise")
    cache, t = device_cache(w)
    g = run_decode(w, cache, t, headwise=True)
    res = oracle_decode(w, headwise=True)
    _check_decode(w, g, res)
    # it differs from the union output wherever a head's set is smaller than the union
    gu = run_decode(w, cache, t)
    some = [(b, h) for (b, h), r in res.items() if any(len(hd["tokens"]) < len(r["union"]) for hd in r["heads"])]
    if some:
        b, h = some[0]
        G = w.group
        assert not np.allclose(g["out"][b, h * G:(h + 1) * G], gu["out"][b, h * G:(h + 1) * G])


def test_decode_topk_headwise_together():
    w = make_custom(**TINY[2])
    _print_case(w.name + " top-25 head-wise")
    cache, t = device_cache(w)
    g = run_decode(w, cache, t, topk=25, headwise=True)
    _check_decode(w, g, oracle_decode(w, topk=25, headwise=True), topk=True)


def test_decode_tied_weights():
    # pages repeat 5 contents, so each weight value is shared by ~60 tokens: the threshold search
    # meets bins of tied keys and keeps every tie at the threshold
    w = make_custom(batch=1, num_q_heads=8, num_kv_heads=2, seq_lens=[16 * 300], kind="normal", seed=23,
                    keep_frac=1.0, p=0.9, name="tied_weights")
    _print_case(w.name)
    npg = int(w.seq_lens[0]) // 16
    phys = w.page_table[0, :npg]
    w.k_pages[phys] = w.k_pages[phys[np.arange(npg) % 5]]
    cache, t = device_cache(w)
    g = run_decode(w, cache, t)
    _check_decode(w, g, oracle_decode(w))
    # the kept set is closed under ties: a token is kept iff every token with the same key is
    for h in range(w.num_kv_heads):
        gt = set(unit_tokens(g, h).tolist())
        for tok in gt:
            twins = [tok % 16 + 16 * pg for pg in range(tok // 16 % 5, npg, 5)]
            assert all(x in gt for x in twins), (h, tok)


@pytest.mark.parametrize("name", ["C1", "C2"])
def test_decode_named_configs(name):
    w = make_config(name)
    _print_case(w.name)
    cache, t = device_cache(w)
    g = run_decode(w, cache, t)
    _check_decode(w, g, oracle_decode(w))


@pytest.mark.parametrize("name", ["C3", "C4"])
def test_decode_full_size_sampled_units(name):
    w = make_config(name)
    _print_case(w.name)
    cache, t = device_cache(w)
    g = run_decode(w, cache, t)
    rng = np.random.default_rng(0)
    U = w.batch * w.num_kv_heads
    units = [(int(u) // w.num_kv_heads, int(u) % w.num_kv_heads) for u in rng.choice(U, size=8, replace=False)]
    res = oracle_decode(w, units=units)
    _check_decode(w, g, res)
    # every unit's list is ascending, inside its sequence, and the CSR is consistent
    assert g["indptr"][0] == 0 and np.all(np.diff(g["indptr"]) >= 0)
    for u in range(U):
        tk = unit_tokens(g, u)
        assert np.all(np.diff(tk) > 0) and (tk.size == 0 or (tk[0] >= 0 and tk[-1] < w.seq_lens[u // w.num_kv_heads]))
    assert np.all(np.isfinite(g["out"]))


def test_fused_equals_split_and_is_deterministic():
    w = make_custom(**TINY[0])
    _print_case(w.name)
    cache, t = device_cache(w)
    a = run_decode(w, cache, t)
    b = run_decode(w, cache, t)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    # split path: select -> estimate -> attention
    ids, cnt = _select_pages_gpu(w, cache, t, w.keep_frac)
    U = w.batch * w.num_kv_heads
    pages = [ids[u, :cnt[u]] for u in range(U)]
    e = _estimate_on_pages(w, cache, t, pages, w.p)
    assert np.array_equal(e["indptr"], a["indptr"])
    n = int(a["indptr"][-1])
    assert np.array_equal(e["tokens"][:n], a["tokens"][:n])
    assert np.array_equal(e["thr"], a["thr"])
    maxsel = int(np.max(np.diff(e["indptr"])))
    maxcand = 16 * max_keep(w, w.keep_frac)
    out = torch.empty((w.batch, w.num_q_heads, 128), device="cuda")
    lse = torch.empty((w.batch, w.num_q_heads), device="cuda")
    ws = workspace(cache, maxcand)
    twl.sparse_attn(cache, t["q"], SM, torch.from_numpy(e["indptr"]).cuda(),
                    torch.from_numpy(e["tokens"][:max(n, 1)]).cuda(), maxcand, out, lse, ws)
    torch.cuda.synchronize()
    # same kept sets; the attention partitions the work differently (candidate-space chunks in the
    # fused call, list chunks in the split one), so the float32 sums agree to rounding
    assert np.allclose(out.cpu().numpy(), a["out"], rtol=1e-5, atol=1e-5)
    assert np.allclose(lse.cpu().numpy(), a["lse"], rtol=1e-5, atol=1e-5)
    _ = maxsel
    # the fused call without the optional kept-list output computes the same attention
    g = run_decode(w, cache, t, with_lists=False)
    assert np.array_equal(g["out"], a["out"]) and np.array_equal(g["lse"], a["lse"]) and np.array_equal(g["thr"], a["thr"])


# Decodes without the base selector (every page a candidate): thresholds and kept lists bitwise those
# of the split call over every page, and both match the oracle, for top-p and the top-k baseline.
# Shapes: C1 (one head, 4096 tokens), groups of 2 and 4 at 4096 / 2048 candidates with ragged and
# empty sequences, and one of 1024 candidates.
NO_SELECTOR = [
    dict(batch=2, num_q_heads=4, num_kv_heads=2, seq_lens=[3000, 1500], kind="outlier", seed=81),
    dict(batch=3, num_q_heads=8, num_kv_heads=2, seq_lens=[2000, 0, 1111], kind="temperature", seed=82),
    dict(batch=2, num_q_heads=4, num_kv_heads=1, seq_lens=[1000, 17], kind="planted", seed=83),
]


@pytest.mark.parametrize("cfg", [None] + NO_SELECTOR, ids=["C1", "g2_4096", "g4_2048", "g4_1024"])
def test_decode_without_selector_equals_split(cfg):
    w = make_config("C1") if cfg is None else make_custom(**cfg, keep_frac=1.0, p=0.9)
    _print_case(w.name + " every page a candidate")
    cache, t = device_cache(w)
    a = run_decode(w, cache, t, keep_frac=1.0)
    U = w.batch * w.num_kv_heads
    pages = [np.arange(-(-int(w.seq_lens[u // w.num_kv_heads]) // 16)) for u in range(U)]
    e = _estimate_on_pages(w, cache, t, pages, w.p)
    assert np.array_equal(e["thr"], a["thr"])
    assert np.array_equal(e["indptr"], a["indptr"])
    n = int(a["indptr"][-1])
    assert np.array_equal(e["tokens"][:n], a["tokens"][:n])
    _check_decode(w, a, oracle_decode(w, keep_frac=1.0))
    # the top-k baseline
    k = run_decode(w, cache, t, keep_frac=1.0, topk=40)
    _check_decode(w, k, oracle_decode(w, keep_frac=1.0, topk=40), topk=True)


@pytest.mark.parametrize("G", [1, 2, 8])
def test_group_sizes(G):
    w = make_custom(batch=2, num_q_heads=2 * G, num_kv_heads=2, seq_lens=[1200, 700], kind="outlier", seed=30 + G,
                    keep_frac=0.25, p=0.85)
    _print_case(w.name)
    cache, t = device_cache(w)
    g = run_decode(w, cache, t)
    _check_decode(w, g, oracle_decode(w))


# Group sizes other than 4 at the launch shapes large layers take: the estimate with four 64-candidate
# batches per block (units x candidates >= 2^19), the one-block top-p with 16 or 32 weights per thread
# (16384 / 32768 candidates), and the attention with 4, 8 and 16 sub-blocks of 16 tokens per wave
# (units x candidates of 2^18, 2^19 and 2^20; groups of 8 stop at 8).
LARGE_G = [
    dict(G=1, batch=4, kv=8, n=65536, seed=71),    # 32 units x 16384: estimate 4 batches, attention 8, top-p 16
    dict(G=2, batch=4, kv=8, n=131072, seed=72),   # 32 x 32768: attention 16, top-p 32
    dict(G=8, batch=4, kv=8, n=65536, seed=73),    # 32 x 16384: attention 8 (the most for groups of 8)
    dict(G=8, batch=2, kv=8, n=65536, seed=74),    # 16 x 16384: attention 4, estimate 2 batches
    dict(G=1, batch=2, kv=8, n=65536, seed=75),    # 16 x 16384: attention 4
]
LARGE_G_IDS = ["g1_nsb8", "g2_nsb16", "g8_nsb8", "g8_nsb4", "g1_nsb4"]


@pytest.mark.parametrize("case", LARGE_G, ids=LARGE_G_IDS)
def test_group_sizes_at_large_launch_shapes(case):
    G = case["G"]
    w = make_custom(batch=case["batch"], num_q_heads=G * case["kv"], num_kv_heads=case["kv"],
                    seq_lens=[case["n"]] * case["batch"], kind="outlier", seed=case["seed"], keep_frac=0.25, p=0.85,
                    name=f"large_g{G}_b{case['batch']}_n{case['n']}")
    _print_case(w.name)
    cache, t = device_cache(w)
    g = run_decode(w, cache, t)
    U = w.batch * w.num_kv_heads
    rng = np.random.default_rng(case["seed"])
    units = [(int(u) // w.num_kv_heads, int(u) % w.num_kv_heads) for u in rng.choice(U, size=3, replace=False)]
    res = oracle_decode(w, units=units)
    _check_decode(w, g, res)
    # per-head sets through the split path on the same pages
    ids, cnt = _select_pages_gpu(w, cache, t, w.keep_frac)
    for (b, h), r in res.items():
        assert np.array_equal(ids[b * w.num_kv_heads + h, :cnt[b * w.num_kv_heads + h]], r["pages"])
    e = _estimate_on_pages(w, cache, t, [ids[u, :cnt[u]] for u in range(U)], w.p)
    st = SetStats(w.name)
    _check_head_sets(w, e, res, w.p, st)
    st.report()
