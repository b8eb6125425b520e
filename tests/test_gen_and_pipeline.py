"""Seeded generator checks and oracle pipeline invariants (CPU only)."""

import math
import os

import numpy as np
import pytest

from gen import CONFIGS, make_config, make_custom
from oracle import attention, numerics, pipeline, topp


def test_generator_is_deterministic_and_paged_consistently():
    a = make_custom(batch=3, num_q_heads=8, num_kv_heads=2, seq_lens=[100, 16, 33], kind="outlier", seed=9)
    b = make_custom(batch=3, num_q_heads=8, num_kv_heads=2, seq_lens=[100, 16, 33], kind="outlier", seed=9)
    assert np.array_equal(a.k_pages, b.k_pages) and np.array_equal(a.q, b.q)
    # every used physical page appears exactly once
    used = np.concatenate([a.page_table[i, :-(-int(n) // 16)] for i, n in enumerate(a.seq_lens)])
    assert np.array_equal(np.sort(used), np.arange(a.num_phys_pages))
    # slots past the end of a sequence hold the fill value
    last = a.page_table[0, 6]
    assert np.all(numerics.bf16_to_f32(a.k_pages[last, :, 4:]) == 5.0)
    assert a.logical("k", 2).shape == (33, 2, 128)


def test_workload_structures():
    w = make_custom(batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=[2000, 1500], kind="planted", seed=1,
                    planted_per_head=16)
    for (b, hq), pos in w.meta["planted_positions"].items():
        h = hq // 4
        k = numerics.bf16_to_f32(w.logical("k", b)[pos, h]).astype(np.float64)
        q = numerics.bf16_to_f32(w.q[b, hq]).astype(np.float64)
        cos = (k @ q) / (np.linalg.norm(k, axis=1) * np.linalg.norm(q))
        assert np.all(np.abs(cos - 0.6) < 0.01)
    w = make_custom(batch=1, num_q_heads=4, num_kv_heads=1, seq_lens=[64], kind="temperature", seed=2)
    assert w.meta["beta"].min() >= 0.05 and w.meta["beta"].max() <= 3.5
    assert set(CONFIGS) == {"C1", "C2", "C3", "C4", "C5"}


def test_named_small_config_shapes():
    w = make_config("C1")
    assert (w.batch, w.num_q_heads, w.num_kv_heads, w.max_seq_len) == (1, 1, 1, 4096)
    w = make_config("C2", seq_len=1000)
    assert (w.num_q_heads, w.num_kv_heads, w.seq_lens.tolist()) == (32, 8, [1000])


@pytest.mark.parametrize("kind,keep", [("normal", 0.25), ("outlier", 0.5), ("temperature", 0.25), ("peaked", 1.0)])
def test_pipeline_invariants(kind, keep):
    w = make_custom(batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=[777, 300], kind=kind, seed=4,
                    keep_frac=keep, p=0.85)
    res = pipeline.decode(w)
    for (b, h), r in res.items():
        n = int(w.seq_lens[b])
        npg = -(-n // 16)
        assert len(r["pages"]) == max(1, min(npg, math.ceil(keep * npg)))
        assert np.all(r["candidates"] < n)
        for hd in r["heads"]:
            assert math.fsum(hd["W"][hd["topp"]["sel"]]) >= 0.85
            assert set(hd["tokens"].tolist()) <= set(r["union"].tolist())
        assert np.all(np.diff(r["union"]) > 0)
        assert np.all(np.isfinite(r["out"]))


def test_pipeline_empty_sequence():
    w = make_custom(batch=2, num_q_heads=4, num_kv_heads=1, seq_lens=[0, 5], seed=1, keep_frac=0.25)
    res = pipeline.decode(w)
    assert res[(0, 0)]["union"].size == 0 and np.all(res[(0, 0)]["out"] == 0)
    assert res[(1, 0)]["union"].size >= 1


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _torch_attention(qbits_g, kbits, vbits, sm, mask=None):
    """float64 torch scaled-dot-product attention of G query heads over n tokens (optional boolean
    mask [G][n] of the tokens each head may attend to), and the log-sum-exp of its scores."""
    import torch
    q = torch.from_numpy(numerics.bf16_to_f32(qbits_g).astype(np.float64))[None, :, None, :]   # [1][G][1][d]
    k = torch.from_numpy(numerics.bf16_to_f32(kbits).astype(np.float64))[None, None].expand(1, q.shape[1], -1, -1)
    v = torch.from_numpy(numerics.bf16_to_f32(vbits).astype(np.float64))[None, None].expand(1, q.shape[1], -1, -1)
    am = None if mask is None else torch.from_numpy(mask)[None, :, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=am, scale=sm)[0, :, 0]
    s = (q[0, :, 0] @ k[0, 0].T) * sm
    if mask is not None:
        s = s.masked_fill(~torch.from_numpy(mask), -math.inf)
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("G", [1, 4, 8])
def test_pipeline_everything_kept_is_dense_attention(G):
    # every page a candidate and p = 1: every head keeps every token, so each head's output is plain
    # attention over the whole sequence (torch's scaled-dot-product attention, float64)
    w = make_custom(batch=2, num_q_heads=2 * G, num_kv_heads=2, seq_lens=[300, 77], kind="outlier", seed=40 + G,
                    keep_frac=1.0, p=1.0)
    sm = float(np.float32(1 / math.sqrt(128)))
    res = pipeline.decode(w)
    for (b, h), r in res.items():
        n = int(w.seq_lens[b])
        assert r["union"].tolist() == list(range(n))
        o, lse = _torch_attention(w.q[b, h * G:(h + 1) * G], w.logical("k", b)[:, h], w.logical("v", b)[:, h], sm)
        assert np.allclose(r["out"], o, rtol=0, atol=1e-12)
        assert np.allclose(r["lse"], lse, rtol=1e-13, atol=0)


def _grid_k_pages(w, seed):
    """Replace every key row by one that sits on its own 4-bit min/max grid (reconstructed exactly
    by the quantisation, so the INT4 estimate equals the exact bf16 logit)."""
    rng = np.random.default_rng(seed)
    shp = w.k_pages.shape[:-1]
    codes = rng.integers(0, 16, size=shp + (4, 32))
    codes[..., 0], codes[..., 1] = 0, 15
    s = 2.0 ** rng.integers(-4, -1, size=shp + (4,))
    m = rng.integers(-15, 240, size=shp + (4,))
    x = (codes + m[..., None]) * s[..., None]
    w.k_pages[...] = numerics.f32_to_bf16_bits(x.reshape(shp + (128,)).astype(np.float32))


@pytest.mark.parametrize("G,p", [(1, 0.9), (4, 0.85), (8, 0.7)])
def test_pipeline_on_grid_keys_is_top_p_of_the_exact_weights(G, p):
    # keys on the INT4 grid make the estimate exact, so with every page a candidate each head keeps
    # the minimal top-p set of its exact attention weights (found here with torch: softmax, sort,
    # cumulative sum), the group attends over the union, and the output is masked attention
    import torch
    w = make_custom(batch=2, num_q_heads=2 * G, num_kv_heads=2, seq_lens=[500, 130], kind="temperature",
                    seed=50 + G, keep_frac=1.0, p=p)
    _grid_k_pages(w, 60 + G)
    sm = float(np.float32(1 / math.sqrt(128)))
    res = pipeline.decode(w)
    for (b, h), r in res.items():
        n = int(w.seq_lens[b])
        kb, vb = w.logical("k", b)[:, h], w.logical("v", b)[:, h]
        K = torch.from_numpy(numerics.bf16_to_f32(kb).astype(np.float64))
        mask = np.zeros((G, n), bool)
        for j in range(G):
            qv = torch.from_numpy(numerics.bf16_to_f32(w.q[b, h * G + j]).astype(np.float64))
            Wt = torch.softmax((K @ qv) * sm, dim=0)
            order = torch.argsort(-Wt, stable=True)
            cum = torch.cumsum(Wt[order], 0)
            kstar = int(torch.searchsorted(cum, torch.tensor([p], dtype=torch.float64))[0]) + 1
            want = np.sort(order[:kstar].numpy())
            got = r["heads"][j]["tokens"]
            # identical away from near-ties and prefix masses within rounding of p
            res_j = r["heads"][j]["topp"]
            diff = np.setxor1d(got, want)
            assert np.all(np.isin(diff, np.union1d(res_j["amb_i"], res_j["amb_ii"]))), (b, h, j)
            mask[j, got] = True
        union = mask.any(0)
        assert r["union"].tolist() == np.nonzero(union)[0].tolist()
        o, lse = _torch_attention(w.q[b, h * G:(h + 1) * G], kb, vb, sm, np.broadcast_to(union, (G, n)).copy())
        assert np.allclose(r["out"], o, rtol=0, atol=1e-12)
        assert np.allclose(r["lse"], lse, rtol=1e-13, atol=0)
