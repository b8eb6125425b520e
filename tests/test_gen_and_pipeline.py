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
