"""The allocation-free decode entry point (twl_decode_noalloc) against twl_decode on the same inputs.

Both run the same kernels, the first on the library's static device scratch, the second on a
caller-given workspace, so every output must be bitwise equal.  Two calls in a row, the second with
a smaller input (so the scratch still holds the first call's contents), then the first again.
"""

import numpy as np
import pytest
import torch

import top_sparse_attention_int4_amd as twl
from gen import make_config, make_custom
from tests.gpu_helpers import device_cache, max_keep, workspace

pytestmark = pytest.mark.gpu


def _outputs(w, t, with_lists):
    B, Hq, U = w.batch, w.num_q_heads, w.batch * w.num_kv_heads
    maxcand = 16 * max_keep(w, w.keep_frac) if w.keep_frac < 1 else w.max_seq_len
    o = {"out": torch.full((B, Hq, 128), float("nan"), device="cuda"),
         "lse": torch.full((B, Hq), float("nan"), device="cuda"),
         "thr": torch.full((B, Hq), float("nan"), device="cuda")}
    if with_lists:
        o["indptr"] = torch.full((U + 1,), -7, dtype=torch.int32, device="cuda")
        o["tokens"] = torch.full((max(U * maxcand, 1),), -7, dtype=torch.int32, device="cuda")
    return o, maxcand


def _run(w, cache, t, noalloc, with_lists=True):
    o, maxcand = _outputs(w, t, with_lists)
    kw = dict(p=w.p, keep_frac=w.keep_frac, out=o["out"], lse=o["lse"], threshold=o["thr"],
              sel_indptr=o.get("indptr"), sel_tokens=o.get("tokens"))
    if noalloc:
        twl.decode_noalloc(cache, t["q"], **kw)
    else:
        twl.decode(cache, t["q"], ws=workspace(cache, maxcand), **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}


def _same(a, b):
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k


def test_noalloc_decode_equals_decode_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = make_config("C2")
    small = make_custom(batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=[1500, 33], kind="outlier", seed=17,
                        keep_frac=0.25, p=0.85)
    print("[case] C2 then a two-sequence 1500/33-token layer", flush=True)
    cb, tb = device_cache(big)
    cs, ts = device_cache(small)
    first = _run(big, cb, tb, noalloc=True)
    _same(first, _run(big, cb, tb, noalloc=False))
    second = _run(small, cs, ts, noalloc=True)
    _same(second, _run(small, cs, ts, noalloc=False))
    # the timed form (no token list) and a repeat of the first call over the second's leftovers
    _same(_run(small, cs, ts, noalloc=True, with_lists=False), _run(small, cs, ts, noalloc=False, with_lists=False))
    _same(_run(big, cb, tb, noalloc=True), first)
    assert np.all(np.isfinite(first["out"])) and np.all(np.isfinite(second["out"]))


def test_noalloc_decode_refuses_a_step_beyond_its_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = make_custom(batch=1, num_q_heads=4, num_kv_heads=1, seq_lens=[600], seed=3, keep_frac=0.25, p=0.9)
    print("[case] refusal of a step beyond the scratch", flush=True)
    cache, t = device_cache(w)
    # a cache description claiming 4M-token sequences needs far more workspace than the scratch holds
    c = cache.struct()
    saved = (c.max_pages_per_seq, c.max_seq_len)
    c.max_pages_per_seq, c.max_seq_len = 262144, 262144 * 16
    try:
        with pytest.raises(twl.TwlError) as e:
            twl.decode_noalloc(cache, t["q"], p=0.9, keep_frac=1.0, out=torch.empty((1, 4, 128), device="cuda"))
        assert e.value.status == twl.TWL_EWORKSPACE
    finally:
        c.max_pages_per_seq, c.max_seq_len = saved
