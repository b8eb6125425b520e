"""CPU checks of the C ABI: the library loads without a GPU, exports every symbol the header
declares, and rejects invalid arguments with the documented status before any HIP call."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def twl():
    import top_sparse_attention_int4_amd as t
    if not os.path.exists(t.LIB_PATH):
        from top_sparse_attention_int4_amd import build
        build.build()
    t.lib()
    return t


def _declared():
    src = open(os.path.join(ROOT, "include", "twl.h")).read()
    return sorted(set(re.findall(r"^\s*(?:twl_status|size_t|const char\*|int32_t)\s+(twl_\w+)\s*\(", src, re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["twl_quantize_k", "twl_select_pages", "twl_estimate_topp", "twl_sparse_attn", "twl_decode",
              "twl_decode_profiled", "twl_select_clusters_topp", "twl_decode_clusters", "twl_workspace_bytes",
              "twl_status_str", "twl_version", "twl_keep_pages", "twl_decode_noalloc"]:
        assert n in names


def test_library_exports_every_declared_symbol(twl):
    L = twl.lib()
    for n in _declared():
        assert hasattr(L, n), n


def _fake_cache(twl, **kw):
    fake = ctypes.c_void_p(0x10000)
    c = twl.CacheC(1, 32, 8, 128, 16, 32, 2048, 2048, 32768, fake, fake, fake, fake, fake, fake, fake)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_status_strings(twl):
    for s in range(5):
        assert twl.status_str(s).startswith("TWL_")
    assert "gfx950" in twl.version()


def test_version_names_the_source_hash(twl):
    # the loaded library was built from this tree's kernel and ABI sources (the binding refuses others)
    from top_sparse_attention_int4_amd.build import source_hash
    assert twl.version().endswith(" src " + source_hash())


def test_keep_pages_rule(twl):
    # clamp(ceil(fp32(keep) * fp32(P)), 1, P): the budget of the base selector, computed in the library
    import numpy as np
    for P, kf in [(2048, 0.25), (8192, 0.25), (7, 0.3), (1, 0.01), (5, 1.0), (5, 3.0), (3, 1e-9)]:
        want = max(1, min(P, int(np.ceil(min(np.float32(kf) * np.float32(P), np.float32(P))))))
        assert twl.keep_count(P, kf) == want, (P, kf)
    assert twl.keep_count(0, 0.25) == 0
    assert twl.lib().twl_keep_pages(10, float("nan")) == -1
    assert twl.lib().twl_keep_pages(10, 0.0) == -1


def test_workspace_bytes(twl):
    L = twl.lib()
    c = _fake_cache(twl)
    a = L.twl_workspace_bytes(ctypes.byref(c), 8192)
    b = L.twl_workspace_bytes(ctypes.byref(c), 32768)
    assert 0 < a < b
    assert a % 256 == 0
    assert L.twl_workspace_bytes(None, 8192) == 0
    bad = _fake_cache(twl, head_dim=64)
    assert L.twl_workspace_bytes(ctypes.byref(bad), 8192) == 0


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, 2), ("page_size", 32, 2), ("quant_group", 64, 2), ("num_kv_heads", 5, 1),
    ("num_kv_heads", 2, 2), ("batch", 0, 1), ("max_seq_len", 2048 * 16 + 1, 1), ("page_table", None, 1),
    ("key_bits", 3, 2), ("key_bits", 16, 2), ("key_bits", -4, 2),
])
def test_decode_rejects_bad_cache(twl, field, value, status):
    L = twl.lib()
    c = _fake_cache(twl, **{field: value})
    prm = twl.ParamsC(0.85, 0.25, 0.088, 32)
    fake = ctypes.c_void_p(0x10000)
    st = L.twl_decode(ctypes.byref(c), fake, ctypes.byref(prm), fake, None, None, None, None, 0, fake, 1 << 40, None)
    assert st == status


@pytest.mark.parametrize("p,kf,iters,status", [
    (0.0, 0.25, 32, 1), (1.5, 0.25, 32, 1), (float("nan"), 0.25, 32, 1), (0.85, 0.0, 32, 1),
    (0.85, float("inf"), 32, 1), (0.85, 0.25, 0, 1), (0.85, 0.25, 65, 1),
])
def test_decode_rejects_bad_params(twl, p, kf, iters, status):
    L = twl.lib()
    c = _fake_cache(twl)
    prm = twl.ParamsC(p, kf, 0.088, iters)
    fake = ctypes.c_void_p(0x10000)
    st = L.twl_decode(ctypes.byref(c), fake, ctypes.byref(prm), fake, None, None, None, None, 0, fake, 1 << 40, None)
    assert st == status


@pytest.mark.parametrize("topk,headwise,status", [(-1, 0, 1), (0, 2, 1), (0, -1, 1)])
def test_decode_rejects_bad_baseline_params(twl, topk, headwise, status):
    L = twl.lib()
    c = _fake_cache(twl)
    prm = twl.ParamsC(0.85, 0.25, 0.088, 32, topk, headwise)
    fake = ctypes.c_void_p(0x10000)
    st = L.twl_decode(ctypes.byref(c), fake, ctypes.byref(prm), fake, None, None, None, None, 0, fake, 1 << 40, None)
    assert st == status


def test_decode_rejects_misaligned_query(twl):
    L = twl.lib()
    c = _fake_cache(twl)
    prm = twl.ParamsC(0.85, 0.25, 0.088, 32)
    fake = ctypes.c_void_p(0x10000)
    st = L.twl_decode(ctypes.byref(c), ctypes.c_void_p(0x10004), ctypes.byref(prm), fake, None, None, None, None, 0,
                      fake, 1 << 40, None)
    assert st == 1


def test_workspace_and_capacity_checks(twl):
    L = twl.lib()
    c = _fake_cache(twl)
    prm = twl.ParamsC(0.85, 0.25, 0.088, 32)
    fake = ctypes.c_void_p(0x10000)
    need = L.twl_workspace_bytes(ctypes.byref(c), 16 * 512)
    # too small, NULL, misaligned workspace
    assert L.twl_decode(ctypes.byref(c), fake, ctypes.byref(prm), fake, None, None, None, None, 0, fake, need - 1, None) == 3
    assert L.twl_decode(ctypes.byref(c), fake, ctypes.byref(prm), fake, None, None, None, None, 0, None, need, None) == 3
    assert L.twl_decode(ctypes.byref(c), fake, ctypes.byref(prm), fake, None, None, None, None, 0,
                        ctypes.c_void_p(0x10010), need, None) == 3
    # CSR outputs need both pointers and enough capacity
    assert L.twl_decode(ctypes.byref(c), fake, ctypes.byref(prm), fake, None, None, fake, None, 0, fake, need, None) == 1
    assert L.twl_decode(ctypes.byref(c), fake, ctypes.byref(prm), fake, None, None, fake, fake, 8 * 8192 - 1, fake,
                        need, None) == 1


def test_split_entry_points_validate(twl):
    L = twl.lib()
    c = _fake_cache(twl)
    fake = ctypes.c_void_p(0x10000)
    assert L.twl_quantize_k(ctypes.byref(c), None, fake, 16, None) == 1
    assert L.twl_quantize_k(ctypes.byref(c), fake, fake, -1, None) == 1
    assert L.twl_select_pages(ctypes.byref(c), fake, 0.25, 511, fake, fake, fake, 1 << 40, None) == 1  # needs 512
    cand = twl.CandC(fake, fake, fake, 4)  # both pages and ranges
    assert L.twl_estimate_topp(ctypes.byref(c), fake, 0.088, 0.9, 32, ctypes.byref(cand), fake, None, None, 0,
                               fake, fake, 1 << 30, fake, 1 << 40, None) == 1
    cand = twl.CandC(fake, None, None, 4)  # count missing
    assert L.twl_estimate_topp(ctypes.byref(c), fake, 0.088, 0.9, 32, ctypes.byref(cand), fake, None, None, 0,
                               fake, fake, 1 << 30, fake, 1 << 40, None) == 1
    assert L.twl_sparse_attn(ctypes.byref(c), fake, 0.088, fake, fake, -1, fake, None, fake, 1 << 40, None) == 1
    assert L.twl_select_clusters_topp(ctypes.byref(c), fake, 0.088, 0.0, 32, fake, fake, fake, 64, fake, fake,
                                      fake, 1 << 40, None) == 1
    assert L.twl_select_clusters_topp(ctypes.byref(c), fake, 0.088, 0.95, 32, fake, fake, fake, 65537, fake, fake,
                                      fake, 1 << 40, None) == 2


def test_workspace_grows_into_the_wide_top_p():
    """Candidate capacities above 65536 per unit use the multi-pass top-p and its extra state."""
    import top_sparse_attention_int4_amd as t
    L = t.lib()
    c = _fake_cache(t, max_pages_per_seq=1 << 15, num_phys_pages=1 << 15, max_seq_len=1 << 19)
    a = L.twl_workspace_bytes(ctypes.byref(c), 65536)
    b = L.twl_workspace_bytes(ctypes.byref(c), 65537)
    assert b > a * 65537 / 65536  # the wide state comes on top of the per-candidate buffers


def test_decode_clusters_validates():
    import top_sparse_attention_int4_amd as t
    L = t.lib()
    c = _fake_cache(t)
    fake = ctypes.c_void_p(0x10000)
    prm = t.ParamsC(0.9, 1.0, 0.088, 32)
    args = lambda p1, ncl, ws_bytes: (ctypes.byref(c), fake, ctypes.byref(prm), p1, fake, fake, fake, ncl, fake, None,
                                      None, None, None, 0, fake, ws_bytes, None, None)
    assert L.twl_decode_clusters(*args(0.0, 4096, 1 << 40)) == 1      # p1 out of range
    assert L.twl_decode_clusters(*args(0.95, 0, 1 << 40)) == 1        # no clusters
    assert L.twl_decode_clusters(*args(0.95, 16385, 1 << 40)) == 2    # more than half the capacity
    need = L.twl_workspace_bytes(ctypes.byref(c), 32768)
    assert L.twl_decode_clusters(*args(0.95, 4096, need - 256)) == 3  # workspace too small
    nulls = (ctypes.byref(c), fake, ctypes.byref(prm), 0.95, None, fake, fake, 4096, fake, None, None, None, None, 0,
             fake, 1 << 40, None, None)
    assert L.twl_decode_clusters(*nulls) == 1                         # centroids missing
    prm.topk = 8                                                      # baselines are for the page path only
    assert L.twl_decode_clusters(*args(0.95, 4096, 1 << 40)) == 2
    prm.topk, prm.headwise = 0, 1
    assert L.twl_decode_clusters(*args(0.95, 4096, 1 << 40)) == 2


def test_cluster_approx_entry_points_validate():
    import top_sparse_attention_int4_amd as t
    L = t.lib()
    c = _fake_cache(t)
    fake = ctypes.c_void_p(0x10000)
    assert L.twl_cluster_value_means(ctypes.byref(c), fake, fake, 0, fake, None) == 1       # no clusters
    assert L.twl_cluster_value_means(ctypes.byref(c), None, fake, 64, fake, None) == 1      # csize missing
    ok = (ctypes.byref(c), fake, 0.088, 0.95, 32, fake, fake, 64, fake, fake, fake, fake, 1 << 40, None)
    bad_p1 = ok[:3] + (1.5,) + ok[4:]
    assert L.twl_cluster_approx_unkept(*bad_p1) == 1
    no_lse = ok[:10] + (None,) + ok[11:]
    assert L.twl_cluster_approx_unkept(*no_lse) == 1
    small_ws = ok[:12] + (256,) + ok[13:]
    assert L.twl_cluster_approx_unkept(*small_ws) == 3


def test_noalloc_decode_rejects_steps_beyond_its_scratch(twl):
    # validated on the host before any HIP call: a step whose workspace exceeds the static scratch,
    # and the usual argument errors, are refused without touching a GPU
    L = twl.lib()
    fake = ctypes.c_void_p(0x10000)
    prm = twl.ParamsC(0.9, 1.0, 0.088, 32, 0, 0)
    big = twl.CacheC(4, 32, 8, 128, 16, 32, 16384, 65536, 262144, fake, fake, fake, fake, fake, fake, fake, 4)
    need = L.twl_workspace_bytes(ctypes.byref(big), 262144)
    assert need > twl.NOALLOC_SCRATCH_BYTES
    r = L.twl_decode_noalloc(ctypes.byref(big), fake, ctypes.byref(prm), fake, None, None, None, None, 0, None)
    assert r == twl.TWL_EWORKSPACE
    small = _fake_cache(twl)
    bad = twl.ParamsC(1.5, 0.25, 0.088, 32, 0, 0)
    assert L.twl_decode_noalloc(ctypes.byref(small), fake, ctypes.byref(bad), fake, None, None, None, None, 0,
                                None) == twl.TWL_EINVAL
    assert L.twl_decode_noalloc(ctypes.byref(small), ctypes.c_void_p(0x10001), ctypes.byref(prm), fake, None, None,
                                None, None, 0, None) == twl.TWL_EINVAL
