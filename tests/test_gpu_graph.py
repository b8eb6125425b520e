"""The fused decode captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

The decode enqueues kernels only (no memsets, no allocation, no synchronisation; every kernel
initialises the workspace words it reads), so a captured step must give, on every replay, bitwise
the outputs of the same step run eagerly.  Each replay is separated from the next by the program's
own eager decodes on other inputs and a synchronisation, and every replay is checked."""

import numpy as np
import pytest
import torch

import top_sparse_attention_int4_amd as twl
from gen import make_config, make_custom
from tests.gpu_helpers import device_cache, max_keep, workspace

pytestmark = pytest.mark.gpu


def _buffers(w, maxcand):
    B, Hq, U = w.batch, w.num_q_heads, w.batch * w.num_kv_heads
    return {"out": torch.full((B, Hq, 128), float("nan"), device="cuda"),
            "lse": torch.full((B, Hq), float("nan"), device="cuda"),
            "thr": torch.full((B, Hq), float("nan"), device="cuda"),
            "indptr": torch.full((U + 1,), -7, dtype=torch.int32, device="cuda"),
            "tokens": torch.full((max(U * maxcand, 1),), -7, dtype=torch.int32, device="cuda")}


def _decode(w, cache, t, o, ws, lists):
    twl.decode(cache, t["q"], p=w.p, keep_frac=w.keep_frac, out=o["out"], lse=o["lse"], threshold=o["thr"],
               sel_indptr=o["indptr"] if lists else None, sel_tokens=o["tokens"] if lists else None, ws=ws)


def _host(o):
    return {k: v.cpu().numpy() for k, v in o.items()}


@pytest.mark.parametrize("lists", [False, True], ids=["no_lists", "lists"])
def test_captured_decode_replays_bitwise(lists):
    w = make_config("C2")
    other = make_custom(batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=[1500, 700], kind="outlier", seed=31,
                        keep_frac=0.25, p=0.85)
    print(f"[case] C2 decode captured in a graph, lists={lists}", flush=True)
    cache, t = device_cache(w)
    c2, t2 = device_cache(other)
    maxcand = 16 * max_keep(w, w.keep_frac)
    ws = workspace(cache, maxcand)
    ws2 = workspace(c2, 16 * max_keep(other, other.keep_frac))
    eager = _buffers(w, maxcand)
    _decode(w, cache, t, eager, ws, lists)
    torch.cuda.synchronize()
    want = _host(eager)
    graph_out = _buffers(w, maxcand)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _decode(w, cache, t, graph_out, ws, lists)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _decode(w, cache, t, graph_out, ws, lists)
    torch.cuda.synchronize()
    scratch = _buffers(other, 16 * max_keep(other, other.keep_frac))
    for r in range(4):
        for v in graph_out.values():
            v.fill_(-3)  # every replay rewrites what it is checked on
        g.replay()
        torch.cuda.synchronize()
        got = _host(graph_out)
        for k in want:
            if k in ("indptr", "tokens") and not lists:
                continue
            if k == "tokens":
                n = int(want["indptr"][-1])
                assert np.array_equal(got[k][:n], want[k][:n]), (r, k)
            else:
                assert np.array_equal(got[k], want[k], equal_nan=True), (r, k)
        # the program's own eager work between replays, on other inputs and another workspace
        _decode(other, c2, t2, scratch, ws2, True)
        torch.cuda.synchronize()
