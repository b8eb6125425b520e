"""Python binding of libtwl: top-p sparse decode attention with an INT4 K estimate for MI355X.

This module only marshals arguments: it turns torch device tensors into the plain pointers and
sizes of the C ABI declared in ``include/twl.h`` and raises on a non-OK status.  Every step of the
decode path runs in the HIP kernels of ``_lib/libtwl.so``; there is no Python or CPU fallback.  If
the library is missing, importing the functions raises.

Names follow the C ABI: ``quantize_k``, ``select_pages``, ``estimate_topp``, ``sparse_attn``,
``decode``, ``decode_profiled``, ``select_clusters_topp``, ``workspace_bytes``.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = [
    "LIB_PATH", "TwlError", "PagedCache", "lib", "workspace_bytes", "quantize_k", "select_pages",
    "estimate_topp", "sparse_attn", "decode", "decode_profiled", "select_clusters_topp", "status_str",
    "version", "keep_count", "NUM_STAGES", "STAGE_NAMES", "DEFAULT_SM_SCALE", "decode_clusters",
    "cluster_value_means", "cluster_approx_unkept", "decode_noalloc", "NOALLOC_SCRATCH_BYTES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libtwl.so")
NUM_STAGES = 6
STAGE_NAMES = ("page_score", "page_select", "estimate", "topp_union", "attn_splitk", "attn_merge")
DEFAULT_SM_SCALE = float(torch.tensor(1.0 / math.sqrt(128.0), dtype=torch.float32))

TWL_OK, TWL_EINVAL, TWL_EUNSUPPORTED, TWL_EWORKSPACE, TWL_EHIP = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 64 << 20  # TWL_NOALLOC_SCRATCH_BYTES

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float


class TwlError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class CacheC(ctypes.Structure):
    _fields_ = [
        ("batch", _i32), ("num_q_heads", _i32), ("num_kv_heads", _i32), ("head_dim", _i32),
        ("page_size", _i32), ("quant_group", _i32), ("max_pages_per_seq", _i32),
        ("num_phys_pages", _i32), ("max_seq_len", _i32),
        ("page_table", _p), ("seq_lens", _p), ("k", _p), ("v", _p),
        ("k4", _p), ("k4_meta", _p), ("kbound", _p), ("key_bits", _i32),
    ]


class CandC(ctypes.Structure):
    _fields_ = [("page_ids", _p), ("ranges", _p), ("count", _p), ("max_items", _i32)]


class ParamsC(ctypes.Structure):
    _fields_ = [("p", _f32), ("keep_frac", _f32), ("sm_scale", _f32), ("iters", _i32), ("topk", _i32),
                ("headwise", _i32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtwl.so (built in-tree by ``build.py``); raise if it is missing or was built from other
    sources than the ones in this tree (its version string carries their hash)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libtwl.so not found at {LIB_PATH}; build it with "
                          "`python -m top_sparse_attention_int4_amd.build` (no CPU fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    from .build import source_hash
    L.twl_version.restype = ctypes.c_char_p
    L.twl_version.argtypes = []
    ver = L.twl_version().decode()
    want = source_hash()
    if not ver.endswith(" src " + want):
        raise ImportError(f"{LIB_PATH} ({ver}) was not built from the sources in this tree (src {want}); "
                          "rebuild it with `python -m top_sparse_attention_int4_amd.build`")
    C = ctypes.POINTER(CacheC)
    sig = {
        "twl_workspace_bytes": (ctypes.c_size_t, [C, _i64]),
        "twl_quantize_k": (_i32, [C, _p, _p, _i32, _p]),
        "twl_select_pages": (_i32, [C, _p, _f32, _i32, _p, _p, _p, ctypes.c_size_t, _p]),
        "twl_estimate_topp": (_i32, [C, _p, _f32, _f32, _i32, ctypes.POINTER(CandC), _p, _p, _p, _i32, _p, _p,
                                     _i64, _p, ctypes.c_size_t, _p]),
        "twl_sparse_attn": (_i32, [C, _p, _f32, _p, _p, _i32, _p, _p, _p, ctypes.c_size_t, _p]),
        "twl_decode": (_i32, [C, _p, ctypes.POINTER(ParamsC), _p, _p, _p, _p, _p, _i64, _p, ctypes.c_size_t, _p]),
        "twl_decode_profiled": (_i32, [C, _p, ctypes.POINTER(ParamsC), _p, _p, _p, _p, _p, _i64, _p,
                                       ctypes.c_size_t, _p, ctypes.POINTER(_p)]),
        "twl_decode_noalloc": (_i32, [C, _p, ctypes.POINTER(ParamsC), _p, _p, _p, _p, _p, _i64, _p]),
        "twl_select_clusters_topp": (_i32, [C, _p, _f32, _f32, _i32, _p, _p, _p, _i32, _p, _p, _p,
                                            ctypes.c_size_t, _p]),
        "twl_decode_clusters": (_i32, [C, _p, ctypes.POINTER(ParamsC), _f32, _p, _p, _p, _i32, _p, _p, _p, _p, _p,
                                       _i64, _p, ctypes.c_size_t, _p, ctypes.POINTER(_p)]),
        "twl_cluster_value_means": (_i32, [C, _p, _p, _i32, _p, _p]),
        "twl_cluster_approx_unkept": (_i32, [C, _p, _f32, _f32, _i32, _p, _p, _i32, _p, _p, _p, _p, ctypes.c_size_t,
                                             _p]),
        "twl_status_str": (ctypes.c_char_p, [_i32]),
        "twl_version": (ctypes.c_char_p, []),
        "twl_keep_pages": (_i32, [_i32, _f32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().twl_status_str(int(status)).decode()


def version() -> str:
    return lib().twl_version().decode()


def _check(status: int) -> None:
    if status != TWL_OK:
        raise TwlError(status, status_str(status))


def _host_mapped_ptr(t: torch.Tensor) -> ctypes.c_void_p:
    """Device address of a pinned host tensor (the HIP runtime's mapping of that host memory)."""
    fn = lib().hipHostGetDevicePointer
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
    out = ctypes.c_void_p()
    if fn(ctypes.byref(out), ctypes.c_void_p(t.data_ptr()), 0) != 0 or not out.value:
        raise ValueError("the pinned host tensor has no device mapping")
    return out


def _ptr(t: Optional[torch.Tensor], allow_host: bool = False):
    if t is None:
        return None
    if allow_host and t.device.type == "cpu":
        if not t.is_pinned():
            raise ValueError("host-resident K/V must be pinned (pin_memory=True)")
        if not t.is_contiguous():
            raise ValueError("libtwl takes contiguous tensors")
        return _host_mapped_ptr(t)
    if t.device.type != "cuda":
        raise ValueError("libtwl takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libtwl takes contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def keep_count(num_pages: int, keep_frac: float) -> int:
    """Pages the base selector keeps for a sequence of ``num_pages`` pages (``twl_keep_pages``)."""
    k = int(lib().twl_keep_pages(int(num_pages), float(keep_frac)))
    if k < 0:
        raise TwlError(TWL_EINVAL, "keep_frac must be finite and > 0")
    return k


class PagedCache:
    """Device tensors of one layer's paged KV cache and its INT4 shadow.

    ``k_pages``/``v_pages``: bf16 (or their uint16 bits viewed as int16) [P][Hkv][16][128];
    ``page_table`` int32 [B][max_pages]; ``seq_lens`` int32 [B].  The key codes (``key_bits`` wide:
    4, or 2 / 8 for the estimator's precision ablation), fp16 scale/zero and page bounds are allocated
    here by (sequence, logical page) -- ``k4`` [B][max_pages][Hkv][16][16*key_bits], ``k4_meta``
    [B][max_pages][Hkv][16][4][2], ``kbound`` [B][max_pages][Hkv][4][2][32] (channel quarter, min/max,
    channel) -- and filled by
    :func:`quantize_k`.  ``k_pages``/``v_pages`` may instead be pinned host tensors
    (the offloading scenario): the kernels then read them over PCIe through the runtime's mapping of
    that memory, while the codes, bounds and everything else stay in device memory.
    """

    def __init__(self, k_pages: torch.Tensor, v_pages: torch.Tensor, page_table: torch.Tensor,
                 seq_lens: torch.Tensor, num_q_heads: int, max_seq_len: Optional[int] = None,
                 key_bits: int = 4):
        P, Hkv, S, D = k_pages.shape
        if (S, D) != (16, 128) or v_pages.shape != k_pages.shape:
            raise ValueError("k/v pages must be [P][Hkv][16][128]")
        dev = page_table.device
        if dev.type != "cuda":
            raise ValueError("page_table must be a device tensor")
        self.k = k_pages
        self.v = v_pages
        self.page_table = page_table
        self.seq_lens = seq_lens
        self.batch = int(page_table.shape[0])
        self.max_pages = int(page_table.shape[1])
        self.num_q_heads = int(num_q_heads)
        self.num_kv_heads = int(Hkv)
        self.num_phys_pages = int(P)
        self.max_seq_len = int(max_seq_len if max_seq_len is not None else self.max_pages * 16)
        if key_bits not in (2, 4, 8):
            raise ValueError("key_bits must be 2, 4 or 8")
        self.key_bits = int(key_bits)
        B, MP = self.batch, self.max_pages
        self.k4 = torch.zeros((B, MP, Hkv, 16, 16 * key_bits), dtype=torch.uint8, device=dev)
        self.k4_meta = torch.zeros((B, MP, Hkv, 16, 4, 2), dtype=torch.int16, device=dev)
        self.kbound = torch.zeros((B, MP, Hkv, 4, 2, 32), dtype=torch.int16, device=dev)
        self._c = CacheC(self.batch, self.num_q_heads, self.num_kv_heads, 128, 16, 32, self.max_pages,
                         self.num_phys_pages, self.max_seq_len, _ptr(page_table), _ptr(seq_lens),
                         _ptr(k_pages, allow_host=True), _ptr(v_pages, allow_host=True), _ptr(self.k4),
                         _ptr(self.k4_meta), _ptr(self.kbound), self.key_bits)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def units(self) -> int:
        return self.batch * self.num_kv_heads

    def struct(self) -> CacheC:
        return self._c


def workspace_bytes(cache: PagedCache, max_candidates_per_group: int) -> int:
    n = lib().twl_workspace_bytes(ctypes.byref(cache.struct()), int(max_candidates_per_group))
    if n == 0:
        raise TwlError(TWL_EINVAL, "invalid cache description")
    return int(n)


def quantize_k(cache: PagedCache, tok_begin: torch.Tensor, tok_end: torch.Tensor, max_span: int, stream=None):
    _check(lib().twl_quantize_k(ctypes.byref(cache.struct()), _ptr(tok_begin), _ptr(tok_end), int(max_span),
                                _stream(stream)))


def select_pages(cache: PagedCache, q: torch.Tensor, keep_frac: float, max_keep: int, page_ids: torch.Tensor,
                 count: torch.Tensor, ws: torch.Tensor, stream=None):
    _check(lib().twl_select_pages(ctypes.byref(cache.struct()), _ptr(q), float(keep_frac), int(max_keep),
                                  _ptr(page_ids), _ptr(count), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)))


def estimate_topp(cache: PagedCache, q: torch.Tensor, sm_scale: float, p: float, iters: int, *,
                  page_ids: Optional[torch.Tensor] = None, ranges: Optional[torch.Tensor] = None,
                  count: Optional[torch.Tensor] = None, max_items: int = 0, threshold: torch.Tensor,
                  mass: Optional[torch.Tensor] = None, head_mask: Optional[torch.Tensor] = None,
                  mask_words: int = 0, sel_indptr: torch.Tensor, sel_tokens: torch.Tensor, ws: torch.Tensor,
                  stream=None):
    cand = CandC(_ptr(page_ids), _ptr(ranges), _ptr(count), int(max_items))
    _check(lib().twl_estimate_topp(ctypes.byref(cache.struct()), _ptr(q), float(sm_scale), float(p), int(iters),
                                   ctypes.byref(cand), _ptr(threshold), _ptr(mass), _ptr(head_mask),
                                   int(mask_words), _ptr(sel_indptr), _ptr(sel_tokens), int(sel_tokens.numel()),
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def sparse_attn(cache: PagedCache, q: torch.Tensor, sm_scale: float, sel_indptr: torch.Tensor,
                sel_tokens: torch.Tensor, max_selected_per_group: int, out: torch.Tensor,
                lse: Optional[torch.Tensor], ws: torch.Tensor, stream=None):
    _check(lib().twl_sparse_attn(ctypes.byref(cache.struct()), _ptr(q), float(sm_scale), _ptr(sel_indptr),
                                 _ptr(sel_tokens), int(max_selected_per_group), _ptr(out), _ptr(lse), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)))


def _params(p, keep_frac, sm_scale, iters, topk=0, headwise=False) -> ParamsC:
    return ParamsC(float(p), float(keep_frac), float(sm_scale), int(iters), int(topk), int(bool(headwise)))


def decode(cache: PagedCache, q: torch.Tensor, *, p: float, keep_frac: float, sm_scale: float = DEFAULT_SM_SCALE,
           iters: int = 32, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
           threshold: Optional[torch.Tensor] = None, sel_indptr: Optional[torch.Tensor] = None,
           sel_tokens: Optional[torch.Tensor] = None, ws: torch.Tensor, stream=None, topk: int = 0,
           headwise: bool = False):
    prm = _params(p, keep_frac, sm_scale, iters, topk, headwise)
    cap = 0 if sel_tokens is None else int(sel_tokens.numel())
    _check(lib().twl_decode(ctypes.byref(cache.struct()), _ptr(q), ctypes.byref(prm), _ptr(out), _ptr(lse),
                            _ptr(threshold), _ptr(sel_indptr), _ptr(sel_tokens), cap, _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(stream)))


def decode_noalloc(cache: PagedCache, q: torch.Tensor, *, p: float, keep_frac: float,
                   sm_scale: float = DEFAULT_SM_SCALE, iters: int = 32, out: torch.Tensor,
                   lse: Optional[torch.Tensor] = None, threshold: Optional[torch.Tensor] = None,
                   sel_indptr: Optional[torch.Tensor] = None, sel_tokens: Optional[torch.Tensor] = None,
                   stream=None, topk: int = 0, headwise: bool = False):
    """:func:`decode` on the library's static device workspace (no workspace argument, nothing
    allocated); raises TwlError(TWL_EWORKSPACE) when the step needs more than NOALLOC_SCRATCH_BYTES."""
    prm = _params(p, keep_frac, sm_scale, iters, topk, headwise)
    cap = 0 if sel_tokens is None else int(sel_tokens.numel())
    _check(lib().twl_decode_noalloc(ctypes.byref(cache.struct()), _ptr(q), ctypes.byref(prm), _ptr(out), _ptr(lse),
                                    _ptr(threshold), _ptr(sel_indptr), _ptr(sel_tokens), cap, _stream(stream)))


def _event_array(events):
    """2*NUM_STAGES timing events as a hipEvent_t array: torch.cuda.Event objects, or raw hipEvent_t
    handles given as integers."""
    if len(events) != 2 * NUM_STAGES:
        raise ValueError("need 2*NUM_STAGES events")
    ptrs = []
    for e in events:
        if isinstance(e, int):
            ptrs.append(ctypes.c_void_p(e))
            continue
        if e.cuda_event == 0:  # make sure the underlying hipEvent_t exists
            e.record()
        ptrs.append(ctypes.c_void_p(e.cuda_event))
    return (_p * (2 * NUM_STAGES))(*ptrs)


def decode_profiled(cache: PagedCache, q: torch.Tensor, events, *, p: float, keep_frac: float,
                    sm_scale: float = DEFAULT_SM_SCALE, iters: int = 32, out: torch.Tensor,
                    lse: Optional[torch.Tensor] = None, threshold: Optional[torch.Tensor] = None,
                    sel_indptr: Optional[torch.Tensor] = None, sel_tokens: Optional[torch.Tensor] = None,
                    ws: torch.Tensor, stream=None, topk: int = 0, headwise: bool = False):
    """``events``: 2*NUM_STAGES timing events (torch.cuda.Event(enable_timing=True), or hipEvent_t
    handles as integers) recorded around each stage."""
    prm = _params(p, keep_frac, sm_scale, iters, topk, headwise)
    arr = _event_array(events)
    cap = 0 if sel_tokens is None else int(sel_tokens.numel())
    _check(lib().twl_decode_profiled(ctypes.byref(cache.struct()), _ptr(q), ctypes.byref(prm), _ptr(out),
                                     _ptr(lse), _ptr(threshold), _ptr(sel_indptr), _ptr(sel_tokens), cap,
                                     _ptr(ws), ws.numel() * ws.element_size(), _stream(stream), arr))


def select_clusters_topp(cache: PagedCache, q: torch.Tensor, sm_scale: float, p1: float, iters: int,
                         centroids: torch.Tensor, csize: torch.Tensor, coff: torch.Tensor, num_clusters: int,
                         ranges: torch.Tensor, count: torch.Tensor, ws: torch.Tensor, stream=None):
    _check(lib().twl_select_clusters_topp(ctypes.byref(cache.struct()), _ptr(q), float(sm_scale), float(p1),
                                          int(iters), _ptr(centroids), _ptr(csize), _ptr(coff), int(num_clusters),
                                          _ptr(ranges), _ptr(count), _ptr(ws), ws.numel() * ws.element_size(),
                                          _stream(stream)))


def decode_clusters(cache: PagedCache, q: torch.Tensor, *, p: float, p1: float, centroids: torch.Tensor,
                    csize: torch.Tensor, coff: torch.Tensor, sm_scale: float = DEFAULT_SM_SCALE, iters: int = 32,
                    out: torch.Tensor, lse: Optional[torch.Tensor] = None, threshold: Optional[torch.Tensor] = None,
                    sel_indptr: Optional[torch.Tensor] = None, sel_tokens: Optional[torch.Tensor] = None,
                    ws: torch.Tensor, events=None, stream=None):
    """Double-P decode step; ``events`` optionally holds 2*NUM_STAGES timing events."""
    arr = None if events is None else _event_array(events)
    prm = _params(p, 1.0, sm_scale, iters)
    cap = 0 if sel_tokens is None else int(sel_tokens.numel())
    _check(lib().twl_decode_clusters(ctypes.byref(cache.struct()), _ptr(q), ctypes.byref(prm), float(p1),
                                     _ptr(centroids), _ptr(csize), _ptr(coff), int(csize.shape[-1]), _ptr(out),
                                     _ptr(lse), _ptr(threshold), _ptr(sel_indptr), _ptr(sel_tokens), cap, _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream), arr))


def cluster_value_means(cache: PagedCache, csize: torch.Tensor, coff: torch.Tensor, vmean: torch.Tensor,
                        stream=None):
    """Mean value row of every cluster into ``vmean`` (float32 [B][Hkv][C][128])."""
    _check(lib().twl_cluster_value_means(ctypes.byref(cache.struct()), _ptr(csize), _ptr(coff),
                                         int(csize.shape[-1]), _ptr(vmean), _stream(stream)))


def cluster_approx_unkept(cache: PagedCache, q: torch.Tensor, *, p1: float, centroids: torch.Tensor,
                          csize: torch.Tensor, vmean: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                          ws: torch.Tensor, sm_scale: float = DEFAULT_SM_SCALE, iters: int = 32, stream=None):
    """Merge the clusters no head of a group kept into ``out`` / ``lse`` of a :func:`decode_clusters`."""
    _check(lib().twl_cluster_approx_unkept(ctypes.byref(cache.struct()), _ptr(q), float(sm_scale), float(p1),
                                           int(iters), _ptr(centroids), _ptr(csize), int(csize.shape[-1]),
                                           _ptr(vmean), _ptr(out), _ptr(lse), _ptr(ws),
                                           ws.numel() * ws.element_size(), _stream(stream)))
