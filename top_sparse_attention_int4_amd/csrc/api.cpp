// C ABI of libtwl: host-side validation, workspace carving and kernel orchestration.
//
// Every entry point validates its arguments before its first HIP call, then checks that the
// current device is gfx950, carves the caller's workspace and enqueues the kernels on the caller's
// stream.  Nothing here allocates, frees or synchronises.
#include <dlfcn.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "twl.h"
#include "twl_internal.h"

namespace {

using namespace twl;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// ---- argument validation (host only, no HIP calls) -------------------------------------------------
twl_status check_cache(const twl_cache* c, bool need_kv, bool need_quant) {
  if (!c) return TWL_EINVAL;
  if (c->batch < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1) return TWL_EINVAL;
  if (c->num_q_heads % c->num_kv_heads) return TWL_EINVAL;
  const int G = c->num_q_heads / c->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return TWL_EUNSUPPORTED;
  if (c->head_dim != 128 || c->page_size != 16 || c->quant_group != 32) return TWL_EUNSUPPORTED;
  if (c->key_bits != 0 && c->key_bits != 2 && c->key_bits != 4 && c->key_bits != 8) return TWL_EUNSUPPORTED;
  if (c->max_pages_per_seq < 1 || c->num_phys_pages < 1) return TWL_EINVAL;
  if (c->max_seq_len < 0 || (int64_t)c->max_seq_len > 16 * (int64_t)c->max_pages_per_seq) return TWL_EINVAL;
  if ((int64_t)c->num_phys_pages * c->num_kv_heads * 16 >= ((int64_t)1 << 31)) return TWL_EUNSUPPORTED;
  if ((int64_t)c->batch * c->max_pages_per_seq >= ((int64_t)1 << 31)) return TWL_EUNSUPPORTED;
  // rows of the codes (stored by sequence and logical page) are int32
  if ((int64_t)c->batch * c->max_pages_per_seq * c->num_kv_heads * 16 >= ((int64_t)1 << 31)) return TWL_EUNSUPPORTED;
  if ((int64_t)c->batch * c->num_kv_heads > 65535) return TWL_EUNSUPPORTED;
  // int32 CSR offsets and candidate indices over all units (with headroom for padded capacities)
  if ((int64_t)c->batch * c->num_q_heads * c->max_seq_len > ((int64_t)1 << 31) / 4) return TWL_EUNSUPPORTED;
  if (!c->page_table || !c->seq_lens) return TWL_EINVAL;
  if (need_kv && (!c->k || !c->v)) return TWL_EINVAL;
  if (need_quant && (!c->k4 || !c->k4_meta || !c->kbound)) return TWL_EINVAL;
  return TWL_OK;
}

bool finite(float x) { return std::isfinite(x); }

// q rows are read with 16-byte loads
bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Kept-page count bound for the longest sequence (matches the device computation).
int keep_count(int P, float keep_frac) {
  if (P <= 0) return 0;
  const float kf = std::ceil(std::fmin(keep_frac * (float)P, (float)P));
  if (!(kf < (float)P)) return P;  // (float)P may round above P: no out-of-range conversion
  const int k = (int)kf;
  return k < 1 ? 1 : (k > P ? P : k);
}

// ---- device check (first HIP call of an entry point) ------------------------------------------------
twl_status check_device() {
  static std::atomic<int> state[64];  // 0 unknown, 1 gfx950, 2 other
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TWL_EHIP;
  if (dev >= 0 && dev < 64) {
    const int s = state[dev].load(std::memory_order_relaxed);
    if (s == 1) return TWL_OK;
    if (s == 2) return TWL_EUNSUPPORTED;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return TWL_EHIP;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? TWL_OK : TWL_EUNSUPPORTED;
}

CacheView make_view(const twl_cache* c) {
  CacheView v;
  v.B = c->batch;
  v.Hq = c->num_q_heads;
  v.Hkv = c->num_kv_heads;
  v.G = c->num_q_heads / c->num_kv_heads;
  v.maxP = c->max_pages_per_seq;
  v.nphys = c->num_phys_pages;
  v.maxTok = c->max_pages_per_seq * 16;
  v.kbits = c->key_bits == 0 ? 4 : c->key_bits;
  v.page_table = c->page_table;
  v.seq_lens = c->seq_lens;
  v.k = static_cast<const uint16_t*>(c->k);
  v.v = static_cast<const uint16_t*>(c->v);
  v.k4 = static_cast<uint8_t*>(c->k4);
  v.k4_meta = static_cast<uint32_t*>(c->k4_meta);
  v.kbound = static_cast<uint16_t*>(c->kbound);
  return v;
}

// ---- workspace layout ----------------------------------------------------------------------------------
struct Layout {
  int64_t ncap = 0;       // candidate capacity per unit (multiple of 1024)
  int chunk_tokens = 64;  // attention chunk
  int slots = 1;          // attention chunk slots per unit (ceil(ncap / chunk_tokens))
  int64_t max_chunks = 0;
  size_t scores = 0, pages = 0, pcnt = 0, rpre = 0, cfirst = 0, logits = 0, masks = 0, utok = 0, urow = 0,
         ucnt = 0, ctok = 0, pphys = 0, parts = 0, thr = 0, pmax = 0, wstate = 0, wcnt = 0, uwords = 0,
         wkeys = 0, wrcnt = 0, wmass = 0, mpart = 0, mtick = 0, smask = 0, apart = 0, qdig = 0, qmeta = 0, total = 0;
};

// ncap_of(maxcand): up to 65536 candidates the top-p block holds 1024*E of them, E a power of two up
// to 64; beyond, the wide top-p takes multiples of 16384 (four of its 4096-candidate chunks per
// histogram block), up to 2^22.  0 = too many.
int64_t ncap_of(int64_t maxcand) {
  if (maxcand < 1) maxcand = 1;
  if (maxcand <= kNarrowMaxCands) return (int64_t)topp_elems_per_thread(maxcand) * kToppThreads;
  if (maxcand > kWideMaxCands) return 0;
  return (maxcand + kWideAlign - 1) / kWideAlign * kWideAlign;
}

bool is_wide(int64_t ncap) { return ncap > kNarrowMaxCands; }

bool make_layout(const twl_cache* c, int64_t ncap, Layout* L) {
  const int64_t U = (int64_t)c->batch * c->num_kv_heads;
  const int64_t BH = (int64_t)c->batch * c->num_q_heads;
  const int G = c->num_q_heads / c->num_kv_heads;
  L->ncap = ncap;
  L->chunk_tokens = attn_chunk_tokens(U * ncap, G);
  L->slots = (int)((ncap + L->chunk_tokens - 1) / L->chunk_tokens);
  if (L->slots < 1) L->slots = 1;
  L->max_chunks = U * L->slots;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  L->scores = take((size_t)U * c->max_pages_per_seq * 4);
  L->pages = take((size_t)U * c->max_pages_per_seq * 4);
  L->pcnt = take((size_t)U * 4);
  L->pphys = take((size_t)U * c->max_pages_per_seq * 4);
  L->smask = take((size_t)U * c->max_pages_per_seq * 4);  // the cluster stage's slot mask of every page
  L->rpre = take((size_t)U * (ncap + 1) * 4);
  L->cfirst = take((size_t)U * (ncap / kEstCands) * 4);
  L->logits = take((size_t)BH * ncap * 4);
  L->masks = take((size_t)BH * (ncap / 32) * 4);
  L->utok = take((size_t)U * ncap * 4);
  L->urow = take((size_t)U * ncap * 4);
  L->ucnt = take((size_t)U * 4);
  L->ctok = take((size_t)U * ncap * 4);
  L->parts = take((size_t)L->max_chunks * G * kPartFloats * 4);
  L->mpart = take((size_t)BH * kMergeSplits * kPartFloats * 4);  // second merge level
  L->mtick = take((size_t)BH * 4);
  L->thr = take((size_t)BH * 4);
  L->apart = take((size_t)BH * kApproxSlices * kApproxStride * 4);  // unkept-cluster approximation
  L->qdig = take((size_t)BH * kGroups * kQDigits * 32);             // the estimate's query digits
  L->qmeta = take((size_t)BH * kGroups * kQMeta * 4);
  if (is_wide(ncap)) {
    L->pmax = take((size_t)BH * (ncap / kEstCands) * 4);
    L->wstate = take((size_t)BH * kWideStateWords * 8);
    L->wcnt = take((size_t)U * (ncap / kWideChunk) * 4);
    L->uwords = take((size_t)U * (ncap / 32) * 4);
    L->wkeys = take((size_t)BH * ncap * 8);
    L->wrcnt = take((size_t)BH * (ncap / kWideChunk) * 4);
    L->wmass = take((size_t)BH * (ncap / kWideChunk) * 8);
  }
  L->total = off;
  return true;
}

twl_status check_ws(const void* ws, size_t ws_bytes, const Layout& L) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1))) return TWL_EWORKSPACE;
  if (ws_bytes < L.total) return TWL_EWORKSPACE;
  return TWL_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// ---- optional tracing ----------------------------------------------------------------------------
// With TWL_TRACE=1 in the environment when the library first traces, every entry point and every
// stage of the fused decodes is bracketed by a roctx range (host-side ranges: what was enqueued
// when, for rocprofv3 --marker-trace timelines).  The roctx library is looked up at run time, so the
// library does not depend on it; without it, or without the variable, tracing costs one branch.
struct Tracer {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};

const Tracer& tracer() {
  static const Tracer t = [] {
    Tracer x;
    const char* e = std::getenv("TWL_TRACE");
    if (!e || std::strcmp(e, "1") != 0) return x;
    void* h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
    if (!h) h = dlopen("libroctx64.so.4", RTLD_NOW | RTLD_LOCAL);
    if (!h) return x;
    auto push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
    auto pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
    if (push && pop) {
      x.push = push;
      x.pop = pop;
    }
    return x;
  }();
  return t;
}

// A roctx range for the lifetime of the object (a no-op unless tracing).
struct TraceRange {
  const bool on;
  explicit TraceRange(const char* name) : on(tracer().push != nullptr) {
    if (on) tracer().push(name);
  }
  ~TraceRange() {
    if (on) tracer().pop();
  }
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;
};

const char* const kStageNames[TWL_NUM_STAGES] = {"page_score", "page_select", "estimate",
                                                 "topp_union", "attention",   "merge"};
const char* const kClusterStageNames[TWL_NUM_STAGES] = {"cluster_scores_topp", "cluster_pages", "estimate",
                                                        "topp_union",          "attention",     "merge"};

// Stage hook of the fused decodes: caller-owned events for profiled runs (event 2i before stage i,
// 2i + 1 after it), and the stage's trace range.
struct Events {
  void* const* ev = nullptr;
  hipStream_t s = nullptr;
  const char* const* names = kStageNames;
  hipError_t rec(int i) const {
    if (tracer().push) {
      if (i % 2 == 0) tracer().push(names[i / 2]);
      else tracer().pop();
    }
    return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), s) : hipSuccess;
  }
};

twl_status hip_status(hipError_t e) { return e == hipSuccess ? TWL_OK : TWL_EHIP; }

#define TWL_TRY(expr)                          \
  do {                                         \
    const hipError_t e_ = (expr);              \
    if (e_ != hipSuccess) return TWL_EHIP;     \
  } while (0)

MergeWs merge_of(void* ws, const Layout& L) { return MergeWs{at<float>(ws, L.mpart), at<int32_t>(ws, L.mtick)}; }

QDigits qdigits_of(void* ws, const Layout& L) { return QDigits{at<uint8_t>(ws, L.qdig), at<int32_t>(ws, L.qmeta)}; }

WideWs wide_of(void* ws, const Layout& L) {
  return WideWs{at<float>(ws, L.pmax), at<uint64_t>(ws, L.wstate), at<int32_t>(ws, L.wcnt), at<uint32_t>(ws, L.uwords),
                at<uint64_t>(ws, L.wkeys), at<int32_t>(ws, L.wrcnt), at<uint64_t>(ws, L.wmass)};
}

// Estimate, top-p and (when `with_union`) the compacted GQA union of every unit, the narrow or the
// wide top-p by candidate capacity.  Events 4/5 bracket the estimate, 6/7 the rest.
// The query digits must have been written (by the page scores or launch_qdigits) before this runs.
hipError_t estimate_topp(const CacheView& c, float sm, const CandView& cand, void* ws,
                         const Layout& L, float p, int iters, float* thr, float* mass, uint32_t* head_mask,
                         int mask_words, bool with_union, const Events& E, hipStream_t s, int topk = 0) {
  const int ncap = (int)L.ncap;
  const WideWs wd = wide_of(ws, L);
  const bool wide = is_wide(L.ncap);
  hipError_t e;
  if ((e = E.rec(4)) != hipSuccess) return e;
  // token ids of the candidates are read only by the passes that emit the union lists
  const bool need_tok = with_union || (wide && mass);
  e = launch_estimate(c, qdigits_of(ws, L), sm, cand, ncap, at<float>(ws, L.logits),
                      need_tok ? at<int32_t>(ws, L.ctok) : nullptr, wide ? &wd : nullptr, s);
  if (e != hipSuccess) return e;
  if ((e = E.rec(5)) != hipSuccess) return e;
  if ((e = E.rec(6)) != hipSuccess) return e;
  if (wide) {
    e = launch_topp_wide(c, wd, at<float>(ws, L.logits), ncap, p, iters, thr, head_mask, mask_words,
                         with_union || mass || head_mask, s);
    if (e == hipSuccess && (with_union || mass))
      e = launch_wide_emit(c, wd, at<int32_t>(ws, L.ctok), ncap, at<int32_t>(ws, L.utok), at<int32_t>(ws, L.ucnt),
                           mass, s);
  } else {
    e = launch_topp(c, at<float>(ws, L.logits), ncap, p, iters, thr, mass, at<uint32_t>(ws, L.masks), head_mask,
                    mask_words, topk, s);
    if (e == hipSuccess && with_union)
      e = launch_union(c, at<uint32_t>(ws, L.masks), at<int32_t>(ws, L.ctok), ncap, at<int32_t>(ws, L.utok),
                       at<int32_t>(ws, L.ucnt), s);
  }
  if (e != hipSuccess) return e;
  return E.rec(7);
}

// Attention over the top-p bitmaps (no compacted list needed) and the merge; events 8..11.
// `cand` names where the K/V row of each candidate comes from: the selector's physical page list, or
// the page table (every page a candidate page).
hipError_t attend_masked(const CacheView& c, const uint16_t* q, float sm, const CandView& cand, void* ws,
                         const Layout& L, float* out, float* lse, const Events& E, hipStream_t s,
                         bool headwise = false) {
  const bool wide = is_wide(L.ncap);
  MaskView mv{};
  if (wide) {
    mv.union_words = at<uint32_t>(ws, L.uwords);
  } else {
    mv.head_masks = at<uint32_t>(ws, L.masks);
  }
  mv.cand_mode = cand.mode;
  mv.page_phys = cand.phys;
  mv.page_stride = cand.max_items;
  mv.ncap = L.ncap;
  hipError_t e;
  if ((e = E.rec(8)) != hipSuccess) return e;
  if ((e = launch_attn_masked(c, q, sm, mv, L.chunk_tokens, L.slots, at<float>(ws, L.parts), merge_of(ws, L),
                              headwise, s)) != hipSuccess)
    return e;
  if ((e = E.rec(9)) != hipSuccess) return e;
  if ((e = E.rec(10)) != hipSuccess) return e;
  if ((e = launch_merge(c, nullptr, L.chunk_tokens, L.slots, at<float>(ws, L.parts), merge_of(ws, L), out, lse,
                        s)) != hipSuccess)
    return e;
  return E.rec(11);
}

// Host-only validation of a decode call's arguments (everything but the workspace); on success the
// workspace layout it needs is written to *L.
twl_status decode_check(const twl_cache* cache, const void* q, const twl_decode_params* prm, const float* out,
                        const int32_t* sel_indptr, const int32_t* sel_tokens, int64_t capacity, Layout* L) {
  twl_status st = check_cache(cache, true, true);
  if (st != TWL_OK) return st;
  if (!q || misaligned16(q) || !prm || !out) return TWL_EINVAL;
  if (!finite(prm->p) || !(prm->p > 0.f) || prm->p > 1.f) return TWL_EINVAL;
  if (!finite(prm->keep_frac) || !(prm->keep_frac > 0.f)) return TWL_EINVAL;
  if (!finite(prm->sm_scale)) return TWL_EINVAL;
  if (prm->iters < 1 || prm->iters > 64) return TWL_EINVAL;
  if (prm->topk < 0 || (prm->headwise != 0 && prm->headwise != 1)) return TWL_EINVAL;
  if ((sel_indptr == nullptr) != (sel_tokens == nullptr)) return TWL_EINVAL;
  const bool selector = prm->keep_frac < 1.0f;
  const int64_t U = (int64_t)cache->batch * cache->num_kv_heads;
  const int max_keep = keep_count(cache->max_pages_per_seq, prm->keep_frac);
  const int64_t maxcand = selector ? 16 * (int64_t)max_keep : (int64_t)cache->max_seq_len;
  if (sel_tokens && capacity < U * maxcand) return TWL_EINVAL;
  const int64_t ncap = ncap_of(maxcand);
  if (ncap == 0) return TWL_EUNSUPPORTED;
  // the top-k baseline and head-wise attention run on the one-block-per-head search's bitmaps
  if ((prm->topk > 0 || prm->headwise) && is_wide(ncap)) return TWL_EUNSUPPORTED;
  make_layout(cache, ncap, L);
  return TWL_OK;
}

twl_status decode_impl(const twl_cache* cache, const void* q, const twl_decode_params* prm, float* out,
                       float* lse, float* threshold, int32_t* sel_indptr, int32_t* sel_tokens, int64_t capacity,
                       void* ws, size_t ws_bytes, void* stream, void* const* events) {
  Layout L;
  twl_status st = decode_check(cache, q, prm, out, sel_indptr, sel_tokens, capacity, &L);
  if (st != TWL_OK) return st;
  const int64_t ncap = L.ncap;
  const bool selector = prm->keep_frac < 1.0f;
  st = check_ws(ws, ws_bytes, L);
  if (st != TWL_OK) return st;
  if (events) {
    for (int i = 0; i < 2 * TWL_NUM_STAGES; ++i)
      if (!events[i]) return TWL_EINVAL;
  }
  // ---- enqueue ----
  st = check_device();
  if (st != TWL_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const Events E{events, s};
  const CacheView c = make_view(cache);
  const uint16_t* qb = static_cast<const uint16_t*>(q);

  CandView cand{};
  if (selector) {
    TWL_TRY(E.rec(0));
    TWL_TRY(launch_page_score(c, qb, at<float>(ws, L.scores), s));
    TWL_TRY(E.rec(1));
    TWL_TRY(E.rec(2));
    TWL_TRY(launch_page_select(c, at<float>(ws, L.scores), prm->keep_frac, cache->max_pages_per_seq,
                               at<int32_t>(ws, L.pphys), at<int32_t>(ws, L.pages), at<int32_t>(ws, L.pcnt), qb,
                               qdigits_of(ws, L), s));
    TWL_TRY(E.rec(3));
    cand.mode = kCandPages;
    cand.items = at<int32_t>(ws, L.pages);
    cand.count = at<int32_t>(ws, L.pcnt);
    cand.max_items = cache->max_pages_per_seq;
    cand.phys = at<int32_t>(ws, L.pphys);
  } else {
    TWL_TRY(E.rec(0));
    TWL_TRY(launch_qdigits(c, qb, qdigits_of(ws, L), s));
    for (int i = 1; i < 4; ++i) TWL_TRY(E.rec(i));
    cand.mode = kCandAll;
  }
  float* thr = threshold ? threshold : at<float>(ws, L.thr);
  const bool csr = sel_tokens != nullptr;
  TWL_TRY(estimate_topp(c, prm->sm_scale, cand, ws, L, prm->p, prm->iters, thr, nullptr, nullptr, 0, csr, E, s,
                        prm->topk));
  if (csr)
    TWL_TRY(launch_csr_emit(c, at<int32_t>(ws, L.utok), at<int32_t>(ws, L.ucnt), (int)ncap, sel_indptr, sel_tokens,
                            capacity, s));
  TWL_TRY(attend_masked(c, qb, prm->sm_scale, cand, ws, L, out, lse, E, s, prm->headwise != 0));
  return TWL_OK;
}

// Double-P decode: cluster top-p -> ranges -> estimate / token top-p / union -> attention -> merge.
// The kept ranges live in the union-row region (read only before the union overwrites it) and their
// count in the page-count region.
twl_status decode_clusters_impl(const twl_cache* cache, const void* q, const twl_decode_params* prm, float p1,
                                const void* centroids, const int32_t* csize, const int32_t* coff,
                                int32_t num_clusters, float* out, float* lse, float* threshold,
                                int32_t* sel_indptr, int32_t* sel_tokens, int64_t capacity, void* ws,
                                size_t ws_bytes, void* stream, void* const* events) {
  twl_status st = check_cache(cache, true, true);
  if (st != TWL_OK) return st;
  if (!q || misaligned16(q) || !prm || !out || !centroids || !csize || !coff) return TWL_EINVAL;
  if (!finite(prm->p) || !(prm->p > 0.f) || prm->p > 1.f) return TWL_EINVAL;
  if (!finite(p1) || !(p1 > 0.f) || p1 > 1.f) return TWL_EINVAL;
  if (!finite(prm->sm_scale)) return TWL_EINVAL;
  if (prm->iters < 1 || prm->iters > 64 || num_clusters < 1) return TWL_EINVAL;
  if (prm->topk != 0 || prm->headwise != 0) return TWL_EUNSUPPORTED;
  if ((sel_indptr == nullptr) != (sel_tokens == nullptr)) return TWL_EINVAL;
  const int64_t U = (int64_t)cache->batch * cache->num_kv_heads;
  const int64_t maxcand = cache->max_seq_len;
  if (sel_tokens && capacity < U * maxcand) return TWL_EINVAL;
  const int64_t ncap = ncap_of(maxcand);
  if (ncap == 0 || num_clusters > kNarrowMaxCands || 2 * (int64_t)num_clusters > ncap) return TWL_EUNSUPPORTED;
  const int64_t cpad = ncap_of(num_clusters);
  if (cpad > ncap) return TWL_EUNSUPPORTED;
  Layout L;
  make_layout(cache, ncap, &L);
  st = check_ws(ws, ws_bytes, L);
  if (st != TWL_OK) return st;
  if (events) {
    for (int i = 0; i < 2 * TWL_NUM_STAGES; ++i)
      if (!events[i]) return TWL_EINVAL;
  }
  st = check_device();
  if (st != TWL_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const Events E{events, s, kClusterStageNames};
  const CacheView c = make_view(cache);
  const uint16_t* qb = static_cast<const uint16_t*>(q);
  TWL_TRY(E.rec(0));
  TWL_TRY(launch_cluster_scores_topp(c, qb, prm->sm_scale, p1, prm->iters, static_cast<const uint16_t*>(centroids),
                                     csize, num_clusters, (int)cpad, at<float>(ws, L.logits), at<float>(ws, L.thr),
                                     at<uint32_t>(ws, L.masks), qdigits_of(ws, L), s));
  TWL_TRY(E.rec(1));
  TWL_TRY(E.rec(2));
  // the kept clusters' tokens as a slot mask of every page
  TWL_TRY(launch_cluster_slots(c, at<uint32_t>(ws, L.masks), (int)cpad, csize, coff, num_clusters,
                               at<uint32_t>(ws, L.smask), s));
  TWL_TRY(E.rec(3));
  CandView cand{};
  cand.mode = kCandAll;
  cand.slot_mask = at<uint32_t>(ws, L.smask);
  float* thr = threshold ? threshold : at<float>(ws, L.thr);
  const bool csr = sel_tokens != nullptr;
  TWL_TRY(estimate_topp(c, prm->sm_scale, cand, ws, L, prm->p, prm->iters, thr, nullptr, nullptr, 0, csr, E, s));
  if (csr)
    TWL_TRY(launch_csr_emit(c, at<int32_t>(ws, L.utok), at<int32_t>(ws, L.ucnt), (int)ncap, sel_indptr, sel_tokens,
                            capacity, s));
  TWL_TRY(attend_masked(c, qb, prm->sm_scale, cand, ws, L, out, lse, E, s));
  return TWL_OK;
}

}  // namespace

namespace twl {

twl_status decode_workspace_need(const twl_cache* cache, const void* q, const twl_decode_params* params,
                                 const float* out, const int32_t* sel_indptr, const int32_t* sel_tokens,
                                 int64_t capacity, size_t* need) {
  Layout L;
  const twl_status st = decode_check(cache, q, params, out, sel_indptr, sel_tokens, capacity, &L);
  if (st == TWL_OK) *need = L.total;
  return st;
}

twl_status decode_with_workspace(const twl_cache* cache, const void* q, const twl_decode_params* params, float* out,
                                 float* lse, float* threshold, int32_t* sel_indptr, int32_t* sel_tokens,
                                 int64_t capacity, void* ws, size_t ws_bytes, void* stream) {
  return decode_impl(cache, q, params, out, lse, threshold, sel_indptr, sel_tokens, capacity, ws, ws_bytes, stream,
                     nullptr);
}

}  // namespace twl

extern "C" {

size_t twl_workspace_bytes(const twl_cache* cache, int64_t max_candidates_per_group) {
  if (check_cache(cache, false, false) != TWL_OK || max_candidates_per_group < 0) return 0;
  const int64_t ncap = ncap_of(max_candidates_per_group);
  if (ncap == 0) return 0;  // beyond the top-p capacity: no entry point accepts such a unit
  Layout L;
  make_layout(cache, ncap, &L);
  return L.total;
}

twl_status twl_quantize_k(const twl_cache* cache, const int32_t* tok_begin, const int32_t* tok_end,
                          int32_t max_span, void* stream) {
  const TraceRange trace_("twl_quantize_k");
  twl_status st = check_cache(cache, true, true);
  if (st != TWL_OK) return st;
  if (!tok_begin || !tok_end) return TWL_EINVAL;
  if (max_span < 0 || (int64_t)max_span > 16 * (int64_t)cache->max_pages_per_seq) return TWL_EINVAL;
  st = check_device();
  if (st != TWL_OK) return st;
  int span_pages = max_span == 0 ? 0 : (max_span + 15) / 16 + 1;
  if (span_pages > cache->max_pages_per_seq) span_pages = cache->max_pages_per_seq;
  return hip_status(launch_quantize(make_view(cache), tok_begin, tok_end, span_pages, static_cast<hipStream_t>(stream)));
}

twl_status twl_select_pages(const twl_cache* cache, const void* q, float keep_frac, int32_t max_keep,
                            int32_t* page_ids, int32_t* count, void* ws, size_t ws_bytes, void* stream) {
  const TraceRange trace_("twl_select_pages");
  twl_status st = check_cache(cache, false, true);
  if (st != TWL_OK) return st;
  if (!q || misaligned16(q) || !page_ids || !count) return TWL_EINVAL;
  if (!finite(keep_frac) || !(keep_frac > 0.f)) return TWL_EINVAL;
  if (max_keep < keep_count(cache->max_pages_per_seq, keep_frac)) return TWL_EINVAL;
  Layout L;
  make_layout(cache, kToppThreads, &L);
  st = check_ws(ws, ws_bytes, L);
  if (st != TWL_OK) return st;
  st = check_device();
  if (st != TWL_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const CacheView c = make_view(cache);
  TWL_TRY(launch_page_score(c, static_cast<const uint16_t*>(q), at<float>(ws, L.scores), s));
  TWL_TRY(launch_page_select(c, at<float>(ws, L.scores), keep_frac, max_keep, nullptr, page_ids, count, nullptr,
                             QDigits{}, s));
  return TWL_OK;
}

twl_status twl_estimate_topp(const twl_cache* cache, const void* q, float sm_scale, float p, int32_t iters,
                             const twl_candidates* cand, float* threshold, float* mass, uint32_t* head_mask,
                             int32_t mask_words, int32_t* sel_indptr, int32_t* sel_tokens, int64_t capacity,
                             void* ws, size_t ws_bytes, void* stream) {
  const TraceRange trace_("twl_estimate_topp");
  twl_status st = check_cache(cache, false, true);
  if (st != TWL_OK) return st;
  if (!q || misaligned16(q) || !cand || !threshold || !sel_indptr || !sel_tokens) return TWL_EINVAL;
  if (!finite(p) || !(p > 0.f) || p > 1.f) return TWL_EINVAL;
  if (!finite(sm_scale)) return TWL_EINVAL;
  if (iters < 1 || iters > 64) return TWL_EINVAL;
  if (cand->page_ids && cand->ranges) return TWL_EINVAL;
  const int64_t U = (int64_t)cache->batch * cache->num_kv_heads;
  CandView cv{};
  int64_t maxcand;
  if (cand->page_ids || cand->ranges) {
    if (!cand->count || cand->max_items < 1) return TWL_EINVAL;
  }
  if (cand->page_ids) {
    if (cand->max_items > cache->max_pages_per_seq) return TWL_EINVAL;
    cv.mode = kCandPages;
    cv.items = cand->page_ids;
    maxcand = 16 * (int64_t)cand->max_items;
  } else if (cand->ranges) {
    cv.mode = kCandRanges;
    cv.items = cand->ranges;
    maxcand = cache->max_seq_len;
  } else {
    cv.mode = kCandAll;
    maxcand = cache->max_seq_len;
  }
  cv.count = cand->count;
  cv.max_items = cand->max_items;
  if (capacity < U * maxcand) return TWL_EINVAL;
  if (head_mask && (int64_t)mask_words * 32 < maxcand) return TWL_EINVAL;
  const int64_t ncap = ncap_of(maxcand);
  if (ncap == 0) return TWL_EUNSUPPORTED;
  if (cv.mode == kCandRanges && cand->max_items > ncap) return TWL_EINVAL;
  Layout L;
  make_layout(cache, ncap, &L);
  st = check_ws(ws, ws_bytes, L);
  if (st != TWL_OK) return st;
  st = check_device();
  if (st != TWL_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const CacheView c = make_view(cache);
  TWL_TRY(launch_qdigits(c, static_cast<const uint16_t*>(q), qdigits_of(ws, L), s));
  if (cv.mode == kCandRanges) {
    cv.range_prefix = at<int32_t>(ws, L.rpre);
    cv.chunk_first = at<int32_t>(ws, L.cfirst);
    TWL_TRY(launch_range_prefix(c, cv, at<int32_t>(ws, L.rpre), at<int32_t>(ws, L.cfirst), (int)(ncap / kEstCands), s));
  }
  TWL_TRY(estimate_topp(c, sm_scale, cv, ws, L, p, iters, threshold, mass, head_mask, mask_words, true, Events{}, s));
  TWL_TRY(launch_csr_emit(c, at<int32_t>(ws, L.utok), at<int32_t>(ws, L.ucnt), (int)ncap, sel_indptr, sel_tokens,
                          capacity, s));
  return TWL_OK;
}

twl_status twl_sparse_attn(const twl_cache* cache, const void* q, float sm_scale, const int32_t* sel_indptr,
                           const int32_t* sel_tokens, int32_t max_selected_per_group, float* out, float* lse,
                           void* ws, size_t ws_bytes, void* stream) {
  const TraceRange trace_("twl_sparse_attn");
  twl_status st = check_cache(cache, true, false);
  if (st != TWL_OK) return st;
  if (!q || misaligned16(q) || !sel_indptr || !sel_tokens || !out) return TWL_EINVAL;
  if (!finite(sm_scale)) return TWL_EINVAL;
  if (max_selected_per_group < 0) return TWL_EINVAL;
  int64_t ncap = ncap_of(max_selected_per_group);
  if (ncap == 0) ncap = (((int64_t)max_selected_per_group + 1023) / 1024) * 1024;
  Layout L;
  make_layout(cache, ncap, &L);
  st = check_ws(ws, ws_bytes, L);
  if (st != TWL_OK) return st;
  st = check_device();
  if (st != TWL_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const CacheView c = make_view(cache);
  const int64_t U = (int64_t)cache->batch * cache->num_kv_heads;
  TWL_TRY(launch_rows(c, sel_indptr, sel_tokens, at<int32_t>(ws, L.urow), U * ncap, s));
  ListView lv{sel_tokens, at<int32_t>(ws, L.urow), sel_indptr, nullptr, 0, U * ncap};
  TWL_TRY(launch_attn(c, static_cast<const uint16_t*>(q), sm_scale, lv, L.chunk_tokens, L.slots,
                      at<float>(ws, L.parts), merge_of(ws, L), s));
  TWL_TRY(launch_merge(c, &lv, L.chunk_tokens, L.slots, at<float>(ws, L.parts), merge_of(ws, L), out, lse, s));
  return TWL_OK;
}

twl_status twl_decode(const twl_cache* cache, const void* q, const twl_decode_params* params, float* out,
                      float* lse, float* threshold, int32_t* sel_indptr, int32_t* sel_tokens, int64_t capacity,
                      void* ws, size_t ws_bytes, void* stream) {
  const TraceRange trace_("twl_decode");
  return decode_impl(cache, q, params, out, lse, threshold, sel_indptr, sel_tokens, capacity, ws, ws_bytes,
                     stream, nullptr);
}

twl_status twl_decode_profiled(const twl_cache* cache, const void* q, const twl_decode_params* params,
                               float* out, float* lse, float* threshold, int32_t* sel_indptr,
                               int32_t* sel_tokens, int64_t capacity, void* ws, size_t ws_bytes,
                               void* stream, void* const* events) {
  const TraceRange trace_("twl_decode_profiled");
  if (!events) return TWL_EINVAL;
  return decode_impl(cache, q, params, out, lse, threshold, sel_indptr, sel_tokens, capacity, ws, ws_bytes,
                     stream, events);
}

twl_status twl_select_clusters_topp(const twl_cache* cache, const void* q, float sm_scale, float p1,
                                    int32_t iters, const void* centroids, const int32_t* csize,
                                    const int32_t* coff, int32_t num_clusters, int32_t* ranges,
                                    int32_t* count, void* ws, size_t ws_bytes, void* stream) {
  const TraceRange trace_("twl_select_clusters_topp");
  twl_status st = check_cache(cache, false, false);
  if (st != TWL_OK) return st;
  if (!q || misaligned16(q) || !centroids || !csize || !coff || !ranges || !count) return TWL_EINVAL;
  if (!finite(p1) || !(p1 > 0.f) || p1 > 1.f || !finite(sm_scale)) return TWL_EINVAL;
  if (iters < 1 || iters > 64 || num_clusters < 1) return TWL_EINVAL;
  if (num_clusters > kNarrowMaxCands) return TWL_EUNSUPPORTED;
  const int64_t cpad = ncap_of(num_clusters);
  Layout L;
  make_layout(cache, cpad, &L);
  st = check_ws(ws, ws_bytes, L);
  if (st != TWL_OK) return st;
  st = check_device();
  if (st != TWL_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const CacheView c = make_view(cache);
  TWL_TRY(launch_cluster_scores_topp(c, static_cast<const uint16_t*>(q), sm_scale, p1, iters,
                                     static_cast<const uint16_t*>(centroids), csize, num_clusters, (int)cpad,
                                     at<float>(ws, L.logits), at<float>(ws, L.thr), at<uint32_t>(ws, L.masks),
                                     QDigits{}, s));
  return hip_status(launch_cluster_union(c, at<uint32_t>(ws, L.masks), (int)cpad, csize, coff, num_clusters, ranges,
                                         count, nullptr, nullptr, 0, s));
}

twl_status twl_cluster_value_means(const twl_cache* cache, const int32_t* csize, const int32_t* coff,
                                   int32_t num_clusters, float* vmean, void* stream) {
  const TraceRange trace_("twl_cluster_value_means");
  twl_status st = check_cache(cache, true, false);
  if (st != TWL_OK) return st;
  if (!csize || !coff || !vmean || num_clusters < 1 || num_clusters > kNarrowMaxCands) return TWL_EINVAL;
  st = check_device();
  if (st != TWL_OK) return st;
  return hip_status(launch_cluster_vmean(make_view(cache), csize, coff, num_clusters, vmean,
                                         static_cast<hipStream_t>(stream)));
}

twl_status twl_cluster_approx_unkept(const twl_cache* cache, const void* q, float sm_scale, float p1, int32_t iters,
                                     const void* centroids, const int32_t* csize, int32_t num_clusters,
                                     const float* vmean, float* out, float* lse, void* ws, size_t ws_bytes,
                                     void* stream) {
  const TraceRange trace_("twl_cluster_approx_unkept");
  twl_status st = check_cache(cache, false, false);
  if (st != TWL_OK) return st;
  if (!q || misaligned16(q) || !centroids || !csize || !vmean || !out || !lse) return TWL_EINVAL;
  if (!finite(p1) || !(p1 > 0.f) || p1 > 1.f || !finite(sm_scale)) return TWL_EINVAL;
  if (iters < 1 || iters > 64 || num_clusters < 1) return TWL_EINVAL;
  if (num_clusters > kNarrowMaxCands) return TWL_EUNSUPPORTED;
  const int64_t cpad = ncap_of(num_clusters);
  Layout L;
  make_layout(cache, cpad, &L);
  st = check_ws(ws, ws_bytes, L);
  if (st != TWL_OK) return st;
  st = check_device();
  if (st != TWL_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const CacheView c = make_view(cache);
  // the cluster stage again (the same kernels and inputs select the same clusters as the decode did)
  TWL_TRY(launch_cluster_scores_topp(c, static_cast<const uint16_t*>(q), sm_scale, p1, iters,
                                     static_cast<const uint16_t*>(centroids), csize, num_clusters, (int)cpad,
                                     at<float>(ws, L.logits), at<float>(ws, L.thr), at<uint32_t>(ws, L.masks),
                                     QDigits{}, s));
  return hip_status(launch_cluster_approx(c, at<float>(ws, L.logits), at<uint32_t>(ws, L.masks), (int)cpad, csize,
                                          num_clusters, vmean, out, lse, at<float>(ws, L.apart), s));
}

twl_status twl_decode_clusters(const twl_cache* cache, const void* q, const twl_decode_params* params, float p1,
                               const void* centroids, const int32_t* csize, const int32_t* coff,
                               int32_t num_clusters, float* out, float* lse, float* threshold, int32_t* sel_indptr,
                               int32_t* sel_tokens, int64_t capacity, void* ws, size_t ws_bytes, void* stream,
                               void* const* events) {
  const TraceRange trace_("twl_decode_clusters");
  return decode_clusters_impl(cache, q, params, p1, centroids, csize, coff, num_clusters, out, lse, threshold,
                              sel_indptr, sel_tokens, capacity, ws, ws_bytes, stream, events);
}

const char* twl_status_str(twl_status status) {
  switch (status) {
    case TWL_OK: return "TWL_OK: success";
    case TWL_EINVAL: return "TWL_EINVAL: invalid argument";
    case TWL_EUNSUPPORTED: return "TWL_EUNSUPPORTED: unsupported shape or device (needs gfx950, head_dim 128, page 16, group 32, G in {1,2,4,8})";
    case TWL_EWORKSPACE: return "TWL_EWORKSPACE: workspace missing, misaligned or too small";
    case TWL_EHIP: return "TWL_EHIP: HIP launch failed";
  }
  return "unknown twl_status";
}

#ifndef TWL_SOURCE_HASH
#define TWL_SOURCE_HASH "unknown"
#endif
const char* twl_version(void) { return "twl 0.2.0 (gfx950) src " TWL_SOURCE_HASH; }

int32_t twl_keep_pages(int32_t num_pages, float keep_frac) {
  if (!finite(keep_frac) || !(keep_frac > 0.f)) return -1;
  return keep_count(num_pages, keep_frac);
}

}  // extern "C"
