/*
 * twl.h -- C ABI of the top-p sparse decode attention library (HIP, gfx950 / MI355X).
 *
 * The library implements the decode-time select-then-prune path of Twilight ("Twilight: Adaptive
 * Attention Sparsity with Hierarchical Top-p Pruning", arXiv 2502.02770):
 *   base page selector (Quest-style key bounds) -> INT4-K weight estimate -> per-head top-p
 *   pruning (binary search of the weight threshold, no sort) -> sparse attention on the survivors,
 * and the cluster-level first stage of Double-P ("Double-P: Hierarchical Top-P Sparse Attention for
 * Long-Context LLMs").  Citations below name the page and the section they follow.
 *
 * Conventions (apply to every entry point)
 * ---------------------------------------
 * - Every pointer argument is a DEVICE pointer owned by the caller, unless it is a pointer to one of
 *   the structs below or to twl_decode_params, which are read on the host during the call only.
 *   The query q must be 16-byte aligned (TWL_EINVAL otherwise; any hipMalloc/torch allocation is).
 * - The library never allocates, frees or synchronises.  Calls enqueue kernels on `stream` (a
 *   hipStream_t; NULL = the default stream) and return once enqueued.  Scratch memory is the
 *   caller's workspace `ws` (>= 256-byte aligned, `ws_bytes` long, contents need not be initialised);
 *   size it with twl_workspace_bytes().  A workspace must not be shared by calls that may run
 *   concurrently.
 * - Arguments are validated synchronously on the host BEFORE any HIP call.  On a non-TWL_OK return
 *   nothing has been enqueued and no output has been written.  Device-resident values (seq_lens,
 *   page tables, candidate lists) cannot be validated on the host: out-of-range values there are
 *   skipped by the kernels where stated, otherwise the behaviour is undefined.
 * - TWL_EUNSUPPORTED: head_dim != 128, page_size != 16, quant_group != 32, key_bits not in
 *   {0, 2, 4, 8}, a GQA group size not in {1, 2, 4, 8}, or a current device that is not gfx950.  TWL_EHIP: a kernel launch failed (the
 *   HIP error is left for hipGetLastError()).  Device faults surface at the caller's next
 *   synchronisation.
 * - Results are deterministic: the same inputs give bitwise identical outputs on every run.  The
 *   fused entry points select bitwise the same pages, top-p sets and thresholds as the split entry
 *   points; their attention outputs agree to float32 rounding (the work is partitioned differently).
 *
 * Data layout of the paged cache (B = batch, Hq/Hkv = query/KV heads, G = Hq/Hkv)
 * ------------------------------------------------------------------------------
 *   k, v      bf16 [num_phys_pages][Hkv][16][128]     token t of sequence b: physical page
 *                                                     page_table[b][t/16], slot t%16
 *   k4        u8   [B][max_pages_per_seq][Hkv][16][16*kb]   key codes of token t of sequence b at
 *                                                     [b][t/16][.][t%16], kb = key_bits bits, 8/kb per byte
 *                                                     with the lowest channel in the lowest bits (kb = 4:
 *                                                     byte j = code(2j) | code(2j+1)<<4)
 *   k4_meta   fp16 [B][max_pages_per_seq][Hkv][16][4][2]  per 32-channel group: (scale, zero)
 *   kbound    bf16 [B][max_pages_per_seq][Hkv][4][2][32] per logical page: channel-wise key min and max,
 *                                                     by channel quarter (32 channels of min, then the
 *                                                     same 32 of max: one 128-byte line per quarter)
 *   The INT4 shadow is the library's own derived data: it is stored by (sequence, logical page), not
 *   paged, so that the page selector and the weight estimate address it without a page-table lookup
 *   (only the attention, which reads the paged K and V, translates pages).
 *   q         bf16 [B][Hq][128]; query head hq belongs to kv-head hq / G
 */
#ifndef TWL_H
#define TWL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum twl_status {
  TWL_OK = 0,
  TWL_EINVAL = 1,        /* an argument is out of its documented range or a required pointer is NULL */
  TWL_EUNSUPPORTED = 2,  /* a shape or device this library does not implement                      */
  TWL_EWORKSPACE = 3,    /* ws is NULL, misaligned or smaller than twl_workspace_bytes()             */
  TWL_EHIP = 4           /* a HIP launch failed                                                      */
} twl_status;

/* The paged KV cache of one decode layer and its INT4 shadow (layouts above). */
typedef struct twl_cache {
  int32_t batch;              /* B >= 1                                                          */
  int32_t num_q_heads;        /* Hq >= 1                                                         */
  int32_t num_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0, G = Hq/Hkv in {1,2,4,8}                */
  int32_t head_dim;           /* must be 128                                                     */
  int32_t page_size;          /* must be 16                                                      */
  int32_t quant_group;        /* must be 32                                                      */
  int32_t max_pages_per_seq;  /* row stride of page_table, >= 1                                  */
  int32_t num_phys_pages;     /* >= 1                                                            */
  int32_t max_seq_len;        /* host upper bound of seq_lens[b], <= 16 * max_pages_per_seq      */
  const int32_t* page_table;  /* [B][max_pages_per_seq] logical page -> physical page            */
  const int32_t* seq_lens;    /* [B] tokens per sequence, 0 <= seq_lens[b] <= max_seq_len         */
  const void* k;              /* bf16 keys                                                       */
  const void* v;              /* bf16 values                                                     */
  void* k4;                   /* key codes, key_bits wide (written by twl_quantize_k)            */
  void* k4_meta;              /* fp16 scale/zero (written by twl_quantize_k)                     */
  void* kbound;               /* bf16 page key bounds (written by twl_quantize_k)                */
  int32_t key_bits;           /* code width of k4: 4 (0 means 4), or 2 / 8 for the estimator's    */
                              /* precision ablation (paperlayer §4.2, Fig. 6)                    */
} twl_cache;

/* Candidate tokens of each (sequence b, kv-head h) unit, i.e. the base selector's output.
 * Exactly one of page_ids / ranges may be non-NULL; both NULL means every token of the sequence.
 *   page_ids  [B][Hkv][max_items]     ascending logical page ids; candidates = their valid slots
 *   ranges    [B][Hkv][max_items][2]  (token_begin, length), ascending and non-overlapping
 *   count     [B][Hkv]                items used per unit (<= max_items)
 * Candidate index k of a unit enumerates the items' tokens in order; slots at or past seq_lens[b]
 * (and page ids >= ceil(seq_lens[b]/16)) are not candidates. */
typedef struct twl_candidates {
  const int32_t* page_ids;
  const int32_t* ranges;
  const int32_t* count;
  int32_t max_items;
} twl_candidates;

typedef struct twl_decode_params {
  float p;          /* top-p threshold, 0 < p <= 1 (p = 1 keeps every candidate)                    */
  float keep_frac;  /* base selector budget as a fraction of pages, > 0 (>= 1: no selector)         */
  float sm_scale;   /* softmax scale, finite (usually 1/sqrt(128))                                 */
  int32_t iters;    /* bisection steps, 1..64 (32 always converges)                                 */
  /* Baselines the pages compare top-p against (paperlayer §3, Fig. 2-3; §B.2 on GQA); 0 = off.
   * topk > 0: each head keeps its topk largest estimated weights (ties at the topk-th kept) instead
   *   of its top-p set; p is then unused.  The search counts only weights of at least 2^-40 of the
   *   head's largest, so when fewer than topk weights reach that, every candidate is kept.
   * headwise = 1: each query head attends over its own kept set instead of the group's union (the
   *   union's rows are still read once per group).
   * Both need at most 65536 candidates per group (TWL_EUNSUPPORTED otherwise, and in
   * twl_decode_clusters); negative topk or headwise outside {0, 1}: TWL_EINVAL. */
  int32_t topk;
  int32_t headwise;
} twl_decode_params;

/* Number of stages twl_decode_profiled() brackets with events (see there). */
#define TWL_NUM_STAGES 6

/* Workspace size, in bytes, sufficient for every entry point on `cache` when no unit has more than
 * `max_candidates_per_group` candidates (for twl_decode: 16 * ceil(keep_frac * max_pages_per_seq),
 * or 16 * max_pages_per_seq without a selector; for ranges: max_seq_len).  Returns 0 when `cache`
 * fails validation, or when max_candidates_per_group is negative or above the top-p capacity of 2^22
 * candidates per unit (no entry point accepts such a unit). */
size_t twl_workspace_bytes(const twl_cache* cache, int64_t max_candidates_per_group);

/* INT4 K cache append (Twilight 4-bit K cache: Paper-Notes "关键设计 / 4-bit K缓存量化";
 * paperlayer §4.2 and §B.1 -- dynamic quantisation with fp16 scales and zero points, two 4-bit
 * values per byte).  For every sequence b and token t in [tok_begin[b], tok_end[b]) and every
 * kv-head: asymmetric min/max quantisation of each 32-channel group of the bf16 key row,
 *   scale = fp16_rne(fp32(max-min)/L), zero = fp16_rne(min), L = 2^key_bits - 1 (15 for 4 bits),
 *   code  = 0 if scale == 0 else clamp(rint_even(fp32(x-zero)/scale), 0, L),
 * written to k4 / k4_meta; and for every page the range touches, kbound = channel-wise min and max
 * over the page's slots holding tokens < tok_end[b] (the Quest-style page bound).
 *   tok_begin, tok_end  device int32 [B]; 0 <= tok_begin <= tok_end <= 16*max_pages_per_seq
 *                       (units violating this are skipped)
 *   max_span            host bound of max_b (tok_end[b] - tok_begin[b]), >= 0; sizes the grid
 * Keys must be finite with |x| <= 65504 (fp16 range); otherwise the codes are undefined. */
twl_status twl_quantize_k(const twl_cache* cache, const int32_t* tok_begin, const int32_t* tok_end,
                          int32_t max_span, void* stream);

/* Base selector (Paper-Notes "整体框架": a generous budget, e.g. 1/4; paperlayer §4.1 Fig. 5),
 * Quest-style: page score of query head h = sum_c max(q_c*kmin_c, q_c*kmax_c); the group score,
 * their sum over the G heads, equals sum_c (P_c*kmax_c + N_c*kmin_c) with P_c / N_c the heads'
 * max(q_c, 0) / min(q_c, 0) summed in float32 in head order, and is evaluated so: one float32
 * left-to-right fold over c from +0 adding P_c*kmax_c, then N_c*kmin_c, each rounded once (fused
 * multiply-add); keep K_b = clamp(ceil(fp32(keep_frac)*fp32(P_b)), 1, P_b) pages
 * (P_b = ceil(seq_lens[b]/16), 0 if empty) with the largest group score, ties to the lower page id;
 * list them ascending.
 *   q          bf16 [B][Hq][128]
 *   keep_frac  > 0, finite
 *   max_keep   row stride of page_ids, >= clamp(ceil(keep_frac*max_pages_per_seq), 1, max_pages_per_seq)
 *   page_ids   int32 [B][Hkv][max_keep] (out; entries past count are left untouched)
 *   count      int32 [B][Hkv] (out) */
twl_status twl_select_pages(const twl_cache* cache, const void* q, float keep_frac, int32_t max_keep,
                            int32_t* page_ids, int32_t* count, void* ws, size_t ws_bytes, void* stream);

/* Weight estimate + top-p pruning + GQA union (Twilight pruner).
 * - Estimate (paperlayer §4.2, §B.1: mixed-precision SpGEMV of the query against dequantised INT4
 *   keys): logit_i = sm_scale * sum_c q_c * (code_ic * s_g + z_g), the query's bf16 values against the
 *   exactly dequantised keys (fp16 scale s_g and zero z_g per 32-channel group g).  The query is held
 *   per head and group in fixed point,
 *     E_g = floor(log2 max_{c in g} |q_c|) (>= -100),  Q_c = rne(q_c * 2^(20 - E_g)),
 *   which is exact for every channel within 2^12 of its group's largest magnitude (so for ordinary
 *   bf16 queries q~ = q); the group sums sum_c Q_c*code_c are exact integers, the rest is float64 --
 *     t_g = s_g*a_g + z_g*b_g,  a_g = 2^(E_g-20) sum Q_c*code_c,  b_g = 2^(E_g-20) sum Q_c,
 *     logit = float32(sm_scale * ((t_0 + t_1) + (t_2 + t_3)))
 *   -- so the logit is the exact estimate for the grid query, rounded once to float32.
 * - Weights: softmax of the logits over the unit's candidates only.
 * - Top-p (Paper-Notes "关键设计 / 高效Top-p": binary search of the threshold m with
 *   sum_{W_i >= m} W_i >= p, no sort): the weights are searched on the scale where the largest is 1
 *   (e_i = exp(l_i - max l), target p * sum e); the threshold is a float32 value whose bit pattern is
 *   bisected over [0, 2^31), one bit per step from the top, keeping the largest threshold whose kept
 *   mass still reaches the target; the kept set is {e_i >= m}.  p = 1 keeps every candidate.  With
 *   iters >= 31 the search has converged: the set is the minimal top-p set up to ties and the
 *   precision of the weights; fewer steps keep the threshold's top `iters` bits, a superset whose
 *   mass still reaches p.  Masses are summed in 64-bit fixed point (2^-40 units of the largest
 *   weight; weights below 2^-40 of it carry no mass).  The search decides 11 bits per pass from mass
 *   histograms; above 65536 candidates per unit (up to 2^22) the first pass runs over all the weights
 *   in many blocks and the remaining 20 bits over the keys inside the chosen bin.
 * - Union (paperlayer §B.2): the kept tokens of a unit are the union over its G query heads.
 * Outputs:
 *   threshold  f32 [B][Hq]   the weight threshold m (required)
 *   mass       f32 [B][Hq]   estimated weight mass of the head's kept set, or NULL
 *   head_mask  u32 [B][Hq][mask_words], bit k%32 of word k/32 = candidate k kept by that head, or NULL;
 *              mask_words >= ceil(max candidates per unit / 32)
 *   sel_indptr int32 [B*Hkv+1] CSR offsets (unit u = b*Hkv + h)
 *   sel_tokens int32 [capacity] logical token ids, ascending within each unit
 *   capacity   >= B*Hkv*(max candidates per unit) */
twl_status twl_estimate_topp(const twl_cache* cache, const void* q, float sm_scale, float p, int32_t iters,
                             const twl_candidates* cand, float* threshold, float* mass,
                             uint32_t* head_mask, int32_t mask_words, int32_t* sel_indptr,
                             int32_t* sel_tokens, int64_t capacity, void* ws, size_t ws_bytes,
                             void* stream);

/* Sparse attention over the kept tokens (Paper-Notes "整体框架"; paperlayer §4.1, §B.2: group-wise
 * variable-length attention on the flattened paged cache).  Every query head of unit u attends over
 * the unit's token list: out = sum_i softmax_i(sm*q.k_i) v_i (bf16 K/V, fp32 accumulation),
 * lse = ln sum_i exp(sm*q.k_i).  An empty list gives out = 0, lse = -inf.  Token ids outside
 * [0, seq_lens[b]) are skipped.
 *   sel_indptr, sel_tokens  CSR as produced by twl_estimate_topp (any token order works)
 *   max_selected_per_group  host bound of the longest unit list, >= 0
 *   out  f32 [B][Hq][128];  lse  f32 [B][Hq] or NULL */
twl_status twl_sparse_attn(const twl_cache* cache, const void* q, float sm_scale, const int32_t* sel_indptr,
                           const int32_t* sel_tokens, int32_t max_selected_per_group, float* out, float* lse,
                           void* ws, size_t ws_bytes, void* stream);

/* The whole decode step for one layer, Twilight's select-then-prune path (Paper-Notes "整体框架";
 * paperlayer §4.1, Fig. 5: an existing selector with a generous budget, then top-p pruning of its
 * candidates, then sparse attention): twl_select_pages (skipped when keep_frac >= 1), then
 * twl_estimate_topp over the kept pages, then the sparse attention over the union.  Pages, top-p
 * sets and thresholds are bitwise those of the split calls; the attention reads the top-p bitmaps
 * directly (chunks of the candidate index space), so its outputs agree with twl_sparse_attn on the
 * same kept list to float32 rounding.
 *   q          bf16 [B][Hq][128], 16-byte aligned
 *   params     p, keep_frac, sm_scale, iters and the baseline switches (see twl_decode_params)
 *   out        f32 [B][Hq][128] (required); lse f32 [B][Hq] (natural log) or NULL
 *   threshold  f32 [B][Hq] the weight threshold (W scale) or NULL
 *   sel_indptr int32 [B*Hkv+1] and sel_tokens int32 [capacity]: the kept tokens' CSR, or both NULL
 *              (the kept list is then not compacted at all and capacity is ignored);
 *              capacity >= B*Hkv*(max candidates per unit)
 *   ws, ws_bytes  workspace of twl_workspace_bytes(cache, max candidates per unit)
 * Errors: TWL_EINVAL for p outside (0, 1], keep_frac <= 0, a non-finite scale, iters outside 1..64,
 * a misaligned q, or only one of sel_indptr / sel_tokens; TWL_EWORKSPACE for a small or misaligned
 * workspace; nothing is enqueued then. */
twl_status twl_decode(const twl_cache* cache, const void* q, const twl_decode_params* params, float* out,
                      float* lse, float* threshold, int32_t* sel_indptr, int32_t* sel_tokens, int64_t capacity,
                      void* ws, size_t ws_bytes, void* stream);

/* twl_decode without a workspace argument, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The workspace is a static
 * device array of TWL_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until the
 * process ends; its device address is looked up once per device, on the first call there.  Calls
 * whose twl_workspace_bytes() would exceed that size return TWL_EWORKSPACE before any HIP call (the
 * Llama-shaped layer, B = 1, 32/8 heads, 32K context with a 1/4 page budget, needs 3.3 MiB; B = 16 at
 * 32K 47 MiB, B = 4 at 128K 41 MiB).  Everything else is as for twl_decode, with the same
 * kernels and bitwise the same outputs.  This function allocates nothing; calls that overlap on one
 * GPU share the array and race, so serialise them (one stream, or events). */
#define TWL_NOALLOC_SCRATCH_BYTES (64u << 20)
twl_status twl_decode_noalloc(const twl_cache* cache, const void* q, const twl_decode_params* params, float* out,
                              float* lse, float* threshold, int32_t* sel_indptr, int32_t* sel_tokens,
                              int64_t capacity, void* stream);

/* twl_decode with timing hooks: `events` holds 2*TWL_NUM_STAGES hipEvent_t created by the caller;
 * events[2i] / events[2i+1] are recorded on `stream` immediately before / after stage i's kernel:
 * 0 page scoring, 1 page top-K, 2 INT4 estimate, 3 top-p + union, 4 split-K attention, 5 merge.
 * Stages that do not run (no selector) record both events back to back. */
twl_status twl_decode_profiled(const twl_cache* cache, const void* q, const twl_decode_params* params,
                               float* out, float* lse, float* threshold, int32_t* sel_indptr,
                               int32_t* sel_tokens, int64_t capacity, void* ws, size_t ws_bytes,
                               void* stream, void* const* events);

/* Double-P first stage ("Double-P", 方法详解: coarse cluster-level top-p on size-weighted
 * centroids).  Per query head: cluster logit l_c = fl(sm * fold_c'(acc + q_c' mu_c,c')) (float32
 * from +0), weight u_c = n_c exp(l_c - M) / sum (M = largest logit of a non-empty cluster), top-p
 * over the clusters with the same bisection as twl_estimate_topp; then the union over the GQA
 * group, written as (begin, length) ranges of the kept non-empty clusters in ascending order --
 * the `ranges` candidate form of twl_estimate_topp.
 *   centroids  bf16 [B][Hkv][num_clusters][128]; csize int32 [B][Hkv][num_clusters];
 *   coff       int32 [B][Hkv][num_clusters+1] token offsets (cluster c = tokens coff[c]..coff[c+1]-1)
 *   ranges     int32 [B][Hkv][num_clusters][2] (out);  count int32 [B][Hkv] (out)
 *   num_clusters  1..65536; the workspace is sized by twl_workspace_bytes(cache, m), m >= num_clusters */
twl_status twl_select_clusters_topp(const twl_cache* cache, const void* q, float sm_scale, float p1,
                                    int32_t iters, const void* centroids, const int32_t* csize,
                                    const int32_t* coff, int32_t num_clusters, int32_t* ranges,
                                    int32_t* count, void* ws, size_t ws_bytes, void* stream);

/* Optional approximation of the clusters that no head of a group keeps (the Double-P abstract refines
 * to token level only where the cluster level does not suffice; the pages give no formula, so this
 * reading is an option and twl_decode_clusters does not apply it): a cluster c not kept enters the
 * softmax as its n_c members collapsed onto (centroid mu_c, mean value vbar_c).
 * twl_cluster_value_means: vbar_c of every cluster, the float32 mean of its value rows in token order
 *   (tokens outside the sequence are skipped; an empty cluster gets zeros), at cache-append time.
 *   csize, coff as in twl_select_clusters_topp; vmean float32 [B][Hkv][num_clusters][128] (out).
 * twl_cluster_approx_unkept: after twl_decode_clusters with the same cache, q, sm_scale, p1, iters,
 *   centroids and csize, merges into its out / lse (in place, natural-log lse) the unkept non-empty
 *   clusters: with l_c the cluster logit and M = max(lse, max_c (l_c + ln n_c)),
 *     den = exp(lse - M) + sum_c n_c exp(l_c - M),  out <- (exp(lse - M) out + sum_c n_c exp(l_c - M)
 *     vbar_c) / den,  lse <- M + ln den.
 *   It repeats the cluster stage in `ws` (sized by twl_workspace_bytes(cache, m), m >= num_clusters),
 *   so it selects the decode's clusters; heads whose group keeps every cluster are left unchanged. */
twl_status twl_cluster_value_means(const twl_cache* cache, const int32_t* csize, const int32_t* coff,
                                   int32_t num_clusters, float* vmean, void* stream);
twl_status twl_cluster_approx_unkept(const twl_cache* cache, const void* q, float sm_scale, float p1, int32_t iters,
                                     const void* centroids, const int32_t* csize, int32_t num_clusters,
                                     const float* vmean, float* out, float* lse, void* ws, size_t ws_bytes,
                                     void* stream);

/* The whole Double-P decode step ("Double-P", 方法详解 and 关键设计): the cluster stage of
 * twl_select_clusters_topp with p1, then the token-level estimate and top-p with params->p
 * (keep_frac is ignored) over the kept clusters' tokens, then the sparse attention over the union.
 * The candidates are the same tokens as twl_estimate_topp over the kept ranges (so are the kept sets
 * and token lists); here they are handed on as the pages the kept clusters touch, each with a mask
 * of its kept slots.  Unkept clusters are dropped.  Requires 2*num_clusters <= max_seq_len rounded up
 * to the top-p capacity; the workspace is twl_workspace_bytes(cache, max_seq_len).  `events` is NULL
 * or holds 2*TWL_NUM_STAGES events as for twl_decode_profiled, the stages being 0 cluster scores +
 * cluster top-p, 1 kept clusters as pages, 2 INT4 estimate, 3 token top-p + union, 4 attention,
 * 5 merge. */
twl_status twl_decode_clusters(const twl_cache* cache, const void* q, const twl_decode_params* params, float p1,
                               const void* centroids, const int32_t* csize, const int32_t* coff,
                               int32_t num_clusters, float* out, float* lse, float* threshold, int32_t* sel_indptr,
                               int32_t* sel_tokens, int64_t capacity, void* ws, size_t ws_bytes, void* stream,
                               void* const* events);

/* Static description of a status code. */
const char* twl_status_str(twl_status status);

/* Library version string: "twl <version> (gfx950) src <hash>", the hash identifying the kernel and
 * ABI sources the library was built from. */
const char* twl_version(void);

/* The base selector's page budget for a sequence of num_pages pages (Paper-Notes "整体框架": a
 * generous budget such as 1/4 of the pages): clamp(ceil(fp32(keep_frac) * fp32(num_pages)), 1,
 * num_pages), 0 when num_pages <= 0; -1 when keep_frac is not finite and > 0.  Host-only, no HIP
 * call: callers size page lists (max_keep) and candidate capacities with it. */
int32_t twl_keep_pages(int32_t num_pages, float keep_frac);

#ifdef __cplusplus
}
#endif

#endif /* TWL_H */
