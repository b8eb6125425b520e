// Internal declarations shared by the HIP translation units of libtwl (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "twl.h"

namespace twl {

constexpr int kD = 128;     // head dim
constexpr int kPage = 16;   // tokens per page
constexpr int kGroups = 4;  // 32-channel quantisation groups per key row

// Device-side view of the paged cache (plain values, passed by value to kernels).
struct CacheView {
  int B, Hq, Hkv, G, maxP, nphys, maxTok;
  int kbits;  // code width of k4 (2, 4 or 8): rows of 16 * kbits bytes
  const int32_t* page_table;
  const int32_t* seq_lens;
  const uint16_t* k;
  const uint16_t* v;
  uint8_t* k4;
  uint32_t* k4_meta;  // per (row, group): scale bits | zero bits << 16
  uint16_t* kbound;
};

// Candidate enumeration of a unit (b, kv-head).
enum CandMode : int { kCandAll = 0, kCandPages = 1, kCandRanges = 2 };
struct CandView {
  int mode;
  const int32_t* items;         // page ids [U][max_items] or ranges [U][max_items][2]
  const int32_t* count;         // [U]
  const int32_t* range_prefix;  // [U][max_items+1] (ranges only; written by launch_range_prefix)
  const int32_t* chunk_first;   // [U][ncap/kEstCands] (ranges only): range holding each block's first candidate
  int max_items;
  const int32_t* phys;          // pages only, optional: physical page of each listed page id
  const uint32_t* slot_mask;    // optional: which of a page's 16 slots are candidates -- per listed page
                                // (pages) or per page of the sequence, [U][maxP] (all tokens)
};

// Wide top-p (more than 65536 candidates per head): per-head state in 64-bit words -- the first
// histogram level (fine bins, then one coarse sum per 32 bins) and the count of histogram blocks
// done (both zero before the first pass),
// the largest logit M, the resolved first level (the key from which a weight is surely kept, the key
// from which it is recorded, the logit bounds that decide most candidates without their weight,
// total mass, mode, bin, remainder), the kept mass and the threshold.
constexpr int kWideChunk = 4096;  // candidates per chunk of the wide kernels
constexpr int kWideThreads = 256;      // threads of the union emit pass
constexpr int kWidePassThreads = 1024;  // threads of the histogram and mask passes
constexpr int kWideBlockChunks = 4;  // chunks per block of the histogram pass (software-pipelined)
constexpr int kWideAlign = kWideChunk * kWideBlockChunks;  // wide candidate capacities are multiples
constexpr int kWideH1 = 0, kWideC1 = 2048, kWideTicket = 2112, kWideZeroWords = 2113;
// adjacent, read together per head by the mask pass
constexpr int kWideSM = 2113, kWideSKeep = 2114, kWideSLo = 2115, kWideSA = 2116, kWideSB = 2117;
constexpr int kWideSZ = 2118, kWideSMode = 2119, kWideSB1 = 2120, kWideSR1 = 2121, kWideMass = 2122, kWideST = 2123;
constexpr int kWideStateWords = 2124;
constexpr int kNarrowMaxCands = 65536;      // largest candidate count of the register-resident top-p
constexpr int kWideMaxCands = 1 << 22;      // fixed-point mass bound
struct WideWs {
  float* pmax;         // [B*Hq][ncap / (64 * est_batches)] per-estimate-block logit maxima
  uint64_t* state;     // [B*Hq][kWideStateWords]
  int32_t* chunk_cnt;  // [B*Hkv][ncap / kWideChunk]
  uint32_t* uwords;    // [B*Hkv][ncap / 32] union bitmap
  uint64_t* keys;      // [B*Hq][ncap] candidates of the first level's bin, key << 32 | candidate index,
                       // those of chunk ch from slot ch * kWideChunk on
  int32_t* rec_cnt;    // [B*Hq][ncap / kWideChunk] how many each chunk recorded
  uint64_t* chunk_mass;  // [B*Hq][ncap / kWideChunk] kept mass of each chunk's sure candidates
};
constexpr int kEstCands = 256;  // candidate block of the range starts (chunk_first); divides the estimate's blocks

// The estimate's fixed-point query, prepared once per step (by the page selection or the cluster
// scores of each unit, or by k_qdigits): per (sequence, query head) row bh and 32-channel group g,
//   dig[((bh * 4 + g) * 3 + d) * 32 + pos]  digit d (0: the 2^14 digit, 1: 2^7, 2: units) of the
//                                           channel at byte pos (the order in which the code unpack
//                                           feeds the matrix cores: a permutation within each 8)
//   meta[(bh * 4 + g) * 8 + {0, 1, 2, 3, 4}] E_g, sum_c Q_c, and the three digits' sums over the group
constexpr int kQDigits = 3;     // int8 digits of Q = 2^14 d0 + 2^7 d1 + d2
constexpr int kQFracBits = 20;  // Q_c = rne(q_c 2^(kQFracBits - E_g))
constexpr int kQMeta = 8;       // ints of meta per (row, group)
struct QDigits {
  uint8_t* dig;   // [B*Hq][4][3][32]
  int32_t* meta;  // [B*Hq][4][8]
};
// 64-candidate batches per estimate block for a candidate capacity and unit count (2 or 8)
int est_batches(int64_t ncap, int64_t units);

// Token list of each unit for the attention stage: either padded rows (stride) with counts, or CSR.
struct ListView {
  const int32_t* tokens;
  const int32_t* rows;    // K/V row index per listed token (same indexing as tokens), or nullptr
  const int32_t* indptr;  // [U+1] when CSR, else nullptr
  const int32_t* counts;  // [U] when padded, else nullptr
  int64_t stride;         // row stride when padded
  int64_t cap;            // CSR: entries the tokens/rows arrays hold (0 when padded)
};

constexpr int kPartFloats = 4 + kD;  // per (chunk, head): max, sum, 2 pad, output row (16-byte aligned)
// Second level of the chunk merge: up to kMergeSplits blocks per (unit, head), each leaving one
// record (same layout as a chunk partial), and a ticket per (unit, head) that the attention kernel
// clears and the merge counts its finished splits with.
constexpr int kMergeSplits = 16;
struct MergeWs {
  float* part;      // [B*Hq][kMergeSplits][kPartFloats]
  int32_t* ticket;  // [B*Hq]
};
// ---- launchers (each returns the launch status) --------------------------------------------------
hipError_t launch_quantize(const CacheView& c, const int32_t* tok_begin, const int32_t* tok_end,
                           int span_pages, hipStream_t s);
hipError_t launch_page_score(const CacheView& c, const uint16_t* q, float* scores, hipStream_t s);
// the query digits of every (sequence, query head) alone
hipError_t launch_qdigits(const CacheView& c, const uint16_t* q, const QDigits& qd, hipStream_t s);
// page top-K; with qd.dig non-null each unit's block also writes the unit's query digits
hipError_t launch_page_select(const CacheView& c, const float* scores, float keep_frac, int max_keep, int32_t* page_phys,
                              int32_t* page_ids, int32_t* count, const uint16_t* q, const QDigits& qd, hipStream_t s);
hipError_t launch_range_prefix(const CacheView& c, const CandView& cand, int32_t* prefix, int32_t* chunk_first,
                               int nchunk, hipStream_t s);
// wide: when non-null, the estimate also writes the per-block logit maxima and clears the wide state;
// cand_tok may be null when no union list is emitted afterwards
hipError_t launch_estimate(const CacheView& c, const QDigits& qd, float sm, const CandView& cand, int ncap,
                           float* logits, int32_t* cand_tok, const WideWs* wide, hipStream_t s);
// wide top-p: histogram passes and masks (union bitmap in wd.uwords); the emit kernel writes the
// compacted union lists and the threshold/mass outputs
// full: the mask pass also writes the head masks, the kept mass and the per-chunk union counts
// (needed by head_mask, the mass output and the union lists); otherwise union words only
hipError_t launch_topp_wide(const CacheView& c, const WideWs& wd, const float* logits, int ncap, float p, int iters,
                            float* threshold, uint32_t* head_mask, int mask_words, bool full, hipStream_t s);
hipError_t launch_wide_emit(const CacheView& c, const WideWs& wd, const int32_t* cand_tok, int ncap,
                            int32_t* union_tok, int32_t* union_cnt, float* mass, hipStream_t s);
hipError_t launch_topp_weighted(const CacheView& c, const float* logits, int ncap, float p, int iters, float* threshold,
                                uint32_t* mask_ws, const int32_t* mult, int mult_stride, hipStream_t s);
// cluster scores (size-weighted logits) and the per-head cluster top-p (head masks in mask_ws); with
// qd.dig non-null the score blocks also write the query digits of the token-level estimate
hipError_t launch_cluster_scores_topp(const CacheView& c, const uint16_t* q, float sm, float p1, int iters,
                                      const uint16_t* centroids, const int32_t* csize, int C, int cpad, float* lam,
                                      float* thr, uint32_t* mask_ws, const QDigits& qd, hipStream_t s);
// union of a unit's head masks -> kept ranges (first token, length) and count; with prefix non-NULL
// also the ranges' prefix sums [U][C + 1] and the range of each 256-candidate block [U][nchunk]
// optional approximation of unkept clusters: mean value rows [B*Hkv][C][128], then the merge into
// out / lse of every (sequence, query head) from the cluster logits and head masks of the cluster stage
hipError_t launch_cluster_vmean(const CacheView& c, const int32_t* csize, const int32_t* coff, int C, float* vmean,
                                hipStream_t s);
hipError_t launch_cluster_approx(const CacheView& c, const float* lam, const uint32_t* masks, int cpad,
                                 const int32_t* csize, int C, const float* vmean, float* out, float* lse, float* part,
                                 hipStream_t s);
constexpr int kApproxSlices = 16;       // cluster slices per head in the approximation's first pass
constexpr int kApproxStride = 128 + 4;  // floats per slice partial: 128 sums, the weight sum, M
hipError_t launch_cluster_union(const CacheView& c, const uint32_t* mask_ws, int cpad, const int32_t* csize,
                                const int32_t* coff, int C, int32_t* ranges, int32_t* count, int32_t* prefix,
                                int32_t* chunk_first, int nchunk, hipStream_t s);
// union of a unit's head masks -> the mask of kept token slots of every page ([U][maxP], page-indexed;
// 0 for pages past the sequence): the token-level candidates as every page with such a mask
hipError_t launch_cluster_slots(const CacheView& c, const uint32_t* mask_ws, int cpad, const int32_t* csize,
                                const int32_t* coff, int C, uint32_t* smask, hipStream_t s);
// topk > 0: keep each head's topk largest weights (ties kept) instead of its top-p set
hipError_t launch_topp(const CacheView& c, const float* logits, int ncap, float p, int iters, float* threshold,
                       float* mass, uint32_t* mask_ws, uint32_t* head_mask, int mask_words, int topk, hipStream_t s);
hipError_t launch_union(const CacheView& c, const uint32_t* mask_ws, const int32_t* cand_tok, int ncap,
                        int32_t* union_tok, int32_t* union_cnt, hipStream_t s);
hipError_t launch_csr_emit(const CacheView& c, const int32_t* union_tok, const int32_t* union_cnt, int ncap,
                           int32_t* indptr, int32_t* tokens, int64_t capacity, hipStream_t s);
// tokens per attention chunk for an upper bound of the total selected tokens
int attn_chunk_tokens(int64_t total_upper, int group);
// Kept candidates given as bitmaps over the candidate index space (the top-p output), with the K/V
// row of every candidate: the attention then reads no compacted list.
struct MaskView {
  const uint32_t* head_masks;   // [B*Hq][ncap/32] per-head bitmaps (OR-ed over the group), or
  const uint32_t* union_words;  // [B*Hkv][ncap/32] union bitmaps (used when non-null)
  int cand_mode;                // kCandPages / kCandAll: rows from the page list / the page table
  const int32_t* page_phys;     // [B*Hkv][page_stride] physical page of each kept page (pages)
  int page_stride;
  int64_t ncap;
};
// one workgroup per chunk slot: slot k of unit u covers list entries [k*chunk_tokens, (k+1)*chunk_tokens)
hipError_t launch_attn(const CacheView& c, const uint16_t* q, float sm, const ListView& list, int chunk_tokens,
                       int slots, float* partials, const MergeWs& mw, hipStream_t s);
// one workgroup per chunk slot of the candidate space (every slot writes a partial); headwise: each
// query head attends over its own bitmap's tokens (needs head_masks) instead of the group's union
hipError_t launch_attn_masked(const CacheView& c, const uint16_t* q, float sm, const MaskView& mv, int chunk_tokens,
                              int slots, float* partials, const MergeWs& mw, bool headwise, hipStream_t s);
// K/V rows of a CSR token list (into `rows`, same indexing), entries at or past `capacity` skipped
hipError_t launch_rows(const CacheView& c, const int32_t* indptr, const int32_t* tokens, int32_t* rows,
                       int64_t capacity, hipStream_t s);
// list: chunks per unit from the list counts; list == nullptr: every slot holds a partial
hipError_t launch_merge(const CacheView& c, const ListView* list, int chunk_tokens, int slots, const float* partials,
                        const MergeWs& mw, float* out, float* lse, hipStream_t s);
// elements per thread of the top-p block for a candidate capacity (0 = unsupported)
int topp_elems_per_thread(int64_t ncap);
constexpr int kToppThreads = 1024;

// ---- the decode entry point's host side, shared with its allocation-free variant ------------------
// Validates a decode call (everything but the workspace, no HIP call) and gives the workspace bytes it
// needs.
twl_status decode_workspace_need(const twl_cache* cache, const void* q, const twl_decode_params* params,
                                 const float* out, const int32_t* sel_indptr, const int32_t* sel_tokens,
                                 int64_t capacity, size_t* need);
// twl_decode on the given workspace.
twl_status decode_with_workspace(const twl_cache* cache, const void* q, const twl_decode_params* params, float* out,
                                 float* lse, float* threshold, int32_t* sel_indptr, int32_t* sel_tokens,
                                 int64_t capacity, void* ws, size_t ws_bytes, void* stream);

}  // namespace twl
