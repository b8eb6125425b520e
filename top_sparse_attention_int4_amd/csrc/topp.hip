// Top-p pruning by binary search of the weight threshold, and the GQA union of the kept tokens.
//
// Paper-Notes "关键设计 / 高效Top-p": instead of sorting, search the threshold m with
// sum_{W_i >= m} W_i >= p; each round is one parallel pass over the weights.  One 1024-thread block
// handles one (sequence, query head); the head's weights stay in registers (E per thread).
//
// Weights are kept unnormalised, e_i = exp(l_i - M) in (0, 1] (the maximum is exactly 1), with the
// target p*Z, Z = sum e_i, which keeps the same set as comparing W_i = e_i/Z with p.  Midpoints are
// taken on the uint32 image of the non-negative float32 weights and the bracket keeps
// f(lo) >= p*Z > f(hi); the kept set is {e_i >= lo}.  The bracket starts at [min e, 1] (all of the
// mass lies at or above the smallest weight).  Candidates that do not exist carry e = -1.
//
// Two phases share that bisection.  While many weights remain inside the bracket, every step is a
// block-wide pass with one fixed-order reduction of f(mid) and #{e >= mid}; the counts at the two
// ends of the bracket give the number of weights inside it.  Once at most kCap weights are inside,
// they are compacted into LDS together with the mass above the bracket, and a single wave finishes
// the search with DPP reductions and no barriers, compacting the shrinking bracket as it goes
// (weights leaving through the top add their mass to that constant).  Rounding order differs
// between the phases but is fixed, so results are reproducible.
//
// The GQA union (paperlayer §B.2: the union over a group's query heads, read once) is a separate
// small kernel over the head masks.
#include "twl_device.h"
#include "twl_internal.h"

namespace twl {

__device__ int cand_token_topp(const CandView& cand, int u, int k, int n) {
  const int P = (n + kPage - 1) / kPage;
  if (cand.mode == kCandAll) return k < n ? k : -1;
  if (cand.mode == kCandPages) {
    const int cnt = clampi(cand.count[u], 0, cand.max_items);
    const int pi = k >> 4;
    if (pi >= cnt) return -1;
    const int page = cand.items[(size_t)u * cand.max_items + pi];
    if (page < 0 || page >= P) return -1;
    const int t = page * kPage + (k & 15);
    return t < n ? t : -1;
  }
  const int cnt = clampi(cand.count[u], 0, cand.max_items);
  const int32_t* pre = cand.range_prefix + (size_t)u * (cand.max_items + 1);
  if (k >= pre[cnt]) return -1;
  int lo = 0, hi = cnt;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= k) lo = mid; else hi = mid;
  }
  const int t = cand.items[((size_t)u * cand.max_items + lo) * 2] + (k - pre[lo]);
  return (t >= 0 && t < n) ? t : -1;
}

constexpr int kCap = 1024;  // weights handed to the single-wave phase

// One bisection step of the single-wave phase over `n` compacted weights in `buf`; compacts the kept
// bracket into `dst`, updates lo/hi and the mass above hi, and returns the new count.
__device__ __forceinline__ int wave_step(const float* buf, float* dst, int n, uint32_t& lo, uint32_t& hi,
                                         float& c_hi, float target) {
  const int lane = threadIdx.x & 63;
  const uint32_t mid = lo + ((hi - lo) >> 1);
  const float m = __uint_as_float(mid);
  float f = 0.f;
  for (int i = lane; i < n; i += 64) {
    const float x = buf[i];
    f += (x >= m) ? x : 0.f;
  }
  f = c_hi + wave_sum_dpp(f);
  const bool up = f >= target;
  const float klo = __uint_as_float(up ? mid : lo);
  const float khi = __uint_as_float(up ? hi : mid);
  float above = 0.f;
  int base = 0;
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    const float x = (i < n) ? buf[i] : -1.f;
    const bool keep = (i < n) && x >= klo && x < khi;
    if (i < n && x >= khi) above += x;
    const unsigned long long bal = __ballot(keep);
    const int pos =
        base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (keep) dst[pos] = x;
    base += __popcll(bal);
  }
  __builtin_amdgcn_wave_barrier();  // the next step reads what other lanes wrote
  c_hi += wave_sum_dpp(above);
  if (up) lo = mid; else hi = mid;
  return base;
}

template <int E>
__global__ __launch_bounds__(1024) void k_topp(CacheView c, const float* __restrict__ logits, int ncap, float p,
                                               int iters, float* threshold, float* mass, uint32_t* mask_ws,
                                               uint32_t* head_mask, int mask_words) {
  constexpr int NT = kToppThreads, NW = NT / 64;
  __shared__ float red[2 * NW * 4];
  __shared__ int scan_sm[NW + 1];
  __shared__ float buf[2][kCap];
  __shared__ uint32_t s_lo;
  BlockReduce<NW> br{red};

  const int bh = blockIdx.x;
  const float* lg = logits + (size_t)bh * ncap;
  const int tid = threadIdx.x;
  const int wv = tid >> 6;

  float e[E];
  float mloc = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int k = j * NT + tid;
    e[j] = (k < ncap) ? lg[k] : -__builtin_inff();
    mloc = fmaxf(mloc, e[j]);
  }
  const float M = br.max(mloc);
  float Z = 0.f, emin = __builtin_inff(), nval = 0.f;
  if (M != -__builtin_inff()) {
#pragma unroll
    for (int j = 0; j < E; ++j) {
      e[j] = (e[j] == -__builtin_inff()) ? -1.f : exp_diff(e[j], M);
      if (e[j] >= 0.f) {
        Z += e[j];
        emin = fminf(emin, e[j]);
        nval += 1.f;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < E; ++j) e[j] = -1.f;
  }
  br.sum_min(Z, emin);
  nval = br.sum(nval);

  uint32_t lo = 0u;
  if (Z > 0.f && p < 1.0f) {
    const float target = p * Z;
    lo = __float_as_uint(emin);                // f(min e) = Z >= target
    uint32_t hi = __float_as_uint(1.0f) + 1u;  // e <= 1 = exp(0)
    float n_lo = nval, n_hi = 0.f;             // #{e >= lo}, #{e >= hi}
    int it = 0;
    // ---- block phase -------------------------------------------------------------------------
    while (it < iters && hi - lo > 1u && n_lo - n_hi > (float)kCap) {
      const uint32_t mid = lo + ((hi - lo) >> 1);
      const float m = __uint_as_float(mid);
      float f = 0.f, cm = 0.f;
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const bool ge = e[j] >= m;
        f += ge ? e[j] : 0.f;
        cm += ge ? 1.f : 0.f;
      }
      br.sum2(f, cm);
      if (f >= target) {
        lo = mid;
        n_lo = cm;
      } else {
        hi = mid;
        n_hi = cm;
      }
      ++it;
    }
    // ---- single-wave phase --------------------------------------------------------------------
    if (it < iters && hi - lo > 1u) {
      const float mlo = __uint_as_float(lo), mhi = __uint_as_float(hi);
      int local = 0;
      float above = 0.f;
#pragma unroll
      for (int j = 0; j < E; ++j) {
        local += (e[j] >= mlo && e[j] < mhi) ? 1 : 0;
        above += (e[j] >= mhi) ? e[j] : 0.f;
      }
      int total;
      int pos = block_excl_scan<NW>(local, scan_sm, &total);
      float c_hi = br.sum(above);
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (e[j] >= mlo && e[j] < mhi) buf[0][pos++] = e[j];
      __syncthreads();
      if (wv == 0) {
        int n = min(total, kCap), cur = 0;
        while (it < iters && hi - lo > 1u && n > 0) {
          n = wave_step(buf[cur], buf[cur ^ 1], n, lo, hi, c_hi, target);
          cur ^= 1;
          ++it;
        }
        if (tid == 0) s_lo = lo;
      }
      __syncthreads();
      lo = s_lo;
    }
  }
  const float m = __uint_as_float(lo);
  float f = 0.f;
#pragma unroll
  for (int j = 0; j < E; ++j) f += (e[j] >= m) ? e[j] : 0.f;
  f = br.sum(f);
  if (tid == 0) {
    threshold[bh] = (Z > 0.f) ? m / Z : 0.f;
    if (mass) mass[bh] = (Z > 0.f) ? f / Z : 0.f;
  }

  // head mask: bit k of the head's bitmap <=> candidate k kept
  const int mw = ncap / 32;
  const int lane = tid & 63;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const unsigned long long bal = __ballot(e[j] >= m);
    const int w = (j * NT + wv * 64) / 32;
    if (lane == 0) {
      mask_ws[(size_t)bh * mw + w] = (uint32_t)bal;
      mask_ws[(size_t)bh * mw + w + 1] = (uint32_t)(bal >> 32);
      if (head_mask) {
        if (w < mask_words) head_mask[(size_t)bh * mask_words + w] = (uint32_t)bal;
        if (w + 1 < mask_words) head_mask[(size_t)bh * mask_words + w + 1] = (uint32_t)(bal >> 32);
      }
    }
  }
}

// One block per unit: OR the unit's G head masks, write the kept token ids in ascending order, their
// K/V row indices, and the count.  A mask word covers 32 candidates, i.e. two pages when candidates
// are whole pages, so the page-id and page-table lookups are made once per word, not per token.
__global__ __launch_bounds__(1024) void k_union(CacheView c, CandView cand, const uint32_t* __restrict__ mask_ws,
                                                int ncap, int32_t* union_tok, int32_t* union_row,
                                                int32_t* union_cnt) {
  constexpr int NT = 1024, NW = NT / 64;
  __shared__ int scan_sm[NW + 1];
  const int u = blockIdx.x;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int n = clampi(c.seq_lens[b], 0, c.maxTok);
  const int mw = ncap / 32;
  const uint32_t* m0 = mask_ws + ((size_t)b * c.Hq + (size_t)h * c.G) * mw;
  const int wpt = (mw + NT - 1) / NT;  // contiguous words per thread keep the token order
  const int w0 = min(mw, (int)threadIdx.x * wpt), w1 = min(mw, w0 + wpt);
  int local = 0;
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = 0u;
    for (int hh = 0; hh < c.G; ++hh) bits |= m0[(size_t)hh * mw + w];
    local += __popc(bits);
  }
  int total;
  int pos = block_excl_scan<NW>(local, scan_sm, &total);
  int32_t* out = union_tok + (size_t)u * ncap;
  int32_t* rows = union_row + (size_t)u * ncap;
  const int32_t* pt = c.page_table + (size_t)b * c.maxP;
  const int cnt = clampi(cand.mode == kCandAll ? 0 : cand.count[u], 0, cand.max_items);
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = 0u;
    for (int hh = 0; hh < c.G; ++hh) bits |= m0[(size_t)hh * mw + w];
    if (!bits) continue;
    if (cand.mode == kCandRanges) {
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1u;
        const int t = cand_token_topp(cand, u, w * 32 + bit, n);
        out[pos] = t;
        rows[pos] = (pt[t >> 4] * c.Hkv + h) * kPage + (t & 15);
        ++pos;
      }
      continue;
    }
    // the two pages of this word (kept bits are valid candidates, so their pages exist)
    int page0, page1;
    if (cand.mode == kCandPages) {
      const int32_t* items = cand.items + (size_t)u * cand.max_items;
      page0 = (2 * w < cnt) ? items[2 * w] : 0;
      page1 = (2 * w + 1 < cnt) ? items[2 * w + 1] : 0;
    } else {
      page0 = 2 * w;
      page1 = 2 * w + 1;
    }
    const int phys0 = (bits & 0xffffu) ? pt[page0] : 0;
    const int phys1 = (bits >> 16) ? pt[page1] : 0;
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1u;
      const int hi = bit >> 4, slot = bit & 15;
      out[pos] = (hi ? page1 : page0) * kPage + slot;
      rows[pos] = ((hi ? phys1 : phys0) * c.Hkv + h) * kPage + slot;
      ++pos;
    }
  }
  if (threadIdx.x == 0) union_cnt[u] = total;
}

__global__ __launch_bounds__(256) void k_csr_emit(CacheView c, const int32_t* __restrict__ union_tok,
                                                  const int32_t* __restrict__ union_cnt, int ncap,
                                                  int32_t* indptr, int32_t* tokens, int64_t capacity) {
  const int U = c.B * c.Hkv;
  const int u = blockIdx.x;
  __shared__ int s_off;
  if (threadIdx.x < 64) {
    // offset of unit u = sum of the counts of units before it
    int acc = 0;
    for (int i = (int)threadIdx.x; i < u; i += 64) acc += union_cnt[i];
    acc = wave_sum_int(acc);
    if (threadIdx.x == 0) s_off = acc;
  }
  __syncthreads();
  const int off = s_off, cnt = union_cnt[u];
  if (threadIdx.x == 0) {
    indptr[u] = off;
    if (u == U - 1) indptr[U] = off + cnt;
  }
  for (int i = threadIdx.x; i < cnt; i += 256)
    if (off + i < capacity) tokens[off + i] = union_tok[(size_t)u * ncap + i];
}

int topp_elems_per_thread(int64_t ncap) {
  for (int e = 1; e <= 64; e *= 2)
    if (ncap <= (int64_t)e * kToppThreads) return e;
  return 0;
}

hipError_t launch_topp(const CacheView& c, const CandView& cand, const float* logits, int ncap, float p,
                       int iters, float* threshold, float* mass, uint32_t* mask_ws, uint32_t* head_mask,
                       int mask_words, int32_t* union_tok, int32_t* union_row, int32_t* union_cnt,
                       hipStream_t s) {
  const int E = ncap / kToppThreads;
  dim3 grid((unsigned)(c.B * c.Hq)), block(kToppThreads);
#define TWL_TOPP_CASE(EE)                                                                                 \
  case EE:                                                                                                \
    hipLaunchKernelGGL(k_topp<EE>, grid, block, 0, s, c, logits, ncap, p, iters, threshold, mass, mask_ws, \
                       head_mask, mask_words);                                                           \
    break;
  switch (E) {
    TWL_TOPP_CASE(1)
    TWL_TOPP_CASE(2)
    TWL_TOPP_CASE(4)
    TWL_TOPP_CASE(8)
    TWL_TOPP_CASE(16)
    TWL_TOPP_CASE(32)
    TWL_TOPP_CASE(64)
    default: return hipErrorInvalidValue;
  }
#undef TWL_TOPP_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_union, dim3((unsigned)(c.B * c.Hkv)), dim3(1024), 0, s, c, cand, mask_ws, ncap, union_tok,
                     union_row, union_cnt);
  return hipGetLastError();
}

hipError_t launch_csr_emit(const CacheView& c, const int32_t* union_tok, const int32_t* union_cnt, int ncap,
                           int32_t* indptr, int32_t* tokens, int64_t capacity, hipStream_t s) {
  hipLaunchKernelGGL(k_csr_emit, dim3((unsigned)(c.B * c.Hkv)), dim3(256), 0, s, c, union_tok, union_cnt, ncap,
                     indptr, tokens, capacity);
  return hipGetLastError();
}

}  // namespace twl
