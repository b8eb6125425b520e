// Top-p pruning by binary search of the weight threshold, and the GQA union of the kept tokens.
//
// Paper-Notes "关键设计 / 高效Top-p": instead of sorting, search the threshold m with
// sum_{W_i >= m} W_i >= p; each round is one parallel pass over the weights.  One 1024-thread block
// handles one (sequence, query head): the head's weights stay in registers (E per thread), the
// softmax maximum and normaliser are computed from the logits in the same block, and each bisection
// step is one fixed-order block reduction.  Midpoints are taken on the uint32 image of the
// non-negative float32 weights, keeping f(lo) >= p*Z > f(hi); the kept set is {e_i >= lo}.
//
// The weights are kept unnormalised, e_i = exp(l_i - M) in (0, 1] (the maximum is exactly 1), and
// the target is p*Z with Z = sum e_i, which selects the same set as comparing W_i = e_i/Z with p.
// Candidates that do not exist carry e = -1 so no threshold >= 0 ever selects them.
//
// The last of the G blocks of a kv-head (paperlayer §B.2: the union over a GQA group's query heads)
// ORs the G head masks and writes the unit's kept token ids, ascending, with their count.
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

// Union of the G head masks of unit u, compacted to ascending token ids.  Called by a whole block.
template <int NW>
__device__ void group_union(const CacheView& c, const CandView& cand, int u, int b, const uint32_t* mask_ws,
                            int mw, int32_t* union_tok, int32_t* union_cnt, int ncap, int* scan_sm) {
  constexpr int NT = NW * 64;
  const int n = clampi(c.seq_lens[b], 0, c.maxTok);
  const int h = u - b * c.Hkv;
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
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = 0u;
    for (int hh = 0; hh < c.G; ++hh) bits |= m0[(size_t)hh * mw + w];
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1u;
      out[pos++] = cand_token_topp(cand, u, w * 32 + bit, n);
    }
  }
  if (threadIdx.x == 0) union_cnt[u] = total;
}

template <int E>
__global__ __launch_bounds__(1024) void k_topp(CacheView c, CandView cand, const float* __restrict__ logits,
                                               int ncap, float p, int iters, float* threshold, float* mass,
                                               uint32_t* mask_ws, uint32_t* head_mask, int mask_words,
                                               int32_t* counters, int32_t* union_tok, int32_t* union_cnt) {
  constexpr int NT = kToppThreads, NW = NT / 64;
  __shared__ float red[2 * NW];
  __shared__ int scan_sm[NW + 1];
  __shared__ int s_last;
  BlockReduce<NW> br{red};

  const int bh = blockIdx.x;
  const int b = bh / c.Hq, hq = bh - b * c.Hq;
  const int h = hq / c.G, u = b * c.Hkv + h;
  const float* lg = logits + (size_t)bh * ncap;
  const int tid = threadIdx.x;

  float e[E];
  float mloc = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int k = j * NT + tid;
    e[j] = (k < ncap) ? lg[k] : -__builtin_inff();
    mloc = fmaxf(mloc, e[j]);
  }
  const float M = br.max(mloc);
  float zloc = 0.f;
  if (M == -__builtin_inff()) {
#pragma unroll
    for (int j = 0; j < E; ++j) e[j] = -1.f;
  } else {
#pragma unroll
    for (int j = 0; j < E; ++j) {
      e[j] = (e[j] == -__builtin_inff()) ? -1.f : exp_diff(e[j], M);
      zloc += fmaxf(e[j], 0.f);
    }
  }
  const float Z = br.sum(zloc);

  uint32_t lo = 0u;
  if (Z > 0.f && p < 1.0f) {
    const float target = p * Z;
    uint32_t hi = __float_as_uint(1.0f) + 1u;  // e <= 1 = exp(0)
    for (int it = 0; it < iters && hi - lo > 1u; ++it) {
      const uint32_t mid = lo + ((hi - lo) >> 1);
      const float m = __uint_as_float(mid);
      float f = 0.f;
#pragma unroll
      for (int j = 0; j < E; ++j) f += (e[j] >= m) ? e[j] : 0.f;
      f = br.sum(f);
      if (f >= target) lo = mid; else hi = mid;
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
  const int lane = tid & 63, wv = tid >> 6;
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

  // the last block of the group forms the union
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&counters[u], 1) == c.G - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  group_union<NW>(c, cand, u, b, mask_ws, mw, union_tok, union_cnt, ncap, scan_sm);
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
                       int mask_words, int32_t* counters, int32_t* union_tok, int32_t* union_cnt,
                       hipStream_t s) {
  const int E = ncap / kToppThreads;
  dim3 grid((unsigned)(c.B * c.Hq)), block(kToppThreads);
#define TWL_TOPP_CASE(EE)                                                                               \
  case EE:                                                                                              \
    hipLaunchKernelGGL(k_topp<EE>, grid, block, 0, s, c, cand, logits, ncap, p, iters, threshold, mass, \
                       mask_ws, head_mask, mask_words, counters, union_tok, union_cnt);                 \
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
  return hipGetLastError();
}

hipError_t launch_csr_emit(const CacheView& c, const int32_t* union_tok, const int32_t* union_cnt, int ncap,
                           int32_t* indptr, int32_t* tokens, int64_t capacity, hipStream_t s) {
  hipLaunchKernelGGL(k_csr_emit, dim3((unsigned)(c.B * c.Hkv)), dim3(256), 0, s, c, union_tok, union_cnt, ncap,
                     indptr, tokens, capacity);
  return hipGetLastError();
}

}  // namespace twl
