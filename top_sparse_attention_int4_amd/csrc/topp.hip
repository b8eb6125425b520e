// Top-p pruning by a search of the weight threshold, and the GQA union of the kept tokens.
//
// Paper-Notes "关键设计 / 高效Top-p": instead of sorting, search the threshold m with
// sum_{W_i >= m} W_i >= p; each round is one parallel pass over the weights.  One 1024-thread block
// handles one (sequence, query head); the head's weights stay in registers (E per thread).
//
// Weights are kept unnormalised, e_i = exp(l_i - M) in (0, 1] (the maximum is exactly 1), with the
// target p*Z, Z = sum e_i, which keeps the same set as comparing W_i = e_i/Z with p.  The search runs
// on the key of a weight, the uint32 image of the non-negative float32 value (order-preserving).  A
// bisection of the key over [0, 2^31) decides one key bit per step, top bit first, keeping the
// largest threshold whose mass{e >= T} still reaches p*Z.  Here each round decides a digit of the key
// at once from an LDS histogram of the mass per value of the digit (the outcome of as many
// consecutive bisection steps).  Only weights >= 2^-40 carry mass, so the digits run over keys from
// that floor up: 11 bits of (key - floor) >> 18 (exponent and five mantissa bits, which spreads the
// crowded first round over four times as many bins as the key's top 11 bits), then bits 17..9 and
// 8..0; they give the exact threshold T, and the kept set {e >= T} is the converged bisection's.  With fewer steps requested T keeps only its top `iters`
// bits, where a shorter bisection stops: a superset that still reaches p.  p = 1 keeps everything.
//
// Masses are 64-bit fixed point, floor(e * 2^40), added with integer LDS atomics, so the decision does
// not depend on the order of the additions; the cost is at most 2^-40 per weight (below 1e-7 of Z
// for 65536 candidates).  Candidates that do not exist carry e = -1.  The reported threshold is T over
// the fixed-point mass total (the top-k search: over the float32 total); the kept mass is a float32
// sum in a fixed order.
//
// The GQA union (paperlayer §B.2: the union over a group's query heads, read once) is a separate
// small kernel over the head masks.
#include <algorithm>

#include "twl_device.h"
#include "twl_internal.h"

namespace twl {

// W: weighted mode -- candidate k of unit u carries the integer multiplicity mult[u * mult_stride + k]
// (k < mult_stride), its weight being mult * exp(l - M); the largest weight is then not 1.
// topk > 0: the fixed-budget baseline -- every weight >= 2^-40 counts 1 instead of its mass and the
// target is topk, so T is the topk-th largest weight (ties kept); above the count, all are kept.
template <int E, bool W>
__global__ __launch_bounds__(1024) void k_topp(CacheView c, const float* __restrict__ logits, int ncap, float p,
                                               int iters, float* threshold, float* mass, uint32_t* mask_ws,
                                               uint32_t* head_mask, int mask_words,
                                               const int32_t* __restrict__ mult, int mult_stride, int topk) {
  constexpr int NT = kToppThreads, NW = NT / 64;
  __shared__ float red[2 * NW * 4];
  __shared__ uint64_t h1[2048], h2[512], h3[512], cs[64];
  __shared__ uint64_t s_rem;
  __shared__ uint64_t s_zfix;
  __shared__ int s_bin, s_mode;
  BlockReduce<NW> br{red};

  const int bh = blockIdx.x;
  const float* lg = logits + (size_t)bh * ncap;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;

  float e[E];
  float mloc = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int k = j * NT + tid;
    e[j] = (k < ncap) ? lg[k] : -__builtin_inff();
    mloc = fmaxf(mloc, e[j]);
  }
  // weighted mode: the multiplicities in flight together with the logits
  int mk[W ? E : 1];
  if constexpr (W) {
    const int32_t* mu = mult + (size_t)(bh / c.G) * mult_stride;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int k = j * NT + tid;
      mk[j] = (k < mult_stride) ? mu[k] : -1;
    }
  }
  for (int i = tid; i < 2048; i += NT) h1[i] = 0ull;
  if (tid < 512) {
    h2[tid] = 0ull;
    h3[tid] = 0ull;
  }
  const float M = br.max(mloc);  // its barrier also orders the clearing above
  float Z = 0.f;
  if (M != -__builtin_inff()) {
#pragma unroll
    for (int j = 0; j < E; ++j) {
      e[j] = (e[j] == -__builtin_inff()) ? -1.f : exp_diff(e[j], M);
      if constexpr (W) {
        if (e[j] >= 0.f) e[j] = (mk[j] >= 0) ? (float)mk[j] * e[j] : -1.f;
      }
      if (e[j] >= 0.f) Z += e[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < E; ++j) e[j] = -1.f;
  }

  // ---- round 1: first digit (weights carrying mass are >= 2^-40) ---------------------------------------
#pragma unroll
  for (int j = 0; j < E; ++j) {
    if (e[j] >= 0.f) {
      uint64_t f = to_fix(e[j]);
      if (topk > 0) f = f ? 1ull : 0ull;
      if (f) atomicAdd((unsigned long long*)&h1[key_d1(__float_as_uint(e[j]))], (unsigned long long)f);
    }
  }
  __syncthreads();
  // coarse sums (32 bins each): thread t adds bins 2t and 2t+1, a row of 16 lanes scans its 32
  auto coarse = [&](const uint64_t* h, int ncoarse) {
    if (tid < ncoarse * 16) {
      const uint64_t x = row16_incl_scan_u64(h[2 * tid] + h[2 * tid + 1]);
      if ((lane & 15) == 15) cs[tid >> 4] = x;
    }
    __syncthreads();
  };
  coarse(h1, 64);
  if (wv == 0) {
    const uint64_t zf = readlane_u64(wave_incl_scan_u64(cs[lane]), 63);
    int mode = 1, bin = 0;
    uint64_t rem = 0;
    if (zf != 0ull && (topk > 0 ? (uint64_t)topk <= zf : p < 1.0f)) {
      uint64_t target = topk > 0 ? (uint64_t)topk : (uint64_t)ceil((double)p * (double)zf);
      target = target < 1ull ? 1ull : (target > zf ? zf : target);
      wide_find(h1, cs, 64, target, bin, rem);
      mode = 0;
    }
    if (lane == 0) {
      s_mode = mode;
      s_bin = bin;
      s_rem = rem;
      s_zfix = zf;  // the mass total (a count for the top-k search)
    }
  }
  __syncthreads();
  uint32_t T = 0u;
  if (s_mode == 0) {
    const uint32_t b1 = (uint32_t)s_bin;
    const uint64_t rem1 = s_rem;
    // ---- round 2: bits 17..9 inside bin b1 (keys below the floor wrap past every bin) --------------
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const uint32_t key = __float_as_uint(e[j]);
      if (e[j] >= 0.f && key_d1(key) == b1) {
        uint64_t f = to_fix(e[j]);
        if (topk > 0) f = f ? 1ull : 0ull;
        if (f) atomicAdd((unsigned long long*)&h2[key_d2(key)], (unsigned long long)f);
      }
    }
    __syncthreads();
    coarse(h2, 16);
    if (wv == 0) {
      int bin;
      uint64_t rem;
      wide_find(h2, cs, 16, rem1, bin, rem);
      if (lane == 0) {
        s_bin = bin;
        s_rem = rem;
      }
    }
    __syncthreads();
    const uint32_t pre = key_pre2(b1, (uint32_t)s_bin);
    const uint64_t rem2 = s_rem;
    // ---- round 3: bits 8..0 ------------------------------------------------------------------------
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const uint32_t key = __float_as_uint(e[j]);
      if (e[j] >= 0.f && (key >> 9) == pre) {
        uint64_t f = to_fix(e[j]);
        if (topk > 0) f = f ? 1ull : 0ull;
        if (f) atomicAdd((unsigned long long*)&h3[key_d3(key)], (unsigned long long)f);
      }
    }
    __syncthreads();
    coarse(h3, 16);
    if (wv == 0) {
      int bin;
      uint64_t rem;
      wide_find(h3, cs, 16, rem2, bin, rem);
      if (lane == 0) s_bin = bin;
    }
    __syncthreads();
    T = (pre << 9) | (uint32_t)s_bin;
    if (iters < 31) T &= ~((1u << (31 - iters)) - 1u);
  }
  // the reported threshold relative to the fixed-point mass total (an exact sum: it does not depend
  // on where the candidates sit, and the multi-block search reports the same; the top-k search,
  // whose histograms count, over the float32 total); the kept mass as a float32 sum in a fixed order
  const float m = __uint_as_float(T);
  float f = 0.f;
#pragma unroll
  for (int j = 0; j < E; ++j) f += (e[j] >= m) ? e[j] : 0.f;
  br.sum2(Z, f);
  if (tid == 0) {
    if (topk > 0)
      threshold[bh] = (Z > 0.f) ? m / Z : 0.f;
    else
      threshold[bh] = s_zfix ? m / (float)((double)s_zfix / 1099511627776.0) : 0.f;
    if (mass) mass[bh] = (Z > 0.f) ? f / Z : 0.f;
  }

  // head mask: bit k of the head's bitmap <=> candidate k kept.  Element j of the wave's lanes covers
  // candidates j NT + 64 wv .. + 63, words 2j, 2j + 1 of the wave's 2E; lane l writes word l (and
  // 64 + l), so each wave stores its words with one or two instructions
  const int mw = ncap / 32;
  uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const unsigned long long bal = __ballot(e[j] >= m);
    const uint32_t lo = (uint32_t)bal, hi = (uint32_t)(bal >> 32);
    if (2 * j < 64) {
      if (lane == 2 * j) w0 = lo;
      if (lane == 2 * j + 1) w0 = hi;
    } else {
      if (lane == 2 * j - 64) w1 = lo;
      if (lane == 2 * j - 63) w1 = hi;
    }
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int wn = 64 * r + lane;  // the wave's word number
    if (wn < 2 * E) {
      const int w = (wn >> 1) * (NT / 32) + 2 * wv + (wn & 1);
      const uint32_t x = r ? w1 : w0;
      mask_ws[(size_t)bh * mw + w] = x;
      if (head_mask && w < mask_words) head_mask[(size_t)bh * mask_words + w] = x;
    }
  }
}

// One block per unit: OR the unit's G head masks and write the kept token ids (ascending) and the
// count.  First every thread forms the union of its mask words (all loads in
// flight together) and the block scans their popcounts into per-word output offsets in LDS; then
// thread t of pass j handles candidate j*1024 + t, so the gathers of the ids the estimate recorded,
// and the writes of the kept ones, are coalesced.
template <int E, int G>
__global__ __launch_bounds__(1024) void k_union(CacheView c, const uint32_t* __restrict__ mask_ws,
                                                const int32_t* __restrict__ cand_tok, int ncap, int32_t* union_tok,
                                                int32_t* union_cnt) {
  constexpr int NT = 1024, NW = NT / 64;
  constexpr int MW = E * 32;                 // mask words per head (ncap / 32)
  constexpr int WPT = (MW + NT - 1) / NT;    // words per thread
  __shared__ uint32_t uw[MW];
  __shared__ int woff[MW];
  __shared__ int scan_sm[NW + 1];
  const int u = blockIdx.x;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int tid = threadIdx.x;
  const uint32_t* m0 = mask_ws + ((size_t)b * c.Hq + (size_t)h * G) * MW;
  uint32_t words[WPT];
  int local = 0;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int w = tid * WPT + i;
    uint32_t x = 0u;
    if (w < MW) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) x |= m0[(size_t)hh * MW + w];
    }
    words[i] = x;
    local += __popc(x);
  }
  int total;
  int off = block_excl_scan<NW>(local, scan_sm, &total);
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int w = tid * WPT + i;
    if (w < MW) {
      uw[w] = words[i];
      woff[w] = off;
      off += __popc(words[i]);
    }
  }
  __syncthreads();
  const int32_t* ct = cand_tok + (size_t)u * ncap;
  int32_t* out = union_tok + (size_t)u * ncap;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int k = j * NT + tid;
    const uint32_t x = uw[k >> 5];
    const int bit = k & 31;
    if ((x >> bit) & 1u) {
      const int pos = woff[k >> 5] + __popc(x & ((1u << bit) - 1u));
      out[pos] = ct[k];
    }
  }
  if (tid == 0) union_cnt[u] = total;
}

// CSR of the units' kept lists: block (x, u) copies part x of unit u's list (eight loads in flight per
// thread), its offset being the sum of the counts of the units before it.
__global__ __launch_bounds__(256) void k_csr_emit(CacheView c, const int32_t* __restrict__ union_tok,
                                                  const int32_t* __restrict__ union_cnt, int ncap,
                                                  int32_t* indptr, int32_t* tokens, int64_t capacity) {
  const int U = c.B * c.Hkv;
  const int u = blockIdx.y;
  __shared__ int s_off;
  if (threadIdx.x < 64) {
    int acc = 0;
    for (int i = (int)threadIdx.x; i < u; i += 64) acc += union_cnt[i];
    acc = wave_sum_int(acc);
    if (threadIdx.x == 0) s_off = acc;
  }
  __syncthreads();
  const int off = s_off, cnt = union_cnt[u];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    indptr[u] = off;
    if (u == U - 1) indptr[U] = off + cnt;
  }
  const int32_t* src = union_tok + (size_t)u * ncap;
  for (int base = (int)blockIdx.x * 2048; base < cnt; base += (int)gridDim.x * 2048) {
    int v[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int i = base + r * 256 + (int)threadIdx.x;
      v[r] = (i < cnt) ? src[i] : 0;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int i = base + r * 256 + (int)threadIdx.x;
      if (i < cnt && off + (int64_t)i < capacity) tokens[off + i] = v[r];
    }
  }
}

int topp_elems_per_thread(int64_t ncap) {
  for (int e = 1; e <= 64; e *= 2)
    if (ncap <= (int64_t)e * kToppThreads) return e;
  return 0;
}

hipError_t launch_topp(const CacheView& c, const float* logits, int ncap, float p, int iters, float* threshold,
                       float* mass, uint32_t* mask_ws, uint32_t* head_mask, int mask_words, int topk, hipStream_t s) {
  const int E = ncap / kToppThreads;
  dim3 grid((unsigned)(c.B * c.Hq)), block(kToppThreads);
#define TWL_TOPP_CASE(EE)                                                                                   \
  case EE:                                                                                                  \
    hipLaunchKernelGGL((k_topp<EE, false>), grid, block, 0, s, c, logits, ncap, p, iters, threshold, mass,   \
                       mask_ws, head_mask, mask_words, nullptr, 0, topk);                                  \
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

hipError_t launch_union(const CacheView& c, const uint32_t* mask_ws, const int32_t* cand_tok, int ncap,
                        int32_t* union_tok, int32_t* union_cnt, hipStream_t s) {
  const int E = ncap / kToppThreads;
  dim3 ugrid((unsigned)(c.B * c.Hkv)), block(kToppThreads);
#define TWL_UNION_G(EE, GG)                                                                                \
  case GG:                                                                                                 \
    hipLaunchKernelGGL((k_union<EE, GG>), ugrid, block, 0, s, c, mask_ws, cand_tok, ncap, union_tok,     \
                       union_cnt);                                                                       \
    break;
#define TWL_UNION_CASE(EE)        \
  case EE:                        \
    switch (c.G) {                \
      TWL_UNION_G(EE, 1)          \
      TWL_UNION_G(EE, 2)          \
      TWL_UNION_G(EE, 4)          \
      TWL_UNION_G(EE, 8)          \
      default: return hipErrorInvalidValue; \
    }                             \
    break;
  switch (E) {
    TWL_UNION_CASE(1)
    TWL_UNION_CASE(2)
    TWL_UNION_CASE(4)
    TWL_UNION_CASE(8)
    TWL_UNION_CASE(16)
    TWL_UNION_CASE(32)
    TWL_UNION_CASE(64)
    default: return hipErrorInvalidValue;
  }
#undef TWL_UNION_G
#undef TWL_UNION_CASE
  return hipGetLastError();
}

hipError_t launch_topp_weighted(const CacheView& c, const float* logits, int ncap, float p, int iters, float* threshold,
                                uint32_t* mask_ws, const int32_t* mult, int mult_stride, hipStream_t s) {
  dim3 grid((unsigned)(c.B * c.Hq)), block(kToppThreads);
#define TWL_TOPPW_CASE(EE)                                                                                \
  case EE:                                                                                                \
    hipLaunchKernelGGL((k_topp<EE, true>), grid, block, 0, s, c, logits, ncap, p, iters, threshold, nullptr, \
                       mask_ws, nullptr, 0, mult, mult_stride, 0);                                       \
    break;
  switch (ncap / kToppThreads) {
    TWL_TOPPW_CASE(1)
    TWL_TOPPW_CASE(2)
    TWL_TOPPW_CASE(4)
    TWL_TOPPW_CASE(8)
    TWL_TOPPW_CASE(16)
    TWL_TOPPW_CASE(32)
    TWL_TOPPW_CASE(64)
    default: return hipErrorInvalidValue;
  }
#undef TWL_TOPPW_CASE
  return hipGetLastError();
}

hipError_t launch_csr_emit(const CacheView& c, const int32_t* union_tok, const int32_t* union_cnt, int ncap,
                           int32_t* indptr, int32_t* tokens, int64_t capacity, hipStream_t s) {
  const unsigned parts = (unsigned)std::min<int64_t>(64, ((int64_t)ncap + 2047) / 2048);
  hipLaunchKernelGGL(k_csr_emit, dim3(parts, (unsigned)(c.B * c.Hkv)), dim3(256), 0, s, c, union_tok, union_cnt, ncap,
                     indptr, tokens, capacity);
  return hipGetLastError();
}

}  // namespace twl
