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

constexpr int kCap = 1024;  // weights handed to the single-wave phase (16 per lane)

// W: weighted mode -- candidate k of unit u carries the integer multiplicity mult[u * mult_stride + k]
// (k < mult_stride), its weight being mult * exp(l - M); the largest weight is then not 1.
template <int E, bool W>
__global__ __launch_bounds__(1024) void k_topp(CacheView c, const float* __restrict__ logits, int ncap, float p,
                                               int iters, float* threshold, float* mass, uint32_t* mask_ws,
                                               uint32_t* head_mask, int mask_words,
                                               const int32_t* __restrict__ mult, int mult_stride) {
  constexpr int NT = kToppThreads, NW = NT / 64;
  __shared__ float red[2 * NW * 4];
  __shared__ int cnt_sm[2][NW];
  __shared__ int scan_sm[NW + 1];
  __shared__ float buf[kCap];
  __shared__ uint32_t s_lo;
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
  const float M = br.max(mloc);
  float Z = 0.f, emin = __builtin_inff();
  int nval_w = 0;  // wave-uniform count of existing candidates
  if (M != -__builtin_inff()) {
    const int32_t* mu = W ? mult + (size_t)(bh / c.G) * mult_stride : nullptr;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      e[j] = (e[j] == -__builtin_inff()) ? -1.f : exp_diff(e[j], M);
      if (W) {
        const int k = j * NT + tid;
        if (e[j] >= 0.f) e[j] = (k < mult_stride) ? (float)mu[k] * e[j] : -1.f;
      }
      const bool ok = e[j] >= 0.f;
      if (ok) {
        Z += e[j];
        emin = fminf(emin, e[j]);
      }
      nval_w += __popcll(__ballot(ok));
    }
  } else {
#pragma unroll
    for (int j = 0; j < E; ++j) e[j] = -1.f;
  }
  br.sum_min(Z, emin);
  float emax = 1.0f;  // exp(0): the largest unweighted weight
  if (W) {
    float x = -1.f;
#pragma unroll
    for (int j = 0; j < E; ++j) x = fmaxf(x, e[j]);
    emax = br.max(x);
  }

  // block-wide sum of f and of a wave-uniform count, with one barrier
  int slot = 0;
  auto block_f_count = [&](float& f, int& cnt) {
    f = wave_sum_dpp(f);
    float* r = red + slot * NW * 4;
    int* cs = cnt_sm[slot];
    slot ^= 1;
    if (lane == 0) {
      r[wv] = f;
      cs[wv] = cnt;
    }
    __syncthreads();
    float t = r[0];
    int ct = cs[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
      t += r[i];
      ct += cs[i];
    }
    f = t;
    cnt = ct;
  };
  {
    float dummy = 0.f;
    block_f_count(dummy, nval_w);
  }
  const int nval = nval_w;

  uint32_t lo = 0u;
  if (Z > 0.f && p < 1.0f) {
    const float target = p * Z;
    lo = __float_as_uint(emin);                // f(min e) = Z >= target
    uint32_t hi = __float_as_uint(emax) + 1u;  // every weight is <= emax
    int n_lo = nval, n_hi = 0;                 // #{e >= lo}, #{e >= hi}
    int it = 0;
    // ---- block phase: one fixed-order reduction of f(mid) and #{e >= mid} per step ------------
    while (it < iters && hi - lo > 1u && n_lo - n_hi > kCap) {
      const uint32_t mid = lo + ((hi - lo) >> 1);
      const float m = __uint_as_float(mid);
      float f = 0.f;
      int cm = 0;
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const bool ge = e[j] >= m;
        f += ge ? e[j] : 0.f;
        cm += __popcll(__ballot(ge));
      }
      block_f_count(f, cm);
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
      const float c_hi = br.sum(above);  // mass at or above the bracket
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (e[j] >= mlo && e[j] < mhi) buf[pos++] = e[j];
      __syncthreads();
      if (wv == 0) {
        // the bracket's weights, 16 per lane (-1 marks an empty slot)
        float xs[kCap / 64];
        const int nb0 = min(total, kCap);
#pragma unroll
        for (int i = 0; i < kCap / 64; ++i) xs[i] = (lane + 64 * i < nb0) ? buf[lane + 64 * i] : -1.f;
        int c_lo = nb0, c_hi_n = 0;  // #{x >= lo}, #{x >= hi} among the register weights
        bool exact = false;
        while (it < iters && hi - lo > 1u) {
          const uint32_t need = 32u - (uint32_t)__clz((int)(hi - lo - 1u));  // steps left to converge
          if (c_lo - c_hi_n <= 64 && (uint32_t)(iters - it) >= need) {
            exact = true;
            break;
          }
          const uint32_t mid = lo + ((hi - lo) >> 1);
          const float m = __uint_as_float(mid);
          float f = 0.f;
          int cm = 0;
#pragma unroll
          for (int i = 0; i < kCap / 64; ++i) {
            const bool ge = xs[i] >= m;
            f += ge ? xs[i] : 0.f;
            cm += __popcll(__ballot(ge));
          }
          f = c_hi + wave_sum_dpp(f);
          if (f >= target) {
            lo = mid;
            c_lo = cm;
          } else {
            hi = mid;
            c_hi_n = cm;
          }
          ++it;
        }
        if (exact) {
          // Finish in one step: the converged threshold is the largest weight x in the bracket with
          // f(x) >= target, and every lane evaluates f at one of the (at most 64) bracket weights.
          const float mlo2 = __uint_as_float(lo), mhi2 = __uint_as_float(hi);
          float mabove = 0.f;
          int base = 0;
          float y = -1.f;
#pragma unroll
          for (int i = 0; i < kCap / 64; ++i) {
            const bool inb = xs[i] >= mlo2 && xs[i] < mhi2;
            mabove += (xs[i] >= mhi2) ? xs[i] : 0.f;
            const unsigned long long bal = __ballot(inb);
            const int r = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            if (inb) buf[r] = xs[i];
            base += __popcll(bal);
          }
          __builtin_amdgcn_wave_barrier();
          const int nb = base;
          y = (lane < nb) ? buf[lane] : -1.f;
          float fy = c_hi + wave_sum_dpp(mabove);
          for (int i = 0; i < nb; ++i) {
            const float yi = readlane_f(y, i);
            fy += (yi >= y) ? yi : 0.f;
          }
          const float best = wave_max_dpp((lane < nb && fy >= target) ? y : -1.f);
          if (best >= 0.f) lo = __float_as_uint(best);
        }
        if (lane == 0) s_lo = lo;
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

// One block per unit: OR the unit's G head masks and write the kept token ids (ascending), their K/V
// row indices and the count.  First every thread forms the union of its mask words (all loads in
// flight together) and the block scans their popcounts into per-word output offsets in LDS; then
// thread t of pass j handles candidate j*1024 + t, so the gathers of the ids and rows the estimate
// recorded, and the writes of the kept ones, are coalesced.
template <int E, int G>
__global__ __launch_bounds__(1024) void k_union(CacheView c, const uint32_t* __restrict__ mask_ws,
                                                const int32_t* __restrict__ cand_tok,
                                                const int32_t* __restrict__ cand_row, int ncap, int32_t* union_tok,
                                                int32_t* union_row, int32_t* union_cnt) {
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
  const int32_t* cr = cand_row + (size_t)u * ncap;
  int32_t* out = union_tok + (size_t)u * ncap;
  int32_t* rows = union_row + (size_t)u * ncap;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int k = j * NT + tid;
    const uint32_t x = uw[k >> 5];
    const int bit = k & 31;
    if ((x >> bit) & 1u) {
      const int pos = woff[k >> 5] + __popc(x & ((1u << bit) - 1u));
      out[pos] = ct[k];
      rows[pos] = cr[k];
    }
  }
  if (tid == 0) union_cnt[u] = total;
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

hipError_t launch_topp(const CacheView& c, const int32_t* cand_tok, const int32_t* cand_row, const float* logits,
                       int ncap, float p,
                       int iters, float* threshold, float* mass, uint32_t* mask_ws, uint32_t* head_mask,
                       int mask_words, int32_t* union_tok, int32_t* union_row, int32_t* union_cnt,
                       hipStream_t s) {
  const int E = ncap / kToppThreads;
  dim3 grid((unsigned)(c.B * c.Hq)), block(kToppThreads);
#define TWL_TOPP_CASE(EE)                                                                                   \
  case EE:                                                                                                  \
    hipLaunchKernelGGL((k_topp<EE, false>), grid, block, 0, s, c, logits, ncap, p, iters, threshold, mass,   \
                       mask_ws, head_mask, mask_words, nullptr, 0);                                        \
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
  dim3 ugrid((unsigned)(c.B * c.Hkv));
#define TWL_UNION_G(EE, GG)                                                                                \
  case GG:                                                                                                 \
    hipLaunchKernelGGL((k_union<EE, GG>), ugrid, block, 0, s, c, mask_ws, cand_tok, cand_row, ncap,      \
                       union_tok, union_row, union_cnt);                                                 \
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
                       mask_ws, nullptr, 0, mult, mult_stride);                                          \
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
  hipLaunchKernelGGL(k_csr_emit, dim3((unsigned)(c.B * c.Hkv)), dim3(256), 0, s, c, union_tok, union_cnt, ncap,
                     indptr, tokens, capacity);
  return hipGetLastError();
}

}  // namespace twl
