// Top-p for heads with more candidates than one block holds in registers (more than 65536).
//
// Same threshold search as the block kernel (Paper-Notes "关键设计 / 高效Top-p": find the threshold m
// with sum_{W_i >= m} W_i >= p by repeated parallel passes, no sort), over the same weights
// e_i = exp(l_i - M) and the same key, the uint32 image of the non-negative float32 weight.  A
// bisection of that key over [0, 2^31) decides one key bit per step, top bit first; here a histogram
// of the mass per value of a digit of the key decides several steps at once.  Only weights >= 2^-40
// carry fixed-point mass, so the digits run over keys from that floor: 11 bits of (key - floor) >> 18,
// then bits 17..9 and 8..0, which give the exact largest threshold T with mass{e >= T} >= p * Z, so
// the kept set {e >= T} is the converged bisection's.  With fewer steps requested the threshold keeps only its top `iters`
// bits, the point a shorter bisection stops at: a superset that still reaches p.
//
// Masses are 64-bit fixed point, floor(e * 2^40) (e <= 1, at most 2^22 candidates per head), so the
// histograms can be summed across blocks with integer atomics in any order and still give the same
// result on every run.  Truncation costs at most 2^-40 per weight, below 2.4e-7 of Z for 2^18
// candidates.
//
// Kernels:
//   k_wide_hist1    M from the estimate's per-block maxima; e written over the logits; histogram of
//                   the first digit (four 4096-candidate chunks per block, the next chunk's loads in flight
//                   while one is processed, one flush of integer atomics to the global histogram)
//   k_wide_collect  resolve the first digit; the keys of the candidates inside its bin appended to a
//                   per-head buffer (one atomic per block and chunk; their order does not matter)
//   k_wide_finish   one block per head: bits 17..9 and 8..0 from LDS histograms over the collected keys
//                   (the bisection steps left), the threshold
//   k_wide_mask     per (unit, chunk): head masks, kept mass, union words and their count
//   k_wide_emit     per (unit, chunk): compaction of the union (ascending ids and K/V rows), outputs
#include "twl_device.h"
#include "twl_internal.h"

namespace twl {

namespace {

constexpr int NT = kWideThreads;
constexpr int NW = NT / 64;
constexpr int EPT = kWideChunk / NT;  // candidates per thread
constexpr int QPT = EPT / 4;            // of them as float4 (the histogram passes read 16 B per lane)

// the thread's candidates of a chunk as float4: candidates 4 (j NT + t) .. + 3
__device__ __forceinline__ void load_chunk4(const float* x, float (&v)[EPT]) {
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const float4 q = reinterpret_cast<const float4*>(x)[j * NT + threadIdx.x];
    v[4 * j] = q.x;
    v[4 * j + 1] = q.y;
    v[4 * j + 2] = q.z;
    v[4 * j + 3] = q.w;
  }
}
__device__ __forceinline__ void flush_hist(const uint64_t* h, int nbins, uint64_t* g_fine, uint64_t* g_coarse) {
  for (int i = threadIdx.x; i < nbins; i += NT)
    if (h[i]) atomicAdd((unsigned long long*)&g_fine[i], (unsigned long long)h[i]);
  for (int cb = threadIdx.x; cb < nbins / 32; cb += NT) {
    uint64_t s = 0;
#pragma unroll 8
    for (int i = 0; i < 32; ++i) s += h[32 * cb + i];
    if (s) atomicAdd((unsigned long long*)&g_coarse[cb], (unsigned long long)s);
  }
}

// Lane l of each group of 8 lanes holds the keep bits of candidates 4l .. 4l + 3 of a 32-candidate
// word (bit e for candidate 4l + e); every lane of the group gets the word (bit k <=> candidate k).
__device__ __forceinline__ uint32_t nibbles_to_word(uint32_t nib) {
  uint32_t x = nib << (4 * (threadIdx.x & 7));
  x |= (uint32_t)__shfl_xor((int)x, 1);
  x |= (uint32_t)__shfl_xor((int)x, 2);
  x |= (uint32_t)__shfl_xor((int)x, 4);
  return x;
}

}  // namespace

__global__ __launch_bounds__(kWideThreads) void k_wide_hist1(float* __restrict__ logits, int ncap,
                                                             const float* __restrict__ pmax, int npm,
                                                             uint64_t* __restrict__ state) {
  __shared__ uint64_t h[2048];
  __shared__ float red[2 * NW * 4];
  BlockReduce<NW> br{red};
  const int nbk = ncap / kWideAlign;
  const int bh = blockIdx.x / nbk, bk = blockIdx.x - bh * nbk;
  float* lg = logits + (size_t)bh * ncap + (size_t)bk * kWideAlign;
  float v[2][EPT];
  load_chunk4(lg, v[0]);  // in flight while M is formed
  for (int i = threadIdx.x; i < 2048; i += NT) h[i] = 0ull;
  float m = -__builtin_inff();
  for (int i = threadIdx.x; i < npm; i += NT) m = fmaxf(m, pmax[(size_t)bh * npm + i]);
  const float M = br.max(m);  // (its barrier also orders the clearing of h)
#pragma unroll
  for (int c = 0; c < kWideBlockChunks; ++c) {
    // the next chunk's logits in flight while this one is weighted
    if (c + 1 < kWideBlockChunks) load_chunk4(lg + (size_t)(c + 1) * kWideChunk, v[(c + 1) & 1]);
    float (&x)[EPT] = v[c & 1];
#pragma unroll
    for (int j = 0; j < EPT; ++j)
      x[j] = (x[j] == -__builtin_inff() || M == -__builtin_inff()) ? -1.f : exp_diff(x[j], M);
    float4* out = reinterpret_cast<float4*>(lg + (size_t)c * kWideChunk);
#pragma unroll
    for (int j = 0; j < QPT; ++j) out[j * NT + threadIdx.x] = make_float4(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]);
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const float e = x[j];
      if (e >= 0.f) {
        const uint64_t f = to_fix(e);
        if (f) atomicAdd((unsigned long long*)&h[key_d1(__float_as_uint(e))], (unsigned long long)f);
      }
    }
  }
  __syncthreads();
  uint64_t* st = state + (size_t)bh * kWideStateWords;
  flush_hist(h, 2048, st + kWideH1, st + kWideC1);
}

// Level-1 resolution of one head (whole wave): Z, the trivial cases, target, bin and remainder.
__device__ __forceinline__ void wide_level1(const uint64_t* st, float p, int& mode, uint64_t& Z, int& b1,
                                            uint64_t& rem1) {
  const int lane = threadIdx.x & 63;
  uint64_t z = st[kWideC1 + lane];
  z = wave_suffix_u64(z);
  Z = __shfl(z, 0);
  b1 = 0;
  rem1 = 0;
  if (Z == 0ull || !(p < 1.0f)) {
    mode = 1;  // keep every candidate (threshold 0)
    return;
  }
  mode = 0;
  double t = ceil((double)p * (double)Z);
  uint64_t target = (uint64_t)t;
  if (target < 1ull) target = 1ull;
  if (target > Z) target = Z;
  wide_find(st + kWideH1, st + kWideC1, 64, target, b1, rem1);
}

__global__ __launch_bounds__(kWideThreads) void k_wide_collect(const float* __restrict__ w, int ncap, float p,
                                                               uint64_t* __restrict__ state,
                                                               uint32_t* __restrict__ keys) {
  __shared__ int s_mode, s_b1;
  __shared__ int scan_sm[NW + 1];
  __shared__ int s_base;
  const int nbk = ncap / kWideAlign;
  const int bh = blockIdx.x / nbk, bk = blockIdx.x - bh * nbk;
  uint64_t* st = state + (size_t)bh * kWideStateWords;
  const float* x0 = w + (size_t)bh * ncap + (size_t)bk * kWideAlign;
  uint32_t* kout = keys + (size_t)bh * ncap;
  float v[2][EPT];
  load_chunk4(x0, v[0]);  // in flight during the resolution
  if (threadIdx.x < 64) {
    int mode, b1;
    uint64_t Z, rem1;
    wide_level1(st, p, mode, Z, b1, rem1);
    if (threadIdx.x == 0) {
      s_mode = mode;
      s_b1 = b1;
      if (bk == 0) {
        st[kWideSZ] = Z;
        st[kWideSMode] = (uint64_t)mode;
        st[kWideSB1] = (uint64_t)b1;
        st[kWideSR1] = rem1;
      }
    }
  }
  __syncthreads();
  if (s_mode != 0) return;
  const uint32_t b1 = (uint32_t)s_b1;
#pragma unroll
  for (int c = 0; c < kWideBlockChunks; ++c) {
    if (c + 1 < kWideBlockChunks) load_chunk4(x0 + (size_t)(c + 1) * kWideChunk, v[(c + 1) & 1]);
    const float (&x)[EPT] = v[c & 1];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) cnt += (x[j] >= 0.f && key_d1(__float_as_uint(x[j])) == b1) ? 1 : 0;
    int total;
    const int off = block_excl_scan<NW>(cnt, scan_sm, &total);
    if (total == 0) continue;  // uniform
    if (threadIdx.x == 0)
      s_base = (int)atomicAdd((unsigned long long*)&st[kWideNKeys], (unsigned long long)total);
    __syncthreads();
    int pos = s_base + off;
#pragma unroll
    for (int j = 0; j < EPT; ++j)
      if (x[j] >= 0.f && key_d1(__float_as_uint(x[j])) == b1) kout[pos++] = __float_as_uint(x[j]);
  }
}

// One block per head: the remaining 20 key bits from LDS histograms of the collected keys (all in the
// first level's bin), then the threshold.
__global__ __launch_bounds__(1024) void k_wide_finish(int ncap, int iters, uint64_t* __restrict__ state,
                                                      const uint32_t* __restrict__ keys, float* threshold) {
  constexpr int FT = 1024, FU = 8;
  __shared__ uint64_t h2[512], h3[512], cs[64];
  __shared__ int s_bin;
  __shared__ uint64_t s_rem;
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint64_t* st = state + (size_t)bh * kWideStateWords;
  const uint32_t* kin = keys + (size_t)bh * ncap;
  const uint64_t mode = st[kWideSMode], Z = st[kWideSZ];
  const uint32_t b1 = (uint32_t)st[kWideSB1];
  const uint64_t rem1 = st[kWideSR1];
  const int n = (int)min(st[kWideNKeys], (uint64_t)ncap);
  uint32_t T = 0u;
  if (mode == 0ull) {
    if (tid < 512) {
      h2[tid] = 0ull;
      h3[tid] = 0ull;
    }
    __syncthreads();
    auto coarse = [&](const uint64_t* h, int ncoarse) {
      if (tid < ncoarse * 16) {
        const uint64_t x = row16_incl_scan_u64(h[2 * tid] + h[2 * tid + 1]);
        if ((lane & 15) == 15) cs[tid >> 4] = x;
      }
      __syncthreads();
    };
    // bits 17..9 of every collected key
    for (int i0 = 0; i0 < n; i0 += FT * FU) {
      uint32_t kk[FU];
#pragma unroll
      for (int e = 0; e < FU; ++e) {
        const int i = i0 + e * FT + tid;
        kk[e] = (i < n) ? kin[i] : 0xFFFFFFFFu;  // a weight key never has the sign bit set
      }
#pragma unroll
      for (int e = 0; e < FU; ++e) {
        if (kk[e] != 0xFFFFFFFFu) {
          const uint64_t f = to_fix(__uint_as_float(kk[e]));
          if (f) atomicAdd((unsigned long long*)&h2[key_d2(kk[e])], (unsigned long long)f);
        }
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
    // bits 8..0 of the keys inside that bin
    for (int i0 = 0; i0 < n; i0 += FT * FU) {
      uint32_t kk[FU];
#pragma unroll
      for (int e = 0; e < FU; ++e) {
        const int i = i0 + e * FT + tid;
        kk[e] = (i < n) ? kin[i] : 0xFFFFFFFFu;
      }
#pragma unroll
      for (int e = 0; e < FU; ++e) {
        if (kk[e] != 0xFFFFFFFFu && (kk[e] >> 9) == pre) {
          const uint64_t f = to_fix(__uint_as_float(kk[e]));
          if (f) atomicAdd((unsigned long long*)&h3[key_d3(kk[e])], (unsigned long long)f);
        }
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
  if (tid == 0) {
    st[kWideST] = (uint64_t)T;
    if (threshold) threshold[bh] = Z ? __uint_as_float(T) / (float)((double)Z / 1099511627776.0) : 0.f;
  }
}

// Per (unit, chunk): head masks under the finished thresholds, the kept mass per head, union words and count.
// FULL = false: the union words only (no head masks, kept mass or counts are asked for).
template <int G, bool FULL>
__global__ __launch_bounds__(kWideThreads) void k_wide_mask(CacheView c, const float* __restrict__ w, int ncap,
                                                            uint64_t* __restrict__ state,
                                                            uint32_t* __restrict__ head_mask, int mask_words,
                                                            uint32_t* __restrict__ uwords,
                                                            int32_t* __restrict__ chunk_cnt) {
  __shared__ float s_thr[G];
  __shared__ int s_cnt[NW];
  const int nch = ncap / kWideChunk;
  const int u = blockIdx.x / nch, ch = blockIdx.x - u * nch;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const size_t bh0 = (size_t)b * c.Hq + (size_t)h * G;
  // every weight of the chunk in flight before the thresholds are resolved (thread t holds
  // candidates 4 (j NT + t) .. + 3 of round j)
  float4 x[QPT][G];
#pragma unroll
  for (int j = 0; j < QPT; ++j)
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
      x[j][hh] = reinterpret_cast<const float4*>(w + (bh0 + hh) * ncap + (size_t)ch * kWideChunk)[j * NT + threadIdx.x];
  if (threadIdx.x < G) s_thr[threadIdx.x] = __uint_as_float((uint32_t)state[(bh0 + threadIdx.x) * kWideStateWords + kWideST]);
  __syncthreads();
  float thr[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) thr[hh] = s_thr[hh];
  uint64_t kept[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) kept[hh] = 0ull;
  int cnt = 0;
  const int MW = ncap / 32;
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int wbase = (ch * kWideChunk + 4 * (j * NT + wv * 64)) >> 5;  // first of the wave's 8 words
    const int wd = wbase + (lane >> 3);
    uint32_t unib = 0u;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float xs[4] = {x[j][hh].x, x[j][hh].y, x[j][hh].z, x[j][hh].w};
      uint32_t nib = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool keep = xs[e] >= 0.f && xs[e] >= thr[hh];
        if (FULL && keep) kept[hh] += to_fix(xs[e]);
        nib |= (keep ? 1u : 0u) << e;
      }
      unib |= nib;
      if (FULL && head_mask) {
        const uint32_t word = nibbles_to_word(nib);
        if ((lane & 7) == 0 && wd < mask_words) head_mask[(bh0 + hh) * mask_words + wd] = word;
      }
    }
    cnt += __popc(unib);
    const uint32_t uword = nibbles_to_word(unib);
    if ((lane & 7) == 0) uwords[(size_t)u * MW + wd] = uword;
  }
  if (!FULL) return;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    uint64_t s = wave_suffix_u64(kept[hh]);
    if (lane == 0 && s) atomicAdd((unsigned long long*)&state[(bh0 + hh) * kWideStateWords + kWideMass],
                                  (unsigned long long)s);
  }
  cnt = wave_sum_int(cnt);
  if (lane == 0) s_cnt[wv] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) t += s_cnt[i];
    chunk_cnt[(size_t)u * nch + ch] = t;
  }
}

// Per (unit, chunk): kept candidates of the union in ascending order, with the token ids the estimate
// recorded; chunk 0 also writes each head's threshold and kept mass.
template <int G>
__global__ __launch_bounds__(kWideThreads) void k_wide_emit(CacheView c, int ncap, const uint64_t* __restrict__ state,
                                                            const uint32_t* __restrict__ uwords,
                                                            const int32_t* __restrict__ chunk_cnt,
                                                            const int32_t* __restrict__ cand_tok,
                                                            int32_t* __restrict__ union_tok,
                                                            int32_t* __restrict__ union_cnt, float* mass) {
  constexpr int WPB = kWideChunk / 32;  // union words per chunk
  __shared__ uint32_t uw[WPB];
  __shared__ int woff[WPB];
  __shared__ int scan_sm[NW + 1];
  __shared__ int s_off;
  const int nch = ncap / kWideChunk;
  const int u = blockIdx.x / nch, ch = blockIdx.x - u * nch;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int tid = threadIdx.x;
  const size_t bh0 = (size_t)b * c.Hq + (size_t)h * G;
  if (ch == 0 && tid < G && mass) {
    const uint64_t* st = state + (bh0 + tid) * kWideStateWords;
    const uint64_t Z = st[kWideSZ];
    mass[bh0 + tid] = Z ? (float)((double)st[kWideMass] / (double)Z) : 0.f;
  }
  if (tid < 64) {
    int acc = 0;
    for (int i = tid; i < ch; i += 64) acc += chunk_cnt[(size_t)u * nch + i];
    acc = wave_sum_int(acc);
    if (tid == 0) s_off = acc;
  }
  const uint32_t x = (tid < WPB) ? uwords[(size_t)u * (ncap / 32) + (size_t)ch * WPB + tid] : 0u;
  int total;
  const int off = block_excl_scan<NW>(__popc(x), scan_sm, &total);
  if (tid < WPB) {
    uw[tid] = x;
    woff[tid] = off;
  }
  __syncthreads();
  const int base = s_off;
  if (ch == nch - 1 && tid == 0) union_cnt[u] = base + total;
  const size_t ub = (size_t)u * ncap;
#pragma unroll 4
  for (int j = 0; j < EPT; ++j) {
    const int kl = j * NT + tid;
    const uint32_t wd = uw[kl >> 5];
    const int bit = kl & 31;
    if ((wd >> bit) & 1u) {
      const int pos = base + woff[kl >> 5] + __popc(wd & ((1u << bit) - 1u));
      const size_t k = (size_t)ch * kWideChunk + kl;
      union_tok[ub + pos] = cand_tok[ub + k];
    }
  }
}

hipError_t launch_topp_wide(const CacheView& c, const WideWs& wd, float* logits, int ncap, float p, int iters,
                            float* threshold, uint32_t* head_mask, int mask_words, bool full, hipStream_t s) {
  if (ncap % kWideChunk) return hipErrorInvalidValue;
  const int nch = ncap / kWideChunk;
  if (ncap % kWideAlign) return hipErrorInvalidValue;
  const unsigned hgrid = (unsigned)(c.B * c.Hq * (ncap / kWideAlign)), ugrid = (unsigned)(c.B * c.Hkv * nch);
  const dim3 blk(kWideThreads);
  const int npm = ncap / (64 * est_batches(ncap, (int64_t)c.B * c.Hkv));
  hipLaunchKernelGGL(k_wide_hist1, dim3(hgrid), blk, 0, s, logits, ncap, wd.pmax, npm, wd.state);
  hipLaunchKernelGGL(k_wide_collect, dim3(hgrid), blk, 0, s, logits, ncap, p, wd.state, wd.keys);
  hipLaunchKernelGGL(k_wide_finish, dim3((unsigned)(c.B * c.Hq)), dim3(1024), 0, s, ncap, iters, wd.state, wd.keys,
                     threshold);
#define TWL_WIDE_G(GG)                                                                                      \
  case GG:                                                                                                  \
    if (full)                                                                                               \
      hipLaunchKernelGGL((k_wide_mask<GG, true>), dim3(ugrid), blk, 0, s, c, logits, ncap, wd.state,         \
                         head_mask, mask_words, wd.uwords, wd.chunk_cnt);                                   \
    else                                                                                                    \
      hipLaunchKernelGGL((k_wide_mask<GG, false>), dim3(ugrid), blk, 0, s, c, logits, ncap, wd.state,        \
                         nullptr, 0, wd.uwords, wd.chunk_cnt);                                              \
    break;
  switch (c.G) {
    TWL_WIDE_G(1)
    TWL_WIDE_G(2)
    TWL_WIDE_G(4)
    TWL_WIDE_G(8)
    default: return hipErrorInvalidValue;
  }
#undef TWL_WIDE_G
  return hipGetLastError();
}

hipError_t launch_wide_emit(const CacheView& c, const WideWs& wd, const int32_t* cand_tok, int ncap,
                            int32_t* union_tok, int32_t* union_cnt, float* mass, hipStream_t s) {
  if (ncap % kWideChunk) return hipErrorInvalidValue;
  const int nch = ncap / kWideChunk;
  const unsigned ugrid = (unsigned)(c.B * c.Hkv * nch);
  const dim3 blk(kWideThreads);
#define TWL_WIDE_E(GG)                                                                                      \
  case GG:                                                                                                  \
    hipLaunchKernelGGL(k_wide_emit<GG>, dim3(ugrid), blk, 0, s, c, ncap, wd.state, wd.uwords, wd.chunk_cnt,  \
                       cand_tok, union_tok, union_cnt, mass);                                             \
    break;
  switch (c.G) {
    TWL_WIDE_E(1)
    TWL_WIDE_E(2)
    TWL_WIDE_E(4)
    TWL_WIDE_E(8)
    default: return hipErrorInvalidValue;
  }
#undef TWL_WIDE_E
  return hipGetLastError();
}

}  // namespace twl
