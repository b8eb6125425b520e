// Top-p for heads with more candidates than one block holds in registers (more than 65536).
//
// Same threshold search as the block kernel (Paper-Notes "关键设计 / 高效Top-p": find the threshold m
// with sum_{W_i >= m} W_i >= p by repeated parallel passes, no sort), over the same weights
// e_i = exp(l_i - M) and the same key, the uint32 image of the non-negative float32 weight.  A
// bisection of that key over [0, 2^31) decides one key bit per step, top bit first; here a histogram
// of the mass per value of a digit of the key decides several steps at once.  Only weights >= 2^-40
// carry fixed-point mass, so the digits run over keys from that floor: 11 bits of (key - floor) >> 18,
// then bits 17..9 and 8..0, which give the exact largest threshold T with mass{e >= T} >= p * Z, so
// the kept set {e >= T} is the converged bisection's.  With fewer steps requested the threshold keeps
// only its top `iters` bits, the point a shorter bisection stops at: a superset that still reaches p.
// The first digit fixes key bits 30..18, so up to 13 steps the threshold is known once the first
// level is resolved.
//
// Masses are 64-bit fixed point, floor(e * 2^40) (e <= 1, at most 2^22 candidates per head), so the
// histograms can be summed across blocks with integer atomics in any order and still give the same
// result on every run.  Truncation costs at most 2^-40 per weight, below 2.4e-7 of Z for 2^18
// candidates.
//
// The weights are never stored: each pass forms e = exp(l - M) from the estimate's logits with the
// same instructions, so both passes see the same values, and the logits are read twice in all.
//
// Kernels:
//   k_wide_hist1   M from the estimate's per-block maxima (recorded for the later passes); histogram
//                  of the first digit (four 4096-candidate chunks per block, the next chunk's loads in
//                  flight while one is processed, one flush of integer atomics to the global histogram);
//                  the head's last block resolves the first digit (bin, remainder, and the key and
//                  logit bounds the mask pass sorts by)
//   k_wide_mask    per (unit, chunk): weights above the chosen bin kept (head masks, kept mass, union
//                  words and their count), those inside it recorded with their index in the chunk's
//                  own record range
//   k_wide_finish  one block per head: bits 17..9 and 8..0 from LDS histograms over the recorded keys
//                  (the bisection steps left), the threshold, and the recorded candidates that reach it
//                  set in the union words and head masks by atomic ORs
//   k_wide_emit    per (unit, chunk): compaction of the union (ascending ids)
#include "twl_device.h"
#include "twl_internal.h"

namespace twl {

namespace {

constexpr int NT = kWideThreads;        // threads of the emit pass
constexpr int NW = NT / 64;
constexpr int EPT = kWideChunk / NT;    // candidates per thread of a chunk there
constexpr int HT = kWidePassThreads;    // threads of the histogram and mask passes
constexpr int HW = HT / 64;
constexpr int HEPT = kWideChunk / HT;   // candidates per thread of a chunk there
constexpr int HQPT = HEPT / 4;          // of them as float4 (16 B per lane)

// the thread's candidates of a chunk as float4: candidates 4 (j HT + t) .. + 3
__device__ __forceinline__ void load_chunk4(const float* x, float (&v)[HEPT]) {
#pragma unroll
  for (int j = 0; j < HQPT; ++j) {
    const float4 q = reinterpret_cast<const float4*>(x)[j * HT + threadIdx.x];
    v[4 * j] = q.x;
    v[4 * j + 1] = q.y;
    v[4 * j + 2] = q.z;
    v[4 * j + 3] = q.w;
  }
}
// The block's first-digit histogram added to the head's: thread t takes bins 2t and 2t + 1, adds each
// non-zero one with an integer atomic, and each row of 16 lanes sums its 32 bins (a DPP scan) for the
// coarse histogram, one atomic per row.  Integer sums, so the order of the additions does not matter.
__device__ __forceinline__ void flush_hist1(const uint64_t* h, uint64_t* g_fine, uint64_t* g_coarse) {
  static_assert(2 * HT == 2048, "two bins per thread");
  const int t = threadIdx.x;
  const uint64_t a = h[2 * t], b = h[2 * t + 1];
  if (a) atomicAdd((unsigned long long*)&g_fine[2 * t], (unsigned long long)a);
  if (b) atomicAdd((unsigned long long*)&g_fine[2 * t + 1], (unsigned long long)b);
  const uint64_t rs = row16_incl_scan_u64(a + b);  // lane 15 of the row: its 32 bins
  if ((t & 15) == 15 && rs) atomicAdd((unsigned long long*)&g_coarse[t >> 4], (unsigned long long)rs);
}

// Lane l of each group of 8 lanes holds the keep bits of candidates 4l .. 4l + 3 of a 32-candidate
// word (bit e for candidate 4l + e); every lane of the group gets the word (bit k <=> candidate k).
// (DPP: the quads' ORs, then each quad takes its partner's, four lanes up or down within the row;
// called by whole waves.)
__device__ __forceinline__ uint32_t nibbles_to_word(uint32_t nib) {
  int x = (int)(nib << (4 * (threadIdx.x & 7)));
  x |= dpp_i<kDppXor1>(x);
  x |= dpp_i<kDppXor2>(x);
  const int up = __builtin_amdgcn_update_dpp(0, x, kDppShl4, 0xf, 0xf, true);  // lane n + 4 (0 past the row)
  const int dn = __builtin_amdgcn_update_dpp(0, x, kDppShr4, 0xf, 0xf, true);  // lane n - 4
  return (uint32_t)(x | ((threadIdx.x & 4) ? dn : up));
}

}  // namespace

// The weight of a logit: exp(l - M), or -1 for a candidate that does not exist (l = -inf) and for a
// head without candidates.  Every pass forms it with these same instructions.
__device__ __forceinline__ float wide_weight(float l, float M) {
  return (l == -__builtin_inff() || M == -__builtin_inff()) ? -1.f : exp_diff(l, M);
}

// Bisection steps decided by the first digit alone (it fixes key bits 30..18).
constexpr int kWideKnownSteps = 13;

// The threshold of a resolved first level when at most kWideKnownSteps steps are asked for: the
// bin's lowest key with the bits below the top `iters` cleared (every key of the bin shares them).
__device__ __forceinline__ uint32_t wide_known_threshold(uint32_t b1, int iters) {
  return (kKeyFloor + (b1 << 18)) & ~((1u << (31 - iters)) - 1u);
}

// Level-1 resolution of one head (whole wave): Z, the trivial cases, target, bin and remainder.
template <bool COH>
__device__ __forceinline__ void wide_level1(const uint64_t* st, float p, int& mode, uint64_t& Z, int& b1,
                                            uint64_t& rem1) {
  const int lane = threadIdx.x & 63;
  uint64_t z = hist_load<COH>(st + kWideC1 + lane);
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
  wide_find<COH>(st + kWideH1, st + kWideC1, 64, target, b1, rem1);
}

// float32 bounds of a float64 value: the least float >= x and the greatest float <= x
__device__ __forceinline__ float f32_at_least(double x) {
  float f = (float)x;
  if ((double)f < x) f = nextafterf(f, __builtin_inff());
  return f;
}
__device__ __forceinline__ float f32_at_most(double x) {
  float f = (float)x;
  if ((double)f > x) f = nextafterf(f, -__builtin_inff());
  return f;
}

// One wave: the first level of a head resolved once -- total mass, mode, bin and remainder -- and the
// two keys the mask pass sorts by: a weight whose key reaches `keep` is kept for sure (every key above
// the bin, or the whole threshold when the first level fixes it), one from `lo` up to `keep` lies
// in the bin and is recorded for the finishing pass.  Mode 1 keeps every weight (keep = lo = 0).
// The logit bounds A and B decide without the weight: a logit >= A has a weight >= keep and one
// below B a weight below lo, for any weight within a relative 2^-16 of exp(l - M) (the weight's
// own error is below 2e-7); only logits in [B, A) need it.  With keep = 0 every finite logit is kept.
// The histogram is read with agent-scope loads (its last updates came from other blocks).
__device__ __forceinline__ void wide_resolve_level1(uint64_t* st, float M, float p, int iters) {
  int mode, b1;
  uint64_t Z, rem1;
  wide_level1<true>(st, p, mode, Z, b1, rem1);
  if ((threadIdx.x & 63) == 0) {
    uint32_t keep = 0u, lo = 0u;
    if (mode == 0) {
      if (iters <= kWideKnownSteps) {
        keep = lo = wide_known_threshold((uint32_t)b1, iters);
      } else {
        lo = kKeyFloor + ((uint32_t)b1 << 18);
        keep = lo + (1u << 18);
      }
    }
    float A = -3.402823466e38f, B = -3.402823466e38f;
    if (keep > 0u && M != -__builtin_inff()) {
      constexpr double kMargin = 1.0 / 65536.0;
      A = f32_at_least((double)M + log((double)__uint_as_float(keep)) + kMargin);
      B = f32_at_most((double)M + log((double)__uint_as_float(lo)) - kMargin);
    }
    st[kWideSKeep] = keep;
    st[kWideSLo] = lo;
    st[kWideSA] = (uint64_t)__float_as_uint(A);
    st[kWideSB] = (uint64_t)__float_as_uint(B);
    st[kWideSZ] = Z;
    st[kWideSMode] = (uint64_t)mode;
    st[kWideSB1] = (uint64_t)b1;
    st[kWideSR1] = rem1;
  }
}

// Histogram blocks of a head: M, the first digit's mass histogram; the head's last block to finish
// (a ticket counter) resolves the first level for the mask pass.
__global__ __launch_bounds__(HT) void k_wide_hist1(const float* __restrict__ logits, int ncap,
                                                   const float* __restrict__ pmax, int npm, float p, int iters,
                                                   uint64_t* __restrict__ state) {
  __shared__ int s_last;
  __shared__ uint64_t h[2048];
  __shared__ float red[2 * HW * 4];
  BlockReduce<HW> br{red};
  const int nbk = ncap / kWideAlign;
  const int bh = blockIdx.x / nbk, bk = blockIdx.x - bh * nbk;
  const float* lg = logits + (size_t)bh * ncap + (size_t)bk * kWideAlign;
  uint64_t* st = state + (size_t)bh * kWideStateWords;
  float v[2][HEPT];
  load_chunk4(lg, v[0]);  // in flight while M is formed
  for (int i = threadIdx.x; i < 2048; i += HT) h[i] = 0ull;
  float m = -__builtin_inff();
  for (int i = threadIdx.x; i < npm; i += HT) m = fmaxf(m, pmax[(size_t)bh * npm + i]);
  const float M = br.max(m);  // (its barrier also orders the clearing of h)
  if (bk == 0 && threadIdx.x == 0) st[kWideSM] = (uint64_t)__float_as_uint(M);
#pragma unroll
  for (int c = 0; c < kWideBlockChunks; ++c) {
    // the next chunk's logits in flight while this one is weighted
    if (c + 1 < kWideBlockChunks) load_chunk4(lg + (size_t)(c + 1) * kWideChunk, v[(c + 1) & 1]);
    const float (&x)[HEPT] = v[c & 1];
#pragma unroll
    for (int j = 0; j < HEPT; ++j) {
      const float e = wide_weight(x[j], M);
      if (e >= 0.f) {
        const uint64_t f = to_fix(e);
        if (f) atomicAdd((unsigned long long*)&h[key_d1(__float_as_uint(e))], (unsigned long long)f);
      }
    }
  }
  __syncthreads();
  flush_hist1(h, st + kWideH1, st + kWideC1);
  // this block's histogram atomics performed before its ticket is taken
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = atomicAdd((unsigned long long*)&st[kWideTicket], 1ull) == (unsigned long long)(nbk - 1);
  __syncthreads();
  if (s_last && threadIdx.x < 64) wide_resolve_level1(st, M, p, iters);
}


// Per (unit, chunk): every candidate of the chunk and head is kept when its key reaches the head's
// `keep` key, recorded (key, index) when it lies from `lo` up to there.  Writes the union words (and
// with FULL the head masks, the chunk's kept mass per head and its union count) of what is sure; the
// finishing pass adds the recorded candidates that reach the threshold.  Without FULL no kept mass is
// needed, so the logit bounds decide most candidates and only those between them get their weight.
// The per-head words are uniform loads, so they do not wait behind the chunk's logits.
template <int G, bool FULL>
__global__ __launch_bounds__(HT) void k_wide_mask(CacheView c, const float* __restrict__ logits, int ncap,
                                                  const uint64_t* __restrict__ state, uint64_t* __restrict__ keys,
                                                  int32_t* __restrict__ rec_cnt, uint32_t* __restrict__ head_mask,
                                                  int mask_words, uint32_t* __restrict__ uwords,
                                                  int32_t* __restrict__ chunk_cnt, uint64_t* __restrict__ chunk_mass) {
  static_assert(HEPT == 4, "one float4 per thread and head");
  constexpr int NS = 4 * G;  // slots of a thread: bit 4 hh + e is candidate 4 t + e of head hh
  __shared__ int s_cnt[HW];
  __shared__ int s_wrec[HW][G];  // records per wave and head
  __shared__ uint64_t s_wmass[FULL ? HW : 1][G];
  const int nch = ncap / kWideChunk;
  const int u = blockIdx.x / nch, ch = blockIdx.x - u * nch;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const size_t bh0 = (size_t)b * c.Hq + (size_t)h * G;
  float v[NS];  // logits, then the weights of the recorded slots
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float4 q = reinterpret_cast<const float4*>(logits + (bh0 + hh) * ncap + (size_t)ch * kWideChunk)[threadIdx.x];
    v[4 * hh] = q.x;
    v[4 * hh + 1] = q.y;
    v[4 * hh + 2] = q.z;
    v[4 * hh + 3] = q.w;
  }
  float M[G], A[G], B[G];
  uint32_t keep_key[G], lo_key[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint64_t* st = state + (bh0 + hh) * kWideStateWords;
    M[hh] = __uint_as_float((uint32_t)st[kWideSM]);
    keep_key[hh] = (uint32_t)st[kWideSKeep];
    lo_key[hh] = (uint32_t)st[kWideSLo];
    A[hh] = __uint_as_float((uint32_t)st[kWideSA]);
    B[hh] = __uint_as_float((uint32_t)st[kWideSB]);
  }
  uint32_t keep = 0u, rec = 0u;
  uint64_t kept[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) kept[hh] = 0ull;
  if constexpr (FULL) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int hh = i >> 2;
      const float w = wide_weight(v[i], M[hh]);
      const uint32_t k = __float_as_uint(w);
      const bool valid = w >= 0.f;
      const bool kp = valid && k >= keep_key[hh];
      const bool rc = valid && !kp && k >= lo_key[hh];
      if (kp) kept[hh] += to_fix(w);
      keep |= (kp ? 1u : 0u) << i;
      rec |= (rc ? 1u : 0u) << i;
      v[i] = w;
    }
  } else {
    uint32_t unc = 0u;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int hh = i >> 2;
      keep |= (v[i] >= A[hh] ? 1u : 0u) << i;
      unc |= (v[i] < A[hh] && v[i] >= B[hh] ? 1u : 0u) << i;
    }
    // the exact weights between the bounds, one slot at a time per lane
    while (unc) {
      const int i = __builtin_ctz(unc);
      unc &= unc - 1u;
      float l = 0.f, m = 0.f;
      uint32_t kk = 0u, lk = 0u;
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) l = (s2 == i) ? v[s2] : l;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const bool mine = (i >> 2) == hh;
        m = mine ? M[hh] : m;
        kk = mine ? keep_key[hh] : kk;
        lk = mine ? lo_key[hh] : lk;
      }
      const float w = wide_weight(l, m);
      const uint32_t k = __float_as_uint(w);
      if (w >= 0.f && k >= kk) {
        keep |= 1u << i;
      } else if (w >= 0.f && k >= lk) {
        rec |= 1u << i;
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) v[s2] = (s2 == i) ? w : v[s2];
      }
    }
  }
  // union words (and head masks): lanes 8 q .. 8 q + 7 hold the 32 candidates of word q
  const int MW = ncap / 32;
  const int wd = ch * (kWideChunk / 32) + wv * 8 + (lane >> 3);
  uint32_t unib = 0u;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint32_t nib = (keep >> (4 * hh)) & 15u;
    unib |= nib;
    if (FULL && head_mask) {
      const uint32_t word = nibbles_to_word(nib);
      if ((lane & 7) == 0 && wd < mask_words) head_mask[(bh0 + hh) * mask_words + wd] = word;
    }
  }
  const uint32_t uword = nibbles_to_word(unib);
  if ((lane & 7) == 0) uwords[(size_t)u * MW + wd] = uword;
  // the candidates inside the bins: (key << 32 | index) from slot ch * kWideChunk of the head's
  // records, in thread order (a chunk records at most kWideChunk), and the chunk's count
  int nrec[G], incl[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    nrec[hh] = __popc((rec >> (4 * hh)) & 15u);
    incl[hh] = wave_incl_scan(nrec[hh]);
    if (lane == 63) s_wrec[wv][hh] = incl[hh];
  }
  __syncthreads();
  if (threadIdx.x < G) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < HW; ++w) t += s_wrec[w][threadIdx.x];
    rec_cnt[(bh0 + threadIdx.x) * nch + ch] = t;
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    if (s_wrec[wv][hh] == 0) continue;  // wave-uniform
    int pos = incl[hh] - nrec[hh];
    for (int w = 0; w < wv; ++w) pos += s_wrec[w][hh];
    uint64_t* kr = keys + (bh0 + hh) * ncap + (size_t)ch * kWideChunk;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if ((rec >> (4 * hh + e)) & 1u) {
        const uint32_t idx = (uint32_t)(ch * kWideChunk + 4 * threadIdx.x + e);
        kr[pos++] = ((uint64_t)__float_as_uint(v[4 * hh + e]) << 32) | idx;
      }
    }
  }
  if (!FULL) return;
  // the chunk's kept mass per head and its union count: wave sums, then one store each
  const int cnt = wave_sum_int(__popc(unib));
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint64_t sm = wave_suffix_u64(kept[hh]);
    if (lane == 0) s_wmass[wv][hh] = sm;
  }
  if (lane == 0) s_cnt[wv] = cnt;
  __syncthreads();
  if (threadIdx.x < G) {
    uint64_t t = 0ull;
#pragma unroll
    for (int w = 0; w < HW; ++w) t += s_wmass[w][threadIdx.x];
    chunk_mass[(bh0 + threadIdx.x) * nch + ch] = t;
  }
  if (threadIdx.x == 0) {
    int t = 0;
#pragma unroll
    for (int i = 0; i < HW; ++i) t += s_cnt[i];
    chunk_cnt[(size_t)u * nch + ch] = t;
  }
}

// One block per head: the remaining 18 key bits from LDS histograms of the recorded keys (all in the
// first level's bin), the threshold, and the recorded candidates that reach it added to the union
// words (FULL: also to the head masks, kept mass and union counts).
__global__ __launch_bounds__(1024) void k_wide_finish(int G, int ncap, int iters, bool full,
                                                      uint64_t* __restrict__ state, const uint64_t* __restrict__ keys,
                                                      const int32_t* __restrict__ rec_cnt,
                                                      const uint64_t* __restrict__ chunk_mass, float* threshold,
                                                      uint32_t* __restrict__ uwords, int32_t* __restrict__ chunk_cnt,
                                                      uint32_t* __restrict__ head_mask, int mask_words) {
  constexpr int FT = 1024, FU = 8, FW = FT / 64;
  constexpr int kMaxChunks = kWideMaxCands / kWideChunk;
  static_assert(kMaxChunks <= FT, "one chunk count per thread");
  __shared__ uint64_t h2[512], h3[512], cs[64];
  __shared__ int s_off[kMaxChunks + 1];  // first record of each chunk in the head's record order
  __shared__ int scan_sm[FW + 1];
  __shared__ int s_bin;
  __shared__ uint64_t s_rem;
  __shared__ uint64_t s_mass[FW];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nch = ncap / kWideChunk;
  uint64_t* st = state + (size_t)bh * kWideStateWords;
  const uint64_t* kin = keys + (size_t)bh * ncap;
  // every load that does not depend on another in flight together: the head's words, the chunks'
  // record counts and (FULL) their kept mass, to which the recorded candidates are added below
  const uint64_t mode = st[kWideSMode], Z = st[kWideSZ];
  const uint32_t b1 = (uint32_t)st[kWideSB1];
  const uint64_t rem1 = st[kWideSR1];
  // (loaded by every thread, so no branch makes them wait early)
  const int ci = min(tid, nch - 1);
  const int rc = rec_cnt[(size_t)bh * nch + ci];
  const uint64_t cm = chunk_mass[(size_t)bh * nch + ci];
  const int my_cnt = tid < nch ? clampi(rc, 0, kWideChunk) : 0;
  uint64_t mass = (full && tid < nch) ? cm : 0ull;
  uint32_t T = 0u;
  if (mode == 0ull && iters <= kWideKnownSteps) {
    T = wide_known_threshold(b1, iters);  // nothing was recorded
  } else if (mode == 0ull) {
    if (tid < 512) {
      h2[tid] = 0ull;
      h3[tid] = 0ull;
    }
    int n;
    {
      const int off = block_excl_scan<FW>(my_cnt, scan_sm, &n);
      if (tid < nch) s_off[tid] = off;
      if (tid == 0) s_off[nch] = n;
    }
    __syncthreads();
    // record i of the head: chunk s = the last with s_off[s] <= i, then slot i - s_off[s] of it
    auto record = [&](int i) -> uint64_t {
      if (i >= n) return ~0ull;  // a weight key never has the sign bit set
      int lo = 0, hi = nch;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_off[mid] <= i) lo = mid; else hi = mid;
      }
      return kin[(size_t)lo * kWideChunk + (i - s_off[lo])];
    };
    // up to FT * FU records stay in registers for all three passes (record e * FT + tid here)
    const bool resident = n <= FT * FU;
    uint64_t rr[FU];
#pragma unroll
    for (int e = 0; e < FU; ++e) rr[e] = record(e * FT + tid);
    auto records = [&](int i0, uint64_t (&r)[FU]) {
      if (resident) return;
#pragma unroll
      for (int e = 0; e < FU; ++e) r[e] = record(i0 + e * FT + tid);
    };
    __syncthreads();
    auto coarse = [&](const uint64_t* h, int ncoarse) {
      if (tid < ncoarse * 16) {
        const uint64_t x = row16_incl_scan_u64(h[2 * tid] + h[2 * tid + 1]);
        if ((lane & 15) == 15) cs[tid >> 4] = x;
      }
      __syncthreads();
    };
    // bits 17..9 of every recorded key
    for (int i0 = 0; i0 < n; i0 += FT * FU) {
      records(i0, rr);
#pragma unroll
      for (int e = 0; e < FU; ++e) {
        const uint32_t kk = (uint32_t)(rr[e] >> 32);
        if (rr[e] != ~0ull) {
          const uint64_t f = to_fix(__uint_as_float(kk));
          if (f) atomicAdd((unsigned long long*)&h2[key_d2(kk)], (unsigned long long)f);
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
      records(i0, rr);
#pragma unroll
      for (int e = 0; e < FU; ++e) {
        const uint32_t kk = (uint32_t)(rr[e] >> 32);
        if (rr[e] != ~0ull && (kk >> 9) == pre) {
          const uint64_t f = to_fix(__uint_as_float(kk));
          if (f) atomicAdd((unsigned long long*)&h3[key_d3(kk)], (unsigned long long)f);
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
    // the recorded candidates at or above the threshold
    const int u = bh / G;
    const int MW = ncap / 32;
    for (int i0 = 0; i0 < n; i0 += FT * FU) {
      records(i0, rr);
#pragma unroll
      for (int e = 0; e < FU; ++e) {
        const uint32_t key = (uint32_t)(rr[e] >> 32), idx = (uint32_t)rr[e];
        if (rr[e] != ~0ull && key >= T && idx < (uint32_t)ncap) {
          const uint32_t bit = 1u << (idx & 31u), wd = idx >> 5;
          const uint32_t old = atomicOr(&uwords[(size_t)u * MW + wd], bit);
          if (full) {
            if (!(old & bit)) atomicAdd(&chunk_cnt[(size_t)u * nch + idx / kWideChunk], 1);
            if (head_mask && (int)wd < mask_words) atomicOr(&head_mask[(size_t)bh * mask_words + wd], bit);
            mass += to_fix(__uint_as_float(key));
          }
        }
      }
    }
  }
  if (full) {
    const uint64_t sm = wave_suffix_u64(mass);
    if (lane == 0) s_mass[wv] = sm;
    __syncthreads();
  }
  if (tid == 0) {
    if (full) {
      uint64_t t = 0ull;
#pragma unroll
      for (int w = 0; w < FW; ++w) t += s_mass[w];
      st[kWideMass] = t;
    }
    st[kWideST] = (uint64_t)T;
    if (threshold) threshold[bh] = Z ? __uint_as_float(T) / (float)((double)Z / 1099511627776.0) : 0.f;
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

hipError_t launch_topp_wide(const CacheView& c, const WideWs& wd, const float* logits, int ncap, float p, int iters,
                            float* threshold, uint32_t* head_mask, int mask_words, bool full, hipStream_t s) {
  if (ncap % kWideAlign || ncap > kWideMaxCands) return hipErrorInvalidValue;
  const int nch = ncap / kWideChunk;
  const unsigned hgrid = (unsigned)(c.B * c.Hq * (ncap / kWideAlign)), ugrid = (unsigned)(c.B * c.Hkv * nch);
  const dim3 blk(HT);
  const int npm = ncap / (64 * est_batches(ncap, (int64_t)c.B * c.Hkv));
  hipLaunchKernelGGL(k_wide_hist1, dim3(hgrid), blk, 0, s, logits, ncap, wd.pmax, npm, p, iters, wd.state);
#define TWL_WIDE_G(GG)                                                                                      \
  case GG:                                                                                                  \
    if (full)                                                                                               \
      hipLaunchKernelGGL((k_wide_mask<GG, true>), dim3(ugrid), blk, 0, s, c, logits, ncap, wd.state, wd.keys, \
                         wd.rec_cnt, head_mask, mask_words, wd.uwords, wd.chunk_cnt, wd.chunk_mass);        \
    else                                                                                                    \
      hipLaunchKernelGGL((k_wide_mask<GG, false>), dim3(ugrid), blk, 0, s, c, logits, ncap, wd.state,        \
                         wd.keys, wd.rec_cnt, nullptr, 0, wd.uwords, nullptr, nullptr);                     \
    break;
  switch (c.G) {
    TWL_WIDE_G(1)
    TWL_WIDE_G(2)
    TWL_WIDE_G(4)
    TWL_WIDE_G(8)
    default: return hipErrorInvalidValue;
  }
#undef TWL_WIDE_G
  hipLaunchKernelGGL(k_wide_finish, dim3((unsigned)(c.B * c.Hq)), dim3(1024), 0, s, c.G, ncap, iters, full, wd.state,
                     wd.keys, wd.rec_cnt, wd.chunk_mass, threshold, wd.uwords, wd.chunk_cnt,
                     full ? head_mask : nullptr, full ? mask_words : 0);
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
