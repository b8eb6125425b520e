// Device helpers shared by the kernels: bf16/fp16 unpacking, fixed-order wave and block reductions.
// Every reduction here combines values in an order fixed by lane and wave index, so results are
// bitwise reproducible run to run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "twl_internal.h"

namespace twl {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  _Float16 x = __builtin_bit_cast(_Float16, (uint16_t)h);
  return (float)x;
}
__device__ __forceinline__ uint32_t float_to_half_bits(float f) {
  _Float16 x = (_Float16)f;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, x);
}

// ---- DPP reductions: within each 16-lane row (xor 1, xor 2, rotate 4, rotate 8), then the four
// row results are read from lanes 0/16/32/48 and combined as (r0 + r1) + (r2 + r3).  The order is
// fixed by lane position, so the result is the same on every run; it is uniform across the wave.
// (These patterns give every lane a source, so no old value is kept: plain DPP moves.)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xf, 0xf, false);
}
constexpr int kDppXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;  // row_ror:4
constexpr int kDppRor8 = 0x128;  // row_ror:8

__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

__device__ __forceinline__ float wave_sum_dpp(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppRor4>(x);
  x += dpp_f<kDppRor8>(x);
  const float r0 = readlane_f(x, 0), r1 = readlane_f(x, 16), r2 = readlane_f(x, 32), r3 = readlane_f(x, 48);
  return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = fmaxf(x, dpp_f<kDppXor1>(x));
  x = fmaxf(x, dpp_f<kDppXor2>(x));
  x = fmaxf(x, dpp_f<kDppRor4>(x));
  x = fmaxf(x, dpp_f<kDppRor8>(x));
  const float r0 = readlane_f(x, 0), r1 = readlane_f(x, 16), r2 = readlane_f(x, 32), r3 = readlane_f(x, 48);
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_min_dpp(float x) {
  x = fminf(x, dpp_f<kDppXor1>(x));
  x = fminf(x, dpp_f<kDppXor2>(x));
  x = fminf(x, dpp_f<kDppRor4>(x));
  x = fminf(x, dpp_f<kDppRor8>(x));
  const float r0 = readlane_f(x, 0), r1 = readlane_f(x, 16), r2 = readlane_f(x, 32), r3 = readlane_f(x, 48);
  return fminf(fminf(r0, r1), fminf(r2, r3));
}

// Butterfly all-reduce of an integer over the 64 lanes; every lane ends with the total.
__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
// DPP lane moves for scans: row_shr:n shifts within each row of 16 lanes (lanes with no source read
// 0); row_bcast:15 / row_bcast:31 copy lane 15 / 31 into the rows selected by the row mask.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_scan_move(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xf, true);
}
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppShl4 = 0x104;  // row_shl:4 (lane n reads lane n + 4 of its row)
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

// Inclusive prefix sum over the lanes of a wave (DPP: four in-row steps, two row broadcasts).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_scan_move<kDppShr1, 0xf>(x);
  x += dpp_scan_move<kDppShr2, 0xf>(x);
  x += dpp_scan_move<kDppShr4, 0xf>(x);
  x += dpp_scan_move<kDppShr8, 0xf>(x);
  x += dpp_scan_move<kDppBcast15, 0xa>(x);
  x += dpp_scan_move<kDppBcast31, 0xc>(x);
  return x;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_scan_move_u64(uint64_t x) {
  const uint32_t lo = (uint32_t)dpp_scan_move<CTRL, ROW_MASK>((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)dpp_scan_move<CTRL, ROW_MASK>((int)(uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}
// Inclusive prefix sum of 64-bit integers over the lanes of a wave.
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t x) {
  x += dpp_scan_move_u64<kDppShr1, 0xf>(x);
  x += dpp_scan_move_u64<kDppShr2, 0xf>(x);
  x += dpp_scan_move_u64<kDppShr4, 0xf>(x);
  x += dpp_scan_move_u64<kDppShr8, 0xf>(x);
  x += dpp_scan_move_u64<kDppBcast15, 0xa>(x);
  x += dpp_scan_move_u64<kDppBcast31, 0xc>(x);
  return x;
}
// Inclusive prefix sum of 64-bit integers within each row of 16 lanes (lane 15 of a row holds the
// row's total).
__device__ __forceinline__ uint64_t row16_incl_scan_u64(uint64_t x) {
  x += dpp_scan_move_u64<kDppShr1, 0xf>(x);
  x += dpp_scan_move_u64<kDppShr2, 0xf>(x);
  x += dpp_scan_move_u64<kDppShr4, 0xf>(x);
  x += dpp_scan_move_u64<kDppShr8, 0xf>(x);
  return x;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Block-wide reductions for blocks of NW waves, built on the DPP wave reductions.  `red` must hold
// 2*NW*4 floats of LDS; calls alternate between its two halves, so consecutive calls need only one
// barrier each.  The wave results are combined in wave order, so the result is reproducible and
// identical in every thread.
template <int NW>
struct BlockReduce {
  float* red;
  int slot = 0;
  __device__ float* next() {
    float* r = red + slot * NW * 4;
    slot ^= 1;
    return r;
  }
  __device__ float sum(float x) {
    x = wave_sum_dpp(x);
    float* r = next();
    if ((threadIdx.x & 63) == 0) r[threadIdx.x >> 6] = x;
    __syncthreads();
    float t = r[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) t += r[i];
    return t;
  }
  __device__ float max(float x) {
    x = wave_max_dpp(x);
    float* r = next();
    if ((threadIdx.x & 63) == 0) r[threadIdx.x >> 6] = x;
    __syncthreads();
    float t = r[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) t = fmaxf(t, r[i]);
    return t;
  }
  // sum of a, min of b
  __device__ void sum_min(float& a, float& b) {
    a = wave_sum_dpp(a);
    b = wave_min_dpp(b);
    float* r = next();
    if ((threadIdx.x & 63) == 0) {
      r[threadIdx.x >> 6] = a;
      r[NW + (threadIdx.x >> 6)] = b;
    }
    __syncthreads();
    float ta = r[0], tb = r[NW];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
      ta += r[i];
      tb = fminf(tb, r[NW + i]);
    }
    a = ta;
    b = tb;
  }
  // two sums at once (counts below 2^24 are exact in float)
  __device__ void sum2(float& a, float& b) {
    a = wave_sum_dpp(a);
    b = wave_sum_dpp(b);
    float* r = next();
    if ((threadIdx.x & 63) == 0) {
      r[threadIdx.x >> 6] = a;
      r[NW + (threadIdx.x >> 6)] = b;
    }
    __syncthreads();
    float ta = r[0], tb = r[NW];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
      ta += r[i];
      tb += r[NW + i];
    }
    a = ta;
    b = tb;
  }
  // three sums at once (counts below 2^24 are exact in float)
  __device__ void sum3(float& a, float& b, float& c) {
    a = wave_sum_dpp(a);
    b = wave_sum_dpp(b);
    c = wave_sum_dpp(c);
    float* r = next();
    if ((threadIdx.x & 63) == 0) {
      const int w = threadIdx.x >> 6;
      r[w] = a;
      r[NW + w] = b;
      r[2 * NW + w] = c;
    }
    __syncthreads();
    float ta = r[0], tb = r[NW], tc = r[2 * NW];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
      ta += r[i];
      tb += r[NW + i];
      tc += r[2 * NW + i];
    }
    a = ta;
    b = tb;
    c = tc;
  }
};

// Block-wide exclusive scan of one int per thread (blocks of NW waves).  `sm` holds NW+1 ints.
// Returns the exclusive prefix; *total receives the block total.  Contains three barriers.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int* sm, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = wave_incl_scan(v);
  if (lane == 63) sm[w] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int i = 0; i < NW; ++i) {
      int t = sm[i];
      sm[i] = acc;
      acc += t;
    }
    sm[NW] = acc;
  }
  __syncthreads();
  const int base = sm[w];
  *total = sm[NW];
  __syncthreads();  // sm may be reused by the next call
  return base + incl - v;
}

// exp(a - b) for a <= b with the rounding error of the float32 subtraction carried into the result
// (Knuth's two-sum gives the exact difference as s + err; exp(s + err) ~ exp(s) * (1 + err)).
// exp(s) = 2^(s log2 e) with a Cody-Waite split of log2 e: th = fl(s * L) goes to the hardware
// exp2 and the remainder tl (the fma residual of the product plus s * (log2 e - L)) is applied to
// first order.  Measured on MI355X against float64 over 3.9M pairs with differences down to -90:
// at most 1.4e-7 relative error, the same as the libm expf form (1.3e-7) at half the instructions.
__device__ __forceinline__ float exp_diff(float a, float b) {
  constexpr float kLog2e = 1.44269502162933349609375f;      // float32(log2 e)
  constexpr float kLog2eLo = 1.92596299e-8f;               // log2 e - kLog2e
  constexpr float kLn2 = 0.693147182464599609375f;
  const float s = a - b;
  const float bb = s - a;
  const float err = (a - (s - bb)) + (-b - bb);
  const float th = s * kLog2e;
  const float tl = fmaf(s, kLog2eLo, fmaf(s, kLog2e, -th));
  const float ex = __builtin_amdgcn_exp2f(th);
  return fmaf(ex, fmaf(tl, kLn2, err), ex);
}

// Clamp helpers
__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Block index of a grid over (sequence b, item k, kv-head h) with the kv-head fastest: the blocks that
// take item k of a sequence for its kv-heads are dispatched side by side, so their reads of one page's
// per-head slices, which are adjacent in the paged cache, reach HBM together.  Returns the unit
// u = b * Hkv + h and writes the item.
__device__ __forceinline__ int head_fast_unit(int bid, int Hkv, int items, int& k) {
  const int h = bid % Hkv, r = bid / Hkv;
  const int b = r / items;
  k = r - b * items;
  return b * Hkv + h;
}

// The estimate's fixed-point query for channel group g of query row bh, written by 32 lanes (one half
// of a wave, lane l = channel 32 g + l):  E_g = floor(log2 max |q_c|) (>= -100; 0 for an all-zero
// group), Q_c = rne(q_c 2^(20 - E_g)), |Q_c| <= (2 - 2^-7) 2^20, as the digits Q = 2^14 d0 + 2^7 d1 + d2
// (d0 in [-128, 127], d1 and d2 in [0, 127]); byte pos of a digit row is channel 8 j + w of the group
// with pos = 8 j + perm(w), perm the order in which the code unpack feeds the matrix cores (the low
// nibbles or 2-bit fields of four code bytes first, then the high ones; identity for 8-bit codes).
__device__ __forceinline__ void query_digits_half(const uint16_t* __restrict__ q, int bh, int g, int kbits,
                                                  uint8_t* __restrict__ dig, int32_t* __restrict__ meta) {
  const int l = threadIdx.x & 31;
  const float x = __uint_as_float((uint32_t)q[(size_t)bh * kD + 32 * g + l] << 16);
  float m = fabsf(x);
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 32));
  int E = 0;
  if (m > 0.f) E = max((int)(__float_as_uint(m) >> 23) - 127, -100);
  const int Q = (int)rintf(ldexpf(x, kQFracBits - E));
  const int d0 = Q >> 14;           // floor(Q / 2^14)
  const int rm = Q - d0 * 16384;    // in [0, 2^14)
  const int d1 = rm >> 7, d2 = rm & 127;
  const int w = l & 7;
  const int pos = (l & ~7) + (kbits == 8 ? w : ((w & 1) ? 4 + (w >> 1) : (w >> 1)));
  uint8_t* row = dig + (size_t)(bh * 4 + g) * kQDigits * 32;
  row[pos] = (uint8_t)(d0 & 0xff);
  row[32 + pos] = (uint8_t)d1;
  row[64 + pos] = (uint8_t)d2;
  int sq = Q, s0 = d0, s1 = d1, s2 = d2;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    sq += __shfl_xor(sq, o, 32);
    s0 += __shfl_xor(s0, o, 32);
    s1 += __shfl_xor(s1, o, 32);
    s2 += __shfl_xor(s2, o, 32);
  }
  if (l == 0) {
    int32_t* mt = meta + (size_t)(bh * 4 + g) * kQMeta;
    mt[0] = E;
    mt[1] = sq;
    mt[2] = s0;
    mt[3] = s1;
    mt[4] = s2;
  }
}

// The query digit rows of the G heads of unit (b, h), shared out over the unit's blocks: block blk of
// bpu (nthreads each, a multiple of 32) takes the (head, group) pairs blk * halves + i, i < halves,
// then every bpu * halves-th pair after them.
__device__ __forceinline__ void unit_query_digits(const uint16_t* __restrict__ q, int Hq, int kbits, int b, int h,
                                                  int G, int nthreads, int blk, int bpu, const QDigits& qd) {
  const int halves = nthreads >> 5;
  for (int pr = blk * halves + ((int)threadIdx.x >> 5); pr < 4 * G; pr += bpu * halves)
    query_digits_half(q, b * Hq + h * G + (pr >> 2), pr & 3, kbits, qd.dig, qd.meta);
}

// ---- radix form of the top-p threshold search (shared by the block and the multi-block kernels) ----
// Masses are 64-bit fixed point, floor(w * 2^40): exact integer sums in any order.
constexpr float kFixScale = 1099511627776.0f;  // 2^40

__device__ __forceinline__ uint64_t to_fix(float e) { return (uint64_t)(e * kFixScale); }

// Digits of the threshold key.  Only weights >= 2^-40 carry mass (floor(e 2^40) >= 1), so the search
// runs over keys from the image of 2^-40 up: 11 bits of (key - floor) >> 18 (the exponent and five
// mantissa bits; below 2048 for weights under 2^24, as the fixed-point masses require), then bits
// 17..9 and 8..0 (the floor has no bits below 23, so those are the key's own bits).
constexpr uint32_t kKeyFloor = 87u << 23;  // uint32 image of 2^-40
__device__ __forceinline__ uint32_t key_d1(uint32_t key) { return (key - kKeyFloor) >> 18; }
__device__ __forceinline__ uint32_t key_d2(uint32_t key) { return (key >> 9) & 511u; }
__device__ __forceinline__ uint32_t key_d3(uint32_t key) { return key & 511u; }
// key >> 9 of the keys whose first two digits are d1, d2
__device__ __forceinline__ uint32_t key_pre2(uint32_t d1, uint32_t d2) { return (kKeyFloor >> 9) + (d1 << 9) + d2; }

__device__ __forceinline__ uint64_t wave_suffix_u64(uint64_t x) {
  // sum over lanes >= l: total minus the exclusive prefix
  const uint64_t p = wave_incl_scan_u64(x);
  return readlane_u64(p, 63) - p + x;
}

// A histogram word: a plain load, or (COH) an agent-scope atomic load, which sees every device-scope
// atomic already performed, also those of blocks on other dies, whose L2 this one does not share.
template <bool COH>
__device__ __forceinline__ uint64_t hist_load(const uint64_t* p) {
  if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}

// Largest bin of one histogram level whose suffix mass reaches `target` (>= 1), from its coarse
// sums (one per 32 bins) and then the 32 bins of the chosen coarse block; `rem` is the mass still
// needed inside the bin (target minus everything above it).  Called by a whole wave.
template <bool COH = false>
__device__ __forceinline__ void wide_find(const uint64_t* fine, const uint64_t* coarse, int ncoarse,
                                          uint64_t target, int& bin, uint64_t& rem) {
  const int lane = threadIdx.x & 63;
  const uint64_t x = (lane < ncoarse) ? hist_load<COH>(coarse + lane) : 0ull;
  const uint64_t px = wave_incl_scan_u64(x);
  const uint64_t tx = readlane_u64(px, 63);
  unsigned long long bal = __ballot(lane < ncoarse && tx - px + x >= target);
  const int cb = bal ? 63 - __clzll(bal) : 0;
  const uint64_t above = tx - readlane_u64(px, cb);  // mass of the coarse blocks above cb
  const uint64_t r1 = target - above;
  const uint64_t y = (lane < 32) ? hist_load<COH>(fine + 32 * cb + lane) : 0ull;
  const uint64_t py = wave_incl_scan_u64(y);
  const uint64_t ty = readlane_u64(py, 63);
  bal = __ballot(lane < 32 && ty - py + y >= r1);
  const int fb = bal ? 63 - __clzll(bal) : 0;
  const uint64_t above2 = ty - readlane_u64(py, fb);
  bin = 32 * cb + fb;
  rem = r1 - above2;
}

}  // namespace twl
