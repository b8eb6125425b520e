// Device helpers shared by the kernels: bf16/fp16 unpacking, fixed-order wave and block reductions.
// Every reduction here combines values in an order fixed by lane and wave index, so results are
// bitwise reproducible run to run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Butterfly all-reduce over the 64 lanes; every lane ends with the same bits (fp add/max commute).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
// Inclusive prefix sum over the lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Block-wide reductions for blocks of NW waves.  `red` must hold 2*NW floats of LDS; calls
// alternate between its two halves, so consecutive calls need only one barrier each.
template <int NW>
struct BlockReduce {
  float* red;
  int slot = 0;
  __device__ float sum(float x) {
    x = wave_sum(x);
    const int w = threadIdx.x >> 6;
    float* r = red + slot * NW;
    slot ^= 1;
    if ((threadIdx.x & 63) == 0) r[w] = x;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) t += r[i];
    return t;
  }
  __device__ float max(float x) {
    x = wave_max(x);
    const int w = threadIdx.x >> 6;
    float* r = red + slot * NW;
    slot ^= 1;
    if ((threadIdx.x & 63) == 0) r[w] = x;
    __syncthreads();
    float t = r[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) t = fmaxf(t, r[i]);
    return t;
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
// (Knuth's two-sum gives the exact difference as hi + lo; exp(hi + lo) ~ exp(hi) * (1 + lo)).
__device__ __forceinline__ float exp_diff(float a, float b) {
  const float s = a - b;
  const float bb = s - a;
  const float err = (a - (s - bb)) + (-b - bb);
  const float ex = expf(s);
  return fmaf(ex, err, ex);
}

// Clamp helpers
__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

}  // namespace twl
