// INT4 weight estimate: the mixed-precision SpGEMV of the query against the dequantised 4-bit keys
// (paperlayer §4.2; §B.1, Fig. 12).  One lane per candidate token and quantisation group, the GQA
// group's G query heads in the same lane so each code byte and scale/zero pair is read once.
//
// Per head and 32-channel group g the logit is factorised exactly as
//   sum_{c in g} q_c (code_c s_g + z_g) = s_g * a_g + z_g * b_g,  a_g = sum q_c code_c,  b_g = sum q_c
// and evaluated in this fixed float32 order (the products q_c*code_c are exact, so the fused
// multiply-adds are plain rounded additions):
//   a_g = fold_{c in g}(a + q_c*code_c),  t_g = fl(s_g*a_g) + fl(z_g*b_g),
//   logit = fl(sm * ((t_0 + t_1) + (t_2 + t_3))).
// The file is compiled without floating-point contraction so that t_g rounds each product.
#include "twl_device.h"
#include "twl_internal.h"

namespace twl {

// Map candidate index k of unit u to a logical token id; returns -1 when k is not a candidate.
__device__ __forceinline__ int cand_token(const CandView& cand, int u, int k, int n) {
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
  // ranges: binary search the item whose prefix interval holds k
  const int cnt = clampi(cand.count[u], 0, cand.max_items);
  const int32_t* pre = cand.range_prefix + (size_t)u * (cand.max_items + 1);
  if (k >= pre[cnt]) return -1;
  int lo = 0, hi = cnt;  // pre[lo] <= k < pre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= k) lo = mid; else hi = mid;
  }
  const int t = cand.items[((size_t)u * cand.max_items + lo) * 2] + (k - pre[lo]);
  return (t >= 0 && t < n) ? t : -1;
}

// Prefix sums of range lengths per unit (lengths < 0 count as 0).
__global__ __launch_bounds__(256) void k_range_prefix(CacheView c, CandView cand, int32_t* prefix) {
  constexpr int NW = 4;
  __shared__ int scan_sm[NW + 1];
  const int u = blockIdx.x;
  const int cnt = clampi(cand.count[u], 0, cand.max_items);
  int32_t* pre = prefix + (size_t)u * (cand.max_items + 1);
  int carry = 0;
  for (int base = 0; base < cnt; base += 256) {
    const int i = base + (int)threadIdx.x;
    int len = 0;
    if (i < cnt) len = max(0, cand.items[((size_t)u * cand.max_items + i) * 2 + 1]);
    int total;
    const int ex = block_excl_scan<NW>(len, scan_sm, &total);
    if (i < cnt) pre[i] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) pre[cnt] = carry;
}

// One block = 64 candidates x 4 waves; wave g handles quantisation group g (32 channels) of every
// candidate for all G heads, so each wave reads only its 16-byte slice of the code row and its
// scale/zero pair.  The per-group terms meet in LDS and are combined in the committed order.
template <int G>
__global__ __launch_bounds__(256) void k_estimate(CacheView c, const uint16_t* __restrict__ q, float sm,
                                                  CandView cand, int ncap, int chunks_per_unit,
                                                  float* __restrict__ logits, int32_t* counters) {
  const int u = blockIdx.x / chunks_per_unit;
  const int ck = blockIdx.x - u * chunks_per_unit;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  if (ck == 0 && threadIdx.x == 0) counters[u] = 0;  // arrival counter of the group's top-p blocks

  __shared__ float qs[G][kD];
  __shared__ float bs[G][kGroups];
  __shared__ float T[kGroups][G][64];
  const uint16_t* qg = q + ((size_t)b * c.Hq + (size_t)h * G) * kD;
  for (int i = threadIdx.x; i < G * kD; i += 256) qs[i / kD][i % kD] = __uint_as_float((uint32_t)qg[i] << 16);
  __syncthreads();
  if (threadIdx.x < G * kGroups) {
    const int hh = threadIdx.x / kGroups, g = threadIdx.x % kGroups;
    float acc = 0.f;
    for (int ch = g * 32; ch < g * 32 + 32; ++ch) acc = acc + qs[hh][ch];
    bs[hh][g] = acc;
  }
  __syncthreads();

  const int g = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = clampi(c.seq_lens[b], 0, c.maxTok);
  const int k = ck * 64 + lane;
  const int tok = cand_token(cand, u, k, n);
  if (tok >= 0) {
    const int phys = c.page_table[(size_t)b * c.maxP + (tok >> 4)];
    const size_t row = ((size_t)phys * c.Hkv + h) * kPage + (tok & 15);
    const uint4 cw = reinterpret_cast<const uint4*>(c.k4 + row * 64)[g];
    const uint32_t mw = c.k4_meta[row * kGroups + g];
    const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
    float a[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) a[hh] = 0.f;
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
      const uint32_t lo = words[wi] & 0x0F0F0F0Fu;
      const uint32_t hi = (words[wi] >> 4) & 0x0F0F0F0Fu;
      float code[8];
      code[0] = (float)(lo & 0xFFu);
      code[1] = (float)(hi & 0xFFu);
      code[2] = (float)((lo >> 8) & 0xFFu);
      code[3] = (float)((hi >> 8) & 0xFFu);
      code[4] = (float)((lo >> 16) & 0xFFu);
      code[5] = (float)((hi >> 16) & 0xFFu);
      code[6] = (float)(lo >> 24);
      code[7] = (float)(hi >> 24);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ch = g * 32 + wi * 8 + e;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) a[hh] = fmaf(qs[hh][ch], code[e], a[hh]);
      }
    }
    const float s = half_bits_to_float(mw & 0xffffu);
    const float z = half_bits_to_float(mw >> 16);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float sa = s * a[hh];
      const float zb = z * bs[hh][g];
      T[g][hh][lane] = sa + zb;
    }
  }
  __syncthreads();
  for (int hh = g; hh < G; hh += kGroups) {
    float lg = -__builtin_inff();
    if (tok >= 0) {
      const float r01 = T[0][hh][lane] + T[1][hh][lane];
      const float r23 = T[2][hh][lane] + T[3][hh][lane];
      lg = sm * (r01 + r23);
    }
    if (k < ncap) logits[((size_t)b * c.Hq + (size_t)h * G + hh) * ncap + k] = lg;
  }
}

hipError_t launch_range_prefix(const CacheView& c, const CandView& cand, int32_t* prefix, hipStream_t s) {
  hipLaunchKernelGGL(k_range_prefix, dim3((unsigned)(c.B * c.Hkv)), dim3(256), 0, s, c, cand, prefix);
  return hipGetLastError();
}

hipError_t launch_estimate(const CacheView& c, const uint16_t* q, float sm, const CandView& cand, int ncap,
                           float* logits, int32_t* counters, hipStream_t s) {
  const int cpu = (ncap + 63) / 64;
  dim3 grid((unsigned)(c.B * c.Hkv * cpu));
  switch (c.G) {
    case 1: hipLaunchKernelGGL(k_estimate<1>, grid, dim3(256), 0, s, c, q, sm, cand, ncap, cpu, logits, counters); break;
    case 2: hipLaunchKernelGGL(k_estimate<2>, grid, dim3(256), 0, s, c, q, sm, cand, ncap, cpu, logits, counters); break;
    case 4: hipLaunchKernelGGL(k_estimate<4>, grid, dim3(256), 0, s, c, q, sm, cand, ncap, cpu, logits, counters); break;
    case 8: hipLaunchKernelGGL(k_estimate<8>, grid, dim3(256), 0, s, c, q, sm, cand, ncap, cpu, logits, counters); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace twl
