// INT4 K cache append (2- and 8-bit codes for the estimator's precision ablation) and page key bounds.
//
// Twilight keeps a 4-bit copy of K for weight estimation (Paper-Notes "关键设计 / 4-bit K缓存量化";
// paperlayer §4.2 and §B.1: dynamic quantisation with fp16 scales and zero points, two values per
// byte).  One workgroup handles one (page, kv-head): 64 lanes = 16 slots x 4 groups of 32 channels.
// The codes, scale/zero and bounds are stored by (sequence, logical page), so the selector and the
// estimate read them without a page-table lookup; only K itself comes from the physical page.
// The page tile is read once (4 KB, coalesced) into LDS; each lane quantises its (slot, group) and
// then recomputes two channels of the page's min/max bound (Quest-style key bounds used by the page
// selector) over the slots that hold tokens below tok_end.
#include "twl_device.h"
#include "twl_internal.h"

namespace twl {

// BITS: code width (2, 4 or 8); a group's 32 codes fill BITS words, 32 / BITS codes per word with the
// lowest channel in the lowest bits, and L = 2^BITS - 1 levels.
template <int BITS>
__global__ __launch_bounds__(64) void k_quantize(CacheView c, const int32_t* __restrict__ tok_begin,
                                                 const int32_t* __restrict__ tok_end, int span_pages) {
  const int b = blockIdx.x / span_pages;
  const int jp = blockIdx.x - b * span_pages;
  const int h = blockIdx.y;
  const int t0 = tok_begin[b], t1 = tok_end[b];
  if (t0 < 0 || t1 > c.maxP * kPage || t0 >= t1) return;
  const int page = t0 / kPage + jp;
  if (page * kPage >= t1) return;
  const int phys = c.page_table[(size_t)b * c.maxP + page];
  if (phys < 0 || phys >= c.nphys) return;

  __shared__ uint32_t tile[kPage * kD / 2];  // 16 slots x 128 bf16
  const size_t row0 = ((size_t)phys * c.Hkv + h) * kPage;           // K: the physical page
  const size_t lrow0 = (((size_t)b * c.maxP + page) * c.Hkv + h) * kPage;  // codes: the logical page
  const uint4* src = reinterpret_cast<const uint4*>(c.k + row0 * kD);
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) reinterpret_cast<uint4*>(tile)[tid + 64 * i] = src[tid + 64 * i];
  __syncthreads();

  // ---- quantise slot `slot`, group `g` ---------------------------------------------------------------
  const int slot = tid >> 2, g = tid & 3;
  const int tok = page * kPage + slot;
  if (tok >= t0 && tok < t1) {
    float x[32];
    const uint32_t* w = tile + slot * (kD / 2) + g * 16;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t v = w[i];
      x[2 * i] = bf16_lo(v);
      x[2 * i + 1] = bf16_hi(v);
    }
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) {
      mn = fminf(mn, x[i]);
      mx = fmaxf(mx, x[i]);
    }
    const float range = mx - mn;
    constexpr int L = (1 << BITS) - 1, PER = 32 / BITS;
    const uint32_t sbits = float_to_half_bits(range / (float)L);  // IEEE fp32 division, then fp16 RNE
    const uint32_t zbits = float_to_half_bits(mn);
    const float s = half_bits_to_float(sbits);
    const float z = half_bits_to_float(zbits);
    uint32_t packed[BITS];
#pragma unroll
    for (int i = 0; i < BITS; ++i) packed[i] = 0u;
    if (s != 0.0f) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        float t = rintf((x[i] - z) / s);  // round half to even
        t = fminf(fmaxf(t, 0.0f), (float)L);
        const uint32_t code = (uint32_t)t;
        packed[i / PER] |= code << (BITS * (i % PER));
      }
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(c.k4 + (lrow0 + slot) * (16 * BITS)) + g * BITS;
#pragma unroll
    for (int i = 0; i < BITS; ++i) dst[i] = packed[i];
    c.k4_meta[(lrow0 + slot) * kGroups + g] = sbits | (zbits << 16);
  }

  // ---- page bound over slots holding tokens < tok_end: lane owns channels 2*tid, 2*tid+1 ----------
  const int valid = min(kPage, t1 - page * kPage);
  float mn0 = __builtin_inff(), mn1 = __builtin_inff();
  float mx0 = -__builtin_inff(), mx1 = -__builtin_inff();
  for (int sl = 0; sl < valid; ++sl) {
    const uint32_t v = tile[sl * (kD / 2) + tid];
    const float a = bf16_lo(v), bb = bf16_hi(v);
    mn0 = fminf(mn0, a);
    mn1 = fminf(mn1, bb);
    mx0 = fmaxf(mx0, a);
    mx1 = fmaxf(mx1, bb);
  }
  // quarter-major slice: quarter j = channels 32 j .. 32 j + 31 as 64 B of min then 64 B of max, so a
  // quarter of a page is one 128-byte line (16 words of min, then 16 of max, per quarter)
  uint32_t* kb = reinterpret_cast<uint32_t*>(c.kbound + (((size_t)b * c.maxP + page) * c.Hkv + h) * 2 * kD);
  const int qw = (tid >> 4) * 32 + (tid & 15);
  kb[qw] = (__float_as_uint(mn0) >> 16) | (__float_as_uint(mn1) & 0xffff0000u);
  kb[qw + 16] = (__float_as_uint(mx0) >> 16) | (__float_as_uint(mx1) & 0xffff0000u);
}

hipError_t launch_quantize(const CacheView& c, const int32_t* tok_begin, const int32_t* tok_end,
                           int span_pages, hipStream_t s) {
  if (span_pages <= 0) return hipSuccess;
  dim3 grid((unsigned)(c.B * span_pages), (unsigned)c.Hkv);
  switch (c.kbits) {
    case 2: hipLaunchKernelGGL(k_quantize<2>, grid, dim3(64), 0, s, c, tok_begin, tok_end, span_pages); break;
    case 4: hipLaunchKernelGGL(k_quantize<4>, grid, dim3(64), 0, s, c, tok_begin, tok_end, span_pages); break;
    case 8: hipLaunchKernelGGL(k_quantize<8>, grid, dim3(64), 0, s, c, tok_begin, tok_end, span_pages); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace twl
