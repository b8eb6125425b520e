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
//
// A block holds 2 or 4 batches of 64 candidates x 4 waves; wave g handles group g of every
// candidate, reading only its 16-byte slice of the code row and its scale/zero pair.  The query values of a wave's group are
// wave-uniform and live in scalar registers.  The per-group terms meet in LDS and are combined in the
// committed order.  The block also records, per candidate, its token id and K/V row index, which the
// union of the kept sets then gathers without further lookups.
#include "twl_device.h"
#include "twl_internal.h"

namespace twl {

// Map candidate index k of unit u to a logical token id for the "all" and "pages" forms; returns -1
// when k is not a candidate.  (The ranges form is resolved block-wide inside the estimate.)
__device__ __forceinline__ int cand_token(const CandView& cand, int u, int k, int n) {
  if (cand.mode == kCandAll) return k < n ? k : -1;
  const int P = (n + kPage - 1) / kPage;
  const int cnt = clampi(cand.count[u], 0, cand.max_items);
  const int pi = k >> 4;
  if (pi >= cnt) return -1;
  const int page = cand.items[(size_t)u * cand.max_items + pi];
  if (page < 0 || page >= P) return -1;
  const int t = page * kPage + (k & 15);
  return t < n ? t : -1;
}

// Prefix sums of range lengths per unit (lengths < 0 count as 0), and for every block of kEstCands
// candidates the index of the range holding its first candidate (count when past the last one).
// Up to 4096 ranges (4 per thread, loads issued together with the count) the prefix sums stay in
// LDS and each block start is found there by binary search; longer lists take passes of 4096 and
// each range marks the block starts it holds.
__global__ __launch_bounds__(1024) void k_range_prefix(CacheView c, CandView cand, int32_t* prefix,
                                                       int32_t* chunk_first, int nchunk) {
  constexpr int NT = 1024, NW = NT / 64, IPT = 4, MAXL = NT * IPT;
  __shared__ int scan_sm[NW + 1];
  __shared__ int spre[MAXL + 1];
  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t* pre = prefix + (size_t)u * (cand.max_items + 1);
  int32_t* cf = chunk_first + (size_t)u * nchunk;
  const int32_t* it = cand.items + (size_t)u * cand.max_items * 2;
  const int i0 = tid * IPT;
  int len[IPT];
#pragma unroll
  for (int i = 0; i < IPT; ++i) len[i] = it[(size_t)min(i0 + i, cand.max_items - 1) * 2 + 1];
  const int cnt = clampi(cand.count[u], 0, cand.max_items);
  if (cnt <= MAXL) {
    int local = 0;
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      len[i] = (i0 + i < cnt) ? max(0, len[i]) : 0;
      local += len[i];
    }
    int total;
    int s0 = block_excl_scan<NW>(local, scan_sm, &total);
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      if (i0 + i < cnt) {
        pre[i0 + i] = s0;
        spre[i0 + i] = s0;
      }
      s0 += len[i];
    }
    if (tid == 0) {
      pre[cnt] = total;
      spre[cnt] = total;
    }
    __syncthreads();
    for (int j = tid; j < nchunk; j += NT) {
      const int x = j * kEstCands;
      int r = cnt;
      if (x < total) {
        int lo = 0, hi = cnt;  // largest lo with spre[lo] <= x (a non-empty range: x < total)
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (spre[mid] <= x) lo = mid; else hi = mid;
        }
        r = lo;
      }
      cf[j] = r;
    }
    return;
  }
  int carry = 0;
  for (int base = 0; base < cnt; base += MAXL) {
    const int ib = base + i0;
    int local = 0;
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      len[i] = (ib + i < cnt) ? max(0, it[(size_t)(ib + i) * 2 + 1]) : 0;
      local += len[i];
    }
    int total;
    int s0 = carry + block_excl_scan<NW>(local, scan_sm, &total);
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      if (ib + i < cnt) {
        pre[ib + i] = s0;
        if (len[i] > 0) {
          const int64_t e0 = (int64_t)s0 + len[i];
          for (int j = (s0 + kEstCands - 1) / kEstCands; j < nchunk && (int64_t)j * kEstCands < e0; ++j) cf[j] = ib + i;
        }
        s0 += len[i];
      }
    }
    carry += total;
  }
  if (tid == 0) pre[cnt] = carry;
  for (int j = tid; j < nchunk; j += NT)
    if ((int64_t)j * kEstCands >= carry) cf[j] = cnt;
}

// Token id and K/V row of candidate k (row -1 when k is not a candidate).  `cnt` is the unit's item
// count for the page and range forms.
__device__ __forceinline__ void cand_resolve(const CacheView& c, const CandView& cand, int u, int b, int h, int k,
                                             int n, int cnt, int& tok, int& row) {
  tok = -1;
  row = -1;
  if (cand.mode == kCandPages && cand.phys) {
    // the id loads do not wait for the count: the index is clamped into the unit's row and the
    // entry is discarded afterwards when it lies past the count
    const int pi = k >> 4;
    const size_t idx = (size_t)u * cand.max_items + min(pi, cand.max_items - 1);
    const int page = cand.items[idx];
    const int phys = cand.phys[idx];
    const int t = page * kPage + (k & 15);
    if (pi < cnt && page >= 0 && t < n) {
      tok = t;
      row = (phys * c.Hkv + h) * kPage + (k & 15);
    }
    return;
  }
  tok = cand_token(cand, u, k, n);
  if (tok >= 0) row = (c.page_table[(size_t)b * c.maxP + (tok >> 4)] * c.Hkv + h) * kPage + (tok & 15);
}

// Byte n of x as a float (one conversion instruction each).
__device__ __forceinline__ float ub0(uint32_t x) { float r; asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(x)); return r; }
__device__ __forceinline__ float ub1(uint32_t x) { float r; asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(x)); return r; }
__device__ __forceinline__ float ub2(uint32_t x) { float r; asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(x)); return r; }
__device__ __forceinline__ float ub3(uint32_t x) { float r; asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(x)); return r; }

// NB batches of 64 candidates per block (64 * NB candidates, NB = 2 or 4).
template <int G, int NB>
__global__ __launch_bounds__(256) void k_estimate(CacheView c, const uint16_t* __restrict__ q, float sm,
                                                  CandView cand, int ncap, int chunks_per_unit,
                                                  float* __restrict__ logits, int32_t* __restrict__ cand_tok,
                                                  int32_t* __restrict__ cand_row, float* __restrict__ pmax,
                                                  uint64_t* __restrict__ wstate, size_t wstate_words) {
  constexpr int NC = 64 * NB;
  constexpr int NH = (G + kGroups - 1) / kGroups;  // heads combined per wave
  const int u = blockIdx.x / chunks_per_unit;
  const int ck = blockIdx.x - u * chunks_per_unit;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int g = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  __shared__ float T[2][kGroups][G][64];
  __shared__ int s_row[NB][64];
  if (wstate) {
    // clear the wide top-p state for the passes that follow this kernel
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < wstate_words; i += (size_t)gridDim.x * 256)
      wstate[i] = 0ull;
  }
  const int n = clampi(c.seq_lens[b], 0, c.maxTok);
  const int cnt = (cand.mode == kCandAll) ? 0 : clampi(cand.count[u], 0, cand.max_items);
  const int k0 = ck * NC;

  // ---- candidate resolution: wave w resolves batches w, w + 4, ... (token id and K/V row); the
  // rows meet in LDS so each is resolved once
  if (cand.mode == kCandRanges) {
    // The block's candidates lie in the ranges r0..rmax; their prefix sums and first tokens are
    // staged in LDS when they fit, and every lane searches there.
    __shared__ int s_pre[NC + 1];
    __shared__ int s_beg[NC + 1];
    const int32_t* pre = cand.range_prefix + (size_t)u * (cand.max_items + 1);
    const int nchunk = ncap / kEstCands;
    const int j0 = k0 / kEstCands, j1 = (k0 + NC - 1) / kEstCands;
    const int r0 = clampi(cand.chunk_first[(size_t)u * nchunk + j0], 0, cnt);
    const int r1 = (j1 + 1 < nchunk) ? clampi(cand.chunk_first[(size_t)u * nchunk + j1 + 1], 0, cnt) : cnt;
    const int rmax = min(r1, cnt - 1);
    const int nr = rmax - r0 + 1;
    const int tot = pre[cnt];
    const bool staged = nr >= 1 && nr <= NC + 1;
    if (staged) {
      for (int i = threadIdx.x; i < nr; i += 256) {
        s_pre[i] = pre[r0 + i];
        s_beg[i] = cand.items[((size_t)u * cand.max_items + r0 + i) * 2];
      }
    }
    __syncthreads();
    for (int bt = g; bt < NB; bt += kGroups) {
      const int k = k0 + 64 * bt + lane;
      int t = -1;
      if (nr >= 1 && k < tot) {
        int lo, beg, p0;
        if (staged) {
          lo = 0;
          int hi = nr;  // largest lo with s_pre[lo] <= k
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_pre[mid] <= k) lo = mid; else hi = mid;
          }
          p0 = s_pre[lo];
          beg = s_beg[lo];
        } else {
          lo = r0;
          int hi = rmax + 1;
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (pre[mid] <= k) lo = mid; else hi = mid;
          }
          p0 = pre[lo];
          beg = cand.items[((size_t)u * cand.max_items + lo) * 2];
        }
        if (p0 <= k) t = beg + (k - p0);
      }
      const int tok = (t >= 0 && t < n) ? t : -1;
      const int row = tok >= 0 ? (c.page_table[(size_t)b * c.maxP + (tok >> 4)] * c.Hkv + h) * kPage + (tok & 15) : -1;
      s_row[bt][lane] = row;
      cand_tok[(size_t)u * ncap + k] = tok;
      cand_row[(size_t)u * ncap + k] = row;
    }
  } else {
    for (int bt = g; bt < NB; bt += kGroups) {
      const int k = k0 + 64 * bt + lane;
      int tok, row;
      cand_resolve(c, cand, u, b, h, k, n, cnt, tok, row);
      s_row[bt][lane] = row;
      cand_tok[(size_t)u * ncap + k] = tok;
      cand_row[(size_t)u * ncap + k] = row;
    }
  }
  __syncthreads();

  // ---- this wave's group of every candidate: code and scale/zero loads all in flight together
  int rowv[NB];
  uint4 cwv[NB];
  uint32_t mwv[NB];
#pragma unroll
  for (int bt = 0; bt < NB; ++bt) rowv[bt] = s_row[bt][lane];
#pragma unroll
  for (int bt = 0; bt < NB; ++bt) {
    if (rowv[bt] >= 0) {
      cwv[bt] = reinterpret_cast<const uint4*>(c.k4 + (size_t)rowv[bt] * 64)[g];
      mwv[bt] = c.k4_meta[(size_t)rowv[bt] * kGroups + g];
    } else {
      cwv[bt] = make_uint4(0u, 0u, 0u, 0u);
      mwv[bt] = 0u;
    }
  }

  // this wave's 32 query channels per head, as bf16 pairs (wave-uniform: scalar loads)
  const uint32_t* qw = reinterpret_cast<const uint32_t*>(q + ((size_t)b * c.Hq + (size_t)h * G) * kD) + g * 16;
  float bsum[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t w = qw[hh * 64 + i];
      acc = acc + bf16_lo(w);
      acc = acc + bf16_hi(w);
    }
    bsum[hh] = acc;
  }

  float mx[NH];  // running maxima of this wave's heads (pmax)
#pragma unroll
  for (int i = 0; i < NH; ++i) mx[i] = -__builtin_inff();
#pragma unroll
  for (int bt = 0; bt < NB; ++bt) {
    const int k = k0 + 64 * bt + lane;
    if (rowv[bt] >= 0) {
      // the group's 32 codes as floats (element 2j of byte j is its low nibble)
      const uint32_t words[4] = {cwv[bt].x, cwv[bt].y, cwv[bt].z, cwv[bt].w};
      float code[32];
#pragma unroll
      for (int wi = 0; wi < 4; ++wi) {
        const uint32_t lo = words[wi] & 0x0F0F0F0Fu;
        const uint32_t hi = (words[wi] >> 4) & 0x0F0F0F0Fu;
        code[8 * wi + 0] = ub0(lo);
        code[8 * wi + 1] = ub0(hi);
        code[8 * wi + 2] = ub1(lo);
        code[8 * wi + 3] = ub1(hi);
        code[8 * wi + 4] = ub2(lo);
        code[8 * wi + 5] = ub2(hi);
        code[8 * wi + 6] = ub3(lo);
        code[8 * wi + 7] = ub3(hi);
      }
      const float s = half_bits_to_float(mwv[bt] & 0xffffu);
      const float z = half_bits_to_float(mwv[bt] >> 16);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        // head-outer order keeps only one head's 32 query values in scalar registers at a time
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t w = qw[hh * 64 + i];  // channels 32g + 2i, 2i + 1
          a = fmaf(bf16_lo(w), code[2 * i], a);
          a = fmaf(bf16_hi(w), code[2 * i + 1], a);
        }
        const float sa = s * a;
        const float zb = z * bsum[hh];
        T[bt & 1][g][hh][lane] = sa + zb;
      }
    }
    __syncthreads();  // T[bt & 1] complete; T[(bt + 1) & 1] was last read before this barrier
#pragma unroll
    for (int i = 0; i < NH; ++i) {
      const int hh = g + kGroups * i;
      if (hh < G) {
        float lg = -__builtin_inff();
        if (rowv[bt] >= 0) {
          const float r01 = T[bt & 1][0][hh][lane] + T[bt & 1][1][hh][lane];
          const float r23 = T[bt & 1][2][hh][lane] + T[bt & 1][3][hh][lane];
          lg = sm * (r01 + r23);
        }
        mx[i] = fmaxf(mx[i], lg);
        logits[((size_t)b * c.Hq + (size_t)h * G + hh) * ncap + k] = lg;
      }
    }
  }
  if (pmax) {
#pragma unroll
    for (int i = 0; i < NH; ++i) {
      const int hh = g + kGroups * i;
      if (hh < G) {
        const float m = wave_max_dpp(mx[i]);
        if (lane == 0) pmax[((size_t)b * c.Hq + (size_t)h * G + hh) * chunks_per_unit + ck] = m;
      }
    }
  }
}

hipError_t launch_range_prefix(const CacheView& c, const CandView& cand, int32_t* prefix, int32_t* chunk_first,
                               int nchunk, hipStream_t s) {
  hipLaunchKernelGGL(k_range_prefix, dim3((unsigned)(c.B * c.Hkv)), dim3(1024), 0, s, c, cand, prefix, chunk_first,
                     nchunk);
  return hipGetLastError();
}

// 4 batches for large steps (and always for the wide top-p, whose per-block maxima region holds
// ncap / 256 entries per head), 2 for small ones (more blocks in flight)
int est_batches(int64_t ncap, int64_t units) {
  return (ncap > kNarrowMaxCands || ncap * units >= ((int64_t)1 << 19)) ? 4 : 2;
}

hipError_t launch_estimate(const CacheView& c, const uint16_t* q, float sm, const CandView& cand, int ncap,
                           float* logits, int32_t* cand_tok, int32_t* cand_row, const WideWs* wide, hipStream_t s) {
  const int nb = est_batches(ncap, (int64_t)c.B * c.Hkv);
  if (ncap % (64 * nb) || ncap % kEstCands) return hipErrorInvalidValue;
  const int cpu = ncap / (64 * nb);
  dim3 grid((unsigned)(c.B * c.Hkv * cpu));
  float* pmax = wide ? wide->pmax : nullptr;
  uint64_t* wst = wide ? wide->state : nullptr;
  const size_t wwords = wide ? (size_t)c.B * c.Hq * kWideStateWords : 0;
#define TWL_EST_G(GG, NB)                                                                                     \
  case GG:                                                                                                    \
    hipLaunchKernelGGL((k_estimate<GG, NB>), grid, dim3(256), 0, s, c, q, sm, cand, ncap, cpu, logits,        \
                       cand_tok, cand_row, pmax, wst, wwords);                                               \
    break;
#define TWL_EST_NB(NB)                      \
  case NB:                                  \
    switch (c.G) {                          \
      TWL_EST_G(1, NB)                      \
      TWL_EST_G(2, NB)                      \
      TWL_EST_G(4, NB)                      \
      TWL_EST_G(8, NB)                      \
      default: return hipErrorInvalidValue; \
    }                                       \
    break;
  switch (nb) {
    TWL_EST_NB(2)
    TWL_EST_NB(4)
    default: return hipErrorInvalidValue;
  }
#undef TWL_EST_G
#undef TWL_EST_NB
  return hipGetLastError();
}

}  // namespace twl
