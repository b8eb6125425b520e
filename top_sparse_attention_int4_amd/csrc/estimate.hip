// INT4 weight estimate: the mixed-precision SpGEMV of the query against the dequantised 4-bit keys
// (paperlayer §4.2; §B.1, Fig. 12) as an int8 matrix-core contraction.
//
// Per head and 32-channel group g the query is held in fixed point, Q_c = rne(q_c 2^(20 - E_g)) with
// E_g = floor(log2 max |q_c|) (|Q_c| <= 2088960; exact for channels within 2^12 of the largest, i.e.
// for every channel of an ordinary bf16 query), as three int8 digits Q = 2^14 d2 + 2^7 d1 + d0, so
//   sum_{c in g} q~_c (code_c s_g + z_g) = s_g a_g + z_g b_g,  a_g = 2^(E_g-20) sum Q_c code_c,
//   b_g = 2^(E_g-20) sum Q_c
// has exact integer group sums in any order; then, in float64,
//   t_g = s_g a_g + z_g b_g (both products exact, one rounding),  r = (t_0 + t_1) + (t_2 + t_3),
//   logit = float32(sm * r)
// -- the float64 definition of the estimate for the grid query q~, rounded once to float32.
//
// The sums are v_mfma_i32_16x16x32_i8 products: A = 16 candidates x 32 codes (lane (r, kb) reads the
// code run of group kb of candidate r with one load -- 16 bytes of 4-bit codes; 8 or 32 bytes for the
// 2- and 8-bit widths of the precision ablation, paperlayer §4.2, Fig. 6 -- and feeds 8 codes as bytes
// to each of four MFMAs; 8-bit codes go in as code - 128 with the columns started at 128 x the digit
// sums), B = the query digits, one column per (group, head) and zero outside the lane's group, so
// each output column accumulates one group of one head.  A wave takes 16-candidate tiles; the four
// groups of a (candidate, head) then meet by two lane exchanges in the committed order.  The block
// also records, per candidate, its token id and K/V row index, which the union of the kept sets then
// gathers without further lookups.
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

typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kQDigits = 3;     // int8 digits of the fixed-point query
constexpr int kQFracBits = 20;  // Q = rne(q 2^(kQFracBits - E_g))
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// The BITS words of one (candidate, group) code run: 32 codes of BITS bits, lowest channel lowest.
template <int BITS>
__device__ __forceinline__ void load_codes(const uint8_t* row, int group, uint32_t (&w)[BITS]) {
  const uint8_t* p = row + group * 4 * BITS;
  if constexpr (BITS == 2) {
    const u32x2_t x = *reinterpret_cast<const u32x2_t*>(p);
    w[0] = x.x;
    w[1] = x.y;
  } else {
#pragma unroll
    for (int h = 0; h < BITS / 4; ++h) {
      const u32x4_t x = reinterpret_cast<const u32x4_t*>(p)[h];
      w[4 * h] = x.x;
      w[4 * h + 1] = x.y;
      w[4 * h + 2] = x.z;
      w[4 * h + 3] = x.w;
    }
  }
}

// Four 4-bit fields (nibbles 0..3 of t) to the four bytes of a word.
__device__ __forceinline__ uint32_t nibbles_to_bytes(uint32_t t) {
  return (t & 0xFu) | ((t & 0xF0u) << 4) | ((t & 0xF00u) << 8) | ((t & 0xF000u) << 12);
}

// The 8 int8 operands of MFMA j: channels 8j .. 8j + 7 of the group.  For 2 and 4 bits they come in
// the order (0, 2, 4, 6, 1, 3, 5, 7) of the slice; for 8 bits in channel order, shifted to code - 128.
template <int BITS>
__device__ __forceinline__ long code_operand(const uint32_t (&w)[BITS], int j) {
  if constexpr (BITS == 4) {
    const uint32_t lo = w[j] & 0x0F0F0F0Fu, hi = (w[j] >> 4) & 0x0F0F0F0Fu;
    return (long)((uint64_t)lo | ((uint64_t)hi << 32));
  } else if constexpr (BITS == 2) {
    const uint32_t x = (w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    const uint32_t lo = nibbles_to_bytes(x & 0x3333u), hi = nibbles_to_bytes((x >> 2) & 0x3333u);
    return (long)((uint64_t)lo | ((uint64_t)hi << 32));
  } else {
    return (long)(((uint64_t)w[2 * j] | ((uint64_t)w[2 * j + 1] << 32)) ^ 0x8080808080808080ull);
  }
}

// NB batches of 64 candidates per block (64 * NB candidates, NB = 2 or 4): 4 NB tiles of 16, NB per wave.
// BITS: code width (2, 4 or 8; rows of 16 * BITS bytes).
template <int G, int NB, int BITS>
__global__ __launch_bounds__(256) void k_estimate(CacheView c, const uint16_t* __restrict__ q, float sm,
                                                  CandView cand, int ncap, int chunks_per_unit,
                                                  float* __restrict__ logits, int32_t* __restrict__ cand_tok,
                                                  int32_t* __restrict__ cand_row, float* __restrict__ pmax,
                                                  uint64_t* __restrict__ wstate, size_t wstate_words) {
  constexpr int NC = 64 * NB;
  constexpr int GT = G < 4 ? G : 4;  // heads per 16-column MFMA tile (4 groups x GT heads)
  constexpr int NTL = G / GT;        // column tiles
  const int u = blockIdx.x / chunks_per_unit;
  const int ck = blockIdx.x - u * chunks_per_unit;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  __shared__ int s_row[NB][64];
  // query digits (Q = 2^14 [0] + 2^7 [1] + [2]), channel 8j + w of a group at byte 8j + perm(w), the
  // order in which the nibbles of 4 code bytes are unpacked (low nibbles of bytes 0..3, then high)
  __shared__ __align__(16) int8_t s_qd[kQDigits][G][kD];
  __shared__ int s_qe[G][kGroups];   // group exponents E_g
  __shared__ int s_qs[G][kGroups];   // sum_{c in g} Q_c (|.| < 2^26)
  __shared__ int s_qds[kQDigits][G][kGroups];  // per digit, its sum over the group (8-bit codes: the offset of 128)
  __shared__ float s_max[4][G];
  if (wstate) {
    // clear the wide top-p state for the passes that follow this kernel
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < wstate_words; i += (size_t)gridDim.x * 256)
      wstate[i] = 0ull;
  }
  const int n = clampi(c.seq_lens[b], 0, c.maxTok);
  const int cnt = (cand.mode == kCandAll) ? 0 : clampi(cand.count[u], 0, cand.max_items);
  const int k0 = ck * NC;
  // the query: lane pr < 4 G of wave 0 turns the 32 channels of (head pr / 4, group pr % 4) into fixed
  // point on its own (no cross-lane reductions); its 64 bytes are read first
  const bool qlane = wv == 0 && lane < kGroups * G;
  const int qh = qlane ? lane >> 2 : 0, qg = lane & 3;
  u32x4_t qraw[4];
  if (qlane) {
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(q + ((size_t)b * c.Hq + (size_t)h * G + qh) * kD + qg * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) qraw[i] = qp[i];
  }

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
    for (int bt = wv; bt < NB; bt += kGroups) {
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
      if (cand_tok) cand_tok[(size_t)u * ncap + k] = tok;
      cand_row[(size_t)u * ncap + k] = row;
    }
  } else {
    for (int bt = wv; bt < NB; bt += kGroups) {
      const int k = k0 + 64 * bt + lane;
      int tok, row;
      cand_resolve(c, cand, u, b, h, k, n, cnt, tok, row);
      s_row[bt][lane] = row;
      if (cand_tok) cand_tok[(size_t)u * ncap + k] = tok;
      cand_row[(size_t)u * ncap + k] = row;
    }
  }
  // ---- the fixed-point query (wave 0), ordered before the code loads by the barrier below
  if (qlane) {
    float x[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t wq[4] = {qraw[i].x, qraw[i].y, qraw[i].z, qraw[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[8 * i + 2 * k] = bf16_lo(wq[k]);
        x[8 * i + 2 * k + 1] = bf16_hi(wq[k]);
      }
    }
    float m = 0.f;
#pragma unroll
    for (int cc = 0; cc < 32; ++cc) m = fmaxf(m, fabsf(x[cc]));
    int E = 0;
    if (m > 0.f) E = max((int)(__float_as_uint(m) >> 23) - 127, -100);
    int qs = 0, ds[kQDigits] = {0, 0, 0};
    uint32_t dw[kQDigits][8];  // the digits' bytes, 4 per word, in the unpack order of the codes
#pragma unroll
    for (int d = 0; d < kQDigits; ++d)
#pragma unroll
      for (int k = 0; k < 8; ++k) dw[d][k] = 0u;
#pragma unroll
    for (int cc = 0; cc < 32; ++cc) {
      // |x| < 2^(E+1), so |Q| <= (2 - 2^-7) 2^20 (exact in float32 before and after the rounding)
      const int Qv = (int)rintf(ldexpf(x[cc], kQFracBits - E));
      const int d2 = Qv >> 14;            // floor(Q / 2^14) in [-128, 127]
      const int rm = Qv - d2 * 16384;     // in [0, 2^14)
      const int dg[kQDigits] = {d2, rm >> 7, rm & 127};
      qs += Qv;
      const int w = cc & 7;
      const int pos = (cc & ~7) + (BITS == 8 ? w : ((w & 1) ? 4 + (w >> 1) : (w >> 1)));
#pragma unroll
      for (int d = 0; d < kQDigits; ++d) {
        ds[d] += dg[d];
        dw[d][pos >> 2] |= (uint32_t)(dg[d] & 0xff) << (8 * (pos & 3));
      }
    }
#pragma unroll
    for (int d = 0; d < kQDigits; ++d) {
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(&s_qd[d][qh][qg * 32]);
      dst[0] = u32x4_t{dw[d][0], dw[d][1], dw[d][2], dw[d][3]};
      dst[1] = u32x4_t{dw[d][4], dw[d][5], dw[d][6], dw[d][7]};
    }
    s_qe[qh][qg] = E;
    s_qs[qh][qg] = qs;
    if constexpr (BITS == 8) {
#pragma unroll
      for (int d = 0; d < kQDigits; ++d) s_qds[d][qh][qg] = ds[d];
    }
  }
  __syncthreads();  // rows and query digits in LDS

  // ---- this wave's tiles (wv, wv + 4, ...): code and scale/zero loads all in flight together
  const int kb = lane >> 4, nn = lane & 15, rg = lane >> 4;
  const int gc = nn / GT, hl = nn - gc * GT;
  const bool colok = nn < kGroups * GT;
  uint32_t cw[NB][BITS];
  uint32_t mw[NB][4];
  int rw[NB][4];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int ti = wv + 4 * i;
    const int ra = (&s_row[0][0])[16 * ti + nn];
    load_codes<BITS>(c.k4 + (size_t)max(ra, 0) * (16 * BITS), kb, cw[i]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      rw[i][e] = (&s_row[0][0])[16 * ti + 4 * rg + e];
      mw[i][e] = c.k4_meta[(size_t)max(rw[i][e], 0) * kGroups + (gc & 3)];
    }
  }

  // ---- B operands, the same in every wave: lane (kb, nn) holds column nn = (group gc, head ct GT + hl)
  long Bop[NTL][kQDigits][4];
  double cscale[NTL], bcol[NTL];  // 2^(E_g - 20) and b_g of the lane's column
#pragma unroll
  for (int ct = 0; ct < NTL; ++ct) {
    const int hh = ct * GT + hl;
#pragma unroll
    for (int d = 0; d < kQDigits; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        Bop[ct][d][j] = (colok && kb == gc) ? *reinterpret_cast<const long*>(&s_qd[d][hh][32 * kb + 8 * j]) : 0l;
    cscale[ct] = colok ? ldexp(1.0, s_qe[hh][gc] - kQFracBits) : 0.0;
    bcol[ct] = colok ? (double)s_qs[hh][gc] * cscale[ct] : 0.0;  // exact
  }
  // 8-bit codes enter the contraction as code - 128: each column starts at 128 x its digit sum
  int acc0[NTL][kQDigits];
#pragma unroll
  for (int ct = 0; ct < NTL; ++ct) {
    const int hh = ct * GT + hl;
#pragma unroll
    for (int d = 0; d < kQDigits; ++d) acc0[ct][d] = (BITS == 8 && colok) ? 128 * s_qds[d][hh][gc] : 0;
  }
  const double smd = (double)sm;
  float mx[NTL];
#pragma unroll
  for (int ct = 0; ct < NTL; ++ct) mx[ct] = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int ti = wv + 4 * i;
    i32x4_t acc[NTL][kQDigits];
#pragma unroll
    for (int ct = 0; ct < NTL; ++ct)
#pragma unroll
      for (int d = 0; d < kQDigits; ++d) acc[ct][d] = i32x4_t{acc0[ct][d], acc0[ct][d], acc0[ct][d], acc0[ct][d]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long a = code_operand<BITS>(cw[i], j);
#pragma unroll
      for (int ct = 0; ct < NTL; ++ct)
#pragma unroll
        for (int d = 0; d < kQDigits; ++d)
          acc[ct][d] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, Bop[ct][d][j], acc[ct][d], 0, 0, 0);
    }
    // lane (rg, nn) holds the group sums of candidates 16 ti + 4 rg + e for column nn
#pragma unroll
    for (int ct = 0; ct < NTL; ++ct) {
      float lg4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        double S;
        if constexpr (BITS == 8) {
          // up to 2^34 in magnitude: combined in float64 (exact below 2^53)
          S = (double)acc[ct][0][e] * 16384.0 + (double)acc[ct][1][e] * 128.0 + (double)acc[ct][2][e];
        } else {
          // |S| <= 2^14 * 128 * 15 * 32 + (2^14 - 1) * 15 * 32 < 2^31: exact in int32
          S = (double)(acc[ct][0][e] * 16384 + acc[ct][1][e] * 128 + acc[ct][2][e]);
        }
        const double av = S * cscale[ct];  // exact (a power of two)
        const double s = (double)half_bits_to_float(mw[i][e] & 0xffffu);
        const double z = (double)half_bits_to_float(mw[i][e] >> 16);
        const double t = fma(s, av, z * bcol[ct]);  // s a_g and z b_g are exact: one rounding
        const double t01 = t + __shfl_xor(t, GT);      // groups (0, 1) and (2, 3)
        const double r = t01 + __shfl_xor(t01, 2 * GT);  // (t0 + t1) + (t2 + t3)
        lg4[e] = (rw[i][e] >= 0) ? (float)(smd * r) : -__builtin_inff();
        mx[ct] = fmaxf(mx[ct], lg4[e]);
      }
      if (colok && gc == 0) {
        const int k = k0 + 16 * ti + 4 * rg;
        *reinterpret_cast<float4*>(logits + ((size_t)b * c.Hq + (size_t)h * G + ct * GT + hl) * ncap + k) =
            make_float4(lg4[0], lg4[1], lg4[2], lg4[3]);
      }
    }
  }
  if (pmax) {
    // the block's largest logit per head: over the wave's lanes of the head, then over the waves
#pragma unroll
    for (int ct = 0; ct < NTL; ++ct) {
      float v = (colok && gc == 0) ? mx[ct] : -__builtin_inff();
      v = fmaxf(v, __shfl_xor(v, 16));
      v = fmaxf(v, __shfl_xor(v, 32));
#pragma unroll
      for (int s = GT; s < 16; s <<= 1) v = fmaxf(v, __shfl_xor(v, s));
      if (lane < GT) s_max[wv][ct * GT + lane] = v;
    }
    __syncthreads();
    if (threadIdx.x < G) {
      const float m = fmaxf(fmaxf(s_max[0][threadIdx.x], s_max[1][threadIdx.x]),
                            fmaxf(s_max[2][threadIdx.x], s_max[3][threadIdx.x]));
      pmax[((size_t)b * c.Hq + (size_t)h * G + threadIdx.x) * chunks_per_unit + ck] = m;
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
#define TWL_EST_G(GG, NB, BB)                                                                                 \
  case GG:                                                                                                    \
    hipLaunchKernelGGL((k_estimate<GG, NB, BB>), grid, dim3(256), 0, s, c, q, sm, cand, ncap, cpu, logits,    \
                       cand_tok, cand_row, pmax, wst, wwords);                                               \
    break;
#define TWL_EST_NB(NB, BB)                  \
  case NB:                                  \
    switch (c.G) {                          \
      TWL_EST_G(1, NB, BB)                  \
      TWL_EST_G(2, NB, BB)                  \
      TWL_EST_G(4, NB, BB)                  \
      TWL_EST_G(8, NB, BB)                  \
      default: return hipErrorInvalidValue; \
    }                                       \
    break;
#define TWL_EST_B(BB)                       \
  case BB:                                  \
    switch (nb) {                           \
      TWL_EST_NB(2, BB)                     \
      TWL_EST_NB(4, BB)                     \
      default: return hipErrorInvalidValue; \
    }                                       \
    break;
  switch (c.kbits) {
    TWL_EST_B(2)
    TWL_EST_B(4)
    TWL_EST_B(8)
    default: return hipErrorInvalidValue;
  }
#undef TWL_EST_G
#undef TWL_EST_NB
#undef TWL_EST_B
  return hipGetLastError();
}

}  // namespace twl
