// INT4 weight estimate: the mixed-precision SpGEMV of the query against the dequantised 4-bit keys
// (paperlayer §4.2; §B.1, Fig. 12) as an int8 matrix-core contraction.
//
// Per head and 32-channel group g the query is held in fixed point, Q_c = rne(q_c 2^(20 - E_g)) with
// E_g = floor(log2 max |q_c|) (|Q_c| <= 2088960; exact for channels within 2^12 of the largest, i.e.
// for every channel of an ordinary bf16 query), as three int8 digits Q = 2^14 d0 + 2^7 d1 + d2
// (prepared once per step, see QDigits), so
//   sum_{c in g} q~_c (code_c s_g + z_g) = s_g a_g + z_g b_g,  a_g = 2^(E_g-20) sum Q_c code_c,
//   b_g = 2^(E_g-20) sum Q_c
// has exact integer group sums in any order; then, in float64,
//   t_g = s_g a_g + z_g b_g (both products exact, one rounding),  r = (t_0 + t_1) + (t_2 + t_3),
//   logit = float32(sm * r)
// -- the float64 definition of the estimate for the grid query q~, rounded once to float32.
//
// The sums are v_mfma_i32_16x16x32_i8 products: A = the query digits, one row per (head, group) and
// zero outside the row's group; B = 32 codes x 16 candidates (lane (kb, nn) reads the code run of
// group kb of candidate nn with one load -- 16 bytes of 4-bit codes; 8 or 32 bytes for the 2- and
// 8-bit widths of the precision ablation, paperlayer §4.2, Fig. 6 -- and feeds 8 codes as bytes to
// each of four MFMAs; 8-bit codes go in as code - 128 with the rows started at 128 x the digit sums).
// A wave takes 16-candidate tiles; each result lane holds the four group sums of one (candidate,
// head), so the groups meet in-lane in the committed order.
//
// Candidates given as pages (the base selector's output) or as every page of the sequence (the plain
// decode, and the cluster stage's kept tokens as slot masks): a 16-candidate tile is one page, and
// the codes are stored by (sequence, logical page), so each wave addresses its tiles' codes from the
// page ids alone and works on its own (no exchange, no barrier, no page-table lookup); the attention
// later derives the K/V rows from the same pages.  Candidates given as token ranges (a caller's
// list): the block resolves its candidates' rows together (prefix sums of the range lengths, binary
// search).
#include "twl_device.h"
#include "twl_internal.h"

namespace twl {

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

typedef int i32x4_t __attribute__((ext_vector_type(4)));
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

// One wave's share of the contraction, as products (query digits) x (codes): the A operand row
// i = 4 hh + g holds head hh's digits of group g (zero outside the k-slice of group g), the B operand
// column is a candidate (lane (kb, nn) feeds the code run of group kb of candidate nn), so the
// result lane (rg, nn) holds the four group sums of head rg (of the row tile) for candidate nn and
// forms that candidate's logit itself: the groups meet in-lane in the committed order, and the lane
// reads its candidate's four (scale, zero) words with one load.
template <int G, int BITS>
struct EstWave {
  static constexpr int GT = G < 4 ? G : 4;  // heads per 16-row MFMA tile (GT heads x 4 groups)
  static constexpr int NTL = G / GT;        // row tiles
  int lane, kb, nn, rg;
  bool rowok;                     // head rg of a row tile exists (rg < GT)
  long Aop[NTL][kQDigits][4];     // digits of row nn = (head nn / 4, group nn % 4), zero unless kb is the group
  double cscale[NTL][kGroups], bcol[NTL][kGroups];  // 2^(E_g - 20) and b_g of head rg, group g
  int acc0[NTL][kQDigits][kGroups];  // 8-bit codes: 128 x the digit sums (codes enter as code - 128)
  double smd;

  // the A operands and row constants of query rows bh0 .. bh0 + G - 1 (the unit's heads)
  __device__ __forceinline__ void init(const QDigits& qd, size_t bh0, float sm) {
    lane = threadIdx.x & 63;
    kb = lane >> 4;
    nn = lane & 15;
    rg = lane >> 4;
    rowok = rg < GT;
    smd = (double)sm;
    const int ah = nn >> 2, ag = nn & 3;  // this lane's A row
#pragma unroll
    for (int ct = 0; ct < NTL; ++ct) {
      const bool mine = ah < GT && kb == ag;
      const size_t gi = (bh0 + ct * GT + min(ah, GT - 1)) * kGroups + ag;
      const u32x4_t* dg = reinterpret_cast<const u32x4_t*>(qd.dig + gi * kQDigits * 32);
#pragma unroll
      for (int d = 0; d < kQDigits; ++d) {
        const u32x4_t x0 = mine ? dg[2 * d] : u32x4_t{0u, 0u, 0u, 0u};
        const u32x4_t x1 = mine ? dg[2 * d + 1] : u32x4_t{0u, 0u, 0u, 0u};
        Aop[ct][d][0] = (long)((uint64_t)x0.x | ((uint64_t)x0.y << 32));
        Aop[ct][d][1] = (long)((uint64_t)x0.z | ((uint64_t)x0.w << 32));
        Aop[ct][d][2] = (long)((uint64_t)x1.x | ((uint64_t)x1.y << 32));
        Aop[ct][d][3] = (long)((uint64_t)x1.z | ((uint64_t)x1.w << 32));
      }
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        const int32_t* mt = qd.meta + ((bh0 + ct * GT + min(rg, GT - 1)) * kGroups + g) * kQMeta;
        const int E = rowok ? mt[0] : 0;
        cscale[ct][g] = rowok ? ldexp(1.0, E - kQFracBits) : 0.0;
        bcol[ct][g] = rowok ? (double)mt[1] * cscale[ct][g] : 0.0;  // exact
#pragma unroll
        for (int d = 0; d < kQDigits; ++d) acc0[ct][d][g] = (BITS == 8 && rowok) ? 128 * mt[2 + d] : 0;
      }
    }
  }

  // One tile: cw = this lane's code run (candidate nn, group kb), mw = scale | zero << 16 of candidate
  // nn in groups 0..3, ok = whether candidate nn exists.  The logit of candidate nn for head rg of row
  // tile ct lands in lg[ct] (-inf for a candidate that does not exist).
  __device__ __forceinline__ void tile(const uint32_t (&cw)[BITS], const u32x4_t& mw, bool ok,
                                       float (&lg)[NTL]) const {
    i32x4_t acc[NTL][kQDigits];
#pragma unroll
    for (int ct = 0; ct < NTL; ++ct)
#pragma unroll
      for (int d = 0; d < kQDigits; ++d)
        acc[ct][d] = i32x4_t{acc0[ct][d][0], acc0[ct][d][1], acc0[ct][d][2], acc0[ct][d][3]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long bcode = code_operand<BITS>(cw, j);
#pragma unroll
      for (int ct = 0; ct < NTL; ++ct)
#pragma unroll
        for (int d = 0; d < kQDigits; ++d)
          acc[ct][d] = __builtin_amdgcn_mfma_i32_16x16x32_i8(Aop[ct][d][j], bcode, acc[ct][d], 0, 0, 0);
    }
    const uint32_t mwv[kGroups] = {mw.x, mw.y, mw.z, mw.w};
#pragma unroll
    for (int ct = 0; ct < NTL; ++ct) {
      double t[kGroups];
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        double S;
        if constexpr (BITS == 8) {
          // up to 2^34 in magnitude: combined in float64 (exact below 2^53)
          S = (double)acc[ct][0][g] * 16384.0 + (double)acc[ct][1][g] * 128.0 + (double)acc[ct][2][g];
        } else {
          // |S| <= 2^14 * 128 * 15 * 32 + (2^14 - 1) * 15 * 32 < 2^31: exact in int32
          S = (double)(acc[ct][0][g] * 16384 + acc[ct][1][g] * 128 + acc[ct][2][g]);
        }
        const double s = (double)half_bits_to_float(mwv[g] & 0xffffu);
        const double z = (double)half_bits_to_float(mwv[g] >> 16);
        t[g] = fma(s, S * cscale[ct][g], z * bcol[ct][g]);  // s a_g and z b_g are exact: one rounding
      }
      const double r = (t[0] + t[1]) + (t[2] + t[3]);
      lg[ct] = (ok && rowok) ? (float)(smd * r) : -__builtin_inff();
    }
  }
};

// The block's largest logit per head over its waves' maxima (lanes 16 rg .. 16 rg + 15 hold head rg).
template <int G, int BITS>
__device__ __forceinline__ void block_head_max(const EstWave<G, BITS>& ew, const float (&mx)[EstWave<G, BITS>::NTL],
                                               float (*s_max)[G], int wv, float* pmax_row, int stride) {
  constexpr int GT = EstWave<G, BITS>::GT, NTL = EstWave<G, BITS>::NTL;
#pragma unroll
  for (int ct = 0; ct < NTL; ++ct) {
    float v = ew.rowok ? mx[ct] : -__builtin_inff();
#pragma unroll
    for (int s = 1; s < 16; s <<= 1) v = fmaxf(v, __shfl_xor(v, s));
    if (ew.rowok && ew.nn == 0) s_max[wv][ct * GT + ew.rg] = v;
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const float m = fmaxf(fmaxf(s_max[0][threadIdx.x], s_max[1][threadIdx.x]),
                          fmaxf(s_max[2][threadIdx.x], s_max[3][threadIdx.x]));
    pmax_row[(size_t)threadIdx.x * stride] = m;
  }
}

// Candidates as pages (MODE kCandPages, logical pages listed by the selector) or as every page of the
// sequence (kCandAll), either optionally with a mask of each page's candidate slots (the cluster
// stage's): NB 16-candidate tiles (pages) per wave, 4 waves per block, 64 NB candidates per block.
template <int G, int NB, int BITS, int MODE>
__global__ __launch_bounds__(256) void k_estimate_pages(CacheView c, QDigits qd, float sm, CandView cand, int ncap,
                                                        int chunks_per_unit, float* __restrict__ logits,
                                                        int32_t* __restrict__ cand_tok, float* __restrict__ pmax,
                                                        uint64_t* __restrict__ wstate, size_t wstate_words) {
  using EW = EstWave<G, BITS>;
  constexpr int GT = EW::GT, NTL = EW::NTL;
  int ck;
  const int u = head_fast_unit(blockIdx.x, c.Hkv, chunks_per_unit, ck);
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  if (wstate) {
    // clear the wide top-p state for the passes that follow this kernel
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < wstate_words; i += (size_t)gridDim.x * 256)
      wstate[i] = 0ull;
  }
  // the wave's tiles: pages tp0 .. tp0 + NB - 1 of the unit's candidate list (wave-uniform values)
  const int tp0 = ck * 4 * NB + wv * NB;
  const int n = clampi(c.seq_lens[b], 0, c.maxTok);
  int page[NB];
  uint32_t slots[NB];  // which of the page's 16 tokens are candidates
  if constexpr (MODE == kCandPages) {
    const int cnt = clampi(cand.count[u], 0, cand.max_items);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const size_t idx = (size_t)u * cand.max_items + min(tp0 + i, cand.max_items - 1);
      page[i] = cand.items[idx];
      if (tp0 + i >= cnt) page[i] = -1;
      slots[i] = cand.slot_mask ? cand.slot_mask[idx] : 0xFFFFu;
    }
  } else {
    // every page of the sequence: the codes' addresses need no load (stored by logical page), so
    // they are in flight together with the slot masks
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      page[i] = tp0 + i;
      slots[i] = cand.slot_mask ? cand.slot_mask[(size_t)u * c.maxP + min(tp0 + i, c.maxP - 1)] : 0xFFFFu;
    }
  }
  EW ew;
  ew.init(qd, (size_t)b * c.Hq + (size_t)h * G, sm);
  // a tile exists when its page does; its candidate nn exists when page * 16 + nn is a token of the
  // page's candidate slots
  bool tok_ok[NB];
  uint32_t cw[NB][BITS];
  u32x4_t mw[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const bool pg_ok = page[i] >= 0 && page[i] * kPage < n;
    const int row = (pg_ok ? ((b * c.maxP + page[i]) * c.Hkv + h) * kPage : 0) + ew.nn;
    load_codes<BITS>(c.k4 + (size_t)row * (16 * BITS), ew.kb, cw[i]);
    mw[i] = *reinterpret_cast<const u32x4_t*>(c.k4_meta + (size_t)row * kGroups);
    tok_ok[i] = pg_ok && page[i] * kPage + ew.nn < n && ((slots[i] >> ew.nn) & 1u);
  }
  if (cand_tok && ew.kb == 0) {
    // token ids of the candidates, for the union lists (lane nn of each tile)
#pragma unroll
    for (int i = 0; i < NB; ++i)
      cand_tok[(size_t)u * ncap + (size_t)(tp0 + i) * kPage + ew.nn] = tok_ok[i] ? page[i] * kPage + ew.nn : -1;
  }
  float mx[NTL];
#pragma unroll
  for (int ct = 0; ct < NTL; ++ct) mx[ct] = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    float lg[NTL];
    ew.tile(cw[i], mw[i], tok_ok[i], lg);
#pragma unroll
    for (int ct = 0; ct < NTL; ++ct) {
      mx[ct] = fmaxf(mx[ct], lg[ct]);
      if (ew.rowok)
        logits[((size_t)b * c.Hq + (size_t)h * G + ct * GT + ew.rg) * ncap + (size_t)(tp0 + i) * kPage + ew.nn] = lg[ct];
    }
  }
  if (pmax) {
    __shared__ float s_max[4][G];
    block_head_max<G, BITS>(ew, mx, s_max, wv, pmax + ((size_t)b * c.Hq + (size_t)h * G) * chunks_per_unit + ck,
                            chunks_per_unit);
  }
}

// Candidates as token ranges: NB batches of 64 candidates per block (64 NB candidates); the block
// resolves every candidate's token and K/V row once (batch w by wave w), then each wave takes tiles
// wv, wv + 4, ... of the block.
template <int G, int NB, int BITS>
__global__ __launch_bounds__(256) void k_estimate_ranges(CacheView c, QDigits qd, float sm, CandView cand, int ncap,
                                                         int chunks_per_unit, float* __restrict__ logits,
                                                         int32_t* __restrict__ cand_tok, float* __restrict__ pmax,
                                                         uint64_t* __restrict__ wstate, size_t wstate_words) {
  using EW = EstWave<G, BITS>;
  constexpr int NC = 64 * NB;
  constexpr int GT = EW::GT, NTL = EW::NTL;
  const int u = blockIdx.x / chunks_per_unit;
  const int ck = blockIdx.x - u * chunks_per_unit;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  __shared__ int s_row[NB][64];
  __shared__ int s_pre[NC + 1];
  __shared__ int s_beg[NC + 1];
  if (wstate) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < wstate_words; i += (size_t)gridDim.x * 256)
      wstate[i] = 0ull;
  }
  const int n = clampi(c.seq_lens[b], 0, c.maxTok);
  const int cnt = clampi(cand.count[u], 0, cand.max_items);
  const int k0 = ck * NC;
  EW ew;
  ew.init(qd, (size_t)b * c.Hq + (size_t)h * G, sm);
  // ---- candidate resolution: the block's candidates lie in the ranges r0..rmax; their prefix sums
  // and first tokens are staged in LDS when they fit, and every lane searches there
  {
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
      const int row = tok >= 0 ? ((b * c.maxP + (tok >> 4)) * c.Hkv + h) * kPage + (tok & 15) : -1;
      s_row[bt][lane] = row;
      if (cand_tok) cand_tok[(size_t)u * ncap + k] = row >= 0 ? tok : -1;
    }
  }
  __syncthreads();  // rows in LDS

  // ---- this wave's tiles (wv, wv + 4, ...): code and scale/zero loads all in flight together
  uint32_t cw[NB][BITS];
  u32x4_t mw[NB];
  bool ok[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int ti = wv + 4 * i;
    const int ra = (&s_row[0][0])[16 * ti + ew.nn];
    load_codes<BITS>(c.k4 + (size_t)max(ra, 0) * (16 * BITS), ew.kb, cw[i]);
    mw[i] = *reinterpret_cast<const u32x4_t*>(c.k4_meta + (size_t)max(ra, 0) * kGroups);
    ok[i] = ra >= 0;
  }
  float mx[NTL];
#pragma unroll
  for (int ct = 0; ct < NTL; ++ct) mx[ct] = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int ti = wv + 4 * i;
    float lg[NTL];
    ew.tile(cw[i], mw[i], ok[i], lg);
#pragma unroll
    for (int ct = 0; ct < NTL; ++ct) {
      mx[ct] = fmaxf(mx[ct], lg[ct]);
      if (ew.rowok)
        logits[((size_t)b * c.Hq + (size_t)h * G + ct * GT + ew.rg) * ncap + k0 + 16 * ti + ew.nn] = lg[ct];
    }
  }
  if (pmax) {
    __shared__ float s_max[4][G];
    block_head_max<G, BITS>(ew, mx, s_max, wv, pmax + ((size_t)b * c.Hq + (size_t)h * G) * chunks_per_unit + ck,
                            chunks_per_unit);
  }
}

// The query digits of every (sequence, query head) row: 8 (row, group) pairs per 256-thread block.
__global__ __launch_bounds__(256) void k_qdigits(CacheView c, const uint16_t* __restrict__ q, QDigits qd) {
  const int pr = blockIdx.x * 8 + ((int)threadIdx.x >> 5);
  if (pr < c.B * c.Hq * kGroups) query_digits_half(q, pr >> 2, pr & 3, c.kbits, qd.dig, qd.meta);
}

hipError_t launch_qdigits(const CacheView& c, const uint16_t* q, const QDigits& qd, hipStream_t s) {
  const int pairs = c.B * c.Hq * kGroups;
  hipLaunchKernelGGL(k_qdigits, dim3((unsigned)((pairs + 7) / 8)), dim3(256), 0, s, c, q, qd);
  return hipGetLastError();
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

hipError_t launch_estimate(const CacheView& c, const QDigits& qd, float sm, const CandView& cand, int ncap,
                           float* logits, int32_t* cand_tok, const WideWs* wide, hipStream_t s) {
  const int nb = est_batches(ncap, (int64_t)c.B * c.Hkv);
  if (ncap % (64 * nb) || ncap % kEstCands) return hipErrorInvalidValue;
  const int cpu = ncap / (64 * nb);
  dim3 grid((unsigned)(c.B * c.Hkv * cpu));
  float* pmax = wide ? wide->pmax : nullptr;
  uint64_t* wst = wide ? wide->state : nullptr;
  const size_t wwords = wide ? (size_t)c.B * c.Hq * kWideStateWords : 0;
#define TWL_EST_G(GG, NB, BB)                                                                                    \
  case GG:                                                                                                       \
    if (cand.mode == kCandRanges)                                                                                \
      hipLaunchKernelGGL((k_estimate_ranges<GG, NB, BB>), grid, dim3(256), 0, s, c, qd, sm, cand, ncap, cpu,     \
                         logits, cand_tok, pmax, wst, wwords);                                        \
    else if (cand.mode == kCandPages)                                                                            \
      hipLaunchKernelGGL((k_estimate_pages<GG, NB, BB, kCandPages>), grid, dim3(256), 0, s, c, qd, sm, cand,     \
                         ncap, cpu, logits, cand_tok, pmax, wst, wwords);                                        \
    else                                                                                                         \
      hipLaunchKernelGGL((k_estimate_pages<GG, NB, BB, kCandAll>), grid, dim3(256), 0, s, c, qd, sm, cand, ncap, \
                         cpu, logits, cand_tok, pmax, wst, wwords);                                              \
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
