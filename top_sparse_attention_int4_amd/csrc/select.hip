// Base page selector: Quest-style page bound scores and exact top-K page selection.
//
// The Twilight pages run a base sparse-attention selector with a conservative budget before the
// top-p pruner (Paper-Notes "整体框架"; paperlayer §4.1, Fig. 5) and name Quest among those
// selectors.  The page score of query head h is sum_c max(q_c*kmin_c, q_c*kmax_c); it is evaluated
// as a float32 left-to-right fold over the 128 channels, one lane per page, so the result equals the
// documented operation sequence on every run.  Because q_c*bound is exact in float32 (bf16 x bf16),
// max(q*kmin, q*kmax) = q+ * kmax + q- * kmin with q+ = max(q,0), q- = min(q,0): the second product
// is then an exact zero and adding it changes nothing, so two fused multiply-adds per channel and
// head reproduce the fold bit for bit without a compare.  Two layouts compute the same folds: for
// small steps each wave of a 4-wave block folds one query head for 64 pages (latency bound: every
// head in parallel); for large ones a block is one wave and 64 pages, one lane per page folding all G
// query heads, so each bound is converted once (the bounds staged in LDS in two halves of 64
// channels with coalesced loads, 17 KB of LDS so that several blocks share a compute unit and cover
// each other's loads; q+ and q- broadcast from LDS).  The group score then folds the heads in order.
#include "twl_device.h"
#include "twl_internal.h"

namespace twl {

// Small steps (few blocks, latency bound): each wave of a block folds one query head for the block's
// 64 pages, read from an LDS copy of the bounds that the whole block loads at once.
template <int G>
__global__ __launch_bounds__(64 * (G > 4 ? G : 4)) void k_page_score_heads(CacheView c, const uint16_t* __restrict__ q,
                                                                     float* __restrict__ scores,
                                                                     int blocks_per_unit) {
  constexpr int NT = 64 * (G > 4 ? G : 4);
  const int u = blockIdx.x / blocks_per_unit;
  const int blk = blockIdx.x - u * blocks_per_unit;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  if (blk * 64 >= c.maxP) return;
  const int hh = threadIdx.x >> 6, lane = threadIdx.x & 63;

  // the block's 64 pages of bounds, staged with coalesced loads (row = 32 x 16 B, padded by 16 B)
  __shared__ uint4 tile[64][33];
  __shared__ float qpos[G][kD];
  __shared__ float qneg[G][kD];
  __shared__ float sig[G][64];
  const int32_t* pt = c.page_table + (size_t)b * c.maxP;
  constexpr int R = 64 * 32 / NT;
  int phys[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {  // page-table reads in flight with the sequence length
    const int j = blk * 64 + ((int)threadIdx.x >> 5) + r * (NT / 32);
    phys[r] = pt[min(j, c.maxP - 1)];
  }
  const int n = clampi(c.seq_lens[b], 0, c.maxTok);
  const int P = (n + kPage - 1) / kPage;
  if (blk * 64 >= P) return;
  {
    // then all bound reads, so every load of the tile is in flight at once
    const int part = threadIdx.x & 31;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int j = blk * 64 + ((int)threadIdx.x >> 5) + r * (NT / 32);
      if (j >= P) phys[r] = -1;
    }
    uint4 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint4* src = reinterpret_cast<const uint4*>(c.kbound + ((size_t)max(phys[r], 0) * c.Hkv + h) * 2 * kD);
      v[r] = (phys[r] >= 0) ? src[part] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) tile[((int)threadIdx.x >> 5) + r * (NT / 32)][part] = v[r];
  }
  const uint16_t* qg = q + ((size_t)b * c.Hq + (size_t)h * G) * kD;
  for (int i = threadIdx.x; i < G * kD; i += NT) {
    const float x = __uint_as_float((uint32_t)qg[i] << 16);
    qpos[i / kD][i % kD] = x > 0.f ? x : 0.f;
    qneg[i / kD][i % kD] = x < 0.f ? x : 0.f;
  }
  __syncthreads();

  const int j = blk * 64 + lane;
  if (hh < G && j < P) {
    float acc = 0.f;
#pragma unroll
    for (int c8 = 0; c8 < 16; ++c8) {
      const uint4 mnv = tile[lane][c8], mxv = tile[lane][16 + c8];
      const uint32_t wm[4] = {mnv.x, mnv.y, mnv.z, mnv.w};
      const uint32_t wx[4] = {mxv.x, mxv.y, mxv.z, mxv.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ch = c8 * 8 + e;
        const float mn = (e & 1) ? bf16_hi(wm[e >> 1]) : bf16_lo(wm[e >> 1]);
        const float mx = (e & 1) ? bf16_hi(wx[e >> 1]) : bf16_lo(wx[e >> 1]);
        acc = fmaf(qpos[hh][ch], mx, acc);
        acc = fmaf(qneg[hh][ch], mn, acc);
      }
    }
    sig[hh][lane] = acc;
  }
  __syncthreads();
  if (hh == 0 && j < P) {
    float gs = 0.f;
#pragma unroll
    for (int k = 0; k < G; ++k) gs = gs + sig[k][lane];
    scores[(size_t)u * c.maxP + j] = gs;
  }
}

// Fold 64 channels (ch0 .. ch0 + 63) of one page into the G heads' scores: row = the page's staged
// half (8 x 16 B of kmin, then 8 x 16 B of kmax), q+ / q- broadcast from LDS.
template <int G>
__device__ __forceinline__ void page_fold(const uint4* row, const float4 (*qp)[kD / 4], const float4 (*qn)[kD / 4],
                                          int ch0, float (&acc)[G]) {
#pragma unroll 1
  for (int c8 = 0; c8 < 8; ++c8) {
    const uint4 mnv = row[c8], mxv = row[8 + c8];
    const uint32_t wm[4] = {mnv.x, mnv.y, mnv.z, mnv.w};
    const uint32_t wx[4] = {mxv.x, mxv.y, mxv.z, mxv.w};
    float mn[8], mx[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mn[2 * e] = bf16_lo(wm[e]);
      mn[2 * e + 1] = bf16_hi(wm[e]);
      mx[2 * e] = bf16_lo(wx[e]);
      mx[2 * e + 1] = bf16_hi(wx[e]);
    }
    const int ch4 = (ch0 + 8 * c8) / 4;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float4 p0 = qp[i][ch4], p1 = qp[i][ch4 + 1], n0 = qn[i][ch4], n1 = qn[i][ch4 + 1];
      const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
      const float nv[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
      float a = acc[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a = fmaf(pv[e], mx[e], a);
        a = fmaf(nv[e], mn[e], a);
      }
      acc[i] = a;
    }
  }
}

template <int G>
__global__ __launch_bounds__(64) void k_page_score_pages(CacheView c, const uint16_t* __restrict__ q,
                                                         float* __restrict__ scores, int blocks_per_unit) {
  constexpr int RS = 17;  // LDS row of a page: 16 x 16 B of one half (mn 64 ch, mx 64 ch) + 16 B pad
  const int u = blockIdx.x / blocks_per_unit;
  const int blk = blockIdx.x - u * blocks_per_unit;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int lane = threadIdx.x;
  __shared__ uint4 tile[64 * RS];
  __shared__ float4 qp[G][kD / 4], qn[G][kD / 4];
  // the page-table entry of this lane's page, in flight with the sequence length and q
  const int j = blk * 64 + lane;
  int phys = c.page_table[(size_t)b * c.maxP + min(j, c.maxP - 1)];
  const uint16_t* qg = q + ((size_t)b * c.Hq + (size_t)h * G) * kD;
  uint32_t qw[G * kD / 128];  // two bf16 channels per word, G * 64 words over 64 lanes
#pragma unroll
  for (int i = 0; i < G; ++i) qw[i] = reinterpret_cast<const uint32_t*>(qg)[i * 64 + lane];
  const int n = clampi(c.seq_lens[b], 0, c.maxTok);
  const int P = (n + kPage - 1) / kPage;
  if (blk * 64 >= P) return;  // uniform
  if (j >= P) phys = -1;
  // q+ and q- of every (head, channel) into LDS: lane l holds channels 2l, 2l + 1 of head i
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const float x0 = bf16_lo(qw[i]), x1 = bf16_hi(qw[i]);
    float* pp = reinterpret_cast<float*>(&qp[i][0]);
    float* pn = reinterpret_cast<float*>(&qn[i][0]);
    pp[2 * lane] = x0 > 0.f ? x0 : 0.f;
    pp[2 * lane + 1] = x1 > 0.f ? x1 : 0.f;
    pn[2 * lane] = x0 < 0.f ? x0 : 0.f;
    pn[2 * lane + 1] = x1 < 0.f ? x1 : 0.f;
  }
  // half hf of page p: mn channels 64 hf .. + 63 (128 B) and mx channels 64 hf .. + 63 (128 B);
  // load r covers pages 4r .. 4r + 3, lane l taking 16 B (segment l & 15) of page 4r + (l >> 4)
  const int seg = lane & 15;
  const uint4* rowp[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int pg = __shfl(phys, 4 * r + (lane >> 4));
    rowp[r] = reinterpret_cast<const uint4*>(c.kbound + ((size_t)max(pg, 0) * c.Hkv + h) * 2 * kD) +
              (seg < 8 ? 0 : 16) + (seg & 7);
  }
  // both halves in flight at once (32 x 16 B per lane); the tile then stages one half at a time
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 va[16], vb[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) va[r] = reinterpret_cast<const u32x4*>(rowp[r])[0];
#pragma unroll
  for (int r = 0; r < 16; ++r) vb[r] = reinterpret_cast<const u32x4*>(rowp[r])[8];
  float acc[G];
#pragma unroll
  for (int i = 0; i < G; ++i) acc[i] = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) reinterpret_cast<u32x4*>(tile)[(4 * r + (lane >> 4)) * RS + seg] = va[r];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  page_fold<G>(tile + lane * RS, qp, qn, 0, acc);
  // the first half's reads are done before the second overwrites the tile
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int r = 0; r < 16; ++r) reinterpret_cast<u32x4*>(tile)[(4 * r + (lane >> 4)) * RS + seg] = vb[r];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  page_fold<G>(tile + lane * RS, qp, qn, 64, acc);
  if (j < P) {
    float gs = 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) gs = gs + acc[i];
    scores[(size_t)u * c.maxP + j] = gs;
  }
}

// Ascending key <=> descending score (float order mapped onto uint32).
__device__ __forceinline__ uint32_t desc_key(float f) {
  const uint32_t x = __float_as_uint(f);
  const uint32_t o = (x & 0x80000000u) ? ~x : (x | 0x80000000u);
  return ~o;
}

constexpr int kSelRegKeys = 8192;  // pages per unit held in registers (8 per thread)

// Exact top-K of one unit's page scores: radix select of the K-th smallest key with integer
// histograms of 8-bit digits, starting below the leading bits that all keys share (a block AND/OR
// reduction finds them, so no pass histograms a digit every key has in common); ties at the
// threshold key are resolved towards lower page ids, and an order-preserving compaction writes the
// kept page ids in ascending order.
//
// Up to 8192 pages the keys stay in registers (page r * 1024 + tid in slot r of thread tid); the
// search stops early once every key of the chosen bin is kept, and the compaction is one pass of
// wave ballots: with `lt` / `eq` the pages whose key is below / equal to the threshold T and take_eq
// the number of tied pages kept, a page is kept iff lt, or eq with fewer than take_eq tied pages
// before it, at position (lt pages before it) + min(eq pages before it, take_eq).  Longer units
// read their scores from global memory in every pass.
__global__ __launch_bounds__(1024) void k_page_select(CacheView c, const float* __restrict__ scores,
                                                      float keep_frac, int max_keep, int32_t* page_phys,
                                                      int32_t* page_ids, int32_t* count) {
  constexpr int NT = 1024, NW = NT / 64;
  const int u = blockIdx.x;
  const int b = u / c.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int32_t* pt = c.page_table + (size_t)b * c.maxP;
  int32_t* phys_out = page_phys ? page_phys + (size_t)u * max_keep : nullptr;
  const float* sc = scores + (size_t)u * c.maxP;
  constexpr int R = kSelRegKeys / NT;
  float v[R];
  int ptv[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {  // score and page-table reads in flight with the sequence length
    const int i = tid + r * NT;
    v[r] = (i < c.maxP) ? sc[i] : 0.f;
    ptv[r] = (phys_out && i < c.maxP) ? pt[i] : 0;
  }
  const int n = clampi(c.seq_lens[b], 0, c.maxTok);
  const int P = (n + kPage - 1) / kPage;
  int K = 0;
  if (P > 0) {
    const float kf = ceilf(fminf(keep_frac * (float)P, (float)P));
    K = clampi((int)kf, 1, P);
  }
  if (tid == 0) count[u] = K;
  if (K == 0) return;
  int32_t* out = page_ids + (size_t)u * max_keep;
  if (K == P) {
    for (int i = tid; i < P; i += NT) {
      out[i] = i;
      if (phys_out) phys_out[i] = pt[i];
    }
    return;
  }

  __shared__ int hist[2][256];
  __shared__ uint32_t s_prefix, s_mask, s_and[NW], s_or[NW];
  __shared__ int s_rem, s_cnt;
  __shared__ int scan_sm[NW + 1];
  __shared__ int s_clt[R * NW], s_ceq[R * NW];
  const bool in_regs = P <= kSelRegKeys;
  uint32_t kk[R];
  uint32_t kand = 0xffffffffu, kor = 0u;
  if (in_regs) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      kk[r] = desc_key(v[r]);
      if (tid + r * NT < P) {
        kand &= kk[r];
        kor |= kk[r];
      }
    }
  } else {
    for (int i = tid; i < P; i += NT) {
      const uint32_t k = desc_key(sc[i]);
      kand &= k;
      kor |= k;
    }
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    kand &= (uint32_t)__shfl_xor((int)kand, d);
    kor |= (uint32_t)__shfl_xor((int)kor, d);
  }
  if (lane == 0) {
    s_and[wv] = kand;
    s_or[wv] = kor;
  }
  for (int i = tid; i < 512; i += NT) (&hist[0][0])[i] = 0;
  if (tid == 0) {
    s_rem = K;
    s_cnt = P;
  }
  __syncthreads();
  kand = s_and[0];
  kor = s_or[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    kand &= s_and[i];
    kor |= s_or[i];
  }
  auto key = [&](int i) -> uint32_t { return desc_key(sc[i]); };

  // bits at and above hb are common to every key
  int hb = 32 - __clz((int)(kand ^ kor));
  uint32_t mask = (hb >= 32) ? 0u : ~((1u << hb) - 1u);
  uint32_t prefix = kand & mask;
  bool early = false;
  for (int pass = 0; hb > 0; ++pass) {
    const int shift = hb > 8 ? hb - 8 : 0;
    const uint32_t dmask = (1u << (hb - shift)) - 1u;
    int* hs = hist[pass & 1];
    if (in_regs) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (r * NT >= P) break;  // uniform: the slots past the unit's pages
        if (tid + r * NT < P && (kk[r] & mask) == prefix) atomicAdd(&hs[(kk[r] >> shift) & dmask], 1);
      }
    } else {
      for (int i = tid; i < P; i += NT) {
        const uint32_t k = key(i);
        if ((k & mask) == prefix) atomicAdd(&hs[(k >> shift) & dmask], 1);
      }
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 4l..4l+3; find the bin where the cumulative count first reaches rem
      const int h0 = hs[4 * lane], h1 = hs[4 * lane + 1], h2 = hs[4 * lane + 2], h3 = hs[4 * lane + 3];
      const int sum4 = h0 + h1 + h2 + h3;
      const int incl = wave_incl_scan(sum4);
      const int excl = incl - sum4;
      const int rem = s_rem;
      if (excl < rem && rem <= incl) {
        int acc = excl;
        const int hv[4] = {h0, h1, h2, h3};
        for (int t = 0; t < 4; ++t) {
          if (acc + hv[t] >= rem) {
            s_prefix = prefix | ((uint32_t)(4 * lane + t) << shift);
            s_mask = mask | (dmask << shift);
            s_rem = rem - acc;
            s_cnt = hv[t];
            break;
          }
          acc += hv[t];
        }
      }
    } else {
      int* other = hist[(pass + 1) & 1];
      for (int i = tid - 64; i < 256; i += NT - 64) other[i] = 0;
    }
    __syncthreads();
    prefix = s_prefix;
    mask = s_mask;
    hb = shift;
    if (in_regs && s_cnt == s_rem && hb > 0) {  // every key of the bin is kept: T = the bin's top
      prefix |= ~mask;
      early = true;
      break;
    }
  }
  const uint32_t T = prefix;
  if (in_regs) {
    const int take_eq = early ? P : s_rem;  // tied pages to keep, lowest ids first
    unsigned long long blt[R], beq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool ok = tid + r * NT < P;
      blt[r] = (r * NT < P) ? __ballot(ok && kk[r] < T) : 0ull;
      beq[r] = (r * NT < P) ? __ballot(ok && kk[r] == T) : 0ull;
      if (lane == 0) {
        s_clt[r * NW + wv] = __popcll(blt[r]);
        s_ceq[r * NW + wv] = __popcll(beq[r]);
      }
    }
    __syncthreads();
    if (wv == 0) {  // exclusive prefixes over (slot, wave) in page order, two entries per lane
      const int a0 = s_clt[2 * lane], a1 = s_clt[2 * lane + 1];
      const int e0 = s_ceq[2 * lane], e1 = s_ceq[2 * lane + 1];
      const int ia = wave_incl_scan(a0 + a1), ie = wave_incl_scan(e0 + e1);
      s_clt[2 * lane] = ia - a0 - a1;
      s_clt[2 * lane + 1] = ia - a1;
      s_ceq[2 * lane] = ie - e0 - e1;
      s_ceq[2 * lane + 1] = ie - e1;
    }
    __syncthreads();
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r * NT >= P) break;
      const int lt_before = s_clt[r * NW + wv] + __popcll(blt[r] & below);
      const int eq_before = s_ceq[r * NW + wv] + __popcll(beq[r] & below);
      const bool lt = (blt[r] >> lane) & 1ull, eq = (beq[r] >> lane) & 1ull;
      if (lt || (eq && eq_before < take_eq)) {
        const int pos = lt_before + min(eq_before, take_eq);
        out[pos] = tid + r * NT;
        if (phys_out) phys_out[pos] = ptv[r];
      }
    }
    return;
  }
  const int take_eq = s_rem;  // pages with key == T to keep, lowest ids first
  const int cnt_eq = s_cnt;   // pages with key == T

  // contiguous ranges per thread keep page order = thread order then element order
  const int E = (P + NT - 1) / NT;
  const int i0 = min(P, tid * E), i1 = min(P, i0 + E);
  int total;
  if (cnt_eq == take_eq) {
    int keep_local = 0;
    for (int i = i0; i < i1; ++i) keep_local += (key(i) <= T);
    int pos = block_excl_scan<NW>(keep_local, scan_sm, &total);
    for (int i = i0; i < i1; ++i) {
      if (key(i) <= T) {
        if (phys_out) phys_out[pos] = pt[i];
        out[pos++] = i;
      }
    }
    return;
  }
  int eq_local = 0;
  for (int i = i0; i < i1; ++i) eq_local += (key(i) == T);
  const int eq_rank = block_excl_scan<NW>(eq_local, scan_sm, &total);
  int keep_local = 0;
  {
    int r = eq_rank;
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = key(i);
      keep_local += (k < T || (k == T && r < take_eq));
      r += (k == T);
    }
  }
  int pos = block_excl_scan<NW>(keep_local, scan_sm, &total);
  {
    int r = eq_rank;
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = key(i);
      if (k < T || (k == T && r < take_eq)) {
        if (phys_out) phys_out[pos] = pt[i];
        out[pos++] = i;
      }
      r += (k == T);
    }
  }
}

hipError_t launch_page_score(const CacheView& c, const uint16_t* q, float* scores, hipStream_t s) {
  const int bpu = (c.maxP + 63) / 64;
  dim3 grid((unsigned)(c.B * c.Hkv * bpu));
  // up to two blocks per compute unit the step is latency bound: one wave per head; beyond, one lane
  // per page folds every head so that each bound is converted once
  const bool pages = grid.x > 512u;
#define TWL_PS_G(GG)                                                                                        \
  case GG:                                                                                                  \
    if (pages) hipLaunchKernelGGL(k_page_score_pages<GG>, grid, dim3(64), 0, s, c, q, scores, bpu);         \
    else hipLaunchKernelGGL(k_page_score_heads<GG>, grid, dim3(64 * (GG > 4 ? GG : 4)), 0, s, c, q, scores, bpu); \
    break;
  switch (c.G) {
    TWL_PS_G(1)
    TWL_PS_G(2)
    TWL_PS_G(4)
    TWL_PS_G(8)
    default: return hipErrorInvalidValue;
  }
#undef TWL_PS_G
  return hipGetLastError();
}

hipError_t launch_page_select(const CacheView& c, const float* scores, float keep_frac, int max_keep, int32_t* page_phys,
                              int32_t* page_ids, int32_t* count, hipStream_t s) {
  hipLaunchKernelGGL(k_page_select, dim3((unsigned)(c.B * c.Hkv)), dim3(1024), 0, s, c, scores, keep_frac,
                     max_keep, page_phys, page_ids, count);
  return hipGetLastError();
}

}  // namespace twl
