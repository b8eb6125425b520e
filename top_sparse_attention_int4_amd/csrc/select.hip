// Base page selector: Quest-style page bound scores and exact top-K page selection.
//
// The Twilight pages run an existing sparse-attention selector with a generous budget before the
// top-p pruner (Paper-Notes "整体框架"; paperlayer §4.1, Fig. 5) and name Quest among those
// selectors.  The page score of query head h is sum_c max(q_c*kmin_c, q_c*kmax_c), and a GQA group
// ranks its pages by the sum over its heads.  Since kmin_c <= kmax_c, max(q*kmin, q*kmax) =
// q+ * kmax + q- * kmin with q+ = max(q,0), q- = min(q,0), so the group score is
// sum_c (P_c * kmax_c + N_c * kmin_c) with P_c, N_c the group's q+ and q- summed over its heads: two
// fused multiply-adds per channel for the whole group instead of two per channel and head.  P_c and
// N_c are float32 sums over the heads in order, then one float32 left-to-right fold over the 128
// channels adds P_c*kmax_c and then N_c*kmin_c with one rounding each (one lane per page), so the
// result equals the documented operation sequence on every run.  Two layouts compute the same folds:
// for small steps a 4-wave block stages 64 pages' bounds and P/N, and its first wave folds (latency
// bound: the bounds of the block arrive together); for large ones each wave takes 64 pages, one lane
// per page (the bounds are stored quarter-major, so a quarter of the channels of a page is one
// 128-byte line; two quarters of a wave's loads are in flight and each staged quarter requests the
// next, so the folds overlap the loads; a block is four such waves sharing P and N in LDS, 37 KB with
// the waves' quarter tiles, so that four blocks -- sixteen waves, at most 128 VGPRs each -- share a
// compute unit and a 32K-token, 16-sequence layer's grid is resident at once).
#include "twl_device.h"
#include "twl_internal.h"

namespace twl {

// Small steps (few blocks, latency bound): the block loads its 64 pages' bounds at once into LDS with
// the group's P and N, and its first wave folds them (one lane per page).
template <int G>
__global__ __launch_bounds__(64 * (G > 4 ? G : 4)) void k_page_score_heads(CacheView c, const uint16_t* __restrict__ q,
                                                                     float* __restrict__ scores,
                                                                     int blocks_per_unit) {
  constexpr int NT = 64 * (G > 4 ? G : 4);
  int blk;
  const int u = head_fast_unit(blockIdx.x, c.Hkv, blocks_per_unit, blk);
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  if (blk * 64 >= c.maxP) return;
  const int hh = threadIdx.x >> 6, lane = threadIdx.x & 63;

  // the block's 64 pages of bounds, staged with coalesced loads (row = 32 x 16 B, padded by 16 B)
  __shared__ uint4 tile[64][33];
  __shared__ float qpos[kD];  // P_c: the group's q+ summed over its heads
  __shared__ float qneg[kD];  // N_c: the group's q- summed over its heads
  constexpr int R = 64 * 32 / NT;
  const uint16_t* qg = q + ((size_t)b * c.Hq + (size_t)h * G) * kD;
  // thread ch < 128 holds channel ch of every head of the group
  uint16_t qr[G];
#pragma unroll
  for (int i = 0; i < G; ++i) qr[i] = qg[i * kD + ((int)threadIdx.x & (kD - 1))];
  int P;
  {
    // every bound read of the tile in flight at once, with the sequence length (the bounds are stored
    // by logical page; pages past the sequence are read from its allocated range and dropped)
    const int part = threadIdx.x & 31;
    uint4 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int j = blk * 64 + ((int)threadIdx.x >> 5) + r * (NT / 32);
      const uint4* src =
          reinterpret_cast<const uint4*>(c.kbound + (((size_t)b * c.maxP + min(j, c.maxP - 1)) * c.Hkv + h) * 2 * kD);
      v[r] = src[part];
    }
    const int n = clampi(c.seq_lens[b], 0, c.maxTok);
    P = (n + kPage - 1) / kPage;
    if (blk * 64 >= P) return;  // uniform
    // stored quarter-major (8 words per quarter: 4 of min, then 4 of max); the tile row is all 16
    // words of min, then all 16 of max
    const int col = (part & 4) * 4 + (part >> 3) * 4 + (part & 3);
#pragma unroll
    for (int r = 0; r < R; ++r) tile[((int)threadIdx.x >> 5) + r * (NT / 32)][col] = v[r];
  }
  if (threadIdx.x < kD) {
    float sp = 0.f, sn = 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float x = __uint_as_float((uint32_t)qr[i] << 16);
      sp = sp + (x > 0.f ? x : 0.f);
      sn = sn + (x < 0.f ? x : 0.f);
    }
    qpos[threadIdx.x] = sp;
    qneg[threadIdx.x] = sn;
  }
  __syncthreads();

  // one fold per page (the group's): the first wave's lanes take the block's 64 pages
  const int j = blk * 64 + lane;
  if (hh == 0 && j < P) {
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
        acc = fmaf(qpos[ch], mx, acc);
        acc = fmaf(qneg[ch], mn, acc);
      }
    }
    scores[(size_t)u * c.maxP + j] = acc;
  }
}

// Fold 8 NQ channels (ch0 .. ch0 + 8 NQ - 1) of one page into the group score: row = the page's staged
// part (NQ x 16 B of kmin, then NQ x 16 B of kmax), the group's P_c / N_c broadcast from LDS.
template <int NQ>
__device__ __forceinline__ void page_fold(const uint4* row, const float4* qp, const float4* qn, int ch0, float& acc) {
#pragma unroll 1
  for (int c8 = 0; c8 < NQ; ++c8) {
    const uint4 mnv = row[c8], mxv = row[NQ + c8];
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
    const float4 p0 = qp[ch4], p1 = qp[ch4 + 1], n0 = qn[ch4], n1 = qn[ch4 + 1];
    const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    const float nv[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
    float a = acc;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a = fmaf(pv[e], mx[e], a);
      a = fmaf(nv[e], mn[e], a);
    }
    acc = a;
  }
}

template <int G>
__global__ __launch_bounds__(256, 4) void k_page_score_pages(CacheView c, const uint16_t* __restrict__ q,
                                                         float* __restrict__ scores, int blocks_per_unit) {
  constexpr int NQ = 4;           // 16-byte words of one bound per staged quarter (32 channels)
  constexpr int RS = 2 * NQ + 1;  // LDS row of a page: NQ words of kmin, NQ of kmax, 16 B pad
  int blk;
  const int u = head_fast_unit(blockIdx.x, c.Hkv, blocks_per_unit, blk);
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int lane = threadIdx.x & 63, wq = threadIdx.x >> 6;

  __shared__ uint4 tiles[4][64 * RS];
  __shared__ float4 qp[kD / 4], qn[kD / 4];  // the group's P_c and N_c
  uint4* tile = tiles[wq];
  // this lane's page (the bounds are stored by logical page: no page-table lookup)
  const int j = blk * 256 + wq * 64 + lane;
  const uint16_t* qg = q + ((size_t)b * c.Hq + (size_t)h * G) * kD;
  // the bound reads do not wait for the sequence length: a lane past the sequence reads a page of
  // the sequence's allocated range (stored, perhaps stale) and its score is dropped
  const int lpg = min(j, c.maxP - 1);
  // P_c and N_c (the group's q+ and q- summed over its heads in order) into LDS, shared by the
  // block's four waves: thread ch < 128 sums channel ch
  if (threadIdx.x < kD) {
    float sp = 0.f, sn = 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float x = __uint_as_float((uint32_t)qg[i * kD + threadIdx.x] << 16);
      sp = sp + (x > 0.f ? x : 0.f);
      sn = sn + (x < 0.f ? x : 0.f);
    }
    reinterpret_cast<float*>(qp)[threadIdx.x] = sp;
    reinterpret_cast<float*>(qn)[threadIdx.x] = sn;
  }
  // quarter qq of page p is the 128-byte line 8 qq .. 8 qq + 7 of its slice (4 words of kmin, then 4 of
  // kmax); load r of a quarter covers pages 8 r .. 8 r + 7, lane l taking word l & 7 of page 8 r + (l >> 3)
  const int seg = lane & 7;
  const uint4* rowp[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int pg = __shfl(lpg, 8 * r + (lane >> 3));
    rowp[r] = reinterpret_cast<const uint4*>(c.kbound + (((size_t)b * c.maxP + pg) * c.Hkv + h) * 2 * kD) + seg;
  }
  // two quarters in flight (16 x 16 B per lane): quarter qq + 2 is requested once quarter qq is staged,
  // so its loads overlap the fold and each wave's folds are spread over its loads instead of all
  // running after the last one arrives; the tile stages one quarter at a time
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  constexpr int kAhead = 2;
  u32x4 v[4][8];
#pragma unroll
  for (int qq = 0; qq < kAhead; ++qq)
#pragma unroll
    for (int r = 0; r < 8; ++r) v[qq][r] = reinterpret_cast<const u32x4*>(rowp[r])[2 * NQ * qq];
  const int n = clampi(c.seq_lens[b], 0, c.maxTok);
  const int P = (n + kPage - 1) / kPage;
  __syncthreads();  // the query halves are staged
  if (blk * 256 + wq * 64 >= P) return;  // uniform per wave (no block barrier follows)
  float acc = 0.f;
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    if (qq > 0) {
      // the previous quarter's reads are done before this one overwrites the tile
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) reinterpret_cast<u32x4*>(tile)[(8 * r + (lane >> 3)) * RS + seg] = v[qq][r];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (qq + kAhead < 4) {
#pragma unroll
      for (int r = 0; r < 8; ++r) v[qq + kAhead][r] = reinterpret_cast<const u32x4*>(rowp[r])[2 * NQ * (qq + kAhead)];
    }
    page_fold<NQ>(tile + lane * RS, qp, qn, 32 * qq, acc);
  }
  if (j < P) scores[(size_t)u * c.maxP + j] = acc;
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
                                                      int32_t* page_ids, int32_t* count,
                                                      const uint16_t* __restrict__ q, QDigits qd) {
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
  // while the scores arrive: the unit's query digits for the estimate (one pair per half wave)
  if (qd.dig) unit_query_digits(q, c.Hq, c.kbits, b, u - b * c.Hkv, c.G, NT, 0, 1, qd);
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
  const int bpu4 = (c.maxP + 255) / 256;
  dim3 grid4((unsigned)(c.B * c.Hkv * bpu4));
  // up to two blocks per compute unit the step is latency bound: one wave per head; beyond, one lane
  // per page folds every head so that each bound is converted once
  const bool pages = grid.x > 512u;
#define TWL_PS_G(GG)                                                                                        \
  case GG:                                                                                                  \
    if (pages) hipLaunchKernelGGL(k_page_score_pages<GG>, grid4, dim3(256), 0, s, c, q, scores, bpu4);      \
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
                              int32_t* page_ids, int32_t* count, const uint16_t* q, const QDigits& qd, hipStream_t s) {
  hipLaunchKernelGGL(k_page_select, dim3((unsigned)(c.B * c.Hkv)), dim3(1024), 0, s, c, scores, keep_frac,
                     max_keep, page_phys, page_ids, count, q, qd);
  return hipGetLastError();
}

}  // namespace twl
