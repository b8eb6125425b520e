// Sparse attention over the kept tokens: gather split-K flash-decode plus a fixed-order LSE merge.
//
// The pages compute attention only on the top-p survivors, group-wise for GQA over a flattened
// paged cache, with FlashInfer's balancing across heads whose budgets differ widely (Paper-Notes
// "关键设计 / 负载均衡": per-head budgets from ~2% to ~50%; paperlayer §4.2 and §B.2).  Here the
// token lists of all (sequence, kv-head) units are cut into equal chunks of CH tokens, numbered
// across units (head-flattened), and every chunk is one workgroup of four waves; the hardware
// dispatcher hands chunks to compute units as they free up, so a unit with a long list simply owns
// more chunks and no compute unit waits on a slow one.
//
// Each wave takes a contiguous quarter of its chunk in 16-token sub-blocks, software-pipelined: the
// quarter's row indices are read up front, and the K/V data of sub-block i+1 is in flight while
// sub-block i is computed.  K/V are read with the non-temporal hint (each row is used once per step).
// Loads are unconditional (the row of a list entry past the chunk is clamped to a real row and masked
// afterwards) so the compiler can count outstanding loads exactly.  Per sub-block:
//   * S = K q^T with bf16 MFMA (v_mfma_f32_16x16x32_bf16): A = 16 tokens x 32 dims of K loaded
//     straight into registers, B = the G query heads (padded to 16 columns);
//   * online softmax in the log2 domain per head, P and the rescale factor shared through LDS
//     within the wave;
//   * O += P V on the vector ALU in fp32: lane (g, n) owns dims 8n..8n+7 of tokens g, g+4, ...
// The four waves' (max, sum, output) meet in LDS and the chunk's partial goes to the workspace; the
// merge combines a unit's chunks in chunk order.
#include <algorithm>

#include "twl_device.h"
#include "twl_internal.h"

namespace twl {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kPartStride = kPartFloats;  // (m, l, pad, pad, o[128]) per head

// 16 bytes of K or V, read with the non-temporal hint: every row is read once per step, and keeping
// the stream out of the caches' retained set lifts the gather from ~5.9 to ~6.8 TB/s on MI355X
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t stream_load(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ int list_count(const ListView& L, int u) {
  return L.indptr ? (L.indptr[u + 1] - L.indptr[u]) : L.counts[u];
}
__device__ __forceinline__ const int32_t* list_ptr(const ListView& L, int u) {
  return L.indptr ? (L.tokens + L.indptr[u]) : (L.tokens + (size_t)u * L.stride);
}
__device__ __forceinline__ const int32_t* list_rows(const ListView& L, int u) {
  return L.indptr ? (L.rows + L.indptr[u]) : (L.rows + (size_t)u * L.stride);
}

constexpr int kAttnWaves = 4;
constexpr int kAttnSB = 16;  // tokens per sub-block

// NSB: sub-blocks per wave (chunk = 4 waves x NSB x 16 tokens); the sequence is fully unrolled so
// the count of loads in flight is known at every wait.
// MK: the chunk is a range of the candidate index space whose kept entries come from bitmaps (each
// wave compacts its kept candidates' rows in LDS first); otherwise it is a range of a token list.
// HW (with MK): head-wise -- a row read for the group's union counts for head h only when h's own
// bitmap keeps it (the row's head bits travel with it through the compaction).
// With MK the candidates are pages (the selector's list, or every page of the sequence), so a
// sub-block's K/V rows follow from its page.
template <int G, int NSB, bool MK, bool HW = false>
__global__ __launch_bounds__(64 * kAttnWaves) void k_attn(CacheView c, const uint16_t* __restrict__ q,
                                                          float sm_log2, ListView L, MaskView MV, int slots,
                                                          float* __restrict__ partials,
                                                          int32_t* __restrict__ merge_ticket, int nticket) {
  constexpr int NWV = kAttnWaves, SB = kAttnSB, VS = SB / 4, CH = NWV * NSB * SB, QL = CH / NWV;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nn = lane & 15, grp = lane >> 4;
  __shared__ float Pl[NWV][SB * G];
  __shared__ float Al[NWV][G];
  __shared__ float sm_m[NWV][G], sm_l[NWV][G];
  __shared__ float4 so[NWV][G][32];
  __shared__ int cr[MK ? NWV : 1][MK ? QL : 1];
  __shared__ int crh[HW ? NWV : 1][HW ? QL : 1];

  // the merge's split tickets start from zero
  if (blockIdx.x == 0)
    for (int i = tid; i < nticket; i += 64 * NWV) merge_ticket[i] = 0;
  // chunk slot k of unit u (the unit's chunks are its first ceil(count / CH) slots)
  int k;
  const int u = head_fast_unit(blockIdx.x, c.Hkv, slots, k);
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int t_begin = k * CH;
  const int w_begin = t_begin + wv * QL;
  // B operand: q of head nn (zero for padding columns), dims 32kb + 8grp .. +7
  bf16x8_t qv[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    if (nn < G) {
      qv[kb] = *reinterpret_cast<const bf16x8_t*>(q + ((size_t)b * c.Hq + (size_t)h * G + nn) * kD + kb * 32 + grp * 8);
    } else {
      qv[kb] = bf16x8_t{};
    }
  }
  int rows[NSB];
  int hrow[NSB] = {};  // head bits of each row (head-wise only)
  int w_end;
  if constexpr (MK) {
    // the quarter's candidate rows and kept bits (one round trip with q), then the kept rows compacted.
    // Sub-block i covers candidates w_begin + 16 i .. + 15: half of mask word (w_begin + 16 i) / 32, and
    // one page of the candidate list (w_begin is a multiple of 16).  One vector load per wave brings
    // the quarter's mask words (lane hh * NWQ + j: word j of head hh, or of the union) and another its
    // pages' physical ids (lane i: sub-block i); each sub-block then takes them with readlanes.
    const int mw = (int)(MV.ncap >> 5);
    constexpr int NWQ = NSB / 2 + 1;  // words a quarter can touch
    const int w0 = w_begin >> 5;
    // every lane loads from a valid address (no branches, so the loads stay in flight together); only
    // lanes hh * NWQ + j with hh < G (j < NWQ for the union) are read back
    const bool use_union = !HW && MV.union_words;
    const int hh_l = lane / NWQ, j_l = lane - hh_l * NWQ;
    const uint32_t* mbase = use_union ? MV.union_words + (int64_t)u * mw
                                      : MV.head_masks + ((int64_t)b * c.Hq + h * G + min(hh_l, G - 1)) * mw;
    const uint32_t mword = mbase[min(w0 + j_l, mw - 1)];
    int crw[NSB];
    int ph_l = 0;
    {
      const bool sel = MV.cand_mode == kCandPages;
      const int32_t* pbase = sel ? MV.page_phys + (int64_t)u * MV.page_stride : c.page_table + (int64_t)b * c.maxP;
      const int plim = sel ? MV.page_stride : c.maxP;
      ph_l = pbase[min((w_begin >> 4) + min(lane, NSB - 1), plim - 1)];
    }
    uint32_t wd[NSB];
    int hb[NSB];
#pragma unroll
    for (int i = 0; i < NSB; ++i) {
      const int cidx = w_begin + i * SB + (lane & 15);
      const int jw = ((w_begin & 16) + i * SB) >> 5;  // the sub-block's word within the quarter's
      hb[i] = 0;
      if (use_union) {
        wd[i] = (uint32_t)__builtin_amdgcn_readlane((int)mword, jw);
      } else {
        uint32_t x = 0u;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)mword, hh * NWQ + jw);
          x |= y;
          if (HW) hb[i] |= (int)((y >> (cidx & 31)) & 1u) << hh;
        }
        wd[i] = x;
      }
      crw[i] = (__builtin_amdgcn_readlane(ph_l, i) * c.Hkv + h) * kPage + (lane & 15);
    }
    int kept = 0;
#pragma unroll
    for (int i = 0; i < NSB; ++i) {
      const int cidx = w_begin + i * SB + (lane & 15);
      const bool f = lane < SB && ((wd[i] >> (cidx & 31)) & 1u);
      const unsigned long long bal = __ballot(f);
      const int pos = kept + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      if (f) {
        cr[wv][pos] = crw[i];
        if (HW) crh[HW ? wv : 0][HW ? pos : 0] = hb[i];
      }
      kept += __popcll(bal);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int kl = kept > 0 ? kept - 1 : 0;
#pragma unroll
    for (int i = 0; i < NSB; ++i) {
      rows[i] = cr[wv][min(i * SB + (lane & 15), kl)];
      hrow[i] = HW ? crh[HW ? wv : 0][HW ? min(i * SB + (lane & 15), kl) : 0] : 0;
    }
    w_end = kept;
  } else {
    // The rows of this wave's quarter are read together with the count and q (one round trip).
    // Entries past the count may hold anything: a row is used as an address only after a range
    // check, and whether it counts is decided from its index.
    const int32_t* rws;
    int lim;
    if (L.indptr) {
      const int64_t a = __builtin_amdgcn_readfirstlane(L.indptr[u]);
      const bool ok = a >= 0 && a < L.cap;
      rws = L.rows + (ok ? a : 0);
      lim = ok ? (int)min(L.cap - a, (int64_t)1 << 30) - 1 : -1;
    } else {
      rws = L.rows + (size_t)u * L.stride;
      lim = (int)L.stride - 1;
    }
#pragma unroll
    for (int i = 0; i < NSB; ++i) rows[i] = (lim >= 0) ? rws[min(w_begin + i * SB + lane, lim)] : -1;
    int cnt = __builtin_amdgcn_readfirstlane(max(0, list_count(L, u)));
    cnt = min(cnt, lim + 1);  // a CSR list that breaks its declared bound is cut at the arrays' end
    if (t_begin >= cnt) return;  // an unused slot
    const int t_end = min(cnt, t_begin + CH);
    w_end = min(t_end, w_begin + QL);
  }
  const int w_first = MK ? 0 : w_begin;  // list index of the first entry of sub-block 0
  const int nrows = c.nphys * c.Hkv * kPage;
  float m_run = -__builtin_inff(), l_run = 0.f;
  float acc[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[hh][i] = 0.f;

  auto issue = [&](int row, bf16x8_t (&kv)[4], uint4 (&vv)[VS]) {
    const int rs = ((unsigned)row < (unsigned)nrows) ? row : 0;
    const int r = __shfl(rs, nn);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      kv[kb] = __builtin_bit_cast(bf16x8_t, stream_load(c.k + (size_t)r * kD + kb * 32 + grp * 8));
#pragma unroll
    for (int s2 = 0; s2 < VS; ++s2) {
      const int rv = __shfl(rs, grp + 4 * s2);
      vv[s2] = __builtin_bit_cast(uint4, stream_load(c.v + (size_t)rv * kD + nn * 8));
    }
  };
  auto consume = [&](int sb, int row, int hr, const bf16x8_t (&kv)[4], const uint4 (&vv)[VS]) {
    const unsigned long long vmask = __ballot(lane < SB && sb + lane < w_end && row >= 0);
    floatx4_t sacc = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[kb], qv[kb], sacc, 0, 0, 0);
    // lane holds S[token 4*grp + e][head nn]
    float sv[4];
    float mx = -__builtin_inff();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * grp + e;
      bool keep = (vmask >> t) & 1ull;
      if (HW) keep = keep && ((__shfl(hr, t) >> nn) & 1);  // head nn's own bitmap keeps token t
      const float x = keep ? sacc[e] * sm_log2 : -__builtin_inff();
      sv[e] = x;
      mx = fmaxf(mx, x);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == -__builtin_inff()) ? 1.f : exp2f(m_run - m_new);
    // once the running maxima settle most sub-blocks leave every head's scale at exactly 1: the
    // rescaling of the accumulators is then skipped (wave-uniform; multiplying by 1 changes nothing)
    const bool rescale = __ballot(nn < G && alpha != 1.f) != 0ull;
    float ps = 0.f;
    float pv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pv[e] = (sv[e] == -__builtin_inff()) ? 0.f : exp2f(sv[e] - m_new);
      ps += pv[e];
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    if (nn < G) {
#pragma unroll
      for (int e = 0; e < 4; ++e) Pl[wv][(4 * grp + e) * G + nn] = pv[e];
      if (grp == 0) Al[wv][nn] = alpha;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (rescale) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float a = Al[wv][hh];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[hh][i] *= a;
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < VS; ++s2) {
      const int t = grp + 4 * s2;
      const bool ok = (vmask >> t) & 1ull;  // rows past the list or outside the sequence contribute 0
      const uint32_t w[4] = {ok ? vv[s2].x : 0u, ok ? vv[s2].y : 0u, ok ? vv[s2].z : 0u, ok ? vv[s2].w : 0u};
      float vf[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vf[2 * i] = bf16_lo(w[i]);
        vf[2 * i + 1] = bf16_hi(w[i]);
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float pp = Pl[wv][t * G + hh];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[hh][i] = fmaf(pp, vf[i], acc[hh][i]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  if (w_end > w_first) {
    // the data of sub-block i + 1 in flight while sub-block i is computed; sub-blocks past the list
    // read in-range rows and are masked
    bf16x8_t kv[2][4];
    uint4 vv[2][VS];
    issue(rows[0], kv[0], vv[0]);
#pragma unroll
    for (int i = 0; i < NSB; ++i) {
      if (i + 1 < NSB) issue(rows[i + 1], kv[(i + 1) & 1], vv[(i + 1) & 1]);
      consume(w_first + i * SB, rows[i], hrow[i], kv[i & 1], vv[i & 1]);
    }
  }

  // sum the four token groups of the wave, then combine the block's waves in wave order
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x = acc[hh][i];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[hh][i] = x;
    }
  if (grp == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      so[wv][hh][2 * nn] = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
      so[wv][hh][2 * nn + 1] = make_float4(acc[hh][4], acc[hh][5], acc[hh][6], acc[hh][7]);
    }
    if (nn < G) {
      sm_m[wv][nn] = m_run;
      sm_l[wv][nn] = l_run;
    }
  }
  __syncthreads();
  float* part = partials + ((size_t)u * slots + k) * G * kPartStride;
  for (int t = tid; t < G * 32; t += 64 * NWV) {
    const int hh = t >> 5, d4 = t & 31;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, sm_m[w][hh]);
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float l = 0.f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        if (sm_m[w][hh] != -__builtin_inff()) {
          const float sc = exp2f(sm_m[w][hh] - M);
          const float4 x = so[w][hh][d4];
          o.x += x.x * sc;
          o.y += x.y * sc;
          o.z += x.z * sc;
          o.w += x.w * sc;
          l += sm_l[w][hh] * sc;
        }
      }
    }
    reinterpret_cast<float4*>(part + hh * kPartStride + 4)[d4] = o;
    if (d4 == 0) {
      part[hh * kPartStride] = M;
      part[hh * kPartStride + 1] = l;
    }
  }
}

// K/V row of every entry of a CSR token list (-1 for ids outside the sequence), so the attention's
// loads never wait on a page-table lookup.
__global__ __launch_bounds__(256) void k_rows(CacheView c, const int32_t* __restrict__ indptr,
                                              const int32_t* __restrict__ tokens, int32_t* __restrict__ rows,
                                              int64_t capacity) {
  const int u = blockIdx.y;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int a = indptr[u], e = indptr[u + 1];
  const int n = clampi(c.seq_lens[b], 0, c.maxTok);
  for (int i = a + (int)(blockIdx.x * 256 + threadIdx.x); i < e; i += (int)(gridDim.x * 256)) {
    if (i < 0 || i >= capacity) continue;
    const int tok = tokens[i];
    int r = -1;
    if (tok >= 0 && tok < n) r = (c.page_table[(size_t)b * c.maxP + (tok >> 4)] * c.Hkv + h) * kPage + (tok & 15);
    rows[i] = r;
  }
}

// Blocks per (unit, head): split sb of S merges the unit's chunk partials [sb per, (sb + 1) per) by
// NR rows of 32 threads (8, 16 or 32 rows as the count needs), row r taking chunks r, r + NR, ... in
// order with a running maximum and thread j owning dims 4j..4j+3 (UNR chunks' loads in flight per
// thread); the NR row results are then combined in row order.  With a token list the unit has
// ceil(count / CH) chunks; without one every slot holds a partial.  With S > 1 each split leaves its
// (max, sum, row) record with agent-scope stores (seen by every die), takes a ticket, and the head's
// last split combines the S records in split order, so the result does not depend on which finishes
// last.
template <int G, int NR, int UNR>
__global__ __launch_bounds__(NR * 32) void k_merge(CacheView c, ListView L, bool use_list, int CH, int slots, int S,
                                                   const float* __restrict__ partials, float* __restrict__ part2,
                                                   int32_t* __restrict__ ticket, float* out, float* lse) {
  const int hb = blockIdx.x / S, sb = blockIdx.x - hb * S;  // (unit, head) row and split
  const int u = hb / G, hh = hb - u * G;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int tid = threadIdx.x, r = tid >> 5, j = tid & 31;
  __shared__ float sM[NR], sL[NR];
  __shared__ float4 sO[NR][32];
  __shared__ int s_last;
  const int nch = use_list ? min((max(0, list_count(L, u)) + CH - 1) / CH, slots) : slots;
  const int per = (slots + S - 1) / S;
  const int k_lo = sb * per, k_hi = min(slots, k_lo + per), k_end = min(nch, k_hi);
  const float* base = partials + ((size_t)u * slots * G + hh) * kPartStride;
  constexpr size_t kStep = (size_t)G * kPartStride;
  float M = -__builtin_inff(), Ls = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = k_lo + r; k0 < k_hi; k0 += NR * UNR) {
    float mk[UNR], lk[UNR];
    float4 ok[UNR];
    // every load unconditional (a chunk past the split reads the split's first record, and any chunk
    // past the count is dropped after), so the row's loads are all in flight at once
#pragma unroll
    for (int i = 0; i < UNR; ++i) {
      const int k = k0 + NR * i;
      const float* pk = base + (size_t)(k < k_hi ? k : k_lo) * kStep;
      mk[i] = pk[0];
      lk[i] = pk[1];
      ok[i] = reinterpret_cast<const float4*>(pk + 4)[j];
    }
#pragma unroll
    for (int i = 0; i < UNR; ++i)
      if (k0 + NR * i >= k_end) mk[i] = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < UNR; ++i) {
      if (mk[i] != -__builtin_inff()) {
        const float Mn = fmaxf(M, mk[i]);
        const float sa = exp2f(M - Mn), sb2 = exp2f(mk[i] - Mn);
        Ls = Ls * sa + lk[i] * sb2;
        o.x = o.x * sa + ok[i].x * sb2;
        o.y = o.y * sa + ok[i].y * sb2;
        o.z = o.z * sa + ok[i].z * sb2;
        o.w = o.w * sa + ok[i].w * sb2;
        M = Mn;
      }
    }
  }
  if (j == 0) {
    sM[r] = M;
    sL[r] = Ls;
  }
  sO[r][j] = o;
  __syncthreads();
  float Mt = -__builtin_inff(), num = 0.f, den = 0.f;
  if (tid < kD) {
#pragma unroll 8
    for (int i = 0; i < NR; ++i) Mt = fmaxf(Mt, sM[i]);
    if (Mt != -__builtin_inff()) {
      const float* so = reinterpret_cast<const float*>(&sO[0][0]);
#pragma unroll 8
      for (int i = 0; i < NR; ++i) {
        if (sM[i] != -__builtin_inff()) {
          const float s = exp2f(sM[i] - Mt);
          num += so[i * kD + tid] * s;
          den += sL[i] * s;
        }
      }
    }
  }
  if (S > 1) {
    float* rec = part2 + ((size_t)hb * kMergeSplits + sb) * kPartStride;
    if (tid < kD) {
      __hip_atomic_store(reinterpret_cast<uint32_t*>(rec) + 4 + tid, __float_as_uint(num), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      if (tid == 0) {
        __hip_atomic_store(reinterpret_cast<uint32_t*>(rec), __float_as_uint(Mt), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(reinterpret_cast<uint32_t*>(rec) + 1, __float_as_uint(den), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // the record's stores performed before the ticket is taken
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&ticket[hb], 1) == S - 1;
    __syncthreads();
    if (!s_last) return;
    if (tid < kD) {
      // every split's (max, sum, dim tid) in flight at once
      const float* r0 = part2 + (size_t)hb * kMergeSplits * kPartStride;
      auto ld = [](const float* x) {
        return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(x), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT));
      };
      float mi[kMergeSplits], li[kMergeSplits], oi[kMergeSplits];
#pragma unroll
      for (int i = 0; i < kMergeSplits; ++i) {
        const float* ri = r0 + (size_t)(i < S ? i : 0) * kPartStride;
        mi[i] = ld(ri);
        li[i] = ld(ri + 1);
        oi[i] = ld(ri + 4 + tid);
      }
      Mt = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < kMergeSplits; ++i)
        if (i < S) Mt = fmaxf(Mt, mi[i]);
      num = 0.f;
      den = 0.f;
      if (Mt != -__builtin_inff()) {
#pragma unroll
        for (int i = 0; i < kMergeSplits; ++i) {
          if (i < S && mi[i] != -__builtin_inff()) {
            const float s = exp2f(mi[i] - Mt);
            num += oi[i] * s;
            den += li[i] * s;
          }
        }
      }
    }
  }
  if (tid < kD) {
    const size_t oh = (size_t)b * c.Hq + (size_t)h * G + hh;
    out[oh * kD + tid] = (den > 0.f) ? num / den : 0.f;
    if (lse && tid == 0) lse[oh] = (den > 0.f) ? (Mt + log2f(den)) * 0.69314718055994530942f : -__builtin_inff();
  }
}

int attn_chunk_tokens(int64_t total_upper, int group) {
  // 256 tokens (four pipelined sub-blocks per wave) up to 1024 (512 for groups of 8, whose larger
  // accumulators would not fit), aiming at about 1024 chunks: every chunk writes a partial, and those
  // writes slow the K/V stream far beyond their byte count.  Small steps keep 256-token chunks: at 65536
  // candidates (a 32K-token layer at keep 1/4) 128-token chunks cost the merge more than they save the
  // attention, and 512-token chunks leave too few blocks
  const int smax = group >= 8 ? 8 : 16;
  int64_t sb = total_upper / (64 * 1024);
  int s = 4;
  while (s * 2 <= sb && s < smax) s *= 2;
  return 64 * s;
}

template <bool MK, bool HW = false>
static hipError_t launch_attn_impl(const CacheView& c, const uint16_t* q, float sm, const ListView& list,
                                   const MaskView& mv, int chunk_tokens, int slots, float* partials,
                                   const MergeWs& mw, hipStream_t s) {
  if (slots < 1) return hipErrorInvalidValue;
  const float sm_log2 = sm * 1.44269504088896340736f;
  const dim3 grid((unsigned)((int64_t)c.B * c.Hkv * slots)), blk(64 * kAttnWaves);
#define TWL_ATTN_G(GG, NS)                                                                                  \
  case GG:                                                                                                  \
    hipLaunchKernelGGL((k_attn<GG, NS, MK, HW>), grid, blk, 0, s, c, q, sm_log2, list, mv, slots, partials,  \
                       mw.ticket, c.B * c.Hq);                                                             \
    break;
#define TWL_ATTN_NSB(NS)                   \
  case NS * kAttnWaves * kAttnSB:          \
    switch (c.G) {                         \
      TWL_ATTN_G(1, NS)                    \
      TWL_ATTN_G(2, NS)                    \
      TWL_ATTN_G(4, NS)                    \
      TWL_ATTN_G(8, NS)                    \
      default: return hipErrorInvalidValue; \
    }                                      \
    break;
#define TWL_ATTN_NSB_SMALL_G(NS)           \
  case NS * kAttnWaves * kAttnSB:          \
    switch (c.G) {                         \
      TWL_ATTN_G(1, NS)                    \
      TWL_ATTN_G(2, NS)                    \
      TWL_ATTN_G(4, NS)                    \
      default: return hipErrorInvalidValue; \
    }                                      \
    break;
  switch (chunk_tokens) {
    TWL_ATTN_NSB(4)
    TWL_ATTN_NSB(8)
    TWL_ATTN_NSB_SMALL_G(16)
    default: return hipErrorInvalidValue;
  }
#undef TWL_ATTN_G
#undef TWL_ATTN_NSB
#undef TWL_ATTN_NSB_SMALL_G
  return hipGetLastError();
}

hipError_t launch_attn(const CacheView& c, const uint16_t* q, float sm, const ListView& list, int chunk_tokens,
                       int slots, float* partials, const MergeWs& mw, hipStream_t s) {
  if (!list.rows || !mw.ticket) return hipErrorInvalidValue;
  return launch_attn_impl<false>(c, q, sm, list, MaskView{}, chunk_tokens, slots, partials, mw, s);
}

hipError_t launch_attn_masked(const CacheView& c, const uint16_t* q, float sm, const MaskView& mv, int chunk_tokens,
                              int slots, float* partials, const MergeWs& mw, bool headwise, hipStream_t s) {
  if ((!mv.head_masks && !mv.union_words) || mv.ncap % chunk_tokens || !mw.ticket) return hipErrorInvalidValue;
  if ((mv.cand_mode != kCandPages && mv.cand_mode != kCandAll) || (mv.cand_mode == kCandPages && !mv.page_phys))
    return hipErrorInvalidValue;
  if (headwise) {
    if (!mv.head_masks) return hipErrorInvalidValue;
    return launch_attn_impl<true, true>(c, q, sm, ListView{}, mv, chunk_tokens, slots, partials, mw, s);
  }
  return launch_attn_impl<true, false>(c, q, sm, ListView{}, mv, chunk_tokens, slots, partials, mw, s);
}

hipError_t launch_rows(const CacheView& c, const int32_t* indptr, const int32_t* tokens, int32_t* rows,
                       int64_t capacity, hipStream_t s) {
  hipLaunchKernelGGL(k_rows, dim3(16, (unsigned)(c.B * c.Hkv)), dim3(256), 0, s, c, indptr, tokens, rows, capacity);
  return hipGetLastError();
}

hipError_t launch_merge(const CacheView& c, const ListView* list, int chunk_tokens, int slots, const float* partials,
                        const MergeWs& mw, float* out, float* lse, hipStream_t s) {
  if (!mw.part || !mw.ticket || slots < 1) return hipErrorInvalidValue;
  const int heads = c.B * c.Hq;
  // splits per head, for long rows only (the split records and the ticket cost about one short
  // row's merge): enough blocks to spread the records over the chip (about 512), at least 32 chunks
  // per split, at most kMergeSplits
  int S = 1;
  if (slots > 128) S = std::max(1, std::min({kMergeSplits, 512 / std::max(heads, 1), slots / 32}));
  const int per = (slots + S - 1) / S;
  dim3 grid((unsigned)(heads * S));
  const ListView lv = list ? *list : ListView{};
  const bool use_list = list != nullptr;
  // rows of 32 threads: enough for about four chunks per row (one round of loads), at least 8 (the
  // final combine uses 128 threads); past 128 chunks, 32 rows of 8 records each in flight
  const int nr = per <= 32 ? 8 : (per <= 64 ? 16 : (per <= 128 ? 32 : 64));
#define TWL_MERGE_NR(GG, NR, RR, UU)                                                                         \
  case NR:                                                                                                   \
    hipLaunchKernelGGL((k_merge<GG, RR, UU>), grid, dim3(RR * 32), 0, s, c, lv, use_list, chunk_tokens,       \
                       slots, S, partials, mw.part, mw.ticket, out, lse);                                   \
    break;
#define TWL_MERGE_CASE(GG)     \
  case GG:                     \
    switch (nr) {              \
      TWL_MERGE_NR(GG, 8, 8, 4)      \
      TWL_MERGE_NR(GG, 16, 16, 4)    \
      TWL_MERGE_NR(GG, 32, 32, 4)    \
      TWL_MERGE_NR(GG, 64, 32, 8)    \
    }                          \
    break;
  switch (c.G) {
    TWL_MERGE_CASE(1)
    TWL_MERGE_CASE(2)
    TWL_MERGE_CASE(4)
    TWL_MERGE_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef TWL_MERGE_CASE
#undef TWL_MERGE_NR
  return hipGetLastError();
}

}  // namespace twl
