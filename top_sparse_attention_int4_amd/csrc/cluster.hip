// Double-P first stage: cluster-level top-p on size-weighted centroids, and the union of the kept
// clusters as token ranges ("Double-P: Hierarchical Top-P Sparse Attention for Long-Context LLMs",
// sections 方法详解 and 关键设计: a coarse top-p over clusters precedes a token-level top-p inside
// the kept clusters).
//
// Clusters of a (sequence, kv-head) unit are contiguous token ranges with a given bf16 centroid mu_c
// and size n_c.  Per query head the cluster logit is l_c = fl(sm * fold_{c'}(acc + q_c' mu_c,c')), a
// float32 left-to-right fold from +0 (bf16 x bf16 products are exact, so each fused multiply-add
// is the rounded addition of the fold); its weight is n_c exp(l_c - M) with M the largest logit of
// a non-empty cluster.  Empty clusters, and the padding up to the top-p block size, carry a logit of
// -inf and are never candidates.  The top-p itself is the weighted mode of the token-level
// bisection kernel.
#include "twl_device.h"
#include "twl_internal.h"

namespace twl {

// One block per (unit, 64 clusters); wave hh folds query head hh for the block's 64 clusters from an
// LDS copy of their centroids (read with coalesced 16-byte loads).
template <int G>
__global__ __launch_bounds__(64 * (G > 4 ? G : 4)) void k_cluster_score(CacheView c, const uint16_t* __restrict__ q,
                                                                        const uint16_t* __restrict__ cent,
                                                                        const int32_t* __restrict__ csize, int C,
                                                                        int cpad, float sm, float* __restrict__ lam,
                                                                        int blocks_per_unit, QDigits qd) {
  constexpr int NT = 64 * (G > 4 ? G : 4);
  const int u = blockIdx.x / blocks_per_unit;
  const int blk = blockIdx.x - u * blocks_per_unit;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int hh = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // the token-level estimate's query digits, shared out over the unit's blocks
  if (qd.dig) unit_query_digits(q, c.Hq, c.kbits, b, h, G, NT, blk, blocks_per_unit, qd);
  __shared__ uint4 tile[64][17];  // 64 centroid rows of 16 x 16 B, padded by 16 B
  __shared__ float qs[G][kD];
  {
    constexpr int R = 64 * 16 / NT;
    const int part = threadIdx.x & 15;
    uint4 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int j = blk * 64 + ((int)threadIdx.x >> 4) + r * (NT / 16);
      v[r] = (j < C) ? reinterpret_cast<const uint4*>(cent + ((size_t)u * C + j) * kD)[part]
                     : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) tile[((int)threadIdx.x >> 4) + r * (NT / 16)][part] = v[r];
  }
  const uint16_t* qg = q + ((size_t)b * c.Hq + (size_t)h * G) * kD;
  for (int i = threadIdx.x; i < G * kD; i += NT) qs[i / kD][i % kD] = __uint_as_float((uint32_t)qg[i] << 16);
  __syncthreads();

  const int j = blk * 64 + lane;
  if (hh < G && j < cpad) {
    float out = -__builtin_inff();
    if (j < C && csize[(size_t)u * C + j] > 0) {
      float acc = 0.f;
#pragma unroll
      for (int c8 = 0; c8 < 16; ++c8) {
        const uint4 w4 = tile[lane][c8];
        const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float mu = (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
          acc = fmaf(qs[hh][c8 * 8 + e], mu, acc);
        }
      }
      out = sm * acc;
    }
    lam[((size_t)b * c.Hq + (size_t)h * G + hh) * cpad + j] = out;
  }
}

// One block per unit: OR of the G head masks over the clusters, then the kept clusters written in
// ascending order as (first token, length) ranges, and their count.
template <int G>
__global__ __launch_bounds__(1024) void k_cluster_union(CacheView c, const uint32_t* __restrict__ mask_ws, int cpad,
                                                        const int32_t* __restrict__ csize,
                                                        const int32_t* __restrict__ coff, int C,
                                                        int32_t* __restrict__ ranges, int32_t* __restrict__ count,
                                                        int32_t* __restrict__ prefix, int32_t* __restrict__ chunk_first,
                                                        int nchunk) {
  constexpr int NT = 1024, NW = NT / 64;
  constexpr int kMaxWords = 65536 / 32;
  constexpr int WPT = kMaxWords / NT;
  __shared__ uint32_t uw[kMaxWords];
  __shared__ int woff[kMaxWords];
  __shared__ int scan_sm[NW + 1];
  __shared__ int spre[4096 + 1];
  const int u = blockIdx.x;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int tid = threadIdx.x;
  const int MW = cpad / 32;
  const uint32_t* m0 = mask_ws + ((size_t)b * c.Hq + (size_t)h * G) * MW;
  uint32_t words[WPT];
  int local = 0;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int w = tid * WPT + i;
    uint32_t x = 0u;
    if (w < MW) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) x |= m0[(size_t)hh * MW + w];
    }
    words[i] = x;
    local += __popc(x);
  }
  int total;
  int off = block_excl_scan<NW>(local, scan_sm, &total);
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int w = tid * WPT + i;
    if (w < MW) {
      uw[w] = words[i];
      woff[w] = off;
      off += __popc(words[i]);
    }
  }
  __syncthreads();
  const int32_t* cs = csize + (size_t)u * C;
  const int32_t* co = coff + (size_t)u * (C + 1);
  int32_t* rg = ranges + (size_t)u * C * 2;
  // each thread takes a contiguous run of clusters, so the kept ones' positions and token offsets
  // follow from block scans; ranges hold (first token, length).  Up to CR clusters per thread their
  // sizes and offsets are read together (one round trip); more take a loop.
  constexpr int CR = 4;
  const int cpt = (C + NT - 1) / NT;
  const int k0 = tid * cpt, k1 = min(k0 + cpt, C);
  const bool regs = cpt <= CR;  // uniform
  int lenr[CR], offr[CR];
#pragma unroll
  for (int i = 0; i < CR; ++i) {
    const int k = min(k0 + i, C - 1);
    lenr[i] = regs ? cs[k] : 0;
    offr[i] = regs ? co[k] : 0;
  }
  auto kept_at = [&](int k, int& pos) {
    const uint32_t x = uw[k >> 5];
    const int bit = k & 31;
    pos = woff[k >> 5] + __popc(x & ((1u << bit) - 1u));
    return ((x >> bit) & 1u) != 0u;
  };
  int tok_local = 0;
  if (regs) {
#pragma unroll
    for (int i = 0; i < CR; ++i) {
      int pos;
      if (k0 + i < k1 && kept_at(k0 + i, pos)) {
        rg[2 * pos] = offr[i];
        rg[2 * pos + 1] = lenr[i];
        tok_local += max(lenr[i], 0);
      }
    }
  } else {
    for (int k = k0; k < k1; ++k) {
      int pos;
      if (kept_at(k, pos)) {
        const int len = cs[k];
        rg[2 * pos] = co[k];
        rg[2 * pos + 1] = len;
        tok_local += max(len, 0);
      }
    }
  }
  if (tid == 0) count[u] = total;
  if (!prefix) return;  // uniform
  // prefix sums of the kept ranges' lengths (negative lengths count as 0), and for every block of
  // kEstCands candidates the range holding its first candidate (the count when past the last one)
  int tok_total;
  int run = block_excl_scan<NW>(tok_local, scan_sm, &tok_total);
  int32_t* pre = prefix + (size_t)u * (C + 1);
  int32_t* cf = chunk_first + (size_t)u * nchunk;
  constexpr int kLdsPre = 4096;
  const bool in_lds = total <= kLdsPre;  // uniform
  auto put = [&](int pos, int len) {
    pre[pos] = run;
    if (in_lds) spre[pos] = run;
    run += len;
  };
  if (regs) {
#pragma unroll
    for (int i = 0; i < CR; ++i) {
      int pos;
      if (k0 + i < k1 && kept_at(k0 + i, pos)) put(pos, max(lenr[i], 0));
    }
  } else {
    for (int k = k0; k < k1; ++k) {
      int pos;
      if (kept_at(k, pos)) put(pos, max(cs[k], 0));
    }
  }
  if (tid == 0) {
    pre[total] = tok_total;
    if (in_lds) spre[total] = tok_total;
  }
  __syncthreads();  // (also orders this block's global writes of pre before the reads below)
  // block j starts at candidate j * kEstCands: the last range whose prefix is <= that (empty ranges
  // share their successor's prefix, so the last of equal ones is the non-empty one)
  const int32_t* sp = in_lds ? spre : pre;
  for (int j = tid; j < nchunk; j += NT) {
    const int x = j * kEstCands;
    int r = total;
    if (x < tok_total) {
      int lo = 0, hi = total;  // sp[lo] <= x < sp[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sp[mid] <= x) lo = mid; else hi = mid;
      }
      r = lo;
    }
    cf[j] = r;
  }
}

hipError_t launch_cluster_union(const CacheView& c, const uint32_t* mask_ws, int cpad, const int32_t* csize,
                                const int32_t* coff, int C, int32_t* ranges, int32_t* count, int32_t* prefix,
                                int32_t* chunk_first, int nchunk, hipStream_t s) {
  dim3 ugrid((unsigned)(c.B * c.Hkv));
#define TWL_CU_G(GG)                                                                                         \
  case GG:                                                                                                   \
    hipLaunchKernelGGL(k_cluster_union<GG>, ugrid, dim3(1024), 0, s, c, mask_ws, cpad, csize, coff, C, ranges, \
                       count, prefix, chunk_first, nchunk);                                                  \
    break;
  switch (c.G) {
    TWL_CU_G(1)
    TWL_CU_G(2)
    TWL_CU_G(4)
    TWL_CU_G(8)
    default: return hipErrorInvalidValue;
  }
#undef TWL_CU_G
  return hipGetLastError();
}

// Slots a .. b - 1 of a page (0 <= a < b <= 16).
__device__ __forceinline__ uint32_t slot_bits(int a, int b) { return ((1u << b) - 1u) & ~((1u << a) - 1u); }

// Per unit and segment of kSlotSeg pages, one block: the mask of kept token slots of every page of the
// segment -- the token-level candidates as every page of the sequence with such a mask (page-indexed,
// [U][maxP]; pages past the sequence get 0), so the estimate and the attention read K by page and
// need no compacted list.  Every kept cluster (OR of the G head masks) is clipped to the segment's
// tokens: its first and last pages get their slot bits by OR, the pages strictly between them a
// +1 / -1 pair in a difference array whose prefix sums count the clusters covering each page whole.
// Clusters may come in any order and overlap; tokens at or past the sequence length are not
// candidates.  Each thread's clusters are read kSlotBatch at a time, their loads in flight together.
constexpr int kSlotSeg = 1024, kSlotThreads = 256, kSlotBatch = 16;
template <int G>
__global__ __launch_bounds__(kSlotThreads) void k_cluster_slots(CacheView c, const uint32_t* __restrict__ mask_ws,
                                                                int cpad, const int32_t* __restrict__ csize,
                                                                const int32_t* __restrict__ coff, int C,
                                                                int seg_blocks, uint32_t* __restrict__ smask) {
  constexpr int NT = kSlotThreads, NW = NT / 64, PPT = kSlotSeg / NT;
  static_assert(PPT == 4, "four pages per thread");
  constexpr int kMaxWords = 65536 / 32;
  __shared__ uint32_t uw[kMaxWords];
  __shared__ __align__(16) uint32_t sp[kSlotSeg / 2];  // slot bits, two pages per word
  __shared__ __align__(16) int sd[kSlotSeg + 4];       // difference counts
  __shared__ int scan_sm[NW + 1];
  const int u = blockIdx.x / seg_blocks, sg = blockIdx.x - u * seg_blocks;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int tid = threadIdx.x;
  const int n = clampi(c.seq_lens[b], 0, min(c.maxTok, 16 * c.maxP));
  const int s0 = sg * kSlotSeg;                           // the segment's first page
  const int t0 = 16 * s0, t1 = min(16 * (s0 + kSlotSeg), n);  // its tokens inside the sequence
  // kept clusters
  const int MW = cpad / 32;
  const uint32_t* m0 = mask_ws + ((size_t)b * c.Hq + (size_t)h * G) * MW;
  for (int w = tid; w < MW; w += NT) {
    uint32_t x = 0u;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) x |= m0[(size_t)hh * MW + w];
    uw[w] = x;
  }
  for (int i = tid; i < kSlotSeg / 2; i += NT) sp[i] = 0u;
  for (int i = tid; i < kSlotSeg + 4; i += NT) sd[i] = 0;
  __syncthreads();
  if (t0 < t1) {  // uniform
    const int32_t* co = coff + (size_t)u * (C + 1);
    const int32_t* cs = csize + (size_t)u * C;
    for (int k0 = 0; k0 < C; k0 += NT * kSlotBatch) {
      int begr[kSlotBatch], lenr[kSlotBatch];
#pragma unroll
      for (int i = 0; i < kSlotBatch; ++i) {
        const int k = min(k0 + i * NT + tid, C - 1);
        begr[i] = co[k];
        lenr[i] = cs[k];
      }
#pragma unroll
      for (int i = 0; i < kSlotBatch; ++i) {
        const int k = k0 + i * NT + tid;
        if (k >= C || !((uw[k >> 5] >> (k & 31)) & 1u)) continue;
        const int lo = max(begr[i], t0);
        const int hi = (int)min((int64_t)begr[i] + (int64_t)max(lenr[i], 0), (int64_t)t1);
        if (hi <= lo) continue;
        const int p0 = (lo >> 4) - s0, p1 = ((hi - 1) >> 4) - s0;
        if (p0 == p1) {
          atomicOr(&sp[p0 >> 1], slot_bits(lo & 15, hi - 16 * (s0 + p0)) << (16 * (p0 & 1)));
        } else {
          atomicOr(&sp[p0 >> 1], slot_bits(lo & 15, 16) << (16 * (p0 & 1)));
          atomicOr(&sp[p1 >> 1], slot_bits(0, hi - 16 * (s0 + p1)) << (16 * (p1 & 1)));
          if (p1 - p0 >= 2) {
            atomicAdd(&sd[p0 + 1], 1);
            atomicAdd(&sd[p1], -1);
          }
        }
      }
    }
  }
  __syncthreads();
  // thread t: pages s0 + 4t .. + 3 (one 16-byte and one 8-byte LDS read)
  const int4 d4 = reinterpret_cast<const int4*>(sd)[tid];
  const uint2 sp2 = reinterpret_cast<const uint2*>(sp)[tid];
  const int dv[PPT] = {d4.x, d4.y, d4.z, d4.w};
  const uint32_t bits[PPT] = {sp2.x & 0xFFFFu, sp2.x >> 16, sp2.y & 0xFFFFu, sp2.y >> 16};
  int tot;
  int run = block_excl_scan<NW>(dv[0] + dv[1] + dv[2] + dv[3], scan_sm, &tot);
  uint32_t* out = smask + (size_t)u * c.maxP;
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int q = s0 + PPT * tid + i;
    run += dv[i];
    uint32_t m = 0u;
    const int tq = 16 * q;
    if (tq < n) {
      m = bits[i] | (run > 0 ? 0xFFFFu : 0u);
      if (tq + 16 > n) m &= slot_bits(0, n - tq);
    }
    if (q < c.maxP) out[q] = m;
  }
}

hipError_t launch_cluster_slots(const CacheView& c, const uint32_t* mask_ws, int cpad, const int32_t* csize,
                                const int32_t* coff, int C, uint32_t* smask, hipStream_t s) {
  if (C < 1 || C > 65536 || cpad > 65536 || c.maxP < 1) return hipErrorInvalidValue;
  const int seg_blocks = (c.maxP + kSlotSeg - 1) / kSlotSeg;
  dim3 grid((unsigned)(c.B * c.Hkv * seg_blocks));
#define TWL_CS_G(GG)                                                                                          \
  case GG:                                                                                                    \
    hipLaunchKernelGGL(k_cluster_slots<GG>, grid, dim3(kSlotThreads), 0, s, c, mask_ws, cpad, csize, coff, C,  \
                       seg_blocks, smask);                                                                    \
    break;
  switch (c.G) {
    TWL_CS_G(1)
    TWL_CS_G(2)
    TWL_CS_G(4)
    TWL_CS_G(8)
    default: return hipErrorInvalidValue;
  }
#undef TWL_CS_G
  return hipGetLastError();
}

hipError_t launch_cluster_scores_topp(const CacheView& c, const uint16_t* q, float sm, float p1, int iters,
                                      const uint16_t* centroids, const int32_t* csize, int C, int cpad, float* lam,
                                      float* thr, uint32_t* mask_ws, const QDigits& qd, hipStream_t s) {
  const int bpu = cpad / 64;
  dim3 grid((unsigned)(c.B * c.Hkv * bpu));
  switch (c.G) {
    case 1:
      hipLaunchKernelGGL(k_cluster_score<1>, grid, dim3(256), 0, s, c, q, centroids, csize, C, cpad, sm, lam, bpu, qd);
      break;
    case 2:
      hipLaunchKernelGGL(k_cluster_score<2>, grid, dim3(256), 0, s, c, q, centroids, csize, C, cpad, sm, lam, bpu, qd);
      break;
    case 4:
      hipLaunchKernelGGL(k_cluster_score<4>, grid, dim3(256), 0, s, c, q, centroids, csize, C, cpad, sm, lam, bpu, qd);
      break;
    case 8:
      hipLaunchKernelGGL(k_cluster_score<8>, grid, dim3(512), 0, s, c, q, centroids, csize, C, cpad, sm, lam, bpu, qd);
      break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topp_weighted(c, lam, cpad, p1, iters, thr, mask_ws, csize, C, s);
}

// ---- optional approximation of the clusters no head of the group keeps ------------------------------
// (Double-P abstract: token-level attention only where the cluster level does not suffice.)  A cluster
// that is not kept enters the softmax as its n members collapsed onto (centroid key, mean value):
// n exp(l_c) joins the normaliser and n exp(l_c) vbar_c the numerator, merged with the attention's
// (out, lse) in log-sum-exp form.

// Mean value row of every cluster: one 1024-thread block per (cluster, unit); thread (j, d) sums dim d
// over the cluster's tokens j, j + 8, ... (four rows in flight), the eight partial sums are added in
// order of j and divided by the member count; empty clusters get zeros.
__global__ __launch_bounds__(1024) void k_cluster_vmean(CacheView c, const int32_t* __restrict__ csize,
                                                        const int32_t* __restrict__ coff, int C, float* vmean) {
  constexpr int NJ = 8, UN = 4;
  __shared__ float s_sum[NJ][kD];
  __shared__ int s_cnt[NJ];
  const int cl = blockIdx.x, u = blockIdx.y;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int d = threadIdx.x & (kD - 1), j = threadIdx.x >> 7;
  const int n = csize[(size_t)u * C + cl];
  const int t0 = coff[(size_t)u * (C + 1) + cl];
  const int seq = clampi(c.seq_lens[b], 0, c.maxTok);
  float acc = 0.f;
  int cnt = 0;
  for (int i0 = j; i0 < n; i0 += NJ * UN) {
    float x[UN];
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      const int i = i0 + NJ * k, t = t0 + i;
      x[k] = 0.f;
      if (i < n && t >= 0 && t < seq) {  // tokens outside the sequence are not members
        const int phys = c.page_table[(size_t)b * c.maxP + (t >> 4)];
        const size_t row = ((size_t)phys * c.Hkv + h) * kPage + (t & 15);
        x[k] = __uint_as_float((uint32_t)c.v[row * kD + d] << 16);
        ++cnt;
      }
    }
#pragma unroll
    for (int k = 0; k < UN; ++k) acc += x[k];
  }
  s_sum[j][d] = acc;
  if (d == 0) s_cnt[j] = cnt;
  __syncthreads();
  if (j == 0) {
    float tot = 0.f;
    int m = 0;
#pragma unroll
    for (int k = 0; k < NJ; ++k) {
      tot += s_sum[k][d];
      m += s_cnt[k];
    }
    vmean[((size_t)u * C + cl) * kD + d] = m > 0 ? tot / (float)m : 0.f;
  }
}

// Per (sequence, query head, slice of kApproxSlices): the unkept non-empty clusters of the slice summed
// as (sum_c w_c vbar_c, sum_c w_c) with w_c = n_c exp(l_c - M), M the head's largest l_c + ln n_c over
// all unkept clusters and its lse (each block finds M itself); then one block per head merges the
// slices in order with the attention's (out, lse).
constexpr int kApproxSliceMax = 1024;  // clusters per slice held in LDS at once

template <int G>
__global__ __launch_bounds__(256) void k_cluster_approx(CacheView c, const float* __restrict__ lam,
                                                        const uint32_t* __restrict__ masks, int cpad,
                                                        const int32_t* __restrict__ csize, int C,
                                                        const float* __restrict__ vmean, const float* __restrict__ lse,
                                                        float* __restrict__ part) {
  constexpr int NT = 256, NW = NT / 64, UN = 8;
  __shared__ float s_w[kApproxSliceMax];
  __shared__ float s_acc[2][kD];
  __shared__ float red[2 * NW * 4];
  BlockReduce<NW> br{red};
  const int bh = blockIdx.x, sl = blockIdx.y;
  const int b = bh / c.Hq, hq = bh - b * c.Hq, h = hq / G;
  const int u = b * c.Hkv + h;
  const int tid = threadIdx.x, d = tid & (kD - 1), half = tid >> 7;
  const int mw = cpad / 32;
  const float* lm = lam + (size_t)bh * cpad;
  const uint32_t* mk = masks + ((size_t)b * c.Hq + (size_t)h * G) * mw;
  const int32_t* cs = csize + (size_t)u * C;
  const float* vm = vmean + (size_t)u * C * kD;
  auto weight_arg = [&](int cl) -> float {  // l_c + ln n_c of an unkept non-empty cluster, else -inf
    const int n = cs[cl];
    if (n <= 0) return -__builtin_inff();
    uint32_t any = 0u;
#pragma unroll
    for (int g = 0; g < G; ++g) any |= mk[(size_t)g * mw + (cl >> 5)];
    if ((any >> (cl & 31)) & 1u) return -__builtin_inff();
    return lm[cl] + logf((float)n);
  };
  float m = -__builtin_inff();
  for (int cl = tid; cl < C; cl += NT) m = fmaxf(m, weight_arg(cl));
  m = br.max(m);
  const float M = fmaxf(m, lse[bh]);
  const int per = (C + kApproxSlices - 1) / kApproxSlices;
  const int c0 = sl * per, c1 = min(C, c0 + per);
  float acc = 0.f, den = 0.f;
  if (m != -__builtin_inff()) {
    for (int cb = c0; cb < c1; cb += kApproxSliceMax) {
      const int nc = min(kApproxSliceMax, c1 - cb);
      for (int i = tid; i < nc; i += NT) {
        const float a = weight_arg(cb + i);
        const float w = (a == -__builtin_inff()) ? 0.f : expf(a - M);
        s_w[i] = w;
        den += w;
      }
      __syncthreads();
      // UN clusters' value rows in flight per step (each half block takes every other cluster)
      for (int i0 = half; i0 < nc; i0 += 2 * UN) {
        float x[UN], wv[UN];
#pragma unroll
        for (int k = 0; k < UN; ++k) {
          const int i = i0 + 2 * k;
          wv[k] = i < nc ? s_w[i] : 0.f;
          x[k] = (wv[k] != 0.f) ? vm[(size_t)(cb + i) * kD + d] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < UN; ++k) acc = fmaf(wv[k], x[k], acc);
      }
      __syncthreads();
    }
  }
  s_acc[half][d] = acc;
  den = br.sum(den);  // (its barrier also orders s_acc)
  if (tid < kD) {
    float* pp = part + ((size_t)bh * kApproxSlices + sl) * kApproxStride;
    pp[d] = s_acc[0][d] + s_acc[1][d];
    if (tid == 0) {
      pp[kD] = den;
      pp[kD + 1] = M;
    }
  }
}

__global__ __launch_bounds__(128) void k_cluster_approx_merge(const float* __restrict__ part, float* out, float* lse) {
  const int bh = blockIdx.x, d = threadIdx.x;
  const float* pp = part + (size_t)bh * kApproxSlices * kApproxStride;
  const float M = pp[kD + 1];  // the same in every slice
  float num = 0.f, den = 0.f;
#pragma unroll 4
  for (int sl = 0; sl < kApproxSlices; ++sl) {
    num += pp[sl * kApproxStride + d];
    den += pp[sl * kApproxStride + kD];
  }
  if (den == 0.f) return;  // every non-empty cluster kept: nothing to add
  const float lse_a = lse[bh];
  const float wa = (lse_a == -__builtin_inff()) ? 0.f : expf(lse_a - M);
  const float tot = wa + den;
  float* o = out + (size_t)bh * kD;
  o[d] = (wa * o[d] + num) / tot;
  __syncthreads();  // every thread has read lse before it is rewritten
  if (d == 0) lse[bh] = M + logf(tot);
}

hipError_t launch_cluster_vmean(const CacheView& c, const int32_t* csize, const int32_t* coff, int C, float* vmean,
                                hipStream_t s) {
  hipLaunchKernelGGL(k_cluster_vmean, dim3((unsigned)C, (unsigned)(c.B * c.Hkv)), dim3(1024), 0, s, c, csize, coff,
                     C, vmean);
  return hipGetLastError();
}

hipError_t launch_cluster_approx(const CacheView& c, const float* lam, const uint32_t* masks, int cpad,
                                 const int32_t* csize, int C, const float* vmean, float* out, float* lse, float* part,
                                 hipStream_t s) {
  const dim3 grid((unsigned)(c.B * c.Hq), kApproxSlices), blk(256);
  switch (c.G) {
    case 1: hipLaunchKernelGGL(k_cluster_approx<1>, grid, blk, 0, s, c, lam, masks, cpad, csize, C, vmean, lse, part); break;
    case 2: hipLaunchKernelGGL(k_cluster_approx<2>, grid, blk, 0, s, c, lam, masks, cpad, csize, C, vmean, lse, part); break;
    case 4: hipLaunchKernelGGL(k_cluster_approx<4>, grid, blk, 0, s, c, lam, masks, cpad, csize, C, vmean, lse, part); break;
    case 8: hipLaunchKernelGGL(k_cluster_approx<8>, grid, blk, 0, s, c, lam, masks, cpad, csize, C, vmean, lse, part); break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(k_cluster_approx_merge, dim3((unsigned)(c.B * c.Hq)), dim3(128), 0, s, part, out, lse);
  return hipGetLastError();
}

}  // namespace twl
