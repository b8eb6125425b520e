// Sparse attention over the kept tokens: gather split-K flash-decode plus a fixed-order LSE merge.
//
// The pages compute attention only on the top-p survivors, group-wise for GQA over a flattened
// paged cache, with FlashInfer's balancing across heads whose budgets differ widely (Paper-Notes
// "关键设计 / 负载均衡": per-head budgets from ~2% to ~50%; paperlayer §4.2 and §B.2).  Here the
// token lists of all (sequence, kv-head) units are cut into equal chunks of CH tokens and the
// chunks are numbered across units (head-flattened); a persistent grid of one-wave workgroups walks
// that numbering with a static stride, so a unit with a long list simply owns more chunks.
//
// Per 64-token sub-block of a chunk (one wave):
//   * each lane resolves one token id to its paged K/V row;
//   * S = K q^T with bf16 MFMA (v_mfma_f32_16x16x32_bf16): A = 16 tokens x 32 dims of K loaded
//     straight into registers, B = the G query heads (padded to 16 columns);
//   * online softmax in the log2 domain per head, P and the rescale factor shared through LDS;
//   * O += P V on the vector ALU in fp32: lane (g, n) owns dims 8n..8n+7 of tokens g, g+4, ...
// The chunk's partial (max, sum, unnormalised output) per head goes to the workspace; the merge
// combines a unit's chunks in chunk order.
#include "twl_device.h"
#include "twl_internal.h"

namespace twl {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kPartStride = 2 + kD;  // (m, l, o[128]) per head

__device__ __forceinline__ int list_count(const ListView& L, int u) {
  return L.indptr ? (L.indptr[u + 1] - L.indptr[u]) : L.counts[u];
}
__device__ __forceinline__ const int32_t* list_ptr(const ListView& L, int u) {
  return L.indptr ? (L.tokens + L.indptr[u]) : (L.tokens + (size_t)u * L.stride);
}
__device__ __forceinline__ const int32_t* list_rows(const ListView& L, int u) {
  return L.indptr ? (L.rows + L.indptr[u]) : (L.rows + (size_t)u * L.stride);
}

// Find the unit owning flattened chunk `cid`: returns u, and its first chunk id and token offset.
// Executed by a whole wave; every lane gets the same answer.  Returns -1 when cid >= total.
__device__ int find_unit(const ListView& L, int U, int CH, int cid, int* chunk0, int* tok0) {
  const int lane = threadIdx.x & 63;
  int cbase = 0, tbase = 0;
  for (int base = 0; base < U; base += 64) {
    const int u = base + lane;
    const int cnt = (u < U) ? max(0, list_count(L, u)) : 0;
    const int nch = (cnt + CH - 1) / CH;
    const int cinc = wave_incl_scan(nch);
    const int tinc = wave_incl_scan(cnt);
    const int cex = cbase + cinc - nch;
    const bool mine = (u < U) && nch > 0 && cid >= cex && cid < cex + nch;
    const unsigned long long bal = __ballot(mine);
    if (bal) {
      const int src = __ffsll((long long)bal) - 1;
      *chunk0 = __shfl(cex, src);
      *tok0 = __shfl(tbase + tinc - cnt, src);
      return base + src;
    }
    cbase += __shfl(cinc, 63);
    tbase += __shfl(tinc, 63);
  }
  return -1;
}

template <int G>
__global__ __launch_bounds__(64) void k_attn(CacheView c, const uint16_t* __restrict__ q, float sm_log2,
                                             ListView L, int CH, int max_chunks, float* __restrict__ partials,
                                             int32_t* csr_indptr, int32_t* csr_tokens, int64_t capacity) {
  const int U = c.B * c.Hkv;
  const int lane = threadIdx.x;
  const int nn = lane & 15, grp = lane >> 4;
  __shared__ float Pl[64 * G];
  __shared__ float Al[G];

  if (csr_indptr && blockIdx.x == 0) {
    int tbase = 0;
    for (int base = 0; base < U; base += 64) {
      const int u = base + lane;
      const int cnt = (u < U) ? max(0, list_count(L, u)) : 0;
      const int tinc = wave_incl_scan(cnt);
      if (u < U) csr_indptr[u] = tbase + tinc - cnt;
      tbase += __shfl(tinc, 63);
    }
    if (lane == 0) csr_indptr[U] = tbase;
  }

  for (int cid = blockIdx.x;; cid += gridDim.x) {
    int chunk0 = 0, tok0 = 0;
    if (cid >= max_chunks) break;  // more chunks than the workspace holds: lists exceed their bound
    const int u = find_unit(L, U, CH, cid, &chunk0, &tok0);
    if (u < 0) break;
    const int b = u / c.Hkv, h = u - b * c.Hkv;
    const int n = clampi(c.seq_lens[b], 0, c.maxTok);
    const int cnt = max(0, list_count(L, u));
    const int32_t* toks = list_ptr(L, u);
    const int t_begin = (cid - chunk0) * CH;
    const int t_end = min(cnt, t_begin + CH);

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
    float m_run = -__builtin_inff(), l_run = 0.f;
    float acc[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[hh][i] = 0.f;

    const int32_t* rws = L.rows ? list_rows(L, u) : nullptr;
    // K/V row of list entry idx (-1 past the chunk or for a token outside the sequence)
    auto row_of = [&](int idx) -> int {
      if (idx >= t_end) return -1;
      if (rws) return rws[idx];
      const int tok = toks[idx];
      if (tok < 0 || tok >= n) return -1;
      return (c.page_table[(size_t)b * c.maxP + (tok >> 4)] * c.Hkv + h) * kPage + (tok & 15);
    };
    int row_next = row_of(t_begin + lane);
    for (int sb = t_begin; sb < t_end; sb += 64) {
      const int row = row_next;  // K/V row index; rows < 2^31 is checked on the host
      const unsigned long long vmask = __ballot(row >= 0);

      bf16x8_t kv[4][4];
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        const int r = __shfl(row, tau * 16 + nn);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          kv[tau][kb] = (r >= 0) ? *reinterpret_cast<const bf16x8_t*>(c.k + (size_t)r * kD + kb * 32 + grp * 8)
                                 : bf16x8_t{};
      }
      uint4 vv[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int r = __shfl(row, grp + 4 * s);
        vv[s] = (r >= 0) ? *reinterpret_cast<const uint4*>(c.v + (size_t)r * kD + nn * 8) : make_uint4(0u, 0u, 0u, 0u);
      }
      row_next = row_of(sb + 64 + lane);  // next sub-block's rows load while this one computes

      floatx4_t sacc[4];
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        sacc[tau] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          sacc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[tau][kb], qv[kb], sacc[tau], 0, 0, 0);
      }

      // lane holds S[token tau*16 + 4*grp + e][head nn]
      float sv[16];
      float mx = -__builtin_inff();
#pragma unroll
      for (int tau = 0; tau < 4; ++tau)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = tau * 16 + 4 * grp + e;
          const float x = ((vmask >> t) & 1ull) ? sacc[tau][e] * sm_log2 : -__builtin_inff();
          sv[tau * 4 + e] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == -__builtin_inff()) ? 1.f : exp2f(m_run - m_new);
      float ps = 0.f;
      float pv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pv[i] = (sv[i] == -__builtin_inff()) ? 0.f : exp2f(sv[i] - m_new);
        ps += pv[i];
      }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      l_run = l_run * alpha + ps;
      m_run = m_new;
      if (nn < G) {
#pragma unroll
        for (int tau = 0; tau < 4; ++tau)
#pragma unroll
          for (int e = 0; e < 4; ++e) Pl[(tau * 16 + 4 * grp + e) * G + nn] = pv[tau * 4 + e];
        if (grp == 0) Al[nn] = alpha;
      }
      __syncthreads();
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float a = Al[hh];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[hh][i] *= a;
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int t = grp + 4 * s;
        const uint32_t w[4] = {vv[s].x, vv[s].y, vv[s].z, vv[s].w};
        float vf[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          vf[2 * i] = bf16_lo(w[i]);
          vf[2 * i + 1] = bf16_hi(w[i]);
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float pp = Pl[t * G + hh];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[hh][i] = fmaf(pp, vf[i], acc[hh][i]);
        }
      }
      __syncthreads();
    }

    // sum the four token groups
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float x = acc[hh][i];
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        acc[hh][i] = x;
      }
    float* part = partials + (size_t)cid * G * kPartStride;
    if (grp == 0) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float4* o4 = reinterpret_cast<float4*>(part + hh * kPartStride + 2 + nn * 8);
        o4[0] = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
        o4[1] = make_float4(acc[hh][4], acc[hh][5], acc[hh][6], acc[hh][7]);
      }
      if (nn < G) {
        part[nn * kPartStride] = m_run;
        part[nn * kPartStride + 1] = l_run;
      }
    }
    if (csr_tokens) {
      for (int i = t_begin + lane; i < t_end; i += 64)
        if (tok0 + i < capacity) csr_tokens[tok0 + i] = toks[i];
    }
  }
}

// One block per (unit, head), one thread per output dim: combine the unit's chunk partials in chunk
// order.  The per-chunk rescale factors are staged in LDS 128 chunks at a time so the output loads
// of many chunks are in flight together.
template <int G>
__global__ __launch_bounds__(128) void k_merge(CacheView c, ListView L, int CH, int max_chunks,
                                               const float* __restrict__ partials, float* out, float* lse) {
  const int u = blockIdx.x / G, hh = blockIdx.x - (blockIdx.x / G) * G;
  const int b = u / c.Hkv, h = u - b * c.Hkv;
  const int tid = threadIdx.x;
  __shared__ int s_c0, s_nch;
  __shared__ float sc[128];
  __shared__ float red[2 * 2 * 4];
  BlockReduce<2> br{red};
  if (tid < 64) {
    int acc = 0;
    for (int i = tid; i < u; i += 64) acc += (max(0, list_count(L, i)) + CH - 1) / CH;
    acc = wave_sum_int(acc);
    if (tid == 0) {
      s_c0 = acc;
      s_nch = (max(0, list_count(L, u)) + CH - 1) / CH;
    }
  }
  __syncthreads();
  const int c0 = s_c0;
  const int nch = max(0, min(s_nch, max_chunks - c0));
  const float* base = partials + ((size_t)c0 * G + hh) * kPartStride;
  constexpr size_t kStep = (size_t)G * kPartStride;
  float mloc = -__builtin_inff();
  for (int k = tid; k < nch; k += 128) mloc = fmaxf(mloc, base[k * kStep]);
  const float M = br.max(mloc);
  float lpart = 0.f, Os = 0.f;
  if (M != -__builtin_inff()) {
    for (int k0 = 0; k0 < nch; k0 += 128) {
      const int k = k0 + tid;
      float s = 0.f;
      if (k < nch) {
        s = exp2f(base[k * kStep] - M);
        lpart += base[k * kStep + 1] * s;
      }
      sc[tid] = s;
      __syncthreads();
      const int kn = min(128, nch - k0);
      const float* po = base + (size_t)k0 * kStep + 2 + tid;
#pragma unroll 16
      for (int i = 0; i < kn; ++i) Os += po[i * kStep] * sc[i];
      __syncthreads();
    }
  }
  const float Ls = br.sum(lpart);
  const size_t oh = (size_t)b * c.Hq + (size_t)h * G + hh;
  out[oh * kD + tid] = (Ls > 0.f) ? Os / Ls : 0.f;
  if (lse && tid == 0) lse[oh] = (Ls > 0.f) ? (M + log2f(Ls)) * 0.69314718055994530942f : -__builtin_inff();
}

int attn_chunk_tokens(int64_t total_upper) {
  int64_t sb = total_upper / (64 * 4096);
  int s = 1;
  while (s * 2 <= sb && s < 8) s *= 2;
  return 64 * s;
}

hipError_t launch_attn(const CacheView& c, const uint16_t* q, float sm, const ListView& list, int chunk_tokens,
                       int64_t max_chunks, float* partials, int32_t* csr_indptr, int32_t* csr_tokens,
                       int64_t capacity, hipStream_t s) {
  const float sm_log2 = sm * 1.44269504088896340736f;
  int64_t grid = max_chunks;
  const int64_t persistent = 256 * 8;
  if (grid > persistent) grid = persistent;
  if (grid < 1) grid = 1;
  switch (c.G) {
    case 1: hipLaunchKernelGGL(k_attn<1>, dim3((unsigned)grid), dim3(64), 0, s, c, q, sm_log2, list, chunk_tokens, (int)max_chunks, partials, csr_indptr, csr_tokens, capacity); break;
    case 2: hipLaunchKernelGGL(k_attn<2>, dim3((unsigned)grid), dim3(64), 0, s, c, q, sm_log2, list, chunk_tokens, (int)max_chunks, partials, csr_indptr, csr_tokens, capacity); break;
    case 4: hipLaunchKernelGGL(k_attn<4>, dim3((unsigned)grid), dim3(64), 0, s, c, q, sm_log2, list, chunk_tokens, (int)max_chunks, partials, csr_indptr, csr_tokens, capacity); break;
    case 8: hipLaunchKernelGGL(k_attn<8>, dim3((unsigned)grid), dim3(64), 0, s, c, q, sm_log2, list, chunk_tokens, (int)max_chunks, partials, csr_indptr, csr_tokens, capacity); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const CacheView& c, const ListView& list, int chunk_tokens, int64_t max_chunks,
                        const float* partials, float* out, float* lse, hipStream_t s) {
  dim3 grid((unsigned)(c.B * c.Hkv * c.G));
  switch (c.G) {
    case 1: hipLaunchKernelGGL(k_merge<1>, grid, dim3(128), 0, s, c, list, chunk_tokens, (int)max_chunks, partials, out, lse); break;
    case 2: hipLaunchKernelGGL(k_merge<2>, grid, dim3(128), 0, s, c, list, chunk_tokens, (int)max_chunks, partials, out, lse); break;
    case 4: hipLaunchKernelGGL(k_merge<4>, grid, dim3(128), 0, s, c, list, chunk_tokens, (int)max_chunks, partials, out, lse); break;
    case 8: hipLaunchKernelGGL(k_merge<8>, grid, dim3(128), 0, s, c, list, chunk_tokens, (int)max_chunks, partials, out, lse); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace twl
