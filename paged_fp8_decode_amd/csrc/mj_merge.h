// Log-sum-exp merge of the split partials of one (sequence, KV head)
// (mjolnir-kernel README "What it does", step 4): with per-split row maxima
// m_s (log2 domain), sums l_s and unnormalised outputs o_s,
// M = max_s m_s, o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s and
// lse = ln 2 * (M + log2 sum_s 2^(m_s - M) l_s); a row no split saw (every
// m_s = -inf) gives o = 0 and lse = -inf.  Shared by the stand-alone merge
// kernel and the decode kernel's fused tail so both round identically.
#pragma once

#include "mj_device.h"
#include "mj_internal.h"

namespace mj {

// Device-coherent (agent-scope) accesses: the stores write through the XCD's
// L2 (the eight XCD L2s are not coherent with each other) and the loads
// bypass it, so a workgroup on another XCD sees the data without a
// whole-L2 writeback or invalidate.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// kCoherent: read the partials with device-coherent loads (the fused merge,
// which runs in the same launch that wrote them).
template <bool kCoherent>
__device__ __forceinline__ float ld_part(const float* p) {
  if constexpr (kCoherent) return load_coherent(p);
  else return *p;
}
template <bool kCoherent>
__device__ __forceinline__ float4 ld_part4(const float* p) {
  if constexpr (kCoherent) {
    return make_float4(load_coherent(p), load_coherent(p + 1), load_coherent(p + 2), load_coherent(p + 3));
  } else {
    return *reinterpret_cast<const float4*>(p);
  }
}

// Thread layout: 256 threads = 8 rows x 32 lanes of 4 channels; a thread
// takes rows (tid >> 5) + 8i, kRU of them at a time, and reads the splits in
// batches of kB: every load of a batch, for all kRU rows, is in flight at
// once (the merge is latency-bound: a memory round trip per row or split
// would dominate; kRU * kB * 6 registers hold a batch).  kB fixes the
// summation order, so every caller uses the same kB (bit-identical merges);
// kRU only groups independent rows.  Batches combine with the usual running-max rescale; a
// single batch (n <= kB) is exactly the two-pass formula above.
template <bool kCoherent, int kRU, int kB>
__device__ __forceinline__ void merge_one(const MergeParams& p, int seq, int g, int tid) {
  const int n = p.n_splits[seq];
  const int w0 = p.split_begin[seq];
  if (n <= 1 || w0 < 0 || w0 + n > p.part_items) return;
  const int c4 = (tid & 31) * 4;
  for (int r0 = tid >> 5; r0 < p.n_q; r0 += 8 * kRU) {
    float M[kRU], den[kRU];
    float4 num[kRU];
#pragma unroll
    for (int u = 0; u < kRU; ++u) {
      M[u] = -INFINITY;
      den[u] = 0.0f;
      num[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    for (int s0 = 0; s0 < n; s0 += kB) {
      float m[kRU][kB], l[kRU][kB];
      float4 o[kRU][kB];
#pragma unroll
      for (int u = 0; u < kRU; ++u) {
        const int r = r0 + 8 * u;
#pragma unroll
        for (int j = 0; j < kB; ++j) {
          if (r < p.n_q && s0 + j < n) {
            const int64_t idx = ((int64_t)(w0 + s0 + j) * p.h_k + g) * p.nqp + r;
            m[u][j] = ld_part<kCoherent>(&p.m_part[idx]);
            l[u][j] = ld_part<kCoherent>(&p.l_part[idx]);
            o[u][j] = ld_part4<kCoherent>(&p.o_part[idx * kHeadDim + c4]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kRU; ++u) {
        if (r0 + 8 * u >= p.n_q) continue;
        float bm = M[u];
#pragma unroll
        for (int j = 0; j < kB; ++j)
          if (s0 + j < n) bm = fmaxf(bm, m[u][j]);
        if (bm != -INFINITY) {
          const float sc = exp2f(M[u] - bm);  // 0 while nothing was seen (M = -inf)
          den[u] *= sc;
          num[u].x *= sc; num[u].y *= sc; num[u].z *= sc; num[u].w *= sc;
#pragma unroll
          for (int j = 0; j < kB; ++j) {
            if (s0 + j < n) {
              const float wt = exp2f(m[u][j] - bm);
              den[u] += wt * l[u][j];
              num[u].x += wt * o[u][j].x; num[u].y += wt * o[u][j].y;
              num[u].z += wt * o[u][j].z; num[u].w += wt * o[u][j].w;
            }
          }
          M[u] = bm;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kRU; ++u) {
      const int r = r0 + 8 * u;
      if (r >= p.n_q) continue;
      const bool seen = M[u] != -INFINITY;
      const int t = r / p.h_r;
      const int h = g * p.h_r + (r - t * p.h_r);
      const float dn = den[u];
      const float o0 = seen ? num[u].x / dn : 0.0f, o1 = seen ? num[u].y / dn : 0.0f;
      const float o2 = seen ? num[u].z / dn : 0.0f, o3 = seen ? num[u].w / dn : 0.0f;
      const int64_t oi = ((int64_t)seq * p.q_len + t) * p.out_ts + (int64_t)h * p.out_hs + c4;
      if (p.out_f32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + oi) = make_float4(o0, o1, o2, o3);
      } else {
        const uint32_t b0 = f32_to_bf16(o0), b1 = f32_to_bf16(o1), b2 = f32_to_bf16(o2), b3 = f32_to_bf16(o3);
        *reinterpret_cast<uint2*>(p.out + oi) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
      }
      if (c4 == 0 && p.lse)
        p.lse[((int64_t)seq * p.q_len + t) * p.h_q + h] = seen ? (M[u] + log2f(dn)) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace mj
