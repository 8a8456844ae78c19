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

// Thread layout: 256 threads = 8 rows x 32 lanes of 4 channels; rows
// (tid >> 5), (tid >> 5) + 8, ...  The splits are read in batches of kB with
// every load of a batch in flight at once (the merge is latency-bound: a
// loop that waits on each partial in turn costs a memory round trip per
// split and row).  Batches combine with the usual running-max rescale; a
// single batch (n <= kB) is exactly the two-pass formula above.
template <bool kCoherent>
__device__ __forceinline__ void merge_one(const MergeParams& p, int seq, int g, int tid) {
  constexpr int kB = 16;
  const int n = p.n_splits[seq];
  const int w0 = p.split_begin[seq];
  if (n <= 1 || w0 < 0 || w0 + n > p.part_items) return;
  const int c4 = (tid & 31) * 4;
  for (int r = tid >> 5; r < p.n_q; r += 8) {
    float M = -INFINITY, den = 0.0f;
    float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int s0 = 0; s0 < n; s0 += kB) {
      float m[kB], l[kB];
      float4 o[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        if (s0 + j < n) {
          const int64_t idx = ((int64_t)(w0 + s0 + j) * p.h_k + g) * p.nqp + r;
          m[j] = ld_part<kCoherent>(&p.m_part[idx]);
          l[j] = ld_part<kCoherent>(&p.l_part[idx]);
          o[j] = ld_part4<kCoherent>(&p.o_part[idx * kHeadDim + c4]);
        }
      }
      float bm = M;
#pragma unroll
      for (int j = 0; j < kB; ++j)
        if (s0 + j < n) bm = fmaxf(bm, m[j]);
      if (bm != -INFINITY) {
        const float sc = exp2f(M - bm);  // 0 while nothing was seen (M = -inf)
        den *= sc;
        num.x *= sc; num.y *= sc; num.z *= sc; num.w *= sc;
#pragma unroll
        for (int j = 0; j < kB; ++j) {
          if (s0 + j < n) {
            const float wt = exp2f(m[j] - bm);
            den += wt * l[j];
            num.x += wt * o[j].x; num.y += wt * o[j].y; num.z += wt * o[j].z; num.w += wt * o[j].w;
          }
        }
        M = bm;
      }
    }
    const bool seen = M != -INFINITY;
    const int t = r / p.h_r;
    const int h = g * p.h_r + (r - t * p.h_r);
    const uint32_t b0 = f32_to_bf16(seen ? num.x / den : 0.0f), b1 = f32_to_bf16(seen ? num.y / den : 0.0f);
    const uint32_t b2 = f32_to_bf16(seen ? num.z / den : 0.0f), b3 = f32_to_bf16(seen ? num.w / den : 0.0f);
    *reinterpret_cast<uint2*>(p.out + ((int64_t)seq * p.q_len + t) * p.out_ts + (int64_t)h * p.out_hs + c4) =
        make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    if (c4 == 0 && p.lse) p.lse[((int64_t)seq * p.q_len + t) * p.h_q + h] = seen ? (M + log2f(den)) * kLn2 : -INFINITY;
  }
}

}  // namespace mj
