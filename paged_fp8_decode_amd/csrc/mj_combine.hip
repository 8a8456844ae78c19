// Context-parallel combine: the per-slice decode results (fp32 O normalized
// over each slice, and its log-sum-exp) merged into the whole context's
// output.
//
// Method: the log-sum-exp merge of the mjolnir-kernel README ("What it
// does", step 4) applied to the slices of a context-parallel group rather
// than to the splits of one GPU's plan: with M = max_p lse_p and
// w_p = exp(lse_p - M), out = sum_p w_p o_p / sum_p w_p and
// lse = M + ln sum_p w_p.
#include "mj_device.h"
#include "mj_internal.h"

namespace mj {

namespace {

constexpr int kCThreads = 256;

// One thread per (token, query head, 4 channels): 32 threads cover a row.
// Slices are taken kB at a time with all their loads issued together; a
// running maximum rescales the sums between batches (one batch, every group
// of up to kB GPUs, is exactly the formula above).
constexpr int kB = 8;

__global__ __launch_bounds__(kCThreads) void combine_kernel(CombineParams p) {
  const int64_t tid = (int64_t)blockIdx.x * kCThreads + threadIdx.x;
  const int64_t rows_h = (int64_t)p.rows * p.h_q;
  if (tid >= rows_h * 32) return;
  const int64_t rh = tid >> 5;
  const int c4 = (int)(tid & 31) * 4;
  const int t = (int)(rh / p.h_q), h = (int)(rh - (int64_t)t * p.h_q);
  float M = -INFINITY, den = 0.0f;
  float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int q0 = 0; q0 < p.parts; q0 += kB) {
    float l[kB];
    float4 o[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int q = q0 + j;
      l[j] = q < p.parts ? p.plse[((int64_t)q * p.rows + t) * p.h_q + h] : -INFINITY;
      o[j] = q < p.parts ? *reinterpret_cast<const float4*>(p.po + q * p.p_ps + t * p.p_ts + h * p.p_hs + c4)
                         : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    float bm = M;
#pragma unroll
    for (int j = 0; j < kB; ++j) bm = fmaxf(bm, l[j]);
    if (bm == -INFINITY) continue;  // no slice so far saw a key of this row
    const float a = expf(M - bm);   // M = -inf -> 0
    den *= a;
    num.x *= a;
    num.y *= a;
    num.z *= a;
    num.w *= a;
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      if (l[j] == -INFINITY) continue;  // the slice saw no key of this row (its O is 0)
      const float w = expf(l[j] - bm);
      den += w;
      num.x += w * o[j].x;
      num.y += w * o[j].y;
      num.z += w * o[j].z;
      num.w += w * o[j].w;
    }
    M = bm;
  }
  const bool seen = M != -INFINITY;
  const float o0 = seen ? num.x / den : 0.0f, o1 = seen ? num.y / den : 0.0f;
  const float o2 = seen ? num.z / den : 0.0f, o3 = seen ? num.w / den : 0.0f;
  const int64_t oi = (int64_t)t * p.out_ts + (int64_t)h * p.out_hs + c4;
  if (p.out_f32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + oi) = make_float4(o0, o1, o2, o3);
  } else {
    const uint32_t b0 = f32_to_bf16(o0), b1 = f32_to_bf16(o1), b2 = f32_to_bf16(o2), b3 = f32_to_bf16(o3);
    *reinterpret_cast<uint2*>(p.out + oi) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
  }
  if (c4 == 0 && p.lse) p.lse[(int64_t)t * p.h_q + h] = seen ? M + logf(den) : -INFINITY;
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  const int64_t threads = (int64_t)p.rows * p.h_q * 32;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((threads + kCThreads - 1) / kCThreads)), dim3(kCThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mj
