// Dynamic e4m3 quantization of Q per (sequence, KV head), one workgroup per
// (sequence, KV head).
//
// Definition (mjolnir-kernel wheel page mjolnir/runner.py,
// T5DecodeRunner.run, fp8-Q branch; README "What it does", step 2): over the
// q_len tokens and h_r query heads of KV head g, x = fp32(q) [* q_mul],
// amax = max(max|x|, 1e-6f), s = amax / 448, code = e4m3(x / s), rows packed
// t*h_r + r.  Every operation is one IEEE fp32 operation: the amax is exact,
// the divisions are correctly rounded (built with
// -fhip-fp32-correctly-rounded-divide-sqrt, never a reciprocal multiply) and
// the e4m3 rounding is done in integer arithmetic, so the codes are
// bit-identical to any other correct evaluation of the definition.
//
// Q is tiny (n_q x 128 values per workgroup), so the kernel simply reads it
// twice (amax pass, quantize pass) with 16-byte loads of 8 bf16 values.
#include "mj_device.h"
#include "mj_internal.h"

namespace mj {

namespace {

constexpr int kQThreads = 256;

__global__ __launch_bounds__(kQThreads) void qquant_kernel(QQuantParams p) {
  const int seq = blockIdx.x;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int nvec = p.n_q * 16;
  __shared__ float red[kQThreads / 64];

  float amax = 0.0f;
  for (int v = tid; v < nvec; v += kQThreads) {
    float x[8];
    q_load8(p.q, p.q_ts, p.q_hs, p.q_mul, p.q_len, p.h_r, seq, g, v >> 4, (v & 15) * 8, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
  }
  // wave64 max, then across the four waves
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  const float s = q_scale_from_amax(amax);
  const float rs = 1.0f / s;
  uint8_t* dst = p.q8 + ((int64_t)seq * p.h_k + g) * p.n_q * kHeadDim;
  for (int v = tid; v < nvec; v += kQThreads) {
    const int row = v >> 4, c0 = (v & 15) * 8;
    float x[8];
    q_load8(p.q, p.q_ts, p.q_hs, p.q_mul, p.q_len, p.h_r, seq, g, row, c0, x);
    *reinterpret_cast<uint2*>(dst + (int64_t)row * kHeadDim + c0) = q_codes8(x, s, rs);
  }
  if (tid == 0) p.q_descale[(int64_t)seq * p.h_k + g] = s;
}

}  // namespace

hipError_t launch_qquant(const QQuantParams& p, hipStream_t s) {
  hipLaunchKernelGGL(qquant_kernel, dim3(p.num_seqs, p.h_k), dim3(kQThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mj
