// Generic paged decode kernel: any n_q (row tiles of up to 64 query rows),
// both KV formats, causal or not.  One workgroup of 256 threads per (plan
// item, KV head, row tile).  It stages 32-token K/V tiles through LDS as fp32
// and runs a textbook online softmax; it is the simple, always-correct path
// the specialised streaming kernels are checked against and fall back to.
//
// Method (mjolnir-kernel README "What it does", steps 3-4; wheel page
// mjolnir/runner.py, T5DecodeRunner.run): keys come from pages through the
// block table and the pool's byte strides; logits are
// softmax_scale * q_descale * k_descale * sum_c dec(q)dec(k), kept in log2
// units (exp2) internally; a sequence with one plan item writes bf16 O and
// the natural-log LSE, a split sequence writes fp32 partials (O unnormalised,
// running max in log2 units, running sum) for the merge.
#include "mj_device.h"
#include "mj_internal.h"
#include "mj_merge.h"

namespace mj {

namespace {

constexpr int kThreads = 256;
constexpr int kKT = 32;  // tokens per LDS tile
constexpr int kRT = 64;  // query rows per workgroup

template <int FMT>
__device__ __forceinline__ void load_row16(const uint8_t* row, int chunk, float out[16]) {
  if constexpr (FMT == 0) {  // e4m3: 16 bytes at chunk*16
    const uint4 raw = *reinterpret_cast<const uint4*>(row + chunk * 16);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 16; ++e) out[e] = e4m3_raw((w[e >> 2] >> (8 * (e & 3))) & 0xFFu);
  } else if constexpr (FMT >= 3) {  // e2m1 (nvfp4 codes): 8 bytes at chunk*8, code e in nibble e
    const uint2 raw = *reinterpret_cast<const uint2*>(row + chunk * 8);
#pragma unroll
    for (int e = 0; e < 16; ++e) out[e] = e2m1_raw(((e < 8 ? raw.x : raw.y) >> (4 * (e & 7))) & 0xFu);
  } else {  // e2m3 / e3m2: 12 bytes at chunk*12 hold codes 16*chunk .. 16*chunk+15
    const uint32_t* src = reinterpret_cast<const uint32_t*>(row + chunk * 12);
    uint32_t c[16];
    unpack16_6bit(src[0], src[1], src[2], c);
#pragma unroll
    for (int e = 0; e < 16; ++e) out[e] = FMT == 1 ? e2m3_raw(c[e]) : e3m2_raw(c[e]);
  }
}

// Power of two that turns a format's raw decode into its value.
// (nvfp4: applied per 16-channel chunk together with the block scale)
template <int FMT>
constexpr float fmt_rescale() {
  return FMT == 0 ? kE4m3Rescale : FMT == 1 ? kE2m3Rescale : FMT == 2 ? kE3m2Rescale : FMT == 3 ? kE2m1Rescale : 1.0f;
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void decode_generic_kernel(DecodeParams p) {
  __shared__ float q_s[kRT][kHeadDim];
  __shared__ float k_s[kKT][kHeadDim + 1];
  __shared__ float v_s[kKT][kHeadDim];
  __shared__ float s_s[kRT][kKT + 1];
  __shared__ float m_s[kRT], l_s[kRT], a_s[kRT];
  __shared__ int ok_s[kKT];

  const int w = blockIdx.x;
  const int g = blockIdx.y % p.h_k;
  const int rt = blockIdx.y / p.h_k;
  const int tid = threadIdx.x;
  const int seq = p.work[4 * w];
  if (seq < 0 || seq >= p.num_seqs) return;
  const int row0 = rt * kRT;
  const int nr = min(kRT, p.n_q - row0);
  if (nr <= 0) return;

  int L = p.seq_lens[seq];
  L = max(0, min(L, p.max_blocks * p.page_size));
  const int j0 = p.work[4 * w + 1] * p.kv_tile;
  const int j1 = min(p.work[4 * w + 2] * p.kv_tile, L);
  const bool single = p.n_splits[seq] <= 1;
  const bool causal = p.causal && p.q_len > 1;
  const int lim0 = L - p.q_len;  // causal: token t sees keys j <= lim0 + t

  const float rescale = fmt_rescale<FMT>();
  const float qs = (p.q_bf16 ? 1.0f : p.q_descale[(int64_t)seq * p.h_k + g]) * p.scale_log2;
  const float kd = load_descale(p.kd, p.kd_kind, seq, g, p.h_k) * rescale;
  const float vd = load_descale(p.vd, p.vd_kind, seq, g, p.h_k) * rescale;
  if (p.q_bf16) {  // bf16 Q as is: packed row t*h_r + r is query head g*h_r + r of token t
    for (int e = tid; e < nr * kHeadDim; e += kThreads) {
      const int r = row0 + (e >> 7), t = r / p.h_r;
      const int64_t tok = (int64_t)seq * p.q_len + t, h = (int64_t)g * p.h_r + (r - t * p.h_r);
      q_s[e >> 7][e & 127] = __uint_as_float((uint32_t)p.qb[tok * p.qb_ts + h * p.qb_hs + (e & 127)] << 16) * qs;
    }
  } else {
    const uint8_t* qsrc = p.q8 + (((int64_t)seq * p.h_k + g) * p.n_q + row0) * kHeadDim;
    for (int e = tid; e < nr * kHeadDim; e += kThreads) q_s[e >> 7][e & 127] = e4m3_value(qsrc[e]) * qs;
  }
  if (tid < kRT) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.0f;
  }
  const int32_t* bt_row = p.bt + (int64_t)seq * p.bt_stride;
  const int c = tid & 127;
  const int rb = tid >> 7;
  float acc[kRT / 2];
#pragma unroll
  for (int k = 0; k < kRT / 2; ++k) acc[k] = 0.0f;
  __syncthreads();

  for (int t0 = j0; t0 < j1; t0 += kKT) {
    {  // K and V tile: thread -> (token, 16-value chunk)
      const int tok = tid >> 3, ch = tid & 7;
      const int j = t0 + tok;
      float kv[16], vv[16];
      bool ok = j < j1;
      int64_t pg = -1;
      if (ok) {
        pg = page_of(bt_row, j, p.page_shift, p.num_pages);
        ok = pg >= 0;
      }
      if (ok) {
        const int slot = j & (p.page_size - 1);
        load_row16<FMT>(p.k + kv_offset(pg, slot, g, p.k_sp, p.k_ss, p.k_sh), ch, kv);
        load_row16<FMT>(p.v + kv_offset(pg, slot, g, p.v_sp, p.v_ss, p.v_sh), ch, vv);
        if constexpr (FMT == 4) {  // nvfp4: chunk ch is block ch; e2m1 value times its e4m3 scale (exact)
          const float ksf = e4m3_value(p.ksb[kv_offset(pg, slot, g, p.ksb_sp, p.ksb_ss, p.ksb_sh) + ch]);
          const float vsf = e4m3_value(p.vsb[kv_offset(pg, slot, g, p.vsb_sp, p.vsb_ss, p.vsb_sh) + ch]);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            kv[e] = kv[e] * kE2m1Rescale * ksf;
            vv[e] = vv[e] * kE2m1Rescale * vsf;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) kv[e] = vv[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        k_s[tok][ch * 16 + e] = kv[e] * kd;
        v_s[tok][ch * 16 + e] = vv[e] * vd;
      }
      if (ch == 0) ok_s[tok] = ok;
    }
    __syncthreads();
    {  // logits (log2 units), masked
      const int tok = tid & 31, rg = tid >> 5;
      const int j = t0 + tok;
      for (int r = rg; r < nr; r += 8) {
        float s = 0.0f;
#pragma unroll 16
        for (int cc = 0; cc < kHeadDim; ++cc) s += q_s[r][cc] * k_s[tok][cc];
        const int t = (row0 + r) / p.h_r;
        const bool vis = ok_s[tok] && (!causal || j <= lim0 + t);
        s_s[r][tok] = vis ? s : -INFINITY;
      }
    }
    __syncthreads();
    if (tid < nr) {  // online softmax row update
      const float m_old = m_s[tid];
      float mx = m_old;
      for (int j = 0; j < kKT; ++j) mx = fmaxf(mx, s_s[tid][j]);
      float alpha = 1.0f, sum = 0.0f;
      if (mx != -INFINITY) {
        alpha = exp2f(m_old - mx);  // m_old = -inf -> 0
        for (int j = 0; j < kKT; ++j) {
          const float pj = exp2f(s_s[tid][j] - mx);  // -inf -> 0
          s_s[tid][j] = pj;
          sum += pj;
        }
      } else {
        for (int j = 0; j < kKT; ++j) s_s[tid][j] = 0.0f;
      }
      l_s[tid] = l_s[tid] * alpha + sum;
      m_s[tid] = mx;
      a_s[tid] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kRT / 2; ++k) {
      const int r = rb + 2 * k;
      if (r < nr) {
        float o = acc[k] * a_s[r];
#pragma unroll 8
        for (int j = 0; j < kKT; ++j) o += s_s[r][j] * v_s[j][c];
        acc[k] = o;
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int k = 0; k < kRT / 2; ++k) {
    const int r = rb + 2 * k;
    if (r >= nr) continue;
    const int row = row0 + r;
    const int t = row / p.h_r;
    const int h = g * p.h_r + (row - t * p.h_r);
    const float om = p.o_mul ? p.o_mul[(int64_t)h * kHeadDim + c] : 1.0f;
    const float l = l_s[r];
    if (single) {
      const float o = l > 0.0f ? acc[k] / l * om : 0.0f;
      store_out(p.out, p.out_f32, ((int64_t)seq * p.q_len + t) * p.out_ts + (int64_t)h * p.out_hs + c, o);
      if (c == 0 && p.lse) p.lse[((int64_t)seq * p.q_len + t) * p.h_q + h] = l > 0.0f ? (m_s[r] + log2f(l)) * kLn2 : -INFINITY;
    } else if (w < p.part_items) {
      const int64_t idx = ((int64_t)w * p.h_k + g) * p.nqp + row;
      p.o_part[idx * kHeadDim + c] = acc[k] * om;
      if (c == 0) {
        p.m_part[idx] = m_s[r];
        p.l_part[idx] = l;
      }
    }
  }
}

// Log-sum-exp merge of split partials: one workgroup per (sequence, KV head).
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeParams p) {
  merge_one<false, 4, 8>(p, blockIdx.x, blockIdx.y, threadIdx.x);
}

// Probe: dense copy of one (sequence, head)'s codes through the same
// page / slot / stride arithmetic the decode kernels use.
__global__ void gather_kernel(GatherParams p) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)p.seq_len * p.row_bytes) return;
  const int j = (int)(e / p.row_bytes);
  const int b = (int)(e - (int64_t)j * p.row_bytes);
  const int64_t pg = page_of(p.bt + (int64_t)p.seq * p.bt_stride, j, p.page_shift, p.num_pages);
  const int page_size = 1 << p.page_shift;
  p.out[e] = pg < 0 ? 0 : p.pool[kv_offset(pg, j & (page_size - 1), p.head, p.sp, p.ss, p.sh) + b];
}

// Probe: the kernels' code decoders on raw codes.
__global__ void decode_codes_kernel(int fmt, const uint8_t* codes, int n, float* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (fmt == 16) {  // e4m3 through the bf16 operand converter of the bf16-Q kernel
    uint32_t h[2];
    e4m3x4_to_bf16(codes[i], h);
    out[i] = __uint_as_float(h[0] << 16);
    return;
  }
  const uint32_t c = codes[i];
  out[i] = fmt == 0 ? e4m3_value(c) : fmt == 1 ? e2m3_value(c & 63u) : fmt == 2 ? e3m2_value(c & 63u) : e2m1_value(c & 15u);
}

}  // namespace

hipError_t launch_decode_generic(const DecodeParams& p, int kv_format, int row_tiles, hipStream_t s) {
  const dim3 grid(p.num_work, p.h_k * row_tiles);
  switch (kv_format) {
    case 0: hipLaunchKernelGGL(decode_generic_kernel<0>, grid, dim3(kThreads), 0, s, p); break;
    case 1: hipLaunchKernelGGL(decode_generic_kernel<1>, grid, dim3(kThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL(decode_generic_kernel<2>, grid, dim3(kThreads), 0, s, p); break;
    case 3: hipLaunchKernelGGL(decode_generic_kernel<3>, grid, dim3(kThreads), 0, s, p); break;
    default: hipLaunchKernelGGL(decode_generic_kernel<4>, grid, dim3(kThreads), 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3(p.num_seqs, p.h_k), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.seq_len * p.row_bytes;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_decode_codes(int kv_format, const uint8_t* codes, int n, float* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_codes_kernel, dim3((n + 255) / 256), dim3(256), 0, s, kv_format, codes, n, out);
  return hipGetLastError();
}

}  // namespace mj

namespace mj {
namespace {

// Probe: read `n16` 16-byte words with non-temporal loads and fold them into
// one xor checksum per workgroup (a plain HBM streaming read, the practical
// bandwidth ceiling the decode kernels are compared with).
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* src, int64_t n16, uint32_t* out) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    const u4 v = __builtin_nontemporal_load(reinterpret_cast<const u4*>(src) + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* out, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const uint4*>(src), bytes / 16, out);
  return hipGetLastError();
}

}  // namespace mj
