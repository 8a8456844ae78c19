// Device-side split-KV planner: the same plan as the host planner
// (mjolnir-kernel README "What it does", step 1; wheel page
// mjolnir/runner.py, T5DecodeRunner.plan), computed by one workgroup from the
// device sequence lengths.  Because it reads only device memory, a hipGraph
// that captured [plan, decode step] replays later steps with new lengths and
// no host work at all (the host planner must run outside capture).
//
// Rule (identical to mj_plan_compute): tiles_i = ceil(min(L_i + margin,
// lmax) / kv_tile) with L_i clamped to [0, lmax], lmax = max_blocks *
// page_size, as the decode kernels clamp it; without a split each sequence is one item; with a split
// the chunk c is the smallest integer >= max(1, ceil(max tiles / max_splits),
// min_chunk) whose item count sum_i max(1, ceil(tiles_i / c)) fits the slots (a
// bisection over the monotone count); items are sequence-major, padded with
// (-1, 0, 0, 0) up to the buffer's capacity.
//
// Latency, not bandwidth, is what this kernel costs: the lengths are read
// from memory once into LDS (up to kCache sequences; beyond that they are
// re-read per bisection round), the reductions and the item-count scan are
// wave64 shuffles plus one LDS exchange between the four waves.
#include "mj_device.h"
#include "mj_internal.h"

namespace mj {

namespace {

constexpr int kPT = 256;
constexpr int kPW = kPT / 64;
constexpr int kCache = 8192;

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  return v;
}

// Sum (or max) over the workgroup; red holds kPW ints and is reused, so the
// leading barrier keeps a previous call's readers ahead of this call's writers.
__device__ __forceinline__ int block_sum(int v, int* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int i = 0; i < kPW; ++i) r += red[i];
  return r;
}
__device__ __forceinline__ int block_max(int v, int* red) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = red[0];
#pragma unroll
  for (int i = 1; i < kPW; ++i) r = max(r, red[i]);
  return r;
}

__global__ __launch_bounds__(kPT) void plan_kernel(PlanParams p) {
  __shared__ int tl[kCache];
  __shared__ int red[kPW];
  __shared__ int wsum[kPW];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int64_t lmax = (int64_t)p.max_blocks * p.page_size;
  const bool cached = p.num_seqs <= kCache;
  auto tiles_mem = [&](int i) -> int {  // the length plus the margin, never past the table row
    const int64_t L = min<int64_t>(max<int64_t>(p.seq_lens[i], 0), lmax);
    return (int)((min<int64_t>(L + p.margin, lmax) + p.kv_tile - 1) / p.kv_tile);
  };
  auto tiles = [&](int i) -> int { return cached ? tl[i] : tiles_mem(i); };

  int mt = 0;
  for (int i = tid; i < p.num_seqs; i += kPT) {
    const int t = tiles_mem(i);
    if (cached) tl[i] = t;
    mt = max(mt, t);
  }
  const int max_tiles = block_max(mt, red);  // its barriers also publish tl[]

  int c = max(1, max_tiles);
  if (p.split) {
    int lo = max(max(1, (max_tiles + p.max_splits - 1) / p.max_splits), p.min_chunk);
    int hi = max(lo, max_tiles);
    while (lo < hi) {  // uniform across the workgroup
      const int mid = lo + (hi - lo) / 2;
      int cnt = 0;
      for (int i = tid; i < p.num_seqs; i += kPT) cnt += max(1, (tiles(i) + mid - 1) / mid);
      if (block_sum(cnt, red) <= p.slots) hi = mid; else lo = mid + 1;
    }
    c = lo;
  }

  // per-thread contiguous run of sequences; exclusive scan of item counts
  const int per = (p.num_seqs + kPT - 1) / kPT;
  const int i0 = min(p.num_seqs, tid * per), i1 = min(p.num_seqs, i0 + per);
  int mine = 0;
  for (int i = i0; i < i1; ++i) mine += p.split ? max(1, (tiles(i) + c - 1) / c) : 1;
  int incl = mine;  // inclusive scan within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kPW; ++i) {
    base += i < wv ? wsum[i] : 0;
    total += wsum[i];
  }
  int wpos = base + incl - mine;
  for (int i = i0; i < i1; ++i) {
    const int t = tiles(i);
    const int n = p.split ? max(1, (t + c - 1) / c) : 1;
    p.n_splits[i] = n;
    p.split_begin[i] = wpos;
    for (int s = 0; s < n; ++s, ++wpos) {
      const int b = p.split ? s * c : 0;
      const int e = p.split ? min((s + 1) * c, t) : t;
      reinterpret_cast<int4*>(p.work)[wpos] = make_int4(i, b, e, s);
    }
  }
  for (int w = total + tid; w < p.cap_max; w += kPT) reinterpret_cast<int4*>(p.work)[w] = make_int4(-1, 0, 0, 0);
  for (int i = p.num_seqs + tid; i < p.max_num_seqs; i += kPT) {
    p.n_splits[i] = 1;
    p.split_begin[i] = 0;
  }
}

}  // namespace

hipError_t launch_plan(const PlanParams& p, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPT), 0, s, p);
  return hipGetLastError();
}

}  // namespace mj
