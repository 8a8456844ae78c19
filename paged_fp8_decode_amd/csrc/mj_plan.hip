// Device-side split-KV planner: the same plan as the host planner
// (mjolnir-kernel README "What it does", step 1; wheel page
// mjolnir/runner.py, T5DecodeRunner.plan), computed by one workgroup from the
// device sequence lengths.  Because it reads only device memory, a hipGraph
// that captured [plan, quantize, decode, merge] replays later steps with new
// lengths and no host work at all (the host planner must run outside
// capture).
//
// Rule (identical to mj_plan_compute): tiles_i = ceil((L_i + margin) /
// kv_tile) with L_i clamped to [0, max_blocks * page_size] as the decode
// kernels clamp it; without a split each sequence is one item; with a split
// the chunk c is the smallest integer >= max(1, ceil(max tiles / max_splits))
// whose item count sum_i max(1, ceil(tiles_i / c)) fits the slots (a
// bisection over the monotone count); items are sequence-major, padded with
// (-1, 0, 0, 0) up to the buffer's capacity.
#include "mj_device.h"
#include "mj_internal.h"

namespace mj {

namespace {

constexpr int kPT = 1024;

__device__ __forceinline__ int block_reduce(int v, bool is_max, int* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int o = __shfl_xor(v, off, 64);
    v = is_max ? max(v, o) : v + o;
  }
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  int r = red[0];
  for (int i = 1; i < nw; ++i) r = is_max ? max(r, red[i]) : r + red[i];
  return r;
}

__global__ __launch_bounds__(kPT) void plan_kernel(PlanParams p) {
  __shared__ int red[kPT / 64];
  __shared__ int scan[kPT];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int64_t lmax = (int64_t)p.max_blocks * p.page_size;
  auto tiles = [&](int i) -> int64_t {
    const int64_t L = min<int64_t>(max<int64_t>(p.seq_lens[i], 0), lmax);
    return (L + p.margin + p.kv_tile - 1) / p.kv_tile;
  };
  int mt = 0;
  for (int i = tid; i < p.num_seqs; i += nt) mt = max(mt, (int)tiles(i));
  const int max_tiles = block_reduce(mt, true, red);

  int c = max(1, max_tiles);
  if (p.split) {
    int lo = max(1, (max_tiles + p.max_splits - 1) / p.max_splits);
    int hi = max(lo, max_tiles);
    while (lo < hi) {  // uniform across the workgroup
      const int mid = lo + (hi - lo) / 2;
      int cnt = 0;
      for (int i = tid; i < p.num_seqs; i += nt) cnt += max(1, (int)((tiles(i) + mid - 1) / mid));
      if (block_reduce(cnt, false, red) <= p.slots) hi = mid; else lo = mid + 1;
    }
    c = lo;
  }

  // per-thread contiguous run of sequences; exclusive scan of item counts
  const int per = (p.num_seqs + nt - 1) / nt;
  const int i0 = min(p.num_seqs, tid * per), i1 = min(p.num_seqs, i0 + per);
  int mine = 0;
  for (int i = i0; i < i1; ++i) mine += p.split ? max(1, (int)((tiles(i) + c - 1) / c)) : 1;
  scan[tid] = mine;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {  // Hillis-Steele inclusive scan
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const int total = scan[nt - 1];
  int wpos = scan[tid] - mine;
  for (int i = i0; i < i1; ++i) {
    const int t = (int)tiles(i);
    const int n = p.split ? max(1, (t + c - 1) / c) : 1;
    p.n_splits[i] = n;
    p.split_begin[i] = wpos;
    for (int s = 0; s < n; ++s, ++wpos) {
      const int b = p.split ? s * c : 0;
      const int e = p.split ? min((s + 1) * c, t) : t;
      int4* item = reinterpret_cast<int4*>(p.work) + wpos;
      *item = make_int4(i, b, e, s);
    }
  }
  for (int w = total + tid; w < p.cap_max; w += nt) reinterpret_cast<int4*>(p.work)[w] = make_int4(-1, 0, 0, 0);
  for (int i = p.num_seqs + tid; i < p.max_num_seqs; i += nt) {
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
