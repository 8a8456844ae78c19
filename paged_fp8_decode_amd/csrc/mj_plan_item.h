// One wave's view of the split-KV plan: the item a decode workgroup serves,
// derived from the device lengths by the same rule as the host and device
// planners (mjolnir-kernel README "What it does", step 1; wheel listing
// mjolnir/runner.py, T5DecodeRunner.plan): tiles_i = ceil(min(clamped L_i +
// margin, lmax) / kv_tile); without a split, item w is sequence w; with a split the
// chunk c is the smallest integer >= max(1, ceil(max tiles / max_splits),
// min_chunk) whose item count sum_i max(1, ceil(tiles_i / c)) fits the slots,
// and items run sequence-major.  Wave-level only (shuffles, ballots, no LDS
// and no barrier); up to kPlanSeqsPerLane * 64 sequences.
#pragma once

#include "mj_device.h"
#include "mj_internal.h"

#include <climits>

namespace mj {

constexpr int kPlanSeqsPerLane = 4;
static_assert(64 * kPlanSeqsPerLane == kPlanMaxSeqs, "the host's limit is the lanes' capacity");

struct PlanItem {
  int seq;    // -1: padding
  int tb, te; // tile range
  int split;  // split index within the sequence
  int n;      // splits of the sequence
  int begin;  // index of the sequence's first item
};

// ceil(a / b) for 0 <= a, 1 <= b, a + b < 2^23: a float quotient corrected
// by integer remainders (the float error is below one unit there).
__device__ __forceinline__ int ceil_div_small(int a, int b) {
  const int num = a + b - 1;
  int q = (int)((float)num * __builtin_amdgcn_rcpf((float)b));
  int r = num - q * b;
  q += (r >= b) - (r < 0);
  r = num - q * b;
  q += (r >= b) - (r < 0);
  return q;
}

// Inclusive scan over the 64 lanes with DPP lane moves (no LDS round trip):
// row_shr 1, 2, 4, 8 scan each row of 16 lanes; row_bcast 15 then 31 carry
// each row's total into the rows above it.  Lanes a move has no source for
// (or whose row the mask leaves out) take the identity.
template <bool kMax>
__device__ __forceinline__ int wave_scan_i(int x) {
  const int id = kMax ? INT_MIN : 0;
  auto op = [](int a, int b) { return kMax ? max(a, b) : a + b; };
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x118, 0xf, 0xf, false));  // row_shr:8
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x142, 0xa, 0xf, false));  // row_bcast:15 into rows 1, 3
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x143, 0xc, 0xf, false));  // row_bcast:31 into rows 2, 3
  return x;
}
__device__ __forceinline__ int wave_sum_i(int v) { return __builtin_amdgcn_readlane(wave_scan_i<false>(v), 63); }
__device__ __forceinline__ int wave_max_i(int v) { return __builtin_amdgcn_readlane(wave_scan_i<true>(v), 63); }

// All lanes of the wave call this with the same arguments and get the same
// item.  lmax = max_blocks * page_size (lengths are clamped to [0, lmax]).
__device__ __forceinline__ PlanItem plan_item_wave(const int32_t* seq_lens, int num_seqs, int w, int margin,
                                                   int kv_tile, int64_t lmax, int max_splits, int slots, bool split,
                                                   int min_chunk) {
  const int lane = threadIdx.x & 63;
  auto tiles_of = [&](int i) -> int {  // the length plus the margin, never past the table row
    const int64_t L = min<int64_t>(max<int64_t>(seq_lens[i], 0), lmax);
    return (int)((min<int64_t>(L + margin, lmax) + kv_tile - 1) / kv_tile);
  };
  PlanItem it;
  if (!split) {
    it.seq = w < num_seqs ? w : -1;
    it.tb = 0;
    it.te = w < num_seqs ? tiles_of(w) : 0;
    it.split = 0;
    it.n = 1;
    it.begin = w;
    return it;
  }
  int t[kPlanSeqsPerLane];
  int mt = 0;
#pragma unroll
  for (int k = 0; k < kPlanSeqsPerLane; ++k) {
    const int i = lane + 64 * k;
    t[k] = i < num_seqs ? tiles_of(i) : -1;  // -1: no sequence
    mt = max(mt, t[k]);
  }
  const int max_tiles = wave_max_i(mt);
  int lo = max(max(1, (max_tiles + max_splits - 1) / max_splits), min_chunk);
  int hi = max(lo, max_tiles);
  it.seq = -1;
  it.tb = it.te = it.split = it.begin = 0;
  it.n = 1;
  {
    // the count falls as the chunk grows, so the count at the smallest
    // allowed chunk bounds the real one: workgroups past it (the padding of
    // the fixed grid) leave after one pass over the lengths
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kPlanSeqsPerLane; ++k) cnt += t[k] >= 0 ? max(1, ceil_div_small(t[k], lo)) : 0;
    if (w >= min(slots, wave_sum_i(cnt))) return it;
  }
  while (lo < hi) {  // wave-uniform
    const int mid = lo + (hi - lo) / 2;
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kPlanSeqsPerLane; ++k) cnt += t[k] >= 0 ? max(1, ceil_div_small(t[k], mid)) : 0;
    if (wave_sum_i(cnt) <= slots) hi = mid; else lo = mid + 1;
  }
  const int c = lo;
  int carry = 0;
#pragma unroll
  for (int k = 0; k < kPlanSeqsPerLane; ++k) {
    const int nk = t[k] >= 0 ? max(1, ceil_div_small(t[k], c)) : 0;
    const int incl = wave_scan_i<false>(nk);  // inclusive scan over the lanes
    const int beg = carry + incl - nk;
    const bool hit = nk > 0 && beg <= w && w < beg + nk;
    const uint64_t m = __builtin_amdgcn_ballot_w64(hit);
    if (m != 0) {
      const int src = __builtin_ctzll(m);
      it.seq = src + 64 * k;
      it.begin = __builtin_amdgcn_readlane(beg, src);
      it.n = __builtin_amdgcn_readlane(nk, src);
      const int tk = __builtin_amdgcn_readlane(t[k], src);
      it.split = w - it.begin;
      it.tb = it.split * c;
      it.te = min((it.split + 1) * c, tk);
    }
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  return it;
}

}  // namespace mj
