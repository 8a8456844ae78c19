// Draft-step advance: the cache slots of the tokens a draft step appends,
// and the device lengths advanced in place.
//
// Method (mjolnir-kernel wheel listing mjolnir/runner.py, T5DecodeRunner.plan
// and its `margin`; mjolnir/backend.py, the builder's comment on fused
// multi-step draft decode): the plan is made `margin` tokens long once, and
// every draft step runs on it while the speculator advances the device
// seq_lens; the decode kernels mask with the live lengths.  This kernel is
// that advance, so that the whole loop stays on the device and in one graph.
#include "mj_internal.h"

namespace mj {

namespace {

constexpr int kDThreads = 256;

// One thread per sequence: it reads the old length once, writes the q_len
// slots, then the new length (no other thread touches the sequence).
__global__ __launch_bounds__(kDThreads) void draft_advance_kernel(DraftParams p) {
  const int i = blockIdx.x * kDThreads + threadIdx.x;
  if (i >= p.num_seqs) return;
  const int L = p.seq_lens[i];
  const int cap = p.max_blocks << p.page_shift;
  const int32_t* row = p.bt + (int64_t)i * p.bt_stride;
  for (int t = 0; t < p.q_len; ++t) {
    const int pos = L + t;
    int64_t slot = -1;
    if (L > 0 && pos < cap) slot = ((int64_t)row[pos >> p.page_shift] << p.page_shift) + (pos & ((1 << p.page_shift) - 1));
    p.slots[(int64_t)i * p.q_len + t] = slot;
  }
  if (L > 0) p.seq_lens[i] = min(L + p.q_len, cap);
}

}  // namespace

hipError_t launch_draft_advance(const DraftParams& p, hipStream_t s) {
  hipLaunchKernelGGL(draft_advance_kernel, dim3((p.num_seqs + kDThreads - 1) / kDThreads), dim3(kDThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mj
