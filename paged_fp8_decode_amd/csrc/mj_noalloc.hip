// mj_decode_step for callers that cannot allocate device memory (code under
// graph capture, tight serving loops, harnesses that forbid allocation):
// the step's plan buffer and workspace live in one static device array,
// `scratch`, instead of caller-owned buffers.
//
// `scratch` is a file-scope __device__ array: each GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code the array's name is not a device address, so the first call on a
// device (with that device current) asks the runtime for the copy's address
// with hipGetSymbolAddress and keeps it per device; every later use -- the
// plan and workspace pointers handed to the step's kernels -- goes through
// that address, never through the name.
//
// Nothing in `scratch` needs to start at zero: the step plans on the device
// (the decode kernel or the planner kernel writes every plan entry the
// merge reads), each split partial is written before it is read, and the
// in-kernel merge with its zero-initialised arrival counters is not used.
// Every call on a GPU shares that GPU's array and leaves its contents to the
// next call: two calls that overlap on one GPU (two streams without an
// ordering between them) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mj.h"

static constexpr size_t kScratchBytes = MJ_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// This device's copy of `scratch`, looked up on its first use.
mj_status scratch_of_current_device(unsigned char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MJ_EHIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MJ_EHIP;
    g_scratch[dev] = ptr;
  }
  *out = static_cast<unsigned char*>(g_scratch[dev]);
  return MJ_OK;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

extern "C" {

size_t mj_noalloc_scratch_bytes(const mj_config* cfg) {
  const size_t plan = mj_plan_buffer_bytes(cfg), ws = mj_workspace_bytes(cfg);
  if (!plan || !ws) return 0;
  return round256(plan) + ws;
}

mj_status mj_decode_step_noalloc(const mj_config* cfg, const mj_step_args* args, hipStream_t stream) {
  mj_status st = mj_config_check(cfg);
  if (st != MJ_OK) return st;
  if (!args) return MJ_EINVAL;
  // the plan buffer and workspace are the library's own here
  if (args->decode.plan || args->decode.workspace || !args->plan_on_device) return MJ_EINVAL;
  if (cfg->step_merge == 1) return MJ_EUNSUPPORTED;  // its arrival counters would have to start at zero
  const size_t need = mj_noalloc_scratch_bytes(cfg);
  if (need == 0) return MJ_EINVAL;
  if (need > kScratchBytes) return MJ_ECAPACITY;
  unsigned char* base = nullptr;
  st = scratch_of_current_device(&base);
  if (st != MJ_OK) return st;
  mj_step_args a = *args;
  a.decode.plan = reinterpret_cast<const int32_t*>(base);
  a.decode.workspace = base + round256(mj_plan_buffer_bytes(cfg));
  a.decode.workspace_bytes = mj_workspace_bytes(cfg);
  return mj_decode_step(cfg, &a, stream);
}

}  // extern "C"
