// Host side of the mj C ABI: configuration checks, the split-KV planner,
// argument validation and kernel launches.  Never allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "mj.h"
#include "mj_internal.h"

namespace {

constexpr int kRowTile = 64;      // query rows one decode workgroup covers
constexpr int kDefaultKvTile = 128;
constexpr int kMaxRows = 1024;    // sanity bound on q_len * h_r

struct Derived {
  int num_cus, kv_tile, h_r, nq_max;
  int cap_max, slots_max;
  int64_t part_rows_max;  // max over q_len of slots(q_len) * q_len * h_r
};

// Planned workgroups per CU and chunk floor (tokens) for a q_len: the config's
// values, or the defaults of the kernel that serves n_q = q_len * h_r.  The
// e4m3 matrix-core kernel for up to 16 rows holds two workgroups per CU;
// planning it four waves deep lets CUs that stream faster take more items
// (the tail of a single wave is set by the slowest CU), and the 2048-token
// floor keeps items long enough to amortise the prologue and partial write.
// The 32-row kernel (one workgroup per CU) and the e2m3 kernel measured
// fastest planned one wave deep, and so did groups of more than 32 rows (row
// tiles: each item is already several workgroups; cfg4c's batch at 40 rows
// 96 -> 79 us, 128 rows 157 -> 130 us against two per CU).  The e2m1 and
// nvfp4 kernels of up to 32 rows plan two per CU.
struct PlanShape {
  int wgs_per_cu, min_chunk_tokens;
};

PlanShape plan_shape(const mj_config* c, const Derived& d, int q_len) {
  const int n_q = q_len * d.h_r;
  const bool small_e4m3 = c->kv_format == MJ_KV_E4M3 && n_q <= 16;
  const bool fp4 = c->kv_format == MJ_KV_E2M1 || c->kv_format == MJ_KV_NVFP4;
  PlanShape ps;
  ps.wgs_per_cu = c->wgs_per_cu ? c->wgs_per_cu : (small_e4m3 ? 8 : (fp4 && n_q <= 32 ? 2 : 1));
  ps.min_chunk_tokens = c->min_chunk_tokens ? c->min_chunk_tokens : (small_e4m3 ? 2048 : 1);
  return ps;
}

int min_chunk_tiles(const mj_config* c, const Derived& d, int q_len) {
  return (plan_shape(c, d, q_len).min_chunk_tokens + d.kv_tile - 1) / d.kv_tile;
}

// Bytes of one packed 128-channel K or V row of each format.
int kv_row_bytes(int kv_format) {
  return kv_format == MJ_KV_E4M3 ? 128 : (kv_format == MJ_KV_E2M1 || kv_format == MJ_KV_NVFP4 ? 64 : 96);
}
constexpr int kBlockScaleRowBytes = 8;  // nvfp4: one e4m3 per 16 channels

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

mj_status check_config(const mj_config* c) {
  if (!c) return MJ_EINVAL;
  if (c->h_q < 1 || c->h_k < 1 || c->max_num_seqs < 1 || c->max_q_len < 1 || c->max_splits < 1) return MJ_EINVAL;
  if (c->num_cus < 0 || c->wgs_per_cu < 0 || c->kv_tile_tokens < 0 || c->slots_override < 0 ||
      c->min_chunk_tokens < 0)
    return MJ_EINVAL;
  if (c->kv_tile_tokens % 16 != 0) return MJ_EINVAL;
  if (c->h_q % c->h_k != 0) return MJ_EUNSUPPORTED;
  if (c->head_dim != 128) return MJ_EUNSUPPORTED;
  if (c->page_size != 16 && c->page_size != 32 && c->page_size != 64 && c->page_size != 128) return MJ_EUNSUPPORTED;
  if (c->kv_format < MJ_KV_E4M3 || c->kv_format > MJ_KV_NVFP4) return MJ_EUNSUPPORTED;
  if (c->q_mode != MJ_Q_FP8 && c->q_mode != MJ_Q_BF16) return MJ_EINVAL;
  if (c->out_f32 != 0 && c->out_f32 != 1) return MJ_EINVAL;
  if (c->decode_kernel < 0 || (c->decode_kernel > 1 && (c->decode_kernel < 10 || c->decode_kernel > 73)))
    return MJ_EINVAL;
  if (c->kv_cache_policy < 0 || c->kv_cache_policy > 4 || c->step_merge < 0 || c->step_merge > 2) return MJ_EINVAL;
  // the packed fp6 / fp4 formats take fp8 Q only
  if (c->q_mode == MJ_Q_BF16 && c->kv_format != MJ_KV_E4M3 && c->kv_format != MJ_KV_NVFP4) return MJ_EUNSUPPORTED;
  if ((int64_t)c->max_q_len * (c->h_q / c->h_k) > kMaxRows) return MJ_ECAPACITY;
  return MJ_OK;
}

int row_tiles(const mj_config* c, int q_len) { return (q_len * (c->h_q / c->h_k) + kRowTile - 1) / kRowTile; }

int slots_for(const mj_config* c, const Derived& d, int q_len) {
  if (c->slots_override > 0) return c->slots_override;
  const int64_t denom = (int64_t)c->h_k * row_tiles(c, q_len);
  return (int)std::max<int64_t>(1, ((int64_t)d.num_cus * plan_shape(c, d, q_len).wgs_per_cu) / denom);
}

// Largest grid of any plan for q_len (the plan buffer is laid out for it).
int cap_for(const mj_config* c, const Derived& d, int q_len) { return std::max(slots_for(c, d, q_len), c->max_num_seqs); }

// Tokens a block-table row of max_blocks pages addresses: no plan covers more.
int64_t table_tokens(const mj_config* c, int max_blocks) { return (int64_t)max_blocks * c->page_size; }

// Can a plan over such rows split at all: a sequence that fills its row must
// be longer than the chunk floor.  Otherwise every sequence is one item
// whatever the lengths (no merge), and the grid needs max_num_seqs items.
bool splittable(const mj_config* c, const Derived& d, int q_len, int max_blocks) {
  return (table_tokens(c, max_blocks) + d.kv_tile - 1) / d.kv_tile > min_chunk_tiles(c, d, q_len);
}

// Workgroups per CU a batch's plan targets: the format's default, except one
// when the batch's (sequence, KV head, row tile) workgroups already reach
// every CU and a split its table width allows could not make more than two
// per CU (one resident round of the four-wave kernel), counting the chunks of
// at least the floor that a full row holds (a shorter remainder adds a short
// workgroup, not a round): such a split balances nothing and only adds the
// merge.  Measured on 32 sequences of 4K tokens x 8 KV heads on 256 CUs: the
// decode kernel 46.7 us whole and 46.9 us in two splits; the graph step 56.3
// and 63.7 us.  Decided by the configuration, the batch size, q_len and the
// table width (fixed when a graph is captured), never by the lengths;
// explicit wgs_per_cu or slots_override settings are kept as given.
int wgs_for(const mj_config* c, const Derived& d, int num_seqs, int q_len, int max_blocks) {
  const int w = plan_shape(c, d, q_len).wgs_per_cu;
  if (c->wgs_per_cu > 0 || c->slots_override > 0 || w <= 1) return w;
  const int64_t per_seq = (int64_t)c->h_k * row_tiles(c, q_len);
  if ((int64_t)num_seqs * per_seq < d.num_cus) return w;
  const int64_t tiles = (table_tokens(c, max_blocks) + d.kv_tile - 1) / d.kv_tile;
  const int64_t mc = min_chunk_tiles(c, d, q_len);
  const int64_t per_row = std::max<int64_t>(1, std::min<int64_t>(c->max_splits, tiles / mc));
  const int64_t most = std::min<int64_t>(slots_for(c, d, q_len), (int64_t)num_seqs * per_row);
  return most * per_seq <= 2 * (int64_t)d.num_cus ? 1 : w;
}

// The slots (work items of one round) of a batch's plan: slots_for at the
// batch's workgroups per CU.
int batch_slots(const mj_config* c, const Derived& d, int num_seqs, int q_len, int max_blocks) {
  if (c->slots_override > 0) return c->slots_override;
  const int64_t denom = (int64_t)c->h_k * row_tiles(c, q_len);
  return (int)std::max<int64_t>(1, ((int64_t)d.num_cus * wgs_for(c, d, num_seqs, q_len, max_blocks)) / denom);
}

bool plan_splits(const mj_config* c, const Derived& d, int num_seqs, int q_len, int max_blocks) {
  return c->max_splits > 1 && num_seqs < batch_slots(c, d, num_seqs, q_len, max_blocks) &&
         splittable(c, d, q_len, max_blocks);
}

// The grid of a plan: fixed by the config, the batch size, q_len and the
// table width (at most cap_for, which the plan buffer is laid out for).
int work_for(const mj_config* c, const Derived& d, int num_seqs, int q_len, int max_blocks) {
  return splittable(c, d, q_len, max_blocks)
             ? std::max(batch_slots(c, d, num_seqs, q_len, max_blocks), c->max_num_seqs)
             : c->max_num_seqs;
}

void shape_info(const mj_config* c, const Derived& d, int num_seqs, int q_len, int max_blocks, mj_plan_info* info) {
  info->num_work = work_for(c, d, num_seqs, q_len, max_blocks);
  info->slots = batch_slots(c, d, num_seqs, q_len, max_blocks);
  info->chunk_tiles = -1;
  info->num_chunks = -1;
  info->with_reduction = plan_splits(c, d, num_seqs, q_len, max_blocks) ? 1 : 0;
  info->num_seqs = num_seqs;
  info->q_len = q_len;
  info->kv_tile_tokens = d.kv_tile;
  info->min_chunk_tiles = min_chunk_tiles(c, d, q_len);
  info->wgs_per_cu = wgs_for(c, d, num_seqs, q_len, max_blocks);
}

mj_status derive(const mj_config* c, Derived* d) {
  mj_status st = check_config(c);
  if (st != MJ_OK) return st;
  d->num_cus = c->num_cus;
  if (d->num_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MJ_EHIP;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return MJ_EHIP;
    d->num_cus = n;
  }
  d->kv_tile = c->kv_tile_tokens ? c->kv_tile_tokens : kDefaultKvTile;
  d->h_r = c->h_q / c->h_k;
  d->nq_max = c->max_q_len * d->h_r;
  d->cap_max = 0;
  d->slots_max = 0;
  d->part_rows_max = 0;
  for (int ql = 1; ql <= c->max_q_len; ++ql) {
    d->cap_max = std::max(d->cap_max, cap_for(c, *d, ql));
    d->slots_max = std::max(d->slots_max, slots_for(c, *d, ql));
    d->part_rows_max = std::max<int64_t>(d->part_rows_max, (int64_t)slots_for(c, *d, ql) * ql * d->h_r);
  }
  return MJ_OK;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace: split partials (o | m | l), then the step's arrival counters
// and its Q staging (codes, scales) for the unfused fallback.  A plan for
// q_len has at most slots(q_len) split items of q_len * h_r rows per KV head,
// laid out [item][KV head][row] with the row stride of that q_len, so the
// partials take the largest slots(q_len) * q_len * h_r over q_len.
struct WorkspaceLayout {
  size_t o_off, m_off, l_off, cnt_off, q8_off, qd_off, total;
};

WorkspaceLayout workspace_layout(const mj_config* c, const Derived& d) {
  const size_t rows = (size_t)d.part_rows_max * c->h_k;
  const size_t pairs = (size_t)c->max_num_seqs * c->h_k;
  WorkspaceLayout w;
  w.o_off = 0;
  w.m_off = round256(rows * 128 * sizeof(float));
  w.l_off = w.m_off + round256(rows * sizeof(float));
  w.cnt_off = w.l_off + round256(rows * sizeof(float));
  w.q8_off = w.cnt_off + round256(pairs * sizeof(int32_t));
  w.qd_off = w.q8_off + round256(pairs * d.nq_max * 128);
  w.total = w.qd_off + round256(pairs * sizeof(float));
  return w;
}

size_t plan_ints(const mj_config* c, const Derived& d) { return (size_t)4 * d.cap_max + 2 * (size_t)c->max_num_seqs; }

int ilog2(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

// Decode kernel choice: 0 = the generic kernel, 1 = the matrix-core kernel.
// The matrix-core kernel addresses a page's rows with 32-bit lane offsets and
// takes whole 16-token tiles inside one page; it serves any row count (tiles
// of 32 rows).  decode_kernel 1 forces the generic kernel.
int kernel_choice(const mj::DecodeParams& p) {
  const bool small_strides = p.k_ss < (1 << 24) && p.v_ss < (1 << 24) && p.ksb_ss < (1 << 24) && p.vsb_ss < (1 << 24);
  const bool tiles_ok = (p.kv_tile % 16) == 0 && small_strides;
  return p.kernel_variant == 1 || !tiles_ok || p.n_q < 1 ? 0 : 1;
}

bool decode_fuses_step(const mj::DecodeParams& p) { return kernel_choice(p) == 1; }

hipError_t launch_decode(const mj::DecodeParams& p, int kv_format, int row_tiles, hipStream_t s) {
  const int k = kernel_choice(p);
  // only the matrix-core kernel fuses the step; bf16 Q is read by it and the generic kernel
  if (k != 1 && ((p.qb && !p.q_bf16) || p.counters)) return hipErrorInvalidValue;
  // the fused merge counts one arrival per (item, KV head): one row tile
  if (p.counters && p.n_q > mj::kMfmaTileRows) return hipErrorInvalidValue;
  if (k == 0) return mj::launch_decode_generic(p, kv_format, row_tiles, s);
  // kv_cache_policy -> the matrix-core kernel's policy bits (bit 0 K
  // non-temporal, bit 1 V non-temporal; -1 the kernel's default)
  static const int kPolicy[5] = {-1, 0, 3, 2, 1};
  return mj::launch_decode_mfma(p, kv_format, kPolicy[p.cache_policy],
                                p.kernel_variant >= 10 ? p.kernel_variant - 10 : -1, s);
}

}  // namespace

extern "C" {

const char* mj_status_string(mj_status s) {
  switch (s) {
    case MJ_OK: return "ok";
    case MJ_EINVAL: return "invalid argument";
    case MJ_EUNSUPPORTED: return "unsupported shape or format";
    case MJ_EALIGN: return "misaligned pointer or stride";
    case MJ_ECAPACITY: return "capacity exceeded";
    case MJ_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t mj_abi_version(void) { return MJ_ABI_VERSION; }

mj_status mj_config_check(const mj_config* cfg) { return check_config(cfg); }

size_t mj_plan_buffer_bytes(const mj_config* cfg) {
  Derived d;
  if (derive(cfg, &d) != MJ_OK) return 0;
  return plan_ints(cfg, d) * sizeof(int32_t);
}

size_t mj_workspace_bytes(const mj_config* cfg) {
  Derived d;
  if (derive(cfg, &d) != MJ_OK) return 0;
  return workspace_layout(cfg, d).total;
}

int32_t mj_plan_capacity(const mj_config* cfg, int32_t q_len) {
  Derived d;
  if (derive(cfg, &d) != MJ_OK || q_len < 1 || q_len > cfg->max_q_len) return -1;
  return cap_for(cfg, d, q_len);
}

mj_status mj_plan_compute(const mj_config* cfg, const int32_t* seq_lens_host, int32_t num_seqs, int32_t q_len,
                          int32_t margin, int32_t max_blocks_per_seq, int32_t* plan_host, mj_plan_info* info) {
  Derived d;
  mj_status st = derive(cfg, &d);
  if (st != MJ_OK) return st;
  if (!seq_lens_host || !plan_host || !info || num_seqs < 1 || q_len < 1 || margin < 0 || max_blocks_per_seq < 1)
    return MJ_EINVAL;
  if (num_seqs > cfg->max_num_seqs || q_len > cfg->max_q_len) return MJ_ECAPACITY;
  const int64_t T = table_tokens(cfg, max_blocks_per_seq);
  // tokens the plan covers: the length plus the margin, never past the table row
  auto tiles = [&](int i) -> int64_t {
    return (std::min<int64_t>((int64_t)seq_lens_host[i] + margin, T) + d.kv_tile - 1) / d.kv_tile;
  };
  int64_t max_tiles = 0;
  for (int i = 0; i < num_seqs; ++i) {
    const int64_t L = seq_lens_host[i];
    if (L < 0) return MJ_EINVAL;
    if ((L + cfg->page_size - 1) / cfg->page_size > max_blocks_per_seq) return MJ_ECAPACITY;
    max_tiles = std::max(max_tiles, tiles(i));
  }
  auto ceil_div = [](int64_t a, int64_t b) -> int64_t { return (a + b - 1) / b; };

  const int S = batch_slots(cfg, d, num_seqs, q_len, max_blocks_per_seq);
  const int cap = work_for(cfg, d, num_seqs, q_len, max_blocks_per_seq);
  const bool split = plan_splits(cfg, d, num_seqs, q_len, max_blocks_per_seq);
  int64_t c = std::max<int64_t>(1, max_tiles);
  if (split) {
    // smallest chunk >= ceil(max_tiles / max_splits) whose item count fits S;
    // the count only falls as the chunk grows, and at c = max_tiles it is
    // num_seqs < S, so a bisection finds it.
    int64_t lo = std::max<int64_t>({1, ceil_div(max_tiles, cfg->max_splits), min_chunk_tiles(cfg, d, q_len)});
    int64_t hi = std::max<int64_t>(lo, max_tiles);
    auto count = [&](int64_t ch) {
      int64_t n = 0;
      for (int i = 0; i < num_seqs; ++i) n += std::max<int64_t>(1, ceil_div(tiles(i), ch));
      return n;
    };
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (count(mid) <= S) hi = mid; else lo = mid + 1;
    }
    c = lo;
  }

  const size_t total = plan_ints(cfg, d);
  std::fill(plan_host, plan_host + total, 0);
  int32_t* work = plan_host;
  int32_t* nspl = plan_host + 4 * (size_t)d.cap_max;
  int32_t* sbeg = nspl + cfg->max_num_seqs;
  int w = 0, chunks = 0;
  for (int i = 0; i < num_seqs; ++i) {
    const int64_t t = tiles(i);
    const int64_t n = split ? std::max<int64_t>(1, ceil_div(t, c)) : 1;
    nspl[i] = (int32_t)n;
    sbeg[i] = w;
    for (int64_t s = 0; s < n; ++s, ++w) {
      const int64_t b = split ? s * c : 0;
      const int64_t e = split ? std::min((s + 1) * c, t) : t;
      work[4 * w + 0] = i;
      work[4 * w + 1] = (int32_t)b;
      work[4 * w + 2] = (int32_t)e;
      work[4 * w + 3] = (int32_t)s;
      chunks += e > b;
    }
  }
  if (w > cap) return MJ_EINVAL;  // cannot happen: split plans fit S <= cap, others use num_seqs <= cap
  for (; w < d.cap_max; ++w) {
    work[4 * w + 0] = -1;
    work[4 * w + 1] = work[4 * w + 2] = work[4 * w + 3] = 0;
  }
  for (int i = num_seqs; i < cfg->max_num_seqs; ++i) {
    nspl[i] = 1;
    sbeg[i] = 0;
  }
  info->num_work = cap;
  info->slots = S;
  info->chunk_tiles = (int32_t)c;
  info->num_chunks = chunks;
  info->with_reduction = split ? 1 : 0;
  info->num_seqs = num_seqs;
  info->q_len = q_len;
  info->kv_tile_tokens = d.kv_tile;
  info->min_chunk_tiles = min_chunk_tiles(cfg, d, q_len);
  info->wgs_per_cu = wgs_for(cfg, d, num_seqs, q_len, max_blocks_per_seq);
  return MJ_OK;
}

mj_status mj_plan_split_kv(const mj_config* cfg, const int32_t* seq_lens_host, int32_t num_seqs, int32_t q_len,
                           int32_t margin, int32_t max_blocks_per_seq, int32_t* host_staging, int32_t* plan_dev,
                           mj_plan_info* info, hipStream_t stream) {
  if (!plan_dev) return MJ_EINVAL;
  mj_status st = mj_plan_compute(cfg, seq_lens_host, num_seqs, q_len, margin, max_blocks_per_seq, host_staging, info);
  if (st != MJ_OK) return st;
  const size_t bytes = mj_plan_buffer_bytes(cfg);
  if (hipMemcpyAsync(plan_dev, host_staging, bytes, hipMemcpyHostToDevice, stream) != hipSuccess) return MJ_EHIP;
  return MJ_OK;
}

static mj_status plan_device(const mj_config* cfg, const Derived& d, const int32_t* seq_lens_dev, int32_t num_seqs,
                             int32_t q_len, int32_t margin, int32_t max_blocks_per_seq, int32_t* plan_dev,
                             mj_plan_info* info, hipStream_t stream);

mj_status mj_plan_shape(const mj_config* cfg, int32_t num_seqs, int32_t q_len, int32_t max_blocks_per_seq,
                        mj_plan_info* info) {
  Derived d;
  mj_status st = derive(cfg, &d);
  if (st != MJ_OK) return st;
  if (!info || num_seqs < 1 || q_len < 1 || max_blocks_per_seq < 1) return MJ_EINVAL;
  if (num_seqs > cfg->max_num_seqs || q_len > cfg->max_q_len) return MJ_ECAPACITY;
  shape_info(cfg, d, num_seqs, q_len, max_blocks_per_seq, info);
  return MJ_OK;
}

mj_status mj_plan_split_kv_device(const mj_config* cfg, const int32_t* seq_lens_dev, int32_t num_seqs, int32_t q_len,
                                  int32_t margin, int32_t max_blocks_per_seq, int32_t* plan_dev, mj_plan_info* info,
                                  hipStream_t stream) {
  Derived d;
  mj_status st = derive(cfg, &d);
  if (st != MJ_OK) return st;
  if (!info) return MJ_EINVAL;
  return plan_device(cfg, d, seq_lens_dev, num_seqs, q_len, margin, max_blocks_per_seq, plan_dev, info, stream);
}

static mj_status plan_device(const mj_config* cfg, const Derived& d, const int32_t* seq_lens_dev, int32_t num_seqs,
                             int32_t q_len, int32_t margin, int32_t max_blocks_per_seq, int32_t* plan_dev,
                             mj_plan_info* info, hipStream_t stream) {
  if (!seq_lens_dev || !plan_dev || num_seqs < 1 || q_len < 1 || margin < 0 || max_blocks_per_seq < 1)
    return MJ_EINVAL;
  if (num_seqs > cfg->max_num_seqs || q_len > cfg->max_q_len) return MJ_ECAPACITY;
  if (!aligned(plan_dev, 16) || !aligned(seq_lens_dev, 4)) return MJ_EALIGN;
  const int S = batch_slots(cfg, d, num_seqs, q_len, max_blocks_per_seq);
  const bool split = plan_splits(cfg, d, num_seqs, q_len, max_blocks_per_seq);
  mj::PlanParams p;
  p.seq_lens = seq_lens_dev;
  p.work = plan_dev;
  p.n_splits = plan_dev + 4 * (size_t)d.cap_max;
  p.split_begin = p.n_splits + cfg->max_num_seqs;
  p.num_seqs = num_seqs;
  p.max_num_seqs = cfg->max_num_seqs;
  p.margin = margin;
  p.kv_tile = d.kv_tile;
  p.page_size = cfg->page_size;
  p.max_blocks = max_blocks_per_seq;
  p.max_splits = cfg->max_splits;
  p.slots = S;
  p.split = split ? 1 : 0;
  p.cap_max = d.cap_max;
  p.min_chunk = min_chunk_tiles(cfg, d, q_len);
  if (mj::launch_plan(p, stream) != hipSuccess) return MJ_EHIP;
  if (info) shape_info(cfg, d, num_seqs, q_len, max_blocks_per_seq, info);  // chunk decided on the device
  return MJ_OK;
}

mj_status mj_quantize_q(const mj_config* cfg, const void* q, int64_t q_tok_stride, int64_t q_head_stride,
                        const float* q_mul, int32_t num_seqs, int32_t q_len, uint8_t* q8, float* q_descale,
                        hipStream_t stream) {
  mj_status st = check_config(cfg);
  if (st != MJ_OK) return st;
  if (!q || !q8 || !q_descale || num_seqs < 1 || q_len < 1 || q_tok_stride < 0 || q_head_stride < 0) return MJ_EINVAL;
  if (num_seqs > cfg->max_num_seqs || q_len > cfg->max_q_len) return MJ_ECAPACITY;
  if (!aligned(q, 16) || q_tok_stride % 8 || q_head_stride % 8 || !aligned(q8, 16) || !aligned(q_descale, 4) ||
      (q_mul && !aligned(q_mul, 16)))
    return MJ_EALIGN;
  mj::QQuantParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.q_ts = q_tok_stride;
  p.q_hs = q_head_stride;
  p.q_mul = q_mul;
  p.q8 = q8;
  p.q_descale = q_descale;
  p.num_seqs = num_seqs;
  p.q_len = q_len;
  p.h_k = cfg->h_k;
  p.h_r = cfg->h_q / cfg->h_k;
  p.n_q = q_len * p.h_r;
  return mj::launch_qquant(p, stream) == hipSuccess ? MJ_OK : MJ_EHIP;
}

static mj_status fill_decode(const mj_config* cfg, const Derived& d, const mj_decode_args* a, mj::DecodeParams* p) {
  const bool qbf = cfg->q_mode == MJ_Q_BF16;
  if (qbf ? !a->q_bf16 : (!a->q8 || !a->q_descale)) return MJ_EINVAL;
  if (qbf && (a->q_tok_stride < 0 || a->q_head_stride < 0)) return MJ_EINVAL;
  if (qbf && (!aligned(a->q_bf16, 16) || a->q_tok_stride % 8 || a->q_head_stride % 8)) return MJ_EALIGN;
  if (!a->k_cache || !a->v_cache || !a->k_descale || !a->v_descale || !a->block_table ||
      !a->seq_lens || !a->plan || !a->out)
    return MJ_EINVAL;
  if (a->num_seqs < 1 || a->q_len < 1) return MJ_EINVAL;
  if (a->num_seqs > cfg->max_num_seqs || a->q_len > cfg->max_q_len) return MJ_ECAPACITY;
  if (a->k_descale_kind < 0 || a->k_descale_kind > 2 || a->v_descale_kind < 0 || a->v_descale_kind > 2)
    return MJ_EINVAL;
  if (a->num_pages < 1 || a->max_blocks_per_seq < 1 || a->bt_row_stride < a->max_blocks_per_seq) return MJ_EINVAL;
  if (!std::isfinite(a->softmax_scale)) return MJ_EINVAL;
  if (a->k_page_stride < 0 || a->k_slot_stride < 0 || a->k_head_stride < 0 || a->v_page_stride < 0 ||
      a->v_slot_stride < 0 || a->v_head_stride < 0 || a->out_tok_stride < 0 || a->out_head_stride < 0)
    return MJ_EINVAL;
  if ((!qbf && !aligned(a->q8, 16)) || !aligned(a->k_cache, 16) || !aligned(a->v_cache, 16) || !aligned(a->out, 16) ||
      a->k_page_stride % 16 || a->k_slot_stride % 16 || a->k_head_stride % 16 || a->v_page_stride % 16 ||
      a->v_slot_stride % 16 || a->v_head_stride % 16 || a->out_tok_stride % 8 || a->out_head_stride % 8 ||
      (a->o_mul && !aligned(a->o_mul, 16)))
    return MJ_EALIGN;
  const bool nv = cfg->kv_format == MJ_KV_NVFP4;
  if (nv) {
    if (!a->k_block_scale || !a->v_block_scale || a->k_bs_page_stride < 0 || a->k_bs_slot_stride < 0 ||
        a->k_bs_head_stride < 0 || a->v_bs_page_stride < 0 || a->v_bs_slot_stride < 0 || a->v_bs_head_stride < 0)
      return MJ_EINVAL;
    if (!aligned(a->k_block_scale, 8) || !aligned(a->v_block_scale, 8) || a->k_bs_page_stride % 8 ||
        a->k_bs_slot_stride % 8 || a->k_bs_head_stride % 8 || a->v_bs_page_stride % 8 || a->v_bs_slot_stride % 8 ||
        a->v_bs_head_stride % 8)
      return MJ_EALIGN;
  }
  if (a->num_work != work_for(cfg, d, a->num_seqs, a->q_len, a->max_blocks_per_seq)) return MJ_EINVAL;
  const bool split = plan_splits(cfg, d, a->num_seqs, a->q_len, a->max_blocks_per_seq);
  if ((a->with_reduction != 0) != split) return MJ_EINVAL;
  const WorkspaceLayout wl = workspace_layout(cfg, d);
  if (split && (!a->workspace || a->workspace_bytes < wl.total)) return MJ_ECAPACITY;
  if (a->workspace && !aligned(a->workspace, 256)) return MJ_EALIGN;

  char* ws = static_cast<char*>(a->workspace);
  const bool has_ws = ws && a->workspace_bytes >= wl.total;
  p->q8 = qbf ? nullptr : a->q8;
  p->q_descale = qbf ? nullptr : a->q_descale;
  p->k = static_cast<const uint8_t*>(a->k_cache);
  p->v = static_cast<const uint8_t*>(a->v_cache);
  p->k_sp = a->k_page_stride;
  p->k_ss = a->k_slot_stride;
  p->k_sh = a->k_head_stride;
  p->v_sp = a->v_page_stride;
  p->v_ss = a->v_slot_stride;
  p->v_sh = a->v_head_stride;
  p->num_pages = a->num_pages;
  p->kd = a->k_descale;
  p->vd = a->v_descale;
  p->kd_kind = a->k_descale_kind;
  p->vd_kind = a->v_descale_kind;
  p->bt = a->block_table;
  p->bt_stride = a->bt_row_stride;
  p->max_blocks = a->max_blocks_per_seq;
  p->seq_lens = a->seq_lens;
  p->work = a->plan;
  p->n_splits = a->plan + 4 * (size_t)d.cap_max;
  p->split_begin = p->n_splits + cfg->max_num_seqs;
  p->o_part = has_ws ? reinterpret_cast<float*>(ws + wl.o_off) : nullptr;
  p->m_part = has_ws ? reinterpret_cast<float*>(ws + wl.m_off) : nullptr;
  p->l_part = has_ws ? reinterpret_cast<float*>(ws + wl.l_off) : nullptr;
  p->nqp = a->q_len * d.h_r;
  p->part_items = has_ws ? slots_for(cfg, d, a->q_len) : 0;
  p->scale_log2 = a->softmax_scale * 1.4426950408889634f;
  p->pos_inf = INFINITY;
  p->o_mul = a->o_mul;
  p->out = static_cast<uint16_t*>(a->out);
  p->out_f32 = cfg->out_f32;
  p->out_ts = a->out_tok_stride;
  p->out_hs = a->out_head_stride;
  p->lse = a->lse;
  p->num_seqs = a->num_seqs;
  p->q_len = a->q_len;
  p->h_q = cfg->h_q;
  p->h_k = cfg->h_k;
  p->h_r = d.h_r;
  p->n_q = a->q_len * d.h_r;
  p->page_size = cfg->page_size;
  p->page_shift = ilog2(cfg->page_size);
  p->kv_tile = d.kv_tile;
  p->causal = a->causal ? 1 : 0;
  // the launch covers the plan's items: at most max_splits per sequence, so
  // a grid of max_num_seqs * max_splits item slots when that is below the
  // plan's capacity (small batches of long sequences: 16 workgroups per KV
  // head instead of 256 for one sequence on 256 CUs); like the capacity it
  // depends on the config only, so a captured step stays valid
  p->num_work = (int)std::min<int64_t>(a->num_work, (int64_t)cfg->max_num_seqs * cfg->max_splits);
  p->head_major = 0;
  p->row_tiles = 1;
  p->q_bf16 = qbf ? 1 : 0;
  p->qb = qbf ? static_cast<const uint16_t*>(a->q_bf16) : nullptr;
  p->qb_ts = qbf ? a->q_tok_stride : 0;
  p->qb_hs = qbf ? a->q_head_stride : 0;
  p->q_mul = nullptr;
  p->counters = nullptr;
  p->plan_in_kernel = 0;
  p->plan_margin = p->plan_max_splits = p->plan_slots = p->plan_split = p->plan_min_chunk = 0;
  p->ns_out = p->sb_out = nullptr;
  p->kernel_variant = cfg->decode_kernel;
  p->num_cus = d.num_cus;
  p->cache_policy = cfg->kv_cache_policy;
  p->ksb = nv ? static_cast<const uint8_t*>(a->k_block_scale) : nullptr;
  p->vsb = nv ? static_cast<const uint8_t*>(a->v_block_scale) : nullptr;
  p->ksb_sp = nv ? a->k_bs_page_stride : 0;
  p->ksb_ss = nv ? a->k_bs_slot_stride : 0;
  p->ksb_sh = nv ? a->k_bs_head_stride : 0;
  p->vsb_sp = nv ? a->v_bs_page_stride : 0;
  p->vsb_ss = nv ? a->v_bs_slot_stride : 0;
  p->vsb_sh = nv ? a->v_bs_head_stride : 0;
  return MJ_OK;
}

mj_status mj_paged_decode(const mj_config* cfg, const mj_decode_args* a, hipStream_t stream) {
  Derived d;
  mj_status st = derive(cfg, &d);
  if (st != MJ_OK) return st;
  if (!a) return MJ_EINVAL;
  mj::DecodeParams p;
  st = fill_decode(cfg, d, a, &p);
  if (st != MJ_OK) return st;
  return launch_decode(p, cfg->kv_format, row_tiles(cfg, a->q_len), stream) == hipSuccess ? MJ_OK : MJ_EHIP;
}

mj_status mj_decode_step(const mj_config* cfg, const mj_step_args* sa, hipStream_t stream) {
  Derived d;
  mj_status st = derive(cfg, &d);
  if (st != MJ_OK) return st;
  if (!sa || !sa->q || sa->q_tok_stride < 0 || sa->q_head_stride < 0) return MJ_EINVAL;
  if (!aligned(sa->q, 16) || sa->q_tok_stride % 8 || sa->q_head_stride % 8 || (sa->q_mul && !aligned(sa->q_mul, 16)))
    return MJ_EALIGN;
  const WorkspaceLayout wl = workspace_layout(cfg, d);
  if (!sa->decode.workspace || sa->decode.workspace_bytes < wl.total) return MJ_ECAPACITY;
  if (!aligned(sa->decode.workspace, 256)) return MJ_EALIGN;
  char* ws = static_cast<char*>(sa->decode.workspace);
  uint8_t* q8 = reinterpret_cast<uint8_t*>(ws + wl.q8_off);
  float* qd = reinterpret_cast<float*>(ws + wl.qd_off);
  const bool qbf = cfg->q_mode == MJ_Q_BF16;
  if (qbf && sa->q_mul) return MJ_EUNSUPPORTED;  // q_mul folds fp6 K scales into quantized Q
  mj_decode_args a = sa->decode;
  a.q8 = q8;
  a.q_descale = qd;
  a.q_bf16 = sa->q;
  a.q_tok_stride = sa->q_tok_stride;
  a.q_head_stride = sa->q_head_stride;
  if (sa->plan_on_device && sa->margin < 0) return MJ_EINVAL;
  mj::DecodeParams p;
  st = fill_decode(cfg, d, &a, &p);
  if (st != MJ_OK) return st;
  const int rt = row_tiles(cfg, a.q_len);
  // Where a fused step merges (cfg->step_merge): 0 automatic, 1 in the decode
  // kernel (the last split item of a pair), 2 a separate merge launch.
  // Automatic is the separate launch: the in-kernel merge makes every split
  // workgroup wait for its write-through stores and a returning atomic
  // before it retires, which costs more than the launch once a plan takes
  // several rounds of workgroups (measured: 32k context -10 us, ragged batch
  // -12 us per step; a single short sequence +1.4 us).
  const bool want_merge_in_kernel = cfg->step_merge == 1;
  // plan in the decode kernel: matrix-core kernel, a batch the wave-level
  // planner covers, tile counts small enough for its float quotients
  const int64_t max_tiles = ((int64_t)a.max_blocks_per_seq * cfg->page_size + sa->margin + d.kv_tile - 1) / d.kv_tile;
  const bool plan_in_kernel = sa->plan_on_device && decode_fuses_step(p) &&
                              a.num_seqs <= mj::kPlanMaxSeqs && 2 * max_tiles < (1 << 22);
  if (sa->plan_on_device && !plan_in_kernel) {
    st = plan_device(cfg, d, a.seq_lens, a.num_seqs, a.q_len, sa->margin, a.max_blocks_per_seq,
                     const_cast<int32_t*>(a.plan), nullptr, stream);
    if (st != MJ_OK) return st;
  }
  if (plan_in_kernel) {
    p.plan_in_kernel = 1;
    p.plan_margin = sa->margin;
    p.plan_max_splits = cfg->max_splits;
    p.plan_slots = batch_slots(cfg, d, a.num_seqs, a.q_len, a.max_blocks_per_seq);
    p.plan_split = a.with_reduction ? 1 : 0;
    p.plan_min_chunk = min_chunk_tiles(cfg, d, a.q_len);
    p.ns_out = const_cast<int32_t*>(p.n_splits);
    p.sb_out = const_cast<int32_t*>(p.split_begin);
  }
  mj_merge_args m;
  m.plan = a.plan;
  m.num_seqs = a.num_seqs;
  m.q_len = a.q_len;
  m.workspace = a.workspace;
  m.workspace_bytes = a.workspace_bytes;
  m.out = a.out;
  m.out_tok_stride = a.out_tok_stride;
  m.out_head_stride = a.out_head_stride;
  m.lse = a.lse;
  if (qbf) {  // nothing to quantize: the decode reads bf16 Q itself
    const bool merge_in_kernel = want_merge_in_kernel && !plan_in_kernel && p.n_q <= mj::kMfmaTileRows &&
                                 decode_fuses_step(p);
    p.counters = a.with_reduction && merge_in_kernel ? reinterpret_cast<int32_t*>(ws + wl.cnt_off) : nullptr;
    if (launch_decode(p, cfg->kv_format, rt, stream) != hipSuccess) return MJ_EHIP;
    return a.with_reduction && !merge_in_kernel ? mj_merge_lse(cfg, &m, stream) : MJ_OK;
  }
  if (decode_fuses_step(p)) {
    p.qb = static_cast<const uint16_t*>(sa->q);
    p.qb_ts = sa->q_tok_stride;
    p.qb_hs = sa->q_head_stride;
    p.q_mul = sa->q_mul;
    // its merge reads this launch's plan, and covers a group of one row tile
    const bool merge_in_kernel = want_merge_in_kernel && !plan_in_kernel && p.n_q <= mj::kMfmaTileRows;
    p.counters = a.with_reduction && merge_in_kernel ? reinterpret_cast<int32_t*>(ws + wl.cnt_off) : nullptr;
    if (launch_decode(p, cfg->kv_format, rt, stream) != hipSuccess) return MJ_EHIP;
    return a.with_reduction && !merge_in_kernel ? mj_merge_lse(cfg, &m, stream) : MJ_OK;
  }
  st = mj_quantize_q(cfg, sa->q, sa->q_tok_stride, sa->q_head_stride, sa->q_mul, a.num_seqs, a.q_len, q8, qd, stream);
  if (st != MJ_OK) return st;
  if (launch_decode(p, cfg->kv_format, rt, stream) != hipSuccess) return MJ_EHIP;
  return a.with_reduction ? mj_merge_lse(cfg, &m, stream) : MJ_OK;
}

mj_status mj_merge_lse(const mj_config* cfg, const mj_merge_args* a, hipStream_t stream) {
  Derived d;
  mj_status st = derive(cfg, &d);
  if (st != MJ_OK) return st;
  if (!a || !a->plan || !a->workspace || !a->out || a->num_seqs < 1 || a->q_len < 1) return MJ_EINVAL;
  if (a->num_seqs > cfg->max_num_seqs || a->q_len > cfg->max_q_len) return MJ_ECAPACITY;
  if (a->out_tok_stride < 0 || a->out_head_stride < 0) return MJ_EINVAL;
  const WorkspaceLayout wl = workspace_layout(cfg, d);
  if (a->workspace_bytes < wl.total) return MJ_ECAPACITY;
  if (!aligned(a->workspace, 256) || !aligned(a->out, 16) || a->out_tok_stride % 8 || a->out_head_stride % 8)
    return MJ_EALIGN;
  const char* ws = static_cast<const char*>(a->workspace);
  mj::MergeParams p;
  p.n_splits = a->plan + 4 * (size_t)d.cap_max;
  p.split_begin = p.n_splits + cfg->max_num_seqs;
  p.o_part = reinterpret_cast<const float*>(ws + wl.o_off);
  p.m_part = reinterpret_cast<const float*>(ws + wl.m_off);
  p.l_part = reinterpret_cast<const float*>(ws + wl.l_off);
  p.nqp = a->q_len * d.h_r;
  p.part_items = slots_for(cfg, d, a->q_len);
  p.out = static_cast<uint16_t*>(a->out);
  p.out_f32 = cfg->out_f32;
  p.out_ts = a->out_tok_stride;
  p.out_hs = a->out_head_stride;
  p.lse = a->lse;
  p.num_seqs = a->num_seqs;
  p.q_len = a->q_len;
  p.h_q = cfg->h_q;
  p.h_k = cfg->h_k;
  p.h_r = d.h_r;
  p.n_q = a->q_len * d.h_r;
  return mj::launch_merge(p, stream) == hipSuccess ? MJ_OK : MJ_EHIP;
}

mj_status mj_write_kv(const mj_config* cfg, const mj_write_args* a, hipStream_t stream) {
  mj_status st = check_config(cfg);
  if (st != MJ_OK) return st;
  if (!a || a->num_tokens < 0) return MJ_EINVAL;
  if (a->num_tokens == 0) return MJ_OK;
  if (!a->key || !a->value || !a->slot_mapping || !a->k_cache || !a->v_cache || !a->k_scale || !a->v_scale ||
      a->num_pages < 1)
    return MJ_EINVAL;
  if (a->key_tok_stride < 0 || a->key_head_stride < 0 || a->value_tok_stride < 0 || a->value_head_stride < 0 ||
      a->k_page_stride < 0 || a->k_slot_stride < 0 || a->k_head_stride < 0 || a->v_page_stride < 0 ||
      a->v_slot_stride < 0 || a->v_head_stride < 0)
    return MJ_EINVAL;
  for (int kind : {a->k_scale_kind, a->v_scale_kind}) {
    if (kind == MJ_SCALE_SEQ_HEAD) return MJ_EUNSUPPORTED;
    if (kind != MJ_SCALE_TENSOR && kind != MJ_SCALE_HEAD && kind != MJ_SCALE_CHANNEL) return MJ_EINVAL;
  }
  if (!aligned(a->key, 16) || !aligned(a->value, 16) || a->key_tok_stride % 8 || a->key_head_stride % 8 ||
      a->value_tok_stride % 8 || a->value_head_stride % 8 || !aligned(a->k_cache, 16) || !aligned(a->v_cache, 16) ||
      a->k_page_stride % 16 || a->k_slot_stride % 16 || a->k_head_stride % 16 || a->v_page_stride % 16 ||
      a->v_slot_stride % 16 || a->v_head_stride % 16 || !aligned(a->slot_mapping, 8) || !aligned(a->k_scale, 4) ||
      !aligned(a->v_scale, 4))
    return MJ_EALIGN;
  const bool nv = cfg->kv_format == MJ_KV_NVFP4;
  if (nv) {
    if (!a->k_block_scale || !a->v_block_scale || a->k_bs_page_stride < 0 || a->k_bs_slot_stride < 0 ||
        a->k_bs_head_stride < 0 || a->v_bs_page_stride < 0 || a->v_bs_slot_stride < 0 || a->v_bs_head_stride < 0)
      return MJ_EINVAL;
    if (!aligned(a->k_block_scale, 8) || !aligned(a->v_block_scale, 8) || a->k_bs_page_stride % 8 ||
        a->k_bs_slot_stride % 8 || a->k_bs_head_stride % 8 || a->v_bs_page_stride % 8 || a->v_bs_slot_stride % 8 ||
        a->v_bs_head_stride % 8)
      return MJ_EALIGN;
  }
  mj::WriteParams p;
  p.key = static_cast<const uint16_t*>(a->key);
  p.value = static_cast<const uint16_t*>(a->value);
  p.k_ts = a->key_tok_stride;
  p.k_hs = a->key_head_stride;
  p.v_ts = a->value_tok_stride;
  p.v_hs = a->value_head_stride;
  p.slots = a->slot_mapping;
  p.kc = static_cast<uint8_t*>(a->k_cache);
  p.vc = static_cast<uint8_t*>(a->v_cache);
  p.kc_sp = a->k_page_stride;
  p.kc_ss = a->k_slot_stride;
  p.kc_sh = a->k_head_stride;
  p.vc_sp = a->v_page_stride;
  p.vc_ss = a->v_slot_stride;
  p.vc_sh = a->v_head_stride;
  p.num_pages = a->num_pages;
  p.ks = a->k_scale;
  p.vs = a->v_scale;
  p.ks_kind = a->k_scale_kind;
  p.vs_kind = a->v_scale_kind;
  p.num_tokens = a->num_tokens;
  p.h_k = cfg->h_k;
  p.page_shift = ilog2(cfg->page_size);
  p.kv_format = cfg->kv_format;
  p.kbs = nv ? static_cast<uint8_t*>(a->k_block_scale) : nullptr;
  p.vbs = nv ? static_cast<uint8_t*>(a->v_block_scale) : nullptr;
  p.kbs_sp = nv ? a->k_bs_page_stride : 0;
  p.kbs_ss = nv ? a->k_bs_slot_stride : 0;
  p.kbs_sh = nv ? a->k_bs_head_stride : 0;
  p.vbs_sp = nv ? a->v_bs_page_stride : 0;
  p.vbs_ss = nv ? a->v_bs_slot_stride : 0;
  p.vbs_sh = nv ? a->v_bs_head_stride : 0;
  return mj::launch_write_kv(p, stream) == hipSuccess ? MJ_OK : MJ_EHIP;
}

mj_status mj_draft_advance(const mj_config* cfg, const mj_draft_args* a, hipStream_t stream) {
  mj_status st = check_config(cfg);
  if (st != MJ_OK) return st;
  if (!a || !a->block_table || !a->seq_lens || !a->slot_mapping || a->num_seqs < 1 || a->q_len < 1 ||
      a->max_blocks_per_seq < 1 || a->bt_row_stride < a->max_blocks_per_seq)
    return MJ_EINVAL;
  if (a->num_seqs > cfg->max_num_seqs || a->q_len > cfg->max_q_len) return MJ_ECAPACITY;
  if (!aligned(a->slot_mapping, 8)) return MJ_EALIGN;
  mj::DraftParams p;
  p.bt = a->block_table;
  p.bt_stride = a->bt_row_stride;
  p.max_blocks = a->max_blocks_per_seq;
  p.page_shift = ilog2(cfg->page_size);
  p.seq_lens = a->seq_lens;
  p.num_seqs = a->num_seqs;
  p.q_len = a->q_len;
  p.slots = a->slot_mapping;
  return mj::launch_draft_advance(p, stream) == hipSuccess ? MJ_OK : MJ_EHIP;
}

mj_status mj_combine_lse(const mj_config* cfg, const mj_combine_args* a, hipStream_t stream) {
  mj_status st = check_config(cfg);
  if (st != MJ_OK) return st;
  if (!a || !a->part_out || !a->part_lse || !a->out || a->num_parts < 1 || a->num_rows < 1) return MJ_EINVAL;
  if (a->part_stride < 0 || a->part_tok_stride < 0 || a->part_head_stride < 0 || a->out_tok_stride < 0 ||
      a->out_head_stride < 0)
    return MJ_EINVAL;
  const int64_t om = cfg->out_f32 ? 4 : 8;
  if (!aligned(a->part_out, 16) || a->part_stride % 4 || a->part_tok_stride % 4 || a->part_head_stride % 4 ||
      !aligned(a->out, 16) || a->out_tok_stride % om || a->out_head_stride % om)
    return MJ_EALIGN;
  mj::CombineParams p;
  p.po = a->part_out;
  p.p_ps = a->part_stride;
  p.p_ts = a->part_tok_stride;
  p.p_hs = a->part_head_stride;
  p.plse = a->part_lse;
  p.out = static_cast<uint16_t*>(a->out);
  p.out_ts = a->out_tok_stride;
  p.out_hs = a->out_head_stride;
  p.out_f32 = cfg->out_f32;
  p.lse = a->lse;
  p.parts = a->num_parts;
  p.rows = a->num_rows;
  p.h_q = cfg->h_q;
  return mj::launch_combine(p, stream) == hipSuccess ? MJ_OK : MJ_EHIP;
}

mj_status mj_debug_gather_kv(const mj_config* cfg, const mj_decode_args* a, int32_t seq, int32_t head,
                             int32_t seq_len, int32_t which, uint8_t* dense_out, hipStream_t stream) {
  mj_status st = check_config(cfg);
  if (st != MJ_OK) return st;
  const bool scales = which == 2 || which == 3;
  if (!a || !dense_out || !a->block_table || which < 0 || which > 3) return MJ_EINVAL;
  if (scales && cfg->kv_format != MJ_KV_NVFP4) return MJ_EINVAL;
  if (seq < 0 || head < 0 || head >= cfg->h_k || seq_len < 0 || a->num_pages < 1) return MJ_EINVAL;
  if ((int64_t)seq_len > (int64_t)a->max_blocks_per_seq * cfg->page_size) return MJ_ECAPACITY;
  mj::GatherParams p;
  const void* pools[4] = {a->k_cache, a->v_cache, a->k_block_scale, a->v_block_scale};
  const int64_t sps[4] = {a->k_page_stride, a->v_page_stride, a->k_bs_page_stride, a->v_bs_page_stride};
  const int64_t sss[4] = {a->k_slot_stride, a->v_slot_stride, a->k_bs_slot_stride, a->v_bs_slot_stride};
  const int64_t shs[4] = {a->k_head_stride, a->v_head_stride, a->k_bs_head_stride, a->v_bs_head_stride};
  p.pool = static_cast<const uint8_t*>(pools[which]);
  if (!p.pool) return MJ_EINVAL;
  p.sp = sps[which];
  p.ss = sss[which];
  p.sh = shs[which];
  p.num_pages = a->num_pages;
  p.bt = a->block_table;
  p.bt_stride = a->bt_row_stride;
  p.seq = seq;
  p.head = head;
  p.seq_len = seq_len;
  p.row_bytes = scales ? kBlockScaleRowBytes : kv_row_bytes(cfg->kv_format);
  p.page_shift = ilog2(cfg->page_size);
  p.out = dense_out;
  return mj::launch_gather(p, stream) == hipSuccess ? MJ_OK : MJ_EHIP;
}

mj_status mj_debug_stream_read(const void* src, int64_t bytes, uint32_t* out, int32_t blocks, hipStream_t stream) {
  if (!src || !out || bytes < 16 || bytes % 16 || blocks < 1 || !aligned(src, 16)) return MJ_EINVAL;
  return mj::launch_stream_read(src, bytes, out, blocks, stream) == hipSuccess ? MJ_OK : MJ_EHIP;
}

mj_status mj_debug_decode_codes(int32_t kv_format, const uint8_t* codes, int32_t n, float* out, hipStream_t stream) {
  if (!codes || !out || n < 0 || ((kv_format < MJ_KV_E4M3 || kv_format > MJ_KV_E2M1) && kv_format != 16))
    return MJ_EINVAL;
  return mj::launch_decode_codes(kv_format, codes, n, out, stream) == hipSuccess ? MJ_OK : MJ_EHIP;
}

}  // extern "C"
