// Internal (host <-> kernel) interface of the mj library.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mj {

// Query rows one matrix-core workgroup serves; groups of more rows run as
// several such tiles, which the fused in-kernel merge does not cover.
constexpr int kMfmaTileRows = 32;

// Parameters of the Q quantization kernel.
struct QQuantParams {
  const uint16_t* q;  // bf16
  int64_t q_ts, q_hs;  // token / head strides, elements
  const float* q_mul;  // nullable (h_q, 128)
  uint8_t* q8;         // (b, h_k, n_q, 128)
  float* q_descale;    // (b, h_k)
  int num_seqs, q_len, h_k, h_r, n_q;
};

// Parameters of the decode kernels.
struct DecodeParams {
  const uint8_t* q8;
  const float* q_descale;
  const uint8_t* k;
  const uint8_t* v;
  int64_t k_sp, k_ss, k_sh;
  int64_t v_sp, v_ss, v_sh;
  int64_t num_pages;
  const float* kd;
  const float* vd;
  int kd_kind, vd_kind;
  const int32_t* bt;
  int64_t bt_stride;
  int max_blocks;
  const int32_t* seq_lens;
  const int32_t* work;         // plan + 0
  const int32_t* n_splits;     // plan + 4*cap_max
  const int32_t* split_begin;  // plan + 4*cap_max + max_num_seqs
  float* o_part;               // (S, h_k, nqp, 128)
  float* m_part;               // (S, h_k, nqp)   log2 domain
  float* l_part;               // (S, h_k, nqp)
  int nqp;                     // partial row stride = q_len * h_r of this call
  int part_items;              // S = slots for this q_len: items that may hold partials
  float scale_log2;            // softmax_scale * log2(e)
  float pos_inf;               // +inf, as an argument: max(a, b) = med3(a, b, pos_inf)
                               // is one instruction only while the compiler
                               // cannot fold the third operand
  const float* o_mul;          // nullable (h_q, 128)
  uint16_t* out;               // bf16, or fp32 when out_f32 (strides in elements)
  int64_t out_ts, out_hs;
  int out_f32;
  float* lse;                  // nullable
  int num_seqs, q_len, h_q, h_k, h_r, n_q;
  int page_size, page_shift, kv_tile;
  int causal;
  int num_work;
  int num_cus;                 // of the config (the matrix-core launch's grid choices)
  // grid: 0 = (num_work, h_k); 1 = (h_k, num_work); 2 = XCD-grouped, one
  // dimension of ceil(num_work / 8) * 8 * h_k workgroups numbered so that
  // the h_k heads of a work item share an XCD (see the matrix-core launch)
  int head_major;
  // matrix-core kernel: workgroups per (item, KV head), each serving a tile
  // of 32 of the group's n_q rows (the last one the remainder); the head
  // dimension of the grid above then counts h_k * row_tiles (head-major
  // order inside).  Set by the matrix-core launcher; 1 elsewhere.
  int row_tiles;
  // q_bf16 = 1: bf16-Q mode.  qb is then the bf16 Q the kernels use as is
  // (q8 / q_descale unused), on every decode kernel.
  // Otherwise (fused step, matrix-core kernel only; null elsewhere) qb is the
  // bf16 Q quantized in the prologue instead of reading q8 / q_descale.  counters:
  // (max_num_seqs, h_k) zero-initialised arrival counters; the last split of
  // a (sequence, KV head) to finish merges the partials and resets its
  // counter to zero.
  int q_bf16;
  const uint16_t* qb;
  int64_t qb_ts, qb_hs;        // elements
  const float* q_mul;          // nullable (h_q, 128)
  int32_t* counters;
  // Plan in the kernel (matrix-core kernel, fused step): every workgroup
  // derives its item from seq_lens with the planner's rule, and the split-0
  // workgroup of KV head 0 writes n_splits / split_begin of its sequence for
  // the merge launch.  `work` is not read then.
  int plan_in_kernel;
  int plan_margin, plan_max_splits, plan_slots, plan_split, plan_min_chunk;
  int32_t* ns_out;
  int32_t* sb_out;
  // kernel selection of the config (mj_config.decode_kernel and
  // kv_cache_policy; 0 = the library's choice)
  int kernel_variant, cache_policy;
  // nvfp4: the e4m3 block-scale pools (8-byte rows, paged like the codes);
  // null for the other formats
  const uint8_t* ksb;
  const uint8_t* vsb;
  int64_t ksb_sp, ksb_ss, ksb_sh;
  int64_t vsb_sp, vsb_ss, vsb_sh;
};

struct MergeParams {
  const int32_t* n_splits;
  const int32_t* split_begin;
  const float* o_part;
  const float* m_part;
  const float* l_part;
  int nqp;
  int part_items;
  uint16_t* out;
  int64_t out_ts, out_hs;
  int out_f32;
  float* lse;
  int num_seqs, q_len, h_q, h_k, h_r, n_q;
};

// Parameters of the KV-cache write kernel.
struct WriteParams {
  const uint16_t* key;      // bf16
  const uint16_t* value;
  int64_t k_ts, k_hs, v_ts, v_hs;   // elements
  const int64_t* slots;
  uint8_t* kc;
  uint8_t* vc;
  int64_t kc_sp, kc_ss, kc_sh, vc_sp, vc_ss, vc_sh;  // bytes
  int64_t num_pages;
  const float* ks;
  const float* vs;
  int ks_kind, vs_kind;     // 0 tensor, 1 head, 3 channel
  int num_tokens, h_k, page_shift, kv_format;
  int tokens_per_thread;    // set by the launcher
  uint8_t* kbs;             // nvfp4 block-scale pools (null otherwise)
  uint8_t* vbs;
  int64_t kbs_sp, kbs_ss, kbs_sh, vbs_sp, vbs_ss, vbs_sh;  // bytes
};

struct GatherParams {
  const uint8_t* pool;
  int64_t sp, ss, sh;
  int64_t num_pages;
  const int32_t* bt;
  int64_t bt_stride;
  int seq, head, seq_len, row_bytes, page_shift;
  uint8_t* out;
};

struct PlanParams {
  const int32_t* seq_lens;  // device
  int32_t* work;            // plan buffer: [cap_max][4]
  int32_t* n_splits;        // [max_num_seqs]
  int32_t* split_begin;     // [max_num_seqs]
  int num_seqs, max_num_seqs, margin, kv_tile, page_size, max_blocks, max_splits, slots, split, cap_max;
  int min_chunk;            // floor of the chunk, KV tiles
};

hipError_t launch_plan(const PlanParams& p, hipStream_t s);
constexpr int kPlanMaxSeqs = 256;  // batches the decode kernel plans itself (mj_plan_item.h)
hipError_t launch_qquant(const QQuantParams& p, hipStream_t s);
hipError_t launch_decode_generic(const DecodeParams& p, int kv_format, int row_tiles, hipStream_t s);
// cache_policy: -1 the default for the format, else bits (0 K non-temporal,
// 1 V non-temporal); tune: -1 the default, else bits (0 two granules of
// prefetch, 1 head-major grid, 2 XCD-grouped grid)
hipError_t launch_decode_mfma(const DecodeParams& p, int kv_format, int cache_policy, int tune, hipStream_t s);
hipError_t launch_merge(const MergeParams& p, hipStream_t s);
hipError_t launch_gather(const GatherParams& p, hipStream_t s);
hipError_t launch_write_kv(const WriteParams& p, hipStream_t s);

// Parameters of the draft-step advance (slot mapping of the appended tokens,
// seq_lens += q_len).
struct DraftParams {
  const int32_t* bt;
  int64_t bt_stride;
  int max_blocks, page_shift;
  int32_t* seq_lens;
  int num_seqs, q_len;
  int64_t* slots;
};
hipError_t launch_draft_advance(const DraftParams& p, hipStream_t s);

// Parameters of the context-parallel combine.
struct CombineParams {
  const float* po;
  int64_t p_ps, p_ts, p_hs;  // elements
  const float* plse;         // [parts][rows][h_q]
  uint16_t* out;             // bf16 or fp32 (out_f32)
  int64_t out_ts, out_hs;
  int out_f32;
  float* lse;
  int parts, rows, h_q;
};
hipError_t launch_combine(const CombineParams& p, hipStream_t s);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* out, int blocks, hipStream_t s);
hipError_t launch_decode_codes(int kv_format, const uint8_t* codes, int n, float* out, hipStream_t s);

}  // namespace mj
