/*
 * mj.h -- paged decode attention over a quantized (e4m3 / packed e2m3) KV
 * cache on AMD Instinct MI355X (gfx950).  C ABI.
 *
 * One decode step is four calls on one HIP stream:
 *
 *   mj_plan_split_kv   host: the split-KV plan, copied (async) into a
 *                      fixed-address device buffer          (outside capture)
 *   mj_quantize_q      device: dynamic e4m3 Q per (sequence, KV head)
 *   mj_paged_decode    device: paged online-softmax attention
 *   mj_merge_lse       device: log-sum-exp merge of the split partials
 *                      (call it iff the plan says with_reduction)
 *
 * or, after the plan, as one call: mj_decode_step (quantize + decode + merge
 * fused into one kernel launch where the matrix-core kernel serves the
 * shape; the same three launches otherwise, with identical results).
 *
 * The method is the one the mjolnir-kernel 0.1.0 pages describe (PyPI project
 * page and sdist README, section "What it does", steps 1-4; wheel listing
 * mjolnir/runner.py, T5DecodeRunner.plan / .run / ._launch).  Their Thor
 * (sm_110) kernel design is prior art only; nothing here follows it.
 *
 * Conventions for every call:
 *  - Ownership: the caller allocates and owns every buffer (device memory,
 *    pinned host staging).  The library never allocates, frees or
 *    synchronizes; device calls only enqueue work on `stream` and borrow the
 *    pointers until that work has run.
 *  - Errors: every call returns an mj_status; invalid arguments are rejected
 *    on the host before anything is enqueued (no partial launches).  Nothing
 *    aborts or throws across the ABI.
 *  - Graph capture: mj_quantize_q, mj_paged_decode, mj_merge_lse,
 *    mj_decode_step and mj_plan_split_kv_device are capture-safe (their grids depend only on the config, q_len and
 *    num_seqs; every per-step value is read from device memory).
 *    mj_plan_split_kv must run outside capture; a captured graph replays any
 *    later plan written to the same plan buffer.
 *  - Shapes: head_dim is 128; page sizes 16, 32, 64, 128 (README
 *    "Requirements"); h_q % h_k == 0.
 */
#ifndef MJ_H
#define MJ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MJ_ABI_VERSION 9

typedef enum mj_status {
  MJ_OK = 0,
  MJ_EINVAL = -1,        /* null pointer, bad value, plan/launch mismatch        */
  MJ_EUNSUPPORTED = -2,  /* head_dim != 128, page size, h_q % h_k, kv format      */
  MJ_EALIGN = -3,        /* a base pointer or stride is not 16-byte aligned       */
  MJ_ECAPACITY = -4,     /* num_seqs / q_len / block table / buffer too small     */
  MJ_EHIP = -5           /* a HIP runtime call or kernel launch failed            */
} mj_status;

typedef enum mj_kv_format {
  MJ_KV_E4M3 = 0,  /* one OCP e4m3 (float8_e4m3fn) byte per value, 128-byte rows  */
  MJ_KV_E2M3 = 1,  /* OCP MX e2m3 6-bit codes, 4 per 3 bytes, 96-byte rows:
                      code k of a row is stream bits [6k, 6k+6), stream bit 8B+j
                      being bit j of byte B (runner.py, comment above
                      RUNNER_KV_FORMATS: "little-endian bitstream")             */
  MJ_KV_E3M2 = 2,  /* OCP MX e3m2 6-bit codes (bias 3, max 28), packed as e2m3
                      (project page, "Beyond fp8: the harness" names fp6
                      e3m2; the pages give no packing, the e2m3 bitstream is
                      taken)                                                    */
  MJ_KV_E2M1 = 3,  /* OCP MX e2m1 4-bit codes (bias 1, max 6), 64-byte rows:
                      code k is stream bits [4k, 4k+4), i.e. the low nibble of
                      byte k/2 for even k, the high nibble for odd k (same
                      section: fp4 e2m1; same bitstream reading)               */
  MJ_KV_NVFP4 = 4  /* block-scaled fp4 (same section: "nvfp4"; the runner
                      passes K and V "nvfp4 scale pointers"): e2m1 rows as
                      MJ_KV_E2M1, plus one e4m3 scale per 16 channels, i.e.
                      an 8-byte row per (token, KV head) in a block-scale
                      pool paged like the codes; value = e2m1(code c) *
                      e4m3(scale c/16) * the fp32 descale.  The pages give no
                      layout: this is the published NVFP4 block format.     */
} mj_kv_format;

/* How the decode takes Q (runner.py, T5DecodeRunner.__init__ `q_mode`, and
 * the backend's MJOLNIR_ATTN_Q_DTYPE): quantized per (sequence, KV head) to
 * e4m3 by mj_quantize_q, or used as is in bf16 with the KV codes converted
 * to bf16 inside the decode kernel (e4m3 and nvfp4 KV: the packed fp6 / fp4
 * caches take fp8 Q only, per the runner's kv_format comment). */
typedef enum mj_q_mode {
  MJ_Q_FP8 = 0,   /* dynamic e4m3 Q: mj_quantize_q, then q8 / q_descale        */
  MJ_Q_BF16 = 1   /* bf16 Q as given: logit = softmax_scale * k_descale *
                     sum_c q_c * dec(k_c); no Q quantization step           */
} mj_q_mode;

/* Shape of a K or V descale tensor (runner.py, T5DecodeRunner.run: k_scale /
 * v_scale are fp32 with 1 element, (h_k,) or (b, h_k)). */
typedef enum mj_scale_kind {
  MJ_SCALE_TENSOR = 0,   /* descale[0]                       */
  MJ_SCALE_HEAD = 1,     /* descale[g], g = KV head          */
  MJ_SCALE_SEQ_HEAD = 2, /* descale[i * h_k + g]             */
  MJ_SCALE_CHANNEL = 3   /* scale[g * 128 + c] (cache write only; backend.py
                            _install_fp6_scales: per (KV head, channel))     */
} mj_scale_kind;

/* Static configuration of one decode site (one KV-cache group).  Every size a
 * captured graph depends on (grid sizes, plan and workspace layout) is a
 * function of this struct and q_len only. */
typedef struct mj_config {
  int32_t h_q;             /* query heads                                      */
  int32_t h_k;             /* KV heads, h_q % h_k == 0                          */
  int32_t head_dim;        /* must be 128                                       */
  int32_t page_size;       /* tokens per page: 16, 32, 64 or 128                */
  int32_t max_num_seqs;    /* largest batch any plan or launch uses             */
  int32_t max_q_len;       /* largest q_len (1 + speculative tokens), >= 1      */
  int32_t max_splits;      /* most KV chunks per sequence; 1 = never split      */
  int32_t num_cus;         /* compute units to plan for; 0 = ask the device     */
  int32_t wgs_per_cu;      /* planned workgroups per CU; 0 = default (below)    */
  int32_t kv_tile_tokens;  /* plan granularity in tokens (multiple of 16); 0=128*/
  int32_t slots_override;  /* work items per plan; 0 = num_cus*wgs_per_cu/h_k   */
  int32_t kv_format;       /* mj_kv_format                                      */
  int32_t min_chunk_tokens;/* floor of a split chunk; 0 = default (below)       */
  int32_t q_mode;          /* mj_q_mode (0 = fp8)                               */
  int32_t out_f32;         /* 0: outputs `out` are bf16; 1: fp32 (a context-
                              parallel slice's result, combined later by
                              mj_combine_lse without rounding in between)    */
  /* Kernel selection of this decode site (0 = the library's choice; the
     other values exist for A/B measurements and for testing every kernel
     on the same inputs; results agree within the output tolerance, plans
     and codes bit for bit):                                               */
  int32_t decode_kernel;   /* 0 automatic (the matrix-core kernel wherever the
                              plan's KV tiles are whole 16-token tiles and
                              slot strides are < 2^24 bytes, else the generic
                              kernel); 1 always the generic LDS-tiled kernel;
                              10..73 the matrix-core kernel with tuning bits
                              (value - 10): bit 0 two granules of prefetch,
                              bit 1 head-major grid, bit 2 XCD-grouped grid
                              (the KV heads of a work item on one XCD; takes
                              precedence over bit 1), bit 3 four waves per
                              workgroup where the default runs eight (a
                              group of exactly one 32-row tile, e4m3 with
                              fp8 Q or e2m1; two granules of prefetch
                              always run four), bits 4-5 KV heads per
                              workgroup (0 the library's choice: four for
                              token-major packed pages, eight for e2m1 when
                              h_k is a multiple of 8; 1 one, 2 two, 3 four;
                              more than one only for the packed formats at
                              up to 16 query rows per KV head, h_k a
                              multiple, no in-kernel merge)                  */
  int32_t kv_cache_policy; /* matrix-core kernel KV loads: 0 the library's
                              choice (K cached, V non-temporal), 1 every load
                              cached, 2 every load non-temporal, 3 K cached
                              and V non-temporal, 4 K non-temporal and V
                              cached                                         */
  int32_t step_merge;      /* where mj_decode_step merges split partials when
                              it fuses the step: 0 automatic (the separate
                              merge launch), 1 in the decode kernel (the last
                              split item of a (sequence, KV head) to finish;
                              host-planned steps with at most 32 rows per KV
                              head, else the merge launch; every split
                              workgroup then issues an agent-scope release,
                              which costs more than the launch on gfx950),
                              2 the separate merge launch                    */
} mj_config;
/* Defaults of wgs_per_cu / min_chunk_tokens, per q_len (n_q = q_len*h_r):
 * e4m3 with n_q <= 16 -> 8 / 2048 (the matrix-core kernel runs two
 * workgroups per CU; four waves of items of >= 2048 tokens balance the tail
 * across CUs and XCDs); e2m1 / nvfp4 with n_q <= 32 -> 2 / 1; everything
 * else (16 < n_q <= 32, fp6 (e2m3 / e3m2), n_q > 32) -> 1 / 1 (one wave).
 * min_chunk_tokens is rounded up to whole KV tiles.  A batch whose
 * num_seqs*h_k*ceil(n_q/64) workgroups already reach every CU, and whose
 * block-table rows allow no split of more than 2*num_cus workgroups
 * (min(S, num_seqs*max(1, min(max_splits, floor(row tiles / min chunk
 * tiles)))) items at the default: the chunks of at least the floor that a
 * full row holds), plans one workgroup per CU instead: such a split
 * balances nothing and only adds the merge (32 sequences of 4K tokens x 8 KV
 * heads on 256 CUs: the same kernel time, a graph step 7 us shorter).  A
 * wgs_per_cu or slots_override given in the config is always kept. */

/* What a plan decided (runner.py, StepPlan). */
typedef struct mj_plan_info {
  int32_t num_work;        /* grid size of mj_paged_decode = capacity for q_len */
  int32_t slots;           /* work items that fill one wave (S)                  */
  int32_t chunk_tiles;     /* chunk length in kv tiles                          */
  int32_t num_chunks;      /* items with a non-empty KV range                   */
  int32_t with_reduction;  /* 1: some sequence is split; call mj_merge_lse      */
  int32_t num_seqs;
  int32_t q_len;
  int32_t kv_tile_tokens;
  int32_t min_chunk_tiles;  /* floor of the chunk for this q_len                */
  int32_t wgs_per_cu;       /* workgroups per CU the slot count was sized with
                               (the config's value or the default above, for
                               this batch size and table width)              */
} mj_plan_info;

/* Arguments of mj_paged_decode.  All strides are in BYTES for the KV cache and
 * in ELEMENTS (bf16) for the output. */
typedef struct mj_decode_args {
  /* Q from mj_quantize_q (MJ_Q_FP8; not read in MJ_Q_BF16 mode)            */
  const uint8_t* q8;          /* (num_seqs, h_k, q_len*h_r, 128) e4m3, contiguous */
  const float* q_descale;     /* (num_seqs, h_k)                                  */
  int32_t num_seqs;
  int32_t q_len;              /* 1 .. max_q_len                                   */
  int32_t causal;             /* q_len > 1: 1 = causal block, 0 = every query
                                 token sees every key (parallel drafter)          */
  /* KV cache: token j of sequence i, KV head g, starts at byte
     page*page_stride + (j % page_size)*slot_stride + g*head_stride of the
     pool, page = block_table[i*bt_row_stride + j/page_size].  HND and NHD
     (and K|V-interleaved pools) differ only in these strides.               */
  const void* k_cache;
  int64_t k_page_stride, k_slot_stride, k_head_stride;
  const void* v_cache;
  int64_t v_page_stride, v_slot_stride, v_head_stride;
  int64_t num_pages;          /* pages in each pool; a block-table entry outside
                                 [0, num_pages) masks its tokens (never read)      */
  const float* k_descale;     /* fp32 per mj_scale_kind                           */
  int32_t k_descale_kind;
  const float* v_descale;
  int32_t v_descale_kind;
  /* paging */
  const int32_t* block_table; /* int32, row i at block_table + i*bt_row_stride    */
  int64_t bt_row_stride;      /* elements                                          */
  int32_t max_blocks_per_seq; /* valid columns per row; tokens beyond
                                 max_blocks_per_seq*page_size are never read       */
  const int32_t* seq_lens;    /* device (num_seqs,), tokens incl. the q_len new   */
  /* plan (device buffer written by mj_plan_split_kv) */
  const int32_t* plan;
  int32_t num_work;           /* mj_plan_info.num_work                            */
  int32_t with_reduction;     /* mj_plan_info.with_reduction                      */
  void* workspace;            /* split partials; >= mj_workspace_bytes(cfg)       */
  size_t workspace_bytes;
  /* math */
  float softmax_scale;        /* natural-log scale of Q.K (1/sqrt(128) usually)   */
  const float* o_mul;         /* nullable (h_q, 128) fp32: O *= o_mul (fp6 V
                                 channel scales folded into the output)           */
  /* outputs */
  void* out;                  /* bf16 (num_seqs*q_len, h_q, 128) through strides  */
  int64_t out_tok_stride, out_head_stride;
  float* lse;                 /* nullable (num_seqs*q_len, h_q) fp32, natural log */
  /* bf16 Q (MJ_Q_BF16 mode only; not read in MJ_Q_FP8 mode): element
     (token, head, c) at q_bf16[token*q_tok_stride + head*q_head_stride + c],
     token = i*q_len + t; 16-byte aligned, strides multiples of 8 elements  */
  const void* q_bf16;
  int64_t q_tok_stride, q_head_stride;
  /* MJ_KV_NVFP4 only (not read otherwise): the 8-byte block-scale row of
     token j, KV head g starts at byte page*page_stride + (j %
     page_size)*slot_stride + g*head_stride of the block-scale pool, page
     from the same block table (each block-scale pool holds num_pages pages
     too); bases 8-byte aligned, strides multiples of 8 bytes (EALIGN),
     non-null (EINVAL)                                                         */
  const void* k_block_scale;
  int64_t k_bs_page_stride, k_bs_slot_stride, k_bs_head_stride;
  const void* v_block_scale;
  int64_t v_bs_page_stride, v_bs_slot_stride, v_bs_head_stride;
} mj_decode_args;

typedef struct mj_merge_args {
  const int32_t* plan;
  int32_t num_seqs;
  int32_t q_len;
  const void* workspace;
  size_t workspace_bytes;
  void* out;                  /* same output as mj_paged_decode                   */
  int64_t out_tok_stride, out_head_stride;
  float* lse;                 /* nullable                                          */
} mj_merge_args;

/* ------------------------------------------------------------------------ */
const char* mj_status_string(mj_status s);
int32_t mj_abi_version(void);

/* Validate a config (shapes, formats, limits).  Host only. */
mj_status mj_config_check(const mj_config* cfg);

/* Byte sizes of the caller-allocated buffers; 0 for an invalid config.
 * Plan buffer: int32 [work: cap_max x 4][n_splits: max_num_seqs]
 * [split_begin: max_num_seqs], cap_max = the largest capacity over q_len.
 * Workspace: fp32 split partials for the largest slots(q_len) * q_len * h_r
 * rows per KV head over q_len, not sized by the batch (the plan splits only
 * batches smaller than one wave), then
 * mj_decode_step's arrival counters (int32, max_num_seqs x h_k) and its Q
 * staging (e4m3 codes and scales, used when the step is not fused).  The
 * counters must be zero before the first mj_decode_step on a workspace (zero
 * the whole buffer once after allocating it); every completed mj_decode_step
 * leaves them zero again.  The other calls never touch them. */
size_t mj_plan_buffer_bytes(const mj_config* cfg);
size_t mj_workspace_bytes(const mj_config* cfg);

/* Largest decode grid (work items) any plan for q_len can have: max(S,
 * max_num_seqs), S as below; -1 on error.  Host only (queries the current
 * device when cfg->num_cus == 0).  A plan's own grid is mj_plan_info.num_work,
 * which is never larger. */
int32_t mj_plan_capacity(const mj_config* cfg, int32_t q_len);

/* The split-KV plan (README "What it does", step 1; runner.py
 * T5DecodeRunner.plan and __init__ "Capacity per q_len"):
 *   slots S = max(1, num_cus*wgs_per_cu / (h_k*ceil(q_len*h_r/64))), or the
 *   override; with T = max_blocks_per_seq * page_size (the tokens a block-table
 *   row addresses; nothing past them is ever read), tiles_i =
 *   ceil(min(seq_lens_host[i] + margin, T) / kv_tile_tokens).  The plan
 *   splits iff max_splits > 1, num_seqs < S and ceil(T / kv_tile_tokens) >
 *   min chunk tiles (a sequence filling its row could be cut in two; else
 *   every sequence is one item whatever the lengths and no merge is
 *   needed).  A split plan takes the smallest chunk c >= max(ceil(max tiles
 *   / max_splits), min chunk tiles) whose item count sum_i
 *   max(1,ceil(tiles_i/c)) fits S; otherwise one item per sequence.  Items
 *   (seq, tile_begin, tile_end, split) are sequence-major and padded with
 *   (-1,0,0,0).  The grid num_work is max(S, max_num_seqs) for a plan that
 *   may split and max_num_seqs for one that cannot: it depends on the
 *   config, q_len, num_seqs and max_blocks_per_seq only, never on the
 *   lengths, so a captured step replays later plans of that batch.
 * mj_plan_compute writes the whole plan image into plan_host
 * (mj_plan_buffer_bytes bytes) without touching the device.
 * mj_plan_split_kv does the same into `host_staging` (pinned, caller-owned;
 * must not be rewritten until the copy has run on `stream`) and enqueues one
 * hipMemcpyAsync of it into `plan_dev`.
 * Errors: EINVAL (null, num_seqs < 1, q_len out of 1..max_q_len, negative
 * length or margin), ECAPACITY (num_seqs > max_num_seqs, a sequence needs
 * more than max_blocks_per_seq pages), EHIP. */
mj_status mj_plan_compute(const mj_config* cfg, const int32_t* seq_lens_host, int32_t num_seqs, int32_t q_len,
                          int32_t margin, int32_t max_blocks_per_seq, int32_t* plan_host, mj_plan_info* info);
mj_status mj_plan_split_kv(const mj_config* cfg, const int32_t* seq_lens_host, int32_t num_seqs, int32_t q_len,
                           int32_t margin, int32_t max_blocks_per_seq, int32_t* host_staging, int32_t* plan_dev,
                           mj_plan_info* info, hipStream_t stream);

/* The same plan computed on the device from device lengths (one workgroup):
 * seq_lens_dev[i] is clamped to [0, max_blocks_per_seq * page_size] as the
 * decode kernels clamp it, then the rule above applies unchanged, so the plan
 * buffer is bit-identical to mj_plan_split_kv's for valid lengths.  It reads
 * only device memory, so it may be captured in a hipGraph together with the
 * other three calls; replays then re-plan from whatever lengths the device
 * buffer holds.  `info` gets everything the host can know from num_seqs and
 * q_len (num_work, slots, with_reduction; chunk_tiles = num_chunks = -1).
 * plan_dev must be 16-byte aligned.  Errors: EINVAL, ECAPACITY, EALIGN, EHIP. */
mj_status mj_plan_split_kv_device(const mj_config* cfg, const int32_t* seq_lens_dev, int32_t num_seqs, int32_t q_len,
                                  int32_t margin, int32_t max_blocks_per_seq, int32_t* plan_dev, mj_plan_info* info,
                                  hipStream_t stream);

/* What a plan for (num_seqs, q_len) over block-table rows of
 * max_blocks_per_seq pages has regardless of the lengths: num_work, slots,
 * with_reduction, kv_tile_tokens, min_chunk_tiles, wgs_per_cu (chunk_tiles =
 * num_chunks = -1).  Host only.  Errors: EINVAL, ECAPACITY. */
mj_status mj_plan_shape(const mj_config* cfg, int32_t num_seqs, int32_t q_len, int32_t max_blocks_per_seq,
                        mj_plan_info* info);

/* Dynamic e4m3 quantization of Q per (sequence, KV head) (README "What it
 * does", step 2; runner.py T5DecodeRunner.run, fp8-Q branch): over the q_len
 * tokens and h_r heads of KV head g, x = fp32(q) [* q_mul], amax =
 * max(max|x|, 1e-6f), s = amax / 448 (IEEE fp32 division), code =
 * RNE_e4m3(x / s) (IEEE division), q_descale[i*h_k+g] = s.  Rows are packed
 * t*h_r + r for token t, query head g*h_r + r.
 *   q: bf16, element (token, head, c) at q[token*q_tok_stride +
 *      head*q_head_stride + c], token = i*q_len + t (a strided view of a
 *      fused QKV buffer works); 16-byte aligned, strides multiples of 8.
 *   q_mul: nullable (h_q, 128) fp32 (fp6 K channel scales folded into Q).
 *   q8: (num_seqs, h_k, q_len*h_r, 128) bytes; q_descale: (num_seqs, h_k).
 * It does not depend on cfg->q_mode (a MJ_Q_BF16 step simply never calls it).
 * Errors: EINVAL, EALIGN, ECAPACITY, EHIP. */
mj_status mj_quantize_q(const mj_config* cfg, const void* q, int64_t q_tok_stride, int64_t q_head_stride,
                        const float* q_mul, int32_t num_seqs, int32_t q_len, uint8_t* q8, float* q_descale,
                        hipStream_t stream);

/* Paged decode attention (README "What it does", step 3): for every plan item
 * (sequence i, token range) and KV head g, logit = softmax_scale *
 * q_descale[i,g] * k_descale * sum_c dec(q8)*dec(k) (MJ_Q_FP8), or
 * softmax_scale * k_descale * sum_c q*dec(k) with the bf16 q_bf16 rows
 * (MJ_Q_BF16; the products are exact in fp32) over the keys the row may
 * see (causal token t of a q_len block sees keys 0 .. L-q_len+t; q_len == 1
 * or non-causal: 0 .. L-1), online softmax, O = v_descale * sum_j p_j dec(v_j)
 * [* o_mul].  A sequence with one item writes bf16 O and LSE directly; a
 * split sequence writes fp32 partials (unnormalized O, running max, sum) to
 * the workspace for mj_merge_lse.  A row that sees no key writes O = 0,
 * LSE = -inf.
 * Errors: EINVAL (nulls, negative strides, descale kind out of range,
 * num_work / with_reduction not those of a plan for this config and q_len),
 * EALIGN (k/v/q8/q_bf16/out bases or byte strides not 16-byte aligned, out
 * and q_bf16 strides not multiples of 8 elements), ECAPACITY (num_seqs, q_len, workspace
 * missing or too small for a split plan), EUNSUPPORTED, EHIP. */
mj_status mj_paged_decode(const mj_config* cfg, const mj_decode_args* args, hipStream_t stream);

/* Log-sum-exp merge of the split partials (README "What it does", step 4):
 * for each split sequence, M = max_s m_s, O = sum_s e^{m_s-M} O_s /
 * sum_s e^{m_s-M} l_s, LSE = M + ln sum_s e^{m_s-M} l_s; writes bf16 O and
 * LSE.  Sequences with a single item are left untouched (mj_paged_decode
 * already wrote them).  Errors: EINVAL, ECAPACITY, EALIGN, EHIP. */
mj_status mj_merge_lse(const mj_config* cfg, const mj_merge_args* args, hipStream_t stream);

/* Arguments of mj_write_kv.  Strides of key/value in ELEMENTS (bf16), of
 * the caches in BYTES (the same pools and strides mj_paged_decode reads). */
typedef struct mj_write_args {
  const void* key;              /* bf16 (num_tokens, h_k, 128), channel stride 1 */
  int64_t key_tok_stride, key_head_stride;
  const void* value;
  int64_t value_tok_stride, value_head_stride;
  int32_t num_tokens;
  const int64_t* slot_mapping;  /* device (num_tokens): page * page_size + row;
                                   negative = padding token, not written     */
  void* k_cache;
  int64_t k_page_stride, k_slot_stride, k_head_stride;
  void* v_cache;
  int64_t v_page_stride, v_slot_stride, v_head_stride;
  int64_t num_pages;            /* slots in pages >= num_pages are skipped   */
  const float* k_scale;         /* divisor(s) of the write                   */
  int32_t k_scale_kind;         /* TENSOR, HEAD or CHANNEL                   */
  const float* v_scale;
  int32_t v_scale_kind;
  /* MJ_KV_NVFP4 only: the block-scale pools, as in mj_decode_args */
  void* k_block_scale;
  int64_t k_bs_page_stride, k_bs_slot_stride, k_bs_head_stride;
  void* v_block_scale;
  int64_t v_bs_page_stride, v_bs_slot_stride, v_bs_head_stride;
} mj_write_args;

/* The KV-cache write of a step's new rows (wheel listing
 * mjolnir/backend.py, do_kv_cache_update: an fp8 cache written with the
 * layer's per-tensor or per-head scale, the fp6 cache with per-(KV head,
 * channel) scales, _install_fp6_scales).  Every value becomes
 * RNE(x / scale) in the config's KV format, saturated at its largest
 * magnitude (448 e4m3, 7.5 e2m3, 28 e3m2, 6 e2m1), x the fp32 value of the
 * bf16 input and the division correctly rounded; sub-byte rows are packed
 * as mj_paged_decode reads them.  nvfp4 (the published NVFP4 recipe; the
 * pages print no writer): with y = x / scale as above, each 16-channel
 * block's e4m3 scale is RNE(amax|y| / 6) saturated at 448, each code
 * RNE_e2m1(y / e4m3(block scale)) (both divisions correctly rounded), and a
 * block whose scale is 0 stores zero codes.  Tokens are
 * independent; two tokens mapped to one slot race (the caller's contract,
 * as in any slot-mapped write).  num_tokens == 0 enqueues nothing.
 * Errors: EINVAL (nulls, negative strides or counts, scale kind), EALIGN
 * (key/value/cache bases not 16-byte aligned, key/value strides not
 * multiples of 8 elements, cache strides not multiples of 16 bytes),
 * EUNSUPPORTED (SEQ_HEAD scales), EHIP. */
mj_status mj_write_kv(const mj_config* cfg, const mj_write_args* args, hipStream_t stream);

/* Multi-step draft decode (runner.py, T5DecodeRunner.plan: a plan made
 * `margin` tokens long stays valid while the device seq_lens grow by up to
 * margin, since the kernels mask with the live lengths; backend.py: the
 * speculator runs every draft step on one metadata build and advances the
 * device seq_lens in place).  mj_draft_advance is that advance, on the
 * device so that a whole draft loop (advance, mj_write_kv of the new rows,
 * mj_decode_step on the margin plan) is one captured graph: for every
 * sequence i < num_seqs with L = seq_lens[i] > 0, slot_mapping[i*q_len + t]
 * = the cache slot of token position L + t (page block_table[i*bt_row_stride
 * + (L+t)/page_size], as mj_write_kv takes it), for t < q_len, and then
 * seq_lens[i] = min(L + q_len, max_blocks_per_seq * page_size).  A length-0
 * sequence (graph padding) stays 0; slots of positions past the block table
 * are -1 (not written).  One thread per sequence; the caller keeps the
 * block table's pages for the new positions valid.
 * Errors: EINVAL (nulls, num_seqs < 1, q_len < 1, bt_row_stride <
 * max_blocks_per_seq, max_blocks_per_seq < 1), ECAPACITY (num_seqs >
 * max_num_seqs, q_len > max_q_len), EALIGN (slot_mapping not 8-byte aligned),
 * EHIP. */
typedef struct mj_draft_args {
  const int32_t* block_table;   /* device, row i at block_table + i*bt_row_stride */
  int64_t bt_row_stride;        /* elements                                   */
  int32_t max_blocks_per_seq;
  int32_t* seq_lens;            /* device (num_seqs,), advanced in place        */
  int32_t num_seqs;
  int32_t q_len;                /* tokens appended per sequence                */
  int64_t* slot_mapping;        /* device (num_seqs * q_len,), written          */
} mj_draft_args;
mj_status mj_draft_advance(const mj_config* cfg, const mj_draft_args* args, hipStream_t stream);

/* Context-parallel combine (the pages' split-KV reduction, README "What it
 * does" step 4, across GPUs instead of within one): every GPU of a context-
 * parallel group holds a slice of each sequence's pages and runs the decode
 * on it (out_f32 = 1 in its config: fp32 O normalized over the slice, and
 * its LSE); after one all-gather of those (the caller's collective), this
 * merges the num_parts slices per (token, query head):
 *   M = max_p lse_p,  w_p = exp(lse_p - M),
 *   out = sum_p w_p o_p / sum_p w_p,  lse = M + ln sum_p w_p,
 * a row no slice saw (every lse_p = -inf) giving out = 0, lse = -inf.  The
 * slices must partition the context; with q_len > 1 and causal masking the
 * last slice must hold each sequence's last q_len tokens (it runs causal,
 * the others non-causal).  Output dtype per cfg->out_f32.
 * Errors: EINVAL (nulls, num_parts < 1, num_rows < 1, negative strides),
 * EALIGN (part_out / out not 16-byte aligned or strides not multiples of 4
 * (fp32) / 8 (bf16) elements), EHIP. */
typedef struct mj_combine_args {
  int32_t num_parts;            /* slices (GPUs of the group)                  */
  int32_t num_rows;             /* tokens: num_seqs * q_len                    */
  const float* part_out;        /* fp32; slice p, token t, query head h,
                                   channel c at part_out[p*part_stride +
                                   t*part_tok_stride + h*part_head_stride + c] */
  int64_t part_stride, part_tok_stride, part_head_stride;  /* elements         */
  const float* part_lse;        /* fp32 [num_parts][num_rows][h_q], natural log */
  void* out;                    /* bf16 or fp32 (cfg->out_f32), (num_rows, h_q,
                                   128) through the strides                    */
  int64_t out_tok_stride, out_head_stride;  /* elements                        */
  float* lse;                   /* nullable [num_rows][h_q]                    */
} mj_combine_args;
mj_status mj_combine_lse(const mj_config* cfg, const mj_combine_args* args, hipStream_t stream);

/* Arguments of one whole decode step after the plan: the decode arguments
 * (decode.q8, decode.q_descale and decode.q_bf16 are not read and may be
 * NULL;
 * decode.workspace is required, >= mj_workspace_bytes(cfg), 256-byte
 * aligned, counters zeroed once as described above) plus bf16 Q as
 * mj_quantize_q takes it. */
typedef struct mj_step_args {
  mj_decode_args decode;
  const void* q;                /* bf16; see mj_quantize_q for layout       */
  int64_t q_tok_stride;         /* elements                                  */
  int64_t q_head_stride;        /* elements                                  */
  const float* q_mul;           /* nullable (h_q, 128); must be NULL in
                                   MJ_Q_BF16 mode (EUNSUPPORTED)             */
  int32_t plan_on_device;       /* 1: plan this step from decode.seq_lens
                                   (as mj_plan_split_kv_device, with margin
                                   below) instead of reading a prepared plan;
                                   decode.plan still receives the plan's
                                   n_splits / split_begin                    */
  int32_t margin;               /* plan margin when plan_on_device           */
} mj_step_args;

/* mj_quantize_q + mj_paged_decode + mj_merge_lse (README "What it does",
 * steps 2-4) as one call with the same results bit for bit.  Where the
 * matrix-core kernel serves the shape (q_len*h_r <= 32, whole 16-token
 * tiles, slot strides < 2^24 bytes), every decode workgroup quantizes its
 * (sequence, KV head)'s Q rows in its prologue with the quantize kernel's
 * arithmetic, so the step is the decode launch plus, for a split plan, the
 * merge launch; optionally (cfg->step_merge = 1) the last split item of
 * a pair to finish merges in the decode kernel itself (device-coherent
 * partials, an arrival counter in the workspace) and the step is one
 * launch.  Otherwise it enqueues the three kernels, staging Q codes in the
 * workspace.  With plan_on_device the step also plans: where the matrix-core
 * kernel serves the shape and num_seqs <= 256, every decode workgroup
 * derives its own work item from the device lengths (the planner's rule,
 * no plan launch, the separate merge launch); otherwise the device planner
 * runs first.  The result is bit-identical to planning with
 * mj_plan_split_kv_device and calling the step on that plan.  In MJ_Q_BF16
 * mode there is nothing to quantize: the step is mj_paged_decode (+ merge)
 * reading `q` as decode.q_bf16.  Calls that
 * share a workspace must not overlap (one stream, or ordered streams).
 * Errors: those of the three calls. */
mj_status mj_decode_step(const mj_config* cfg, const mj_step_args* args, hipStream_t stream);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): mj_decode_step
 * with the plan buffer and the workspace taken from a static device array of
 * the library instead of the caller's buffers.  The array holds
 * MJ_NOALLOC_SCRATCH_BYTES per GPU the library runs on, from the first call
 * on that GPU until the process ends; a config needing more
 * (mj_noalloc_scratch_bytes: the plan buffer rounded up to 256 bytes plus
 * the workspace) is rejected with ECAPACITY before anything is enqueued.
 * args->decode.plan and args->decode.workspace must be NULL and
 * args->plan_on_device 1 (the step plans from the device lengths; num_work
 * and with_reduction come from mj_plan_shape); cfg->step_merge 1 is
 * EUNSUPPORTED.  The call allocates and frees nothing.  Every call on one
 * GPU shares that GPU's array: calls that overlap on one GPU (streams with
 * no ordering between them) race.  Results are those of mj_decode_step on
 * caller-owned buffers, bit for bit.  Errors: those of mj_decode_step,
 * EINVAL (a plan or workspace pointer given, plan_on_device 0), ECAPACITY,
 * EUNSUPPORTED, EHIP. */
#define MJ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
size_t mj_noalloc_scratch_bytes(const mj_config* cfg);
mj_status mj_decode_step_noalloc(const mj_config* cfg, const mj_step_args* args, hipStream_t stream);

/* Test probes (not part of a decode step).
 * mj_debug_gather_kv copies the codes of tokens 0..seq_len-1 of one
 * (sequence, KV head) from the K (which = 0) or V (which = 1) pool, or for
 * nvfp4 the block scales from the K (which = 2) or V (which = 3) block-scale
 * pool, into dense_out (seq_len x row bytes), using the decode kernel's own
 * address computation.  mj_debug_decode_codes decodes n codes (one per byte; 6-
 * and 4-bit codes in the low bits) with the kernel's own decoder of format
 * kv_format (an mj_kv_format) into fp32; kv_format 16 decodes e4m3 codes
 * through the bf16 operand converter of the MJ_Q_BF16 decode (fp32 of the
 * bf16 it yields). */
mj_status mj_debug_gather_kv(const mj_config* cfg, const mj_decode_args* args, int32_t seq, int32_t head,
                             int32_t seq_len, int32_t which, uint8_t* dense_out, hipStream_t stream);
mj_status mj_debug_decode_codes(int32_t kv_format, const uint8_t* codes, int32_t n, float* out, hipStream_t stream);
/* Plain streaming read of `bytes` (a multiple of 16, 16-byte aligned) with
 * non-temporal 16-byte loads by `blocks` workgroups of 256 threads, each
 * writing one xor checksum to out[block]: the practical HBM read ceiling the
 * decode kernels are compared with.  EINVAL on bad arguments. */
mj_status mj_debug_stream_read(const void* src, int64_t bytes, uint32_t* out, int32_t blocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MJ_H */
