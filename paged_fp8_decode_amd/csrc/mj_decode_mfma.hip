// Paged decode for GQA groups of up to 32 query rows (q_len * h_r <= 32)
// with both products on the gfx950 matrix cores; e4m3, packed fp6 (e2m3,
// e3m2) or packed fp4 (e2m1) KV.
// The description below is for the 4-row instance; 8- and 16-row groups use
// one 16-row block (column n = row n), 32-row groups two blocks, with the
// same operand layouts per block and the max raised wave-uniformly.
//
// Fused step (mj_decode_step): the prologue quantizes the pair's Q rows into
// LDS with the stand-alone quantize kernel's arithmetic, and after writing
// its split partials (device-coherent stores) the last split item of a
// (sequence, KV head) to arrive merges them (mj_merge.h).
//
// bf16-Q mode (the runner's q_mode "bf16": Q as is, KV converted in the
// kernel; FMT 2 below): the lane's 32 K codes of a tile become bf16 with the
// hardware converter (exact) and QK^T is four v_mfma_f32_16x16x32_bf16 per
// tile, the lane's codes [32jj + 8i, 32jj + 8i + 8) forming the contraction
// slice of MFMA i; Q's B operands are the same channels of the bf16 rows,
// loaded as they are.  Products of bf16 values are exact in fp32, so only
// the accumulation rounds.  nvfp4 KV (FMT 5 with fp8 Q, FMT 6 with bf16 Q)
// takes the same route: its fp4 codes times their e4m3 block scales are
// bf16 values, and fp8 Q codes become bf16 B operands.
//
// Method: mjolnir-kernel README "What it does", step 3 (stream KV pages,
// online softmax) and the partials step 4 merges.  The pages' Thor design
// (TMA ring into shared memory, TMEM accumulators, fp8 P) is not followed;
// P stays in bf16 here.
//
// Work split: one workgroup (4 waves) per (plan item, KV head); 32-token
// granules are dealt round-robin to the waves, which stream 4 adjacent
// granules at a time and merge their softmax states through LDS at the end.
// Lane l = 16*jj + n.
//
// QK^T (v_mfma_f32_16x16x128_f8f6f4 on e4m3 bytes): A = 16 tokens of K
// (lane (n, jj): token n, codes [32jj, 32jj+32)), B = the Q rows (column n =
// Q row n % 4, i.e. the <= 4 rows replicated four times).  The result puts
// the logits of tokens 4jj..4jj+3 of the tile for Q row n % 4 in lane
// (n, jj).  K goes in as loaded: e4m3 bytes, e2m3 / e3m2 codes (24 bytes per
// lane) as the instruction's fp6 / bf6 operand, or e2m1 codes (16 bytes per
// lane) as its fp4 operand, the Q operand staying e4m3.
//
// PV (v_mfma_f32_16x16x32_bf16): over one granule, lane (n, jj) holds p for
// the 8 tokens tau(jj, e) = 16*(e/4) + 4*jj + e%4, e = 0..7, of row n % 4.
// Taking e as the contraction index of lane group jj makes these 8 values
// exactly the A operand (row n = P of Q row n % 4) -- no data movement.  The
// B operand needs V[tau(jj, e)][channel] for the lane's column: lane (n, jj)
// loads channels 8n..8n+7 of its 8 tokens (one 8-byte load per token, 4
// bytes for e2m1; 4 tokens x whole rows per load instruction), converts them
// to fp32 (exact for every format) and packs
// token pairs of one channel into bf16 words, giving 8 B operands (channel
// 8n + q, q = 0..7).  Eight MFMAs per granule leave O for all 4 rows and
// channel 8n + q in every lane: the sum over tokens happens in the matrix
// core and the accumulators are only 32 values per lane.
//
// Loads run one granule ahead (K and V double-buffered in registers) through
// buffer resources built per tile in scalar registers: the per-lane offsets
// are loop-invariant, and a dead tile (past the range end, invalid page) has
// zero records, so its loads return zeros without a branch and the wait
// before each use only covers the granule being computed.  KV bytes are
// read once, non-temporally.  The softmax max per row is raised lazily (only
// when a granule exceeds it by more than 8 in log2 units), which is exact.
#include <type_traits>

#include "mj_device.h"
#include "mj_internal.h"
#include "mj_merge.h"
#include "mj_plan_item.h"

namespace mj {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// XCDs of the part: consecutive workgroups of a launch go to them in turn
constexpr int kXcds = 8;
constexpr int kGran = 32;
constexpr float kLazyMax = 8.0f;
constexpr int kE8m0One = 127;
// Buffer resource word 3 for raw (untyped) buffer loads on gfx9-family parts.
constexpr int kRsrcWord3 = 0x00020000;

template <int FMT>
struct Fmt;
template <>
struct Fmt<0> {                     // e4m3: 128-byte rows
  static constexpr int kKDw = 8;    // K dwords per lane per tile (32 codes)
  static constexpr int kKOff = 32;  // K bytes per lane group
  static constexpr int kMfmaFmt = 0;  // f8f6f4 operand format of K: fp8 e4m3
  static constexpr uint32_t kRow = 128;  // bytes per 128-channel row
  static constexpr int kVDw = 2;    // V dwords per token per lane (channels 8n..8n+7)
  static constexpr bool kPacked6 = false;
  static constexpr bool kQkBf16 = false;     // QK^T on bf16 MFMAs (K converted in registers)
  static constexpr bool kQBf16 = false;      // Q given in bf16 (no Q quantization)
  static constexpr bool kBlockScaled = false;  // nvfp4: an e4m3 scale per 16 channels
  static constexpr bool kQkF16 = false;      // QK^T on fp16 MFMAs
  static constexpr bool kPvF16 = false;      // PV on fp16 MFMAs (P and V in fp16)
};
template <>
struct Fmt<1> {                     // e2m3: 96-byte rows, 4 codes per 3 bytes
  static constexpr int kKDw = 6;
  static constexpr int kKOff = 24;
  static constexpr int kMfmaFmt = 2;  // fp6 e2m3: 32 codes in 6 dwords, code k at bits [6k, 6k+6)
  static constexpr uint32_t kRow = 96;
  static constexpr int kVDw = 2;    // the 4-aligned 8 bytes holding the lane's 48 bits
  static constexpr bool kPacked6 = true;
  static constexpr bool kQkBf16 = false;
  static constexpr bool kQBf16 = false;
  static constexpr bool kBlockScaled = false;
  static constexpr bool kQkF16 = false;
  static constexpr bool kPvF16 = false;
};
template <>
struct Fmt<2> : Fmt<0> {            // e4m3 KV with bf16 Q (bf16 MFMAs for QK^T)
  static constexpr bool kQkBf16 = true;
  static constexpr bool kQBf16 = true;
};
template <>
struct Fmt<3> : Fmt<1> {            // e3m2: packed like e2m3
  static constexpr int kMfmaFmt = 3;  // bf6 e3m2, same operand layout as fp6
};
template <>
struct Fmt<4> {                     // e2m1: 64-byte rows, 2 codes per byte
  static constexpr int kKDw = 4;
  static constexpr int kKOff = 16;
  static constexpr int kMfmaFmt = 4;  // fp4 e2m1: 32 codes in 4 dwords, code k at bits [4k, 4k+4)
  static constexpr uint32_t kRow = 64;
  static constexpr int kVDw = 1;
  static constexpr bool kPacked6 = false;
  static constexpr bool kQkBf16 = false;
  static constexpr bool kQBf16 = false;
  static constexpr bool kBlockScaled = false;
  static constexpr bool kQkF16 = false;
  static constexpr bool kPvF16 = false;
};
// nvfp4: e2m1 rows as Fmt<4> plus an 8-byte row of e4m3 block scales.  The
// matrix cores' block scales are powers of two per 32 values, so they cannot
// carry e4m3 scales per 16: K and V are scaled in registers.  An e2m1 value
// times an e4m3 scale has at most 6 significant bits and lies in [2^-10,
// 2688], so it is exact in fp16 (and bf16).  The converters apply the power
// of two of their fp32 scale operand only (measured on gfx950), so a block
// scale s = 2^E * M is applied as the converter's 2^E and one packed fp16
// multiply by M (3 fraction bits at most).  Fmt<5> (fp8 Q): QK^T on fp16
// MFMAs with the Q codes converted to fp16 (exact); Fmt<6> (bf16 Q): QK^T on
// bf16 MFMAs with K scaled in fp32.  PV runs on fp16 MFMAs in both, P
// rounded to fp16.
template <>
struct Fmt<5> : Fmt<4> {
  static constexpr int kMfmaFmt = 0;  // Q operands in the fp8 channel order
  static constexpr bool kBlockScaled = true;
  static constexpr bool kQkF16 = true;
  static constexpr bool kPvF16 = true;
};
template <>
struct Fmt<6> : Fmt<5> {
  static constexpr bool kQBf16 = true;
  static constexpr bool kQkBf16 = true;
  static constexpr bool kQkF16 = false;
};
// Byte offsets in a Q row of the two 16-byte halves of lane group jj's fp8
// B operand.  Against fp8 K the lane group's 32 bytes pair with the K codes
// of the same lane group, so they are Q channels [32jj, 32jj + 32).  Against
// fp6, bf6 or fp4 K, measured on gfx950 (the three share one pairing): code
// c of A lane group jj meets byte 16(jj / 2) + c % 16 of fp8 lane group
// 2(jj % 2) + c / 16; with K lane group jj holding channels [32jj, 32jj + 32),
// B lane group jj then needs channels [16jj, 16jj + 16) and
// [64 + 16jj, 64 + 16jj + 16).
template <int FMT>
__device__ __forceinline__ int q_half_offset(int jj, int h) {
  return Fmt<FMT>::kMfmaFmt == 0 ? 32 * jj + 16 * h : 16 * jj + 64 * h;
}

template <int FMT>
struct KRows {  // tile k: this lane's codes [32jj, 32jj+32) of token n
  int pg[2];    // the two tiles' pages (-1: dead), wave-uniform: found once, at the loads
  uint32_t d[2][Fmt<FMT>::kKDw];
  uint32_t s[Fmt<FMT>::kBlockScaled ? 2 : 1];  // nvfp4: scales of blocks 2jj, 2jj + 1 (low 16 bits)
};
template <int FMT>
struct VRows {  // element e: the bytes holding channels 8n..8n+7 of token tau(jj, e)
  uint32_t d[8][Fmt<FMT>::kVDw];
  uint32_t s[Fmt<FMT>::kBlockScaled ? 8 : 1];  // nvfp4: scale of block n / 2 (low byte)
};

__device__ __forceinline__ float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
// max(a, b) as the median of (a, b, inf) with inf = +inf: one instruction,
// where fmaxf first quiets each operand it cannot prove came from
// arithmetic (the logits reach the max through the masking branch),
// doubling the count.  inf must be a run-time value (a kernel argument):
// with the constant the median is folded back into fmaxf.
__device__ __forceinline__ float fmax2(float a, float b, float inf) { return __builtin_amdgcn_fmed3f(a, b, inf); }

// reduce over the 4 lane groups jj (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float max_jj(float x, float inf) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmax2(__uint_as_float(a[0]), __uint_as_float(a[1]), inf);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax2(__uint_as_float(b[0]), __uint_as_float(b[1]), inf);
}
// Keeps the scheduler from hoisting the next granule's computation above the
// loads just issued: the wait before that computation then leaves the new
// loads in flight instead of draining every load.
__device__ __forceinline__ void issue_fence() { __builtin_amdgcn_sched_barrier(0); }

// Head groups on token-major pages: one 128-byte line holds parts of
// neighbouring heads' rows (e2m3's 96-byte rows straddle lines, e2m1 packs two
// heads per line), read by different waves.  Left alone the waves drift apart
// over a long item and a line leaves the L2 between its two readers (cfg3's
// shape in e2m3 fetched 1.35 times its KV bytes).  A workgroup barrier before
// every P-th granule keeps them within P granules of each other (e2m3 1.02
// times).  It is taken only among a wave's first `end` granules, which every
// wave of the workgroup has, so that every wave passes the same barriers;
// global loads stay in flight across it.  P = 0: none.
template <int P>
__device__ __forceinline__ void group_lockstep(int& it, int end) {
  if constexpr (P > 0) {
    static_assert((P & (P - 1)) == 0, "power of two");
    if (it < end && (it & (P - 1)) == 0) __builtin_amdgcn_s_barrier();
    ++it;
  }
}

// 2^x with the hardware instruction alone: arguments are <= 0 (a logit
// minus a running max at least as large) or -inf, and results below the
// smallest normal flush to 0, which no sum of probabilities can see.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// two fp32 -> one word of two bf16 (round to nearest even; exact for KV values)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const v2bf v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

struct Ctx {
  const int32_t* bt_row;
  const uint8_t* kpool;  // pool + head offset (wave-uniform)
  const uint8_t* vpool;
  int64_t k_sp, v_sp;
  uint32_t k_ss, v_ss;
  uint32_t k_rec, v_rec; // bytes a 16-token tile spans from its first row
  uint32_t k_lane;       // n * k_ss + codes offset of lane group jj
  uint32_t v_lane;       // 4 * jj * v_ss + byte offset of channel 8n (4-aligned)
  uint32_t num_pages;    // clamped to 2^31 - 1
  int j0, j1, page_shift, pmask, lim0, causal, n, jj;
  int jcap;              // end of the item's range clamped to the block-table row, not to the length
  int v_shift;           // e2m3: bit offset of channel 8n in the loaded 8 bytes
  float cscale;
  float pos_inf;         // +inf (kernel argument; see fmax2)
  // nvfp4 block-scale pools, addressed like the codes (8-byte rows)
  const uint8_t* ksbpool;
  const uint8_t* vsbpool;
  int64_t ksb_sp, vsb_sp;
  uint32_t ksb_ss, vsb_ss, ksb_rec, vsb_rec;
  uint32_t ksb_lane;     // n * ksb_ss + 2jj: the scales of blocks 2jj, 2jj + 1 of token n
  uint32_t vsb_lane;     // 4jj * vsb_ss + n / 2: the scale of channel 8n's block
};

// Page of the tile starting at token tk (wave-uniform), or -1 if the tile is
// past the range end or its block-table entry is out of range.
__device__ __forceinline__ int tile_page(const Ctx& c, int tk) {
  // clamped into [0, jcap - 1], inside the block-table row; entry 0 of a row
  // always exists (at least one column), so an empty range reads it and
  // stays dead.  The clamp does not use the sequence length, so the entry's
  // load does not wait for the length's: liveness (tk < j1) masks it after
  const int idx = max(min(tk, c.jcap - 1), 0);
  const int pg = c.bt_row[idx >> c.page_shift];
  // all-ones when the tile is live; bit operations keep the block-table
  // load out of any branch
  const int live = ((tk - c.j1) >> 31) & -(int)((uint32_t)pg < c.num_pages);
  return (pg & live) | ~live;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* pool, int64_t sp, uint32_t ss, uint32_t rec,
                                                            int pg, int tk, int pmask) {
  const uint8_t* base = pool + (int64_t)max(pg, 0) * sp + (uint32_t)(tk & pmask) * ss;
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, pg >= 0 ? (int)rec : 0, kRsrcWord3);
}

template <int FMT, bool NT>
__device__ __forceinline__ KRows<FMT> load_k(const Ctx& c, int gi) {
  // non-temporal (stream past the caches) or cached loads; cached K lets
  // the vector L1 serve the second and third touches of a row's lines
  KRows<FMT> R;
  const int t0 = c.j0 + gi * kGran;
  constexpr int aux = NT ? 2 : 0;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int tk = t0 + 16 * k;
    const int pg = __builtin_amdgcn_readfirstlane(tile_page(c, tk));  // wave-uniform: keep it scalar
    R.pg[k] = pg;
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(c.kpool, c.k_sp, c.k_ss, c.k_rec, pg, tk, c.pmask);
    if constexpr (Fmt<FMT>::kBlockScaled) {
      const __amdgpu_buffer_rsrc_t srs = tile_rsrc(c.ksbpool, c.ksb_sp, c.ksb_ss, c.ksb_rec, pg, tk, c.pmask);
      R.s[k] = __builtin_amdgcn_raw_buffer_load_b16(srs, c.ksb_lane, 0, aux);
    }
    if constexpr (Fmt<FMT>::kKDw == 8) {
      const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, c.k_lane, 0, aux);
      const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rs, c.k_lane, 16, aux);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        R.d[k][i] = a[i];
        R.d[k][4 + i] = b[i];
      }
    } else if constexpr (Fmt<FMT>::kKDw == 4) {
      const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, c.k_lane, 0, aux);
#pragma unroll
      for (int i = 0; i < 4; ++i) R.d[k][i] = a[i];
    } else {
      // packed fp6: the lane's 24 bytes (8-byte aligned) as a 16- and an
      // 8-byte load
      const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, c.k_lane, 0, aux);
      const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(rs, c.k_lane, 16, aux);
#pragma unroll
      for (int i = 0; i < 4; ++i) R.d[k][i] = a[i];
      R.d[k][4] = b[0];
      R.d[k][5] = b[1];
    }
  }
  return R;
}

// pgs: the tiles' pages as load_k found them for the same granule
template <int FMT, bool NT>
__device__ __forceinline__ VRows<FMT> load_v(const Ctx& c, int gi, const int (&pgs)[2]) {
  VRows<FMT> R;
  const int t0 = c.j0 + gi * kGran;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int tk = t0 + 16 * t;
    const int pg = pgs[t];
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(c.vpool, c.v_sp, c.v_ss, c.v_rec, pg, tk, c.pmask);
    if constexpr (Fmt<FMT>::kBlockScaled) {
      const __amdgpu_buffer_rsrc_t srs = tile_rsrc(c.vsbpool, c.vsb_sp, c.vsb_ss, c.vsb_rec, pg, tk, c.pmask);
#pragma unroll
      for (int v = 0; v < 4; ++v)
        R.s[4 * t + v] = __builtin_amdgcn_raw_buffer_load_b8(srs, c.vsb_lane, v * c.vsb_ss, NT ? 2 : 0);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if constexpr (Fmt<FMT>::kVDw == 1) {
        R.d[4 * t + v][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, c.v_lane, v * c.v_ss, NT ? 2 : 0);
      } else {
        const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, c.v_lane, v * c.v_ss, NT ? 2 : 0);
        R.d[4 * t + v][0] = x[0];
        R.d[4 * t + v][1] = x[1];
      }
    }
  }
  return R;
}

// K tile k as the A operand of the QK^T MFMA, as loaded: 32 e4m3 bytes, or
// 32 fp6 / fp4 codes in the packed row's own bit order, which is the matrix
// core's fp6 / bf6 / fp4 operand layout (the upper dwords are not read).
template <int FMT>
__device__ __forceinline__ v8i k_operand(const KRows<FMT>& K, int k) {
  v8i a;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = i < Fmt<FMT>::kKDw ? (int)K.d[k][i] : 0;
  return a;
}

// Packed fp6 V of one granule as 8 bf16 B operands: vb[q] = channel 8n + q
// of the 8 tokens tau(jj, 0..7), as 4 words of token pairs (2i, 2i+1).
template <int FMT>
__device__ __forceinline__ void v_operands(const Ctx& c, const VRows<FMT>& V, uint32_t vb[8][4]) {
  {
    // per tile t: the 48-bit channel groups of its 4 tokens form one
    // 192-bit stream of 32 codes (token-major) for the hardware converter
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t d0 = V.d[4 * t + v][0], d1 = V.d[4 * t + v][1];
        lo[v] = __builtin_amdgcn_alignbit(d1, d0, c.v_shift);      // codes 0..4 and 2 bits of 5
        hi[v] = (d1 >> c.v_shift) & 0xFFFFu;                       // the rest of the 48 bits
      }
      v6i src;
      src[0] = (int)lo[0];
      src[1] = (int)(hi[0] | (lo[1] << 16));
      src[2] = (int)((lo[1] >> 16) | (hi[1] << 16));
      src[3] = (int)lo[2];
      src[4] = (int)(hi[2] | (lo[3] << 16));
      src[5] = (int)((lo[3] >> 16) | (hi[3] << 16));
      // f[8 * v + q]
      const v32f f = FMT == 1 ? __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(src, 1.0f)
                              : __builtin_amdgcn_cvt_scalef32_pk32_f32_bf6(src, 1.0f);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        vb[q][2 * t + 0] = pack_bf16(f[q], f[8 + q]);
        vb[q][2 * t + 1] = pack_bf16(f[16 + q], f[24 + q]);
      }
    }
  }
}

// B operands of QK^T per 16-row block: fp8 codes (one MFMA per tile), or
// bf16 Q channels [32jj + 8i, 32jj + 8i + 8) for MFMA i (bf16-Q mode).
template <int FMT, int NRB, int kKind = Fmt<FMT>::kQkF16 ? 2 : (Fmt<FMT>::kQkBf16 ? 1 : 0)>
struct QOps {
  v8i b[NRB];
};
template <int FMT, int NRB>
struct QOps<FMT, NRB, 1> {
  v8bf b[NRB][4];
};
template <int FMT, int NRB>
struct QOps<FMT, NRB, 2> {
  v8h b[NRB][4];
};

// the e2m1 values of byte B of w as fp16, times the power of two of s
template <int B>
__device__ __forceinline__ v2h fp4_f16(uint32_t w, float s) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, B);
}
// the two e2m1 values of byte B of w, as fp32 (low nibble first)
template <int B>
__device__ __forceinline__ v2f fp4_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
}

// Unscaled Q.K dot products of tile k for every row block: lane (n, jj) gets
// tokens 4jj + v of the tile against column n of the block.
template <int FMT, int NRB>
__device__ __forceinline__ void qk_tile(const KRows<FMT>& K, int k, const QOps<FMT, NRB>& q, v4f (&d)[NRB]) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (Fmt<FMT>::kQkF16) {
    // nvfp4 with fp8 Q: dword i holds codes [8i, 8i + 8) of the lane's 32, in
    // block 2jj + i / 2; codes and the two block scales become fp16 exactly,
    // and one packed multiply per code pair applies the scale (exact: at
    // most 6 significant bits, magnitudes in [2^-10, 2688], fp16 normals)
    const v2h sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(K.s[k], 1.0f, false);
    const v2h m0 = {sc[0], sc[0]}, m1 = {sc[1], sc[1]};
    v8h ka[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v2h mm = i < 2 ? m0 : m1;
      const uint32_t w = K.d[k][i];
      const v2h x0 = fp4_f16<0>(w, 1.0f) * mm, x1 = fp4_f16<1>(w, 1.0f) * mm;
      const v2h x2 = fp4_f16<2>(w, 1.0f) * mm, x3 = fp4_f16<3>(w, 1.0f) * mm;
      ka[i] = (v8h){x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
    }
#pragma unroll
    for (int R = 0; R < NRB; ++R) {
      v4f acc = zero;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[i], q.b[R][i], acc, 0, 0, 0);
      d[R] = acc;
    }
  } else if constexpr (Fmt<FMT>::kQkBf16) {
    v8bf ka[4];
    if constexpr (Fmt<FMT>::kBlockScaled) {
      // nvfp4: dword i holds codes [8i, 8i + 8) of the lane's 32, in block
      // 2jj + i / 2; value times its block scale, exact in bf16
      const v2f sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(K.s[k], 1.0f, false);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float bs = i < 2 ? sc[0] : sc[1];
        const uint32_t w = K.d[k][i];
        const v2f x0 = fp4_pair<0>(w), x1 = fp4_pair<1>(w), x2 = fp4_pair<2>(w), x3 = fp4_pair<3>(w);
        const u32x4 h = {pack_bf16(x0[0] * bs, x0[1] * bs), pack_bf16(x1[0] * bs, x1[1] * bs),
                         pack_bf16(x2[0] * bs, x2[1] * bs), pack_bf16(x3[0] * bs, x3[1] * bs)};
        ka[i] = __builtin_bit_cast(v8bf, h);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t h[4];
        e4m3x4_to_bf16(K.d[k][2 * i], h);
        e4m3x4_to_bf16(K.d[k][2 * i + 1], h + 2);
        const u32x4 w = {h[0], h[1], h[2], h[3]};
        ka[i] = __builtin_bit_cast(v8bf, w);
      }
    }
#pragma unroll
    for (int R = 0; R < NRB; ++R) {
      v4f acc = zero;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[i], q.b[R][i], acc, 0, 0, 0);
      d[R] = acc;
    }
  } else {
    const v8i ka = k_operand<FMT>(K, k);
#pragma unroll
    for (int R = 0; R < NRB; ++R)
      d[R] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, q.b[R], zero, Fmt<FMT>::kMfmaFmt, 0, 0, kE8m0One, 0,
                                                              kE8m0One);
  }
}

// Row layout of a tile of up to 32 query rows of a GQA group: NRB blocks of 16 rows;
// a group of NQB < 16 rows (one block) is replicated 16 / NQB times.
//  - softmax layout (QK^T output): lane (n, jj) holds row 16R + n % NQB of
//    block R for the 8 tokens tau(jj, e) of the granule;
//  - O layout (PV output): lane (n, jj) holds rows 16R + (4jj + v) % NQB,
//    v = 0..3, for channels 8n + q.
// With NQB == 4 every lane holds all 4 rows in both layouts, the rows' max
// is wave-uniform and rescaling needs no lane exchange.
template <int NQB, int NRB>
struct State {
  float m[NRB];         // reference max of this lane's softmax row, log2 units
  v4f l[NRB];           // sums of the rounded P of O rows 16R + (4jj + v) % NQB (a
                        // matrix-core product of P with ones: the PV numerator's own P)
  v4f acc[NRB][8];      // O rows 16R + (4jj + v) % NQB, channel 8n + q: acc[R][q][v]
};

// e4m3 PV for channels 2PR and 2PR + 1 of the lane's 8-channel group (bytes
// 2(PR % 2) and 2(PR % 2) + 1 of dword PR / 2).  One byte permute per token
// pair (2i, 2i + 1) puts each channel's two codes side by side, so one packed
// e4m3 -> bf16 conversion (exact) gives a whole B-operand word: the pair's
// two tokens of one channel.
template <int FMT, int PR, int NQB, int NRB>
__device__ __forceinline__ void pv_pair(const VRows<FMT>& V, const v8bf (&pa)[NRB], State<NQB, NRB>& st) {
  typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
  // bytes [t0 c, t1 c, t0 c+1, t1 c+1] of channel bytes c = 2(PR % 2)
  constexpr uint32_t sel = (PR & 1) ? 0x07030602u : 0x05010400u;
  u32x4 wa, wb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = __builtin_amdgcn_perm(V.d[2 * i + 1][PR >> 1], V.d[2 * i][PR >> 1], sel);
    wa[i] = __builtin_bit_cast(uint32_t, (v2bf_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
    wb[i] = __builtin_bit_cast(uint32_t, (v2bf_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true));
  }
#pragma unroll
  for (int R = 0; R < NRB; ++R) {
    st.acc[R][2 * PR] =
        __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[R], __builtin_bit_cast(v8bf, wa), st.acc[R][2 * PR], 0, 0, 0);
    st.acc[R][2 * PR + 1] =
        __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[R], __builtin_bit_cast(v8bf, wb), st.acc[R][2 * PR + 1], 0, 0, 0);
  }
}

// nvfp4 PV for channels 2PR and 2PR + 1, on fp16 MFMAs.  lo[i] / hi[i]:
// the codes of tokens (2i, 2i + 1) nibble-interleaved, so that byte PR holds
// channel 2PR (lo) or 2PR + 1 (hi) of both tokens: one conversion gives a
// B-operand word (a token pair of one channel) and one packed multiply by the
// two tokens' block scales s[i] (fp16, exact) scales it, exactly as in QK^T
template <int FMT, int PR, int NQB, int NRB>
__device__ __forceinline__ void pv_pair_h(const uint32_t (&lo)[4], const uint32_t (&hi)[4], const v2h (&s)[4],
                                          const v8h (&pa)[NRB], State<NQB, NRB>& st) {
  v2h a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = fp4_f16<PR>(lo[i], 1.0f) * s[i];
    b[i] = fp4_f16<PR>(hi[i], 1.0f) * s[i];
  }
  const v8h wa = {a[0][0], a[0][1], a[1][0], a[1][1], a[2][0], a[2][1], a[3][0], a[3][1]};
  const v8h wb = {b[0][0], b[0][1], b[1][0], b[1][1], b[2][0], b[2][1], b[3][0], b[3][1]};
#pragma unroll
  for (int R = 0; R < NRB; ++R) {
    st.acc[R][2 * PR] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[R], wa, st.acc[R][2 * PR], 0, 0, 0);
    st.acc[R][2 * PR + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[R], wb, st.acc[R][2 * PR + 1], 0, 0, 0);
  }
}

// e2m1 PV for channels 2PR and 2PR + 1 from nibble-interleaved token pairs
// (lo / hi as in the nvfp4 PV): one conversion per B-operand word, exact
template <int FMT, int PR, int NQB, int NRB>
__device__ __forceinline__ void pv_pair_fp4(const uint32_t (&lo)[4], const uint32_t (&hi)[4], const v8bf (&pa)[NRB],
                                            State<NQB, NRB>& st) {
  typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
  u32x4 wa, wb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    wa[i] = __builtin_bit_cast(uint32_t, (v2bf_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(lo[i], 1.0f, PR));
    wb[i] = __builtin_bit_cast(uint32_t, (v2bf_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(hi[i], 1.0f, PR));
  }
#pragma unroll
  for (int R = 0; R < NRB; ++R) {
    st.acc[R][2 * PR] =
        __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[R], __builtin_bit_cast(v8bf, wa), st.acc[R][2 * PR], 0, 0, 0);
    st.acc[R][2 * PR + 1] =
        __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[R], __builtin_bit_cast(v8bf, wb), st.acc[R][2 * PR + 1], 0, 0, 0);
  }
}

// the codes of tokens (2i, 2i + 1) nibble-interleaved: byte k of lo[i] holds
// channel 2k of both tokens (low nibble: token 2i), byte k of hi[i] channel 2k + 1
__device__ __forceinline__ void fp4_interleave(const uint32_t a, const uint32_t b, uint32_t& lo, uint32_t& hi) {
  lo = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
  hi = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
}

template <int NQB, int NRB>
__device__ __forceinline__ float row_of(const Ctx& c, int R) {  // softmax-layout row of this lane
  return 16 * R + (c.n % NQB);
}

// MASK: the granule has a dead tile, tokens past the range end or (causal)
// keys some row may not see; without it every logit is kept as is.
template <int FMT, int NQB, int NRB, bool MASK>
__device__ __forceinline__ void granule(const Ctx& c, const QOps<FMT, NRB>& qo, const int (&row_tok)[NRB], int gi,
                                        const KRows<FMT>& K, VRows<FMT>& V, State<NQB, NRB>& st) {
  const int t0 = c.j0 + gi * kGran;
  // ---- logits: lane (n, jj) gets tokens t0 + 16k + 4jj + v of its rows
  float s[NRB][2][4];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    v4f dk[NRB];
    qk_tile<FMT, NRB>(K, k, qo, dk);
    if constexpr (!MASK) {
#pragma unroll
      for (int R = 0; R < NRB; ++R)
#pragma unroll
        for (int v = 0; v < 4; ++v) s[R][k][v] = dk[R][v];
      continue;
    }
    const int tk = t0 + 16 * k;
    // tokens at or past `end` are masked; a dead tile masks all of them
    const int end = K.pg[k] >= 0 ? c.j1 : 0;
    if (tk + 16 > end) {  // wave-uniform: the tile crosses the range end
      // rows past the end hold whatever the page holds (NaN codes too):
      // their V is zeroed so that their zero probabilities add exact zeros
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (tk + 4 * c.jj + v >= end) {
#pragma unroll
          for (int dw = 0; dw < Fmt<FMT>::kVDw; ++dw) V.d[4 * k + v][dw] = 0u;
          if constexpr (Fmt<FMT>::kBlockScaled) V.s[4 * k + v] = 0u;
        }
      }
    }
    // wave-uniform: every token of the tile visible to every row (row 0 of a
    // causal block sees the fewest keys)
    const bool full = tk + 16 <= end && (!c.causal || tk + 15 <= c.lim0);
#pragma unroll
    for (int R = 0; R < NRB; ++R) {
      const v4f d = dk[R];
      if (full) {
#pragma unroll
        for (int v = 0; v < 4; ++v) s[R][k][v] = d[v];
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = tk + 4 * c.jj + v;
          const bool vis = t < end && (!c.causal || t <= c.lim0 + row_tok[R]);
          s[R][k][v] = vis ? d[v] : -INFINITY;
        }
      }
    }
  }
  // ---- online softmax: max of each row over the granule, raised lazily.
  // The logits stay unscaled dot products; cscale > 0 (its sign is folded
  // into the Q operand), so the scaled maximum is cscale times the raw one.
  float M[NRB];
  bool raise = false;
#pragma unroll
  for (int R = 0; R < NRB; ++R) {
    const float inf = c.pos_inf;
    const float mx = fmax2(fmax2(fmax2(s[R][0][0], s[R][0][1], inf), fmax2(s[R][0][2], s[R][0][3], inf), inf),
                           fmax2(fmax2(s[R][1][0], s[R][1][1], inf), fmax2(s[R][1][2], s[R][1][3], inf), inf), inf);
    M[R] = max_jj(mx, inf) * c.cscale;
    raise |= M[R] > st.m[R] + kLazyMax;
  }
  if constexpr (NQB == 4 && NRB == 1) {
    // every lane holds rows 0..3 in the O layout: per-row uniform decisions
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float Mr = lane_f(M[0], r);       // lane r holds row r
      const float mr = lane_f(st.m[0], r);
      if (Mr > mr + kLazyMax) {               // wave-uniform
        const float a = exp2f(mr - Mr);       // m = -inf -> 0
#pragma unroll
        for (int q = 0; q < 8; ++q) st.acc[0][q][r] *= a;
        st.l[0][r] *= a;
        if ((c.n & 3) == r) st.m[0] = Mr;
      }
    }
  } else {
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // rare after the first granules
#pragma unroll
      for (int R = 0; R < NRB; ++R) {
        const bool up = M[R] > st.m[R] + kLazyMax;
        const float a = up ? exp2f(st.m[R] - M[R]) : 1.0f;
        st.m[R] = up ? M[R] : st.m[R];
        // O-layout row 16R + (4jj + v) % NQB lives in softmax-layout lane
        // (jj, (4jj + v) % NQB)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int src = (c.jj << 4) | ((4 * c.jj + v) % NQB);
          const float av = __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(a)));
#pragma unroll
          for (int q = 0; q < 8; ++q) st.acc[R][q][v] *= av;
          st.l[R][v] *= av;
        }
      }
    }
  }
  // ---- P (bf16 A operands; fp16 for nvfp4): p = 2^(cscale * s - m), the
  // scale folded into one fma; and the row sums of the rounded P, as the
  // product of P with a ones operand on the matrix core
  using PA = typename std::conditional<Fmt<FMT>::kPvF16, v8h, v8bf>::type;
  PA pa[NRB];
  const u32x4 ones_w = Fmt<FMT>::kPvF16 ? (u32x4){0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u}
                                        : (u32x4){0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const PA ones = __builtin_bit_cast(PA, ones_w);
#pragma unroll
  for (int R = 0; R < NRB; ++R) {
    const float ms = st.m[R] == -INFINITY ? 0.0f : st.m[R];
    float p[8];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int v = 0; v < 4; ++v) p[4 * k + v] = exp2_fast(__builtin_fmaf(s[R][k][v], c.cscale, -ms));
    u32x4 pw;  // element e = 4k + v, token pairs per word
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (Fmt<FMT>::kPvF16)
        pw[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(((v2f){p[2 * i], p[2 * i + 1]}), v2h));
      else
        pw[i] = pack_bf16(p[2 * i], p[2 * i + 1]);
    }
    pa[R] = __builtin_bit_cast(PA, pw);
    if constexpr (Fmt<FMT>::kPvF16)
      st.l[R] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[R], ones, st.l[R], 0, 0, 0);
    else
      st.l[R] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[R], ones, st.l[R], 0, 0, 0);
  }
  // ---- PV
  if constexpr (Fmt<FMT>::kPvF16) {
    uint32_t lo[4], hi[4];
    v2h sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fp4_interleave(V.d[2 * i][0], V.d[2 * i + 1][0], lo[i], hi[i]);
      // the two tokens' scale bytes (low bytes) side by side, as fp16
      sv[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__builtin_amdgcn_perm(V.s[2 * i + 1], V.s[2 * i], 0x0C0C0400u),
                                                       1.0f, false);
    }
    pv_pair_h<FMT, 0, NQB, NRB>(lo, hi, sv, pa, st);
    pv_pair_h<FMT, 1, NQB, NRB>(lo, hi, sv, pa, st);
    pv_pair_h<FMT, 2, NQB, NRB>(lo, hi, sv, pa, st);
    pv_pair_h<FMT, 3, NQB, NRB>(lo, hi, sv, pa, st);
  } else if constexpr (Fmt<FMT>::kVDw == 1) {
    // e2m1 V: token pairs nibble-interleaved, then one bf16 conversion per
    // B-operand word
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fp4_interleave(V.d[2 * i][0], V.d[2 * i + 1][0], lo[i], hi[i]);
    pv_pair_fp4<FMT, 0, NQB, NRB>(lo, hi, pa, st);
    pv_pair_fp4<FMT, 1, NQB, NRB>(lo, hi, pa, st);
    pv_pair_fp4<FMT, 2, NQB, NRB>(lo, hi, pa, st);
    pv_pair_fp4<FMT, 3, NQB, NRB>(lo, hi, pa, st);
  } else if constexpr (!Fmt<FMT>::kPacked6) {
    // e4m3 V, one channel pair at a time: converting a word's low or
    // high two bytes gives channels (2pr, 2pr + 1) of one
    // token, so the 8 tokens' words give both channels' B operands, used at
    // once (16 floats live, not 64)
    pv_pair<FMT, 0, NQB, NRB>(V, pa, st);
    pv_pair<FMT, 1, NQB, NRB>(V, pa, st);
    pv_pair<FMT, 2, NQB, NRB>(V, pa, st);
    pv_pair<FMT, 3, NQB, NRB>(V, pa, st);
  } else {
    uint32_t vb[8][4];
    v_operands<FMT>(c, V, vb);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const u32x4 w = {vb[q][0], vb[q][1], vb[q][2], vb[q][3]};
      const v8bf b = __builtin_bit_cast(v8bf, w);
#pragma unroll
      for (int R = 0; R < NRB; ++R)
        st.acc[R][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[R], b, st.acc[R][q], 0, 0, 0);
    }
  }
}

// One granule, masked only where it has to be: wave-uniform, a granule whose
// two tiles are live, end before the range end and (causal) hold only keys
// every row may see -- row 0 of the block sees the fewest -- takes the body
// without masking (groups of up to 16 rows).
template <int FMT, int NQB, int NRB, int PF>
__device__ __forceinline__ void granule_any(const Ctx& c, const QOps<FMT, NRB>& qo, const int (&row_tok)[NRB], int gi,
                                            const KRows<FMT>& K, VRows<FMT>& V, State<NQB, NRB>& st) {
  const int t0 = c.j0 + gi * kGran;
  const bool full = (K.pg[0] | K.pg[1]) >= 0 && t0 + kGran <= c.j1 && (!c.causal || t0 + kGran - 1 <= c.lim0);
  // (32-row tiles and the two-granule prefetch: a second copy of the body
  // does not fit their register budget; nvfp4: with two bodies the byte
  // loads of its V block scales get their zero-extension hoisted to the loop
  // head, which then waits for most of the granule's loads.  The masked body
  // alone, whose tile checks are wave-uniform branches, serves those.)
  if (NRB == 1 && PF == 1 && !Fmt<FMT>::kBlockScaled && full)
    granule<FMT, NQB, NRB, false>(c, qo, row_tok, gi, K, V, st);
  else
    granule<FMT, NQB, NRB, true>(c, qo, row_tok, gi, K, V, st);
}

// PF: granules of loads in flight ahead of the one being computed (1 or 2);
// OCC: waves per SIMD the register budget is fitted to.
// CP: cache policy of the KV loads, bit 0 = K non-temporal, bit 1 = V
// non-temporal.
// W: waves per workgroup (4; 8 for a 32-row tile that runs alone on its
// CU, two waves per SIMD without cutting the item into more splits, and for
// two-head groups).
// HG: KV heads per workgroup (1; 2, 4 or 8 (e2m1) for token-major pages of
// packed rows): head h of the group gets waves [h W / HG, (h + 1) W / HG),
// which share its granules as the W waves of a one-head workgroup do.  The
// heads' rows of one token are adjacent in such pages and fill whole
// 128-byte lines together (4 x 96 bytes, 2 x 64), so that each line is
// fetched once, by one CU, instead of once for each of the heads whose rows
// it holds.
template <int FMT, int NQB, int NRB, int CP, int PF, int OCC, int W, int HG = 1>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void decode_mfma_kernel(DecodeParams p) {
  constexpr int kWaves = W;
  constexpr int kThreads = 64 * W;
  constexpr int kWph = W / HG;     // waves per KV head
  constexpr int kTh = 64 * kWph;   // threads per KV head
  static_assert(W % HG == 0 && (HG == 1 || NRB == 1), "head groups: whole waves per head, one row block");
  using F = Fmt<FMT>;
  constexpr int kRows = NQB * NRB;  // rows of the GQA group this instance serves (padded)
  __shared__ float o_s[kWaves][kRows][kHeadDim];
  __shared__ float m_s[kWaves][kRows], l_s[kWaves][kRows], f_s[kWaves][kRows];
  __shared__ __align__(16) uint8_t q_s[HG][kRows][kHeadDim];  // fused step: this item's e4m3 Q rows per head
  __shared__ float red_s[kWaves];
  __shared__ int last_s;

  // head-major grids put the KV heads of one work item in consecutive
  // workgroups, so they are resident together.  The head index hc counts
  // (KV head, row tile) pairs, row tiles innermost: every tile of a group
  // reads the same KV rows
  int w, hc;
  if (p.head_major == 2) {
    // XCD-grouped: workgroup L runs on XCD L % 8; the heads of item w are
    // L = (w / 8) * 8 H + 8 hc + w % 8 (H = h_k / HG * row_tiles), one XCD,
    // dispatched close together
    const int L = blockIdx.x, per = kXcds * (p.h_k / HG) * p.row_tiles;
    const int chunk = L / per, r = L - chunk * per;
    hc = r / kXcds;
    w = chunk * kXcds + (r - hc * kXcds);
    if (w >= p.num_work) return;  // padding of the last chunk
  } else {
    w = p.head_major ? blockIdx.y : blockIdx.x;
    hc = p.head_major ? blockIdx.x : blockIdx.y;
  }
  int g = hc, rt = 0;
  if (p.row_tiles > 1) {
    g = hc / p.row_tiles;
    rt = hc - g * p.row_tiles;
  }
  // this workgroup's rows of the group: [row0, row0 + nq), nq >= 1
  const int row0 = rt * kRows;
  const int nq = min(kRows, p.n_q - row0);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // head groups: this wave's KV head (wave-uniform) and its index in the group
  const int hw = HG > 1 ? wave / kWph : 0;
  const int hc0 = g;  // the group's (first) head index, over HG
  g = g * HG + hw;
  const int n = lane & 15, jj = lane >> 4;
  int seq, tb, te;
  bool single;
  int plan_n = 0, plan_begin = 0;
  bool plan_writer = false;  // this workgroup publishes its sequence's split count (in the epilogue)
  if (p.plan_in_kernel) {
    const PlanItem it = plan_item_wave(p.seq_lens, p.num_seqs, w, p.plan_margin, p.kv_tile,
                                       (int64_t)p.max_blocks * p.page_size, p.plan_max_splits, p.plan_slots,
                                       p.plan_split != 0, p.plan_min_chunk);
    // wave-uniform by construction; said so, so that everything addressed
    // through them (block-table entries above all) stays scalar
    seq = __builtin_amdgcn_readfirstlane(it.seq);
    tb = __builtin_amdgcn_readfirstlane(it.tb);
    te = __builtin_amdgcn_readfirstlane(it.te);
    single = __builtin_amdgcn_readfirstlane(it.n) <= 1;
    plan_n = it.n;
    plan_begin = it.begin;
    plan_writer = it.split == 0 && g == 0 && rt == 0;
  } else {
    seq = p.work[4 * w];
    tb = p.work[4 * w + 1];
    te = p.work[4 * w + 2];
    single = true;  // read below, once seq is known to be valid
  }
  if (seq < 0 || seq >= p.num_seqs) return;
  if (!p.plan_in_kernel) single = p.n_splits[seq] <= 1;

  int L = p.seq_lens[seq];
  L = max(0, min(L, p.max_blocks * p.page_size));
  Ctx c;
  c.j0 = tb * p.kv_tile;
  c.j1 = min(te * p.kv_tile, L);
  c.jcap = min(te * p.kv_tile, p.max_blocks * p.page_size);
  c.causal = p.causal && p.q_len > 1;
  c.lim0 = L - p.q_len;
  c.n = n;
  c.jj = jj;
  c.bt_row = p.bt + (int64_t)seq * p.bt_stride;
  c.kpool = p.k + (int64_t)g * p.k_sh;
  c.vpool = p.v + (int64_t)g * p.v_sh;
  c.k_sp = p.k_sp;
  c.v_sp = p.v_sp;
  c.k_ss = (uint32_t)p.k_ss;
  c.v_ss = (uint32_t)p.v_ss;
  constexpr uint32_t row = F::kRow;
  c.k_rec = 15u * c.k_ss + row;
  c.v_rec = 15u * c.v_ss + row;
  c.k_lane = (uint32_t)(n * p.k_ss + F::kKOff * jj);
  // 4-aligned byte offset holding channel 8n
  const uint32_t vch = F::kPacked6 ? (6u * n) & ~3u : (F::kRow / 16u) * n;
  c.v_lane = (uint32_t)(4 * jj * p.v_ss) + vch;
  c.v_shift = F::kPacked6 ? 16 * (n & 1) : 0;
  c.num_pages = (uint32_t)min<int64_t>(p.num_pages, 0x7FFFFFFF);
  c.pos_inf = p.pos_inf;
  if constexpr (F::kBlockScaled) {
    c.ksbpool = p.ksb + (int64_t)g * p.ksb_sh;
    c.vsbpool = p.vsb + (int64_t)g * p.vsb_sh;
    c.ksb_sp = p.ksb_sp;
    c.vsb_sp = p.vsb_sp;
    c.ksb_ss = (uint32_t)p.ksb_ss;
    c.vsb_ss = (uint32_t)p.vsb_ss;
    c.ksb_rec = 15u * c.ksb_ss + 8u;
    c.vsb_rec = 15u * c.vsb_ss + 8u;
    c.ksb_lane = (uint32_t)n * c.ksb_ss + 2u * jj;
    c.vsb_lane = 4u * jj * c.vsb_ss + ((uint32_t)n >> 1);
  }
  c.page_shift = p.page_shift;
  c.pmask = p.page_size - 1;

  // fused step: fetch this thread's Q words first, then issue the ring's
  // first granules, so that the quantization below (two barriers) waits only
  // on the Q loads (loads retire in issue order) while the KV loads fly
  constexpr int kQV = (kRows * 16 + kTh - 1) / kTh;  // 8-channel vectors per thread (of its head)
  const int th = threadIdx.x % kTh;                  // thread index among its head's
  const int nvec = nq * 16;
  QRaw8 qr[kQV];
  // unfused: the pre-quantized rows' words, fetched before the KV loads too
  // (clamped rows load a valid row and are zeroed below)
  u32x4 qg[NRB][2];
  // bf16-Q mode: this lane's channels [32jj, 32jj + 32) of Q row 16R + n % NQB
  // of the tile (clamped like the codes; zeroed below past the tile's rows)
  u32x4 qh[NRB][4];
  if constexpr (F::kQBf16) {
#pragma unroll
    for (int R = 0; R < NRB; ++R) {
      const int r = row0 + min(16 * R + (n % NQB), nq - 1);
      const int t = r / p.h_r;
      const int64_t tok = (int64_t)seq * p.q_len + t, h = (int64_t)g * p.h_r + (r - t * p.h_r);
      const u32x4* src = reinterpret_cast<const u32x4*>(p.qb + tok * p.qb_ts + h * p.qb_hs + 32 * jj);
#pragma unroll
      for (int i = 0; i < 4; ++i) qh[R][i] = src[i];
    }
  } else if (!p.qb) {
#pragma unroll
    for (int R = 0; R < NRB; ++R) {
      const int r = row0 + min(16 * R + (n % NQB), nq - 1);
      const uint8_t* row_q = p.q8 + (((int64_t)seq * p.h_k + g) * p.n_q + r) * kHeadDim;
      qg[R][0] = *reinterpret_cast<const u32x4*>(row_q + q_half_offset<FMT>(jj, 0));
      qg[R][1] = *reinterpret_cast<const u32x4*>(row_q + q_half_offset<FMT>(jj, 1));
    }
  }
  if (!F::kQBf16 && p.qb) {
#pragma unroll
    for (int k = 0; k < kQV; ++k) {
      const int v = min(th + k * kTh, nvec - 1);  // a repeat changes no max
      qr[k] = q_fetch8(p.qb, p.qb_ts, p.qb_hs, p.q_mul, p.q_len, p.h_r, seq, g, row0 + (v >> 4), (v & 15) * 8);
    }
  }

  // the ring's first granules, issued unconditionally (a wave with no
  // granule loads a dead tile, i.e. zeros) so that the wait counts stay static
  const int ngr = (c.j1 - c.j0 + kGran - 1) / kGran;
  int gi = wave % kWph;
  const bool run = gi < ngr;
  // lockstep period per format (cfg3's shape; with two waves per head,
  // kernel GB/s against none: e2m3 every 4 granules +4.7 %, e2m1 every 2
  // +6.9 %; with one wave per head, kernel us at periods 2 / 4 / 8 (e2m3)
  // and 1 / 2 / 4 (e2m1): 179.9 / 181.8 / 183.7 and 133.2 / 132.9 / 130.0;
  // nvfp4, whose shared lines are its block-scale rows across the two groups
  // of an item, gained nothing at any period)
  constexpr int kLock = HG == 1 || F::kBlockScaled ? 0 : (F::kPacked6 ? 2 : 4);
  const int lock_end = ngr / kWph;
  int lock_it = 0;
  KRows<FMT> K0 = load_k<FMT, (CP & 1) != 0>(c, gi), K1;
  VRows<FMT> V0 = load_v<FMT, (CP & 2) != 0>(c, gi, K0.pg), V1;
  if constexpr (PF == 2) {
    K1 = load_k<FMT, (CP & 1) != 0>(c, gi + kWph);
    V1 = load_v<FMT, (CP & 2) != 0>(c, gi + kWph, K1.pg);
  }

  float qdesc = 1.0f;  // bf16-Q mode: no Q scale
  if (!F::kQBf16 && p.qb) {
    // fused step: quantize this (sequence, KV head)'s Q rows here, with the
    // arithmetic of the stand-alone quantize kernel (every split item of the
    // pair derives the same codes and scale)
    float x[kQV][8];
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < kQV; ++k) {
      q_convert8(qr[k], p.q_mul != nullptr, x[k]);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[k][e]));
    }
    if constexpr (kRows == 32 && HG == 1) {
      // row tiles: the scale covers every row of the pair, so the rows of
      // the other tiles enter the maximum too (loaded after the ring's first
      // granules, which they then wait for; once per workgroup)
      if (p.row_tiles > 1) {
        for (int v = threadIdx.x; v < p.n_q * 16; v += kThreads) {
          const int r = v >> 4;
          if (r >= row0 && r < row0 + nq) continue;  // in this tile: counted above
          float y[8];
          q_convert8(q_fetch8(p.qb, p.qb_ts, p.qb_hs, p.q_mul, p.q_len, p.h_r, seq, g, r, (v & 15) * 8),
                     p.q_mul != nullptr, y);
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[e]));
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if (lane == 0) red_s[wave] = amax;
    __syncthreads();
    amax = red_s[hw * kWph];
#pragma unroll
    for (int i = 1; i < kWph; ++i) amax = fmaxf(amax, red_s[hw * kWph + i]);
    qdesc = q_scale_from_amax(amax);
    const float rq = 1.0f / qdesc;
#pragma unroll
    for (int k = 0; k < kQV; ++k) {
      const int v = th + k * kTh;
      if (v < nvec) *reinterpret_cast<uint2*>(&q_s[hw][v >> 4][(v & 15) * 8]) = q_codes8(x[k], qdesc, rq);
    }
    __syncthreads();
  } else if (!F::kQBf16) {
    qdesc = p.q_descale[(int64_t)seq * p.h_k + g];
  }
  // the logit scale (log2 units) applied to raw dot products; its sign goes
  // into the Q operand below, so that the scale the softmax multiplies by is
  // positive (a zero scale becomes the smallest normal: every logit ~ 0)
  const float craw = qdesc * load_descale(p.kd, p.kd_kind, seq, g, p.h_k) * p.scale_log2;
  const bool qneg = craw < 0.0f;  // wave-uniform
  c.cscale = craw != craw ? craw : fmaxf(fabsf(craw), 1.17549435e-38f);

  // B operands of QK^T: column n of block R = Q row 16R + n % NQB of the
  // tile (zero past its rows)
  QOps<FMT, NRB> qo;
  int row_tok[NRB];
#pragma unroll
  for (int R = 0; R < NRB; ++R) {
    const int r = 16 * R + (n % NQB);
    row_tok[R] = (row0 + r) / p.h_r;
    const u32x4 z = {0u, 0u, 0u, 0u};
    if constexpr (F::kQBf16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) qo.b[R][i] = __builtin_bit_cast(v8bf, r < nq ? qh[R][i] : z);
    } else if (r < nq) {
      u32x4 a, b;
      if (p.qb) {  // LDS reads of the codes quantized above
        a = *reinterpret_cast<const u32x4*>(&q_s[hw][r][q_half_offset<FMT>(jj, 0)]);
        b = *reinterpret_cast<const u32x4*>(&q_s[hw][r][q_half_offset<FMT>(jj, 1)]);
      } else {
        a = qg[R][0];
        b = qg[R][1];
      }
      if constexpr (F::kQkF16) {
        // fp8 codes of channels [32jj, 32jj + 32) as the fp16 operands of
        // the four MFMAs (exact)
        const uint32_t w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const v2h h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[2 * i], 1.0f, false);
          const v2h h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[2 * i], 1.0f, true);
          const v2h h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[2 * i + 1], 1.0f, false);
          const v2h h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[2 * i + 1], 1.0f, true);
          qo.b[R][i] = (v8h){h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
        }
      } else if constexpr (F::kQkBf16) {
        // fp8 codes of channels [32jj, 32jj + 32) as the bf16 operands of
        // the four MFMAs (exact)
        const uint32_t w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t h[4];
          e4m3x4_to_bf16(w[2 * i], h);
          e4m3x4_to_bf16(w[2 * i + 1], h + 2);
          const u32x4 hv = {h[0], h[1], h[2], h[3]};
          qo.b[R][i] = __builtin_bit_cast(v8bf, hv);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qo.b[R][i] = (int)a[i];
          qo.b[R][4 + i] = (int)b[i];
        }
      }
    } else {
      if constexpr (F::kQkF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) qo.b[R][i] = __builtin_bit_cast(v8h, z);
      } else if constexpr (F::kQkBf16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) qo.b[R][i] = __builtin_bit_cast(v8bf, z);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) qo.b[R][i] = 0;
      }
    }
  }

  if (qneg) {  // negate Q exactly: flip the sign bit of every element
#pragma unroll
    for (int R = 0; R < NRB; ++R) {
      if constexpr (Fmt<FMT>::kQkF16 || Fmt<FMT>::kQkBf16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x4 w = __builtin_bit_cast(u32x4, qo.b[R][i]);
          w ^= 0x80008000u;
          qo.b[R][i] = __builtin_bit_cast(std::remove_reference_t<decltype(qo.b[R][i])>, w);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) qo.b[R][i] ^= (int)0x80808080u;
      }
    }
  }

  State<NQB, NRB> st;
#pragma unroll
  for (int R = 0; R < NRB; ++R) {
    st.m[R] = -INFINITY;
    st.l[R] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < 8; ++q) st.acc[R][q] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  }

  if (run) {
    // register ring of PF + 1 granules, rotated by unrolling
    if constexpr (PF == 1) {
      while (true) {
        group_lockstep<kLock>(lock_it, lock_end);
        K1 = load_k<FMT, (CP & 1) != 0>(c, gi + kWph);
        V1 = load_v<FMT, (CP & 2) != 0>(c, gi + kWph, K1.pg);
        issue_fence();
        granule_any<FMT, NQB, NRB, PF>(c, qo, row_tok, gi, K0, V0, st);
        gi += kWph;
        if (gi >= ngr) break;
        group_lockstep<kLock>(lock_it, lock_end);
        K0 = load_k<FMT, (CP & 1) != 0>(c, gi + kWph);
        V0 = load_v<FMT, (CP & 2) != 0>(c, gi + kWph, K0.pg);
        issue_fence();
        granule_any<FMT, NQB, NRB, PF>(c, qo, row_tok, gi, K1, V1, st);
        gi += kWph;
        if (gi >= ngr) break;
      }
    } else {
      while (true) {
        group_lockstep<kLock>(lock_it, lock_end);
        KRows<FMT> K2 = load_k<FMT, (CP & 1) != 0>(c, gi + 2 * kWph);
        VRows<FMT> V2 = load_v<FMT, (CP & 2) != 0>(c, gi + 2 * kWph, K2.pg);
        issue_fence();
        granule_any<FMT, NQB, NRB, PF>(c, qo, row_tok, gi, K0, V0, st);
        gi += kWph;
        if (gi >= ngr) break;
        group_lockstep<kLock>(lock_it, lock_end);
        K0 = load_k<FMT, (CP & 1) != 0>(c, gi + 2 * kWph);
        V0 = load_v<FMT, (CP & 2) != 0>(c, gi + 2 * kWph, K0.pg);
        issue_fence();
        granule_any<FMT, NQB, NRB, PF>(c, qo, row_tok, gi, K1, V1, st);
        gi += kWph;
        if (gi >= ngr) break;
        group_lockstep<kLock>(lock_it, lock_end);
        K1 = load_k<FMT, (CP & 1) != 0>(c, gi + 2 * kWph);
        V1 = load_v<FMT, (CP & 2) != 0>(c, gi + 2 * kWph, K1.pg);
        issue_fence();
        granule_any<FMT, NQB, NRB, PF>(c, qo, row_tok, gi, K2, V2, st);
        gi += kWph;
        if (gi >= ngr) break;
      }
    }
  }

  // per-wave results: O rows x channels and the row sums (both in the O
  // layout) from the lanes holding distinct rows, the max of each row from the
  // softmax layout
#pragma unroll
  for (int R = 0; R < NRB; ++R) {
    if (4 * jj < NQB) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int v = 0; v < 4; ++v) o_s[wave][NQB * R + 4 * jj + v][8 * n + q] = st.acc[R][q][v];
      if (n == 0) {
#pragma unroll
        for (int v = 0; v < 4; ++v) l_s[wave][NQB * R + 4 * jj + v] = st.l[R][v];
      }
    }
    if (jj == 0 && n < NQB) m_s[wave][NQB * R + n] = st.m[R];
  }
  __syncthreads();

  const float vd = HG == 1 ? load_descale(p.vd, p.vd_kind, seq, g, p.h_k) : 0.0f;
  // per row (thread r of head hr of the group): the weights 2^(m_w - M) of
  // the head's waves, divided by the row sum when the item is the
  // sequence's only one; the row's LSE, or its split partial's max and sum
  if (threadIdx.x < kRows * HG) {
    const int hr = threadIdx.x / kRows, r = threadIdx.x - hr * kRows;
    const int w0 = hr * kWph;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWph; ++ww) M = fmaxf(M, m_s[w0 + ww][r]);
    const float Ms = M == -INFINITY ? 0.0f : M;
    float wt[kWph], Lsum = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWph; ++ww) {
      wt[ww] = exp2f(m_s[w0 + ww][r] - Ms);
      Lsum += wt[ww] * l_s[w0 + ww][r];
    }
    const float f = single ? (Lsum > 0.0f ? 1.0f / Lsum : 0.0f) : 1.0f;
#pragma unroll
    for (int ww = 0; ww < kWph; ++ww) f_s[w0 + ww][r] = wt[ww] * f;
    if (r < nq) {
      const int gr = hc0 * HG + hr;  // the row's KV head
      const int rg = row0 + r;
      const int t = rg / p.h_r;
      const int h = gr * p.h_r + (rg - t * p.h_r);
      if (single) {
        if (p.lse)
          p.lse[((int64_t)seq * p.q_len + t) * p.h_q + h] = Lsum > 0.0f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
      } else if (w < p.part_items) {
        // written through to device-coherent memory, for a merge on any XCD
        const int64_t idx = ((int64_t)w * p.h_k + gr) * p.nqp + rg;
        store_coherent(&p.m_part[idx], Lsum > 0.0f ? M : -INFINITY);
        store_coherent(&p.l_part[idx], Lsum);
      }
    }
  }
  __syncthreads();

  // combine the waves: thread -> channel ch of rows tid / 128 + (W / 2) k
  // (rows of head r / kRows of the group), every row's LDS reads issued
  // together (a compile-time row count)
  const int ch = threadIdx.x & 127;
  constexpr int kRowStep = kThreads / 128;
#pragma unroll
  for (int k = 0; k < (kRows * HG + kRowStep - 1) / kRowStep; ++k) {
    const int rr = (threadIdx.x >> 7) + kRowStep * k;
    const int hr = HG == 1 ? 0 : rr / kRows, r = rr - hr * kRows;
    if (hr < HG && r < nq) {
      float O = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kWph; ++ww) O += f_s[hr * kWph + ww][r] * o_s[hr * kWph + ww][r][ch];
      const int gr = hc0 * HG + hr;  // the row's KV head
      const int rg = row0 + r;       // row of the group
      const int t = rg / p.h_r;
      const int h = gr * p.h_r + (rg - t * p.h_r);
      const float vdr = HG == 1 ? vd : load_descale(p.vd, p.vd_kind, seq, gr, p.h_k);
      const float om = (p.o_mul ? p.o_mul[(int64_t)h * kHeadDim + ch] : 1.0f) * vdr;
      if (single) {
        store_out(p.out, p.out_f32, ((int64_t)seq * p.q_len + t) * p.out_ts + (int64_t)h * p.out_hs + ch, O * om);
      } else if (w < p.part_items) {
        const int64_t idx = ((int64_t)w * p.h_k + gr) * p.nqp + rg;
        store_coherent(&p.o_part[idx * kHeadDim + ch], O * om);
      }
    }
  }

  // the in-kernel plan's split count and first item of this sequence, for
  // the merge launch that follows; stored after the main loop so that no
  // integer store precedes the block-table reads (which then stay scalar
  // loads of memory the kernel provably does not write before them)
  if (plan_writer && threadIdx.x == 0) {
    p.ns_out[seq] = plan_n;
    p.sb_out[seq] = plan_begin;
  }

  if (HG == 1 && !single && p.counters) {
    // fused merge.  Publication follows the memory model: every thread's
    // partial stores are ordered before the workgroup barrier by a
    // workgroup-scope release; thread 0 then counts the arrival with one
    // agent-scope release increment, which covers the whole workgroup's
    // stores (cumulativity through the barrier).  The last split to arrive
    // reads the end of that release sequence and takes an agent-scope
    // acquire fence, so every other split's partials are visible to it; its
    // threads order their merge loads after that with a workgroup-scope
    // acquire past the second barrier.  Only the last split acquires: an
    // acquire invalidates its XCD's L2 under every other workgroup there
    // (with an acquire in every split, the ragged batch took 354 us per
    // step instead of 242).
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (threadIdx.x == 0) {
      int32_t* cnt = p.counters + (int64_t)seq * p.h_k + g;
      const int last =
          __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == p.n_splits[seq] - 1;
      if (last) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        // every split of this launch has arrived: reset for the next launch
        __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      last_s = last;
    }
    __syncthreads();
    if (last_s) {  // the partials are read with device-coherent loads
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      MergeParams mp;
      mp.n_splits = p.n_splits;
      mp.split_begin = p.split_begin;
      mp.o_part = p.o_part;
      mp.m_part = p.m_part;
      mp.l_part = p.l_part;
      mp.nqp = p.nqp;
      mp.part_items = p.part_items;
      mp.out = p.out;
      mp.out_f32 = p.out_f32;
      mp.out_ts = p.out_ts;
      mp.out_hs = p.out_hs;
      mp.lse = p.lse;
      mp.num_seqs = p.num_seqs;
      mp.q_len = p.q_len;
      mp.h_q = p.h_q;
      mp.h_k = p.h_k;
      mp.h_r = p.h_r;
      mp.n_q = p.n_q;
      // same batches as the merge kernel: same rounding (its 256-thread layout)
      if (threadIdx.x < 256) merge_one<true, 1, 8>(mp, seq, g, threadIdx.x);
    }
  }
}

template <int FMT, int NQB, int NRB, int PF, int OCC, int W = 4, int HG = 1>
hipError_t launch_shape(const DecodeParams& p, int cp, hipStream_t s) {
  constexpr int kThreads = 64 * W;
  const int heads = p.h_k / HG * p.row_tiles;
  const dim3 grid = p.head_major == 2 ? dim3((unsigned)((p.num_work + kXcds - 1) / kXcds * kXcds * heads))
                    : p.head_major ? dim3(heads, p.num_work) : dim3(p.num_work, heads);
  if constexpr (HG > 1) {
    // head groups: all KV loads cached (the group's waves share lines
    // through the vector L1) or V streamed
    if (cp == 0)
      hipLaunchKernelGGL((decode_mfma_kernel<FMT, NQB, NRB, 0, PF, OCC, W, HG>), grid, dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL((decode_mfma_kernel<FMT, NQB, NRB, 2, PF, OCC, W, HG>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
  }
  switch (cp) {
    case 0: hipLaunchKernelGGL((decode_mfma_kernel<FMT, NQB, NRB, 0, PF, OCC, W>), grid, dim3(kThreads), 0, s, p); break;
    case 1: hipLaunchKernelGGL((decode_mfma_kernel<FMT, NQB, NRB, 1, PF, OCC, W>), grid, dim3(kThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_mfma_kernel<FMT, NQB, NRB, 2, PF, OCC, W>), grid, dim3(kThreads), 0, s, p); break;
    default: hipLaunchKernelGGL((decode_mfma_kernel<FMT, NQB, NRB, 3, PF, OCC, W>), grid, dim3(kThreads), 0, s, p); break;
  }
  return hipGetLastError();
}

// Head groups for the packed formats at up to 16 rows: four KV heads per
// workgroup in four waves, one per head (two workgroups per CU, so that one
// group's prologue and epilogue overlap another's streaming; against eight
// waves, two per head, one workgroup per CU on the ragged batch in
// token-major pages: e2m3 196 -> 183 us, e2m1 140 -> 133, nvfp4 170 -> 164),
// eight heads in eight waves for e2m1 (a token's eight 64-byte rows are one
// 512-byte run: 130.3 -> 127.1 us; e2m3 and nvfp4 were 2-3 % slower so), or
// two heads in eight waves.
template <int FMT, int NQB>
hipError_t launch_groups(const DecodeParams& p, int cp, int hg, hipStream_t s) {
  if constexpr (Fmt<FMT>::kPacked6 || FMT == 4 || FMT == 5 || FMT == 6) {
    if constexpr (FMT == 4) {
      if (hg == 8) return launch_shape<FMT, NQB, 1, 1, 2, 8, 8>(p, cp, s);
    }
    if (hg == 8) return hipErrorInvalidValue;
    return hg == 4 ? launch_shape<FMT, NQB, 1, 1, 2, 4, 4>(p, cp, s) : launch_shape<FMT, NQB, 1, 1, 2, 8, 2>(p, cp, s);
  } else {
    return hipErrorInvalidValue;
  }
}

template <int FMT>
hipError_t launch_fmt(DecodeParams& p, int nt, int tune, bool wide, int hg, hipStream_t s) {
  const bool pf2 = tune & 2;  // two granules of prefetch instead of one
  // more than 32 rows: tiles of 32 rows (the 32-row instance), each
  // workgroup one tile of one (item, KV head)
  p.row_tiles = (p.n_q + kMfmaTileRows - 1) / kMfmaTileRows;
  if (hg > 1) {
    if (p.n_q > 16 || p.h_k % hg || p.counters) return hipErrorInvalidValue;
    return p.n_q <= 4 ? launch_groups<FMT, 4>(p, nt, hg, s)
                      : (p.n_q <= 8 ? launch_groups<FMT, 8>(p, nt, hg, s) : launch_groups<FMT, 16>(p, nt, hg, s));
  }
  if (p.n_q <= 4) return pf2 ? launch_shape<FMT, 4, 1, 2, 2>(p, nt, s) : launch_shape<FMT, 4, 1, 1, 2>(p, nt, s);
  if (p.n_q <= 8) return pf2 ? launch_shape<FMT, 8, 1, 2, 2>(p, nt, s) : launch_shape<FMT, 8, 1, 1, 2>(p, nt, s);
  if (p.n_q <= 16) return pf2 ? launch_shape<FMT, 16, 1, 2, 2>(p, nt, s) : launch_shape<FMT, 16, 1, 1, 2>(p, nt, s);
  // 32 rows (per tile): two waves per SIMD fit the register budget (VGPR accumulators,
  // no copies through AGPRs) except for packed fp6, whose V expansion needs
  // the one-wave budget, and 16-bit Q operands (bf16 Q; nvfp4), which take
  // 32 more registers (the default plan runs 32-row groups one workgroup per
  // CU either way)
  if constexpr (Fmt<FMT>::kPacked6 || Fmt<FMT>::kQkBf16 || Fmt<FMT>::kQkF16)
    return pf2 ? launch_shape<FMT, 16, 2, 2, 1>(p, nt, s) : launch_shape<FMT, 16, 2, 1, 1>(p, nt, s);
  else if (pf2)
    return launch_shape<FMT, 16, 2, 2, 1>(p, nt, s);
  // a group of one 32-row tile is planned one workgroup per CU: eight waves
  // (two per SIMD) share its item; row tiles of larger groups keep four waves
  // so that two of their workgroups fit a CU
  else if (p.row_tiles == 1 && wide)
    return launch_shape<FMT, 16, 2, 1, 2, 8>(p, nt, s);
  else
    return launch_shape<FMT, 16, 2, 1, 2>(p, nt, s);
}

}  // namespace

// tune bits: 1 = two granules of prefetch, 2 = head-major grid, 4 = XCD-
// grouped grid (over 2), 8 = four waves (not eight) for a lone 32-row tile,
// 16-48 = KV heads per workgroup (0: the library's choice, 16: one, 32: two,
// 48: four; more than one where it applies: packed formats, up to 16 rows,
// no in-kernel merge, h_k a multiple); -1 = the default for the format.  cache_policy:
// -1 = the default for the format, else the CP bits (head groups: 0, or V
// non-temporal for any other).
hipError_t launch_decode_mfma(const DecodeParams& p_in, int kv_format, int cache_policy, int tune, hipStream_t s) {
  DecodeParams p = p_in;
  // e2m1 and nvfp4 rows are half the bytes of e4m3 ones: their items are
  // planned two workgroups per CU, and the KV heads of one item run on one
  // XCD close together (XCD-grouped grid), so that rows of neighbouring
  // heads (one 128-byte line in a token-major page) are fetched once into
  // that XCD's L2 and head-major pages are read together.  Measured: 131K
  // context, 4 sequences, head-major pages 117 -> 100 us; ragged batch,
  // token-major pages 199 -> 169 us.
  const bool auto_tune = tune < 0;
  if (auto_tune) tune = kv_format >= 3 ? 4 : 0;
  // Head groups: packed rows (96 or 64 bytes) of adjacent KV heads in
  // token-major pages share 128-byte lines; a workgroup of 4 heads (fp6:
  // 384 bytes, three whole lines; fp4: 256 bytes, two) reads each line once.
  // Chosen where the grid still gives every CU a workgroup.  Measured on the
  // ragged batch in token-major pages: e2m3 230 -> 215 us, e2m1 149 -> 136.5,
  // nvfp4 174 -> 168 (against one head per workgroup with every load
  // cached); HBM bytes fetched per KV byte 1.95 -> 1.36, 1.20 -> 1.01 and
  // 1.43 -> 1.11.  Two heads per workgroup were slower than one (192-252 us).
  const int hsel = (tune >> 4) & 3;
  int hg = hsel >= 2 ? (hsel == 2 ? 2 : 4) : 1;
  if (hsel == 0 && kv_format >= 1) {
    const int64_t row = kv_format <= 2 ? 96 : 64;
    const int want = 4;
    const bool adjacent = p.k_sh == row && p.v_sh == row;
    const bool cp_ok = cache_policy < 0 || cache_policy == 0 || cache_policy == 2;
    if (adjacent && cp_ok && (int64_t)p.num_work * (p.h_k / want) >= p.num_cus) hg = want;
  }
  // e2m1: all eight heads of a token in one workgroup where h_k allows it
  // and the grid still gives every CU a workgroup
  if (hsel == 0 && hg == 4 && kv_format == 3 && p.h_k % 8 == 0 && (int64_t)p.num_work * (p.h_k / 8) >= p.num_cus)
    hg = 8;
  if (kv_format == 0 || p.n_q > 16 || p.counters || p.h_k % hg) hg = 1;
  // head groups share no lines across workgroups: the plain grid (measured:
  // e2m1 143.6 -> 136.5 us, nvfp4 169.5 -> 168.3)
  if (auto_tune && hg > 1) tune &= ~4;
  p.head_major = (tune & 4) ? 2 : ((tune & 2) ? 1 : 0);
  const int t = (tune & 1) ? 2 : 0;
  const bool wide = (tune & 8) == 0;  // eight waves for a lone 32-row tile (bit 3: four)
  // default: K cached, V non-temporal.  A K tile's row lines are touched by
  // two (e4m3) or three (e2m3) load instructions, which the vector L1 then
  // serves after the first; V loads cover whole rows (e4m3) and stream.
  // Measured against all-non-temporal: e2m3 at 131K context 169 -> 144 us,
  // e4m3 at 32K 657 -> 647 us, ragged batch 225 -> 219 us.  Head groups
  // share V lines too: every load cached.
  const int cp = cache_policy >= 0 ? cache_policy : (hg > 1 ? 0 : 2);
  switch (kv_format) {
    case 0: return p.q_bf16 ? launch_fmt<2>(p, cp, t, wide, hg, s) : launch_fmt<0>(p, cp, t, wide, hg, s);
    case 1: return launch_fmt<1>(p, cp, t, wide, hg, s);
    case 2: return launch_fmt<3>(p, cp, t, wide, hg, s);
    case 3: return launch_fmt<4>(p, cp, t, wide, hg, s);
    default: return p.q_bf16 ? launch_fmt<6>(p, cp, t, wide, hg, s) : launch_fmt<5>(p, cp, t, wide, hg, s);
  }
}

}  // namespace mj
