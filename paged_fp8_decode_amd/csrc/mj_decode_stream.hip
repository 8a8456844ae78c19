// Streaming paged decode with the PV product on the VALU, for GQA groups of
// up to 4 query rows (q_len * h_r <= 4) and e4m3 KV, on gfx950.  It is the
// VALU-PV alternative to the matrix-core kernel (mj_decode_mfma.hip), kept
// for A/B measurement; the dispatcher uses it only when asked to.
//
// Method: mjolnir-kernel README "What it does", step 3 (stream KV pages, online
// softmax) and the partials step 4 merges; the Thor kernel design on those
// pages (TMA ring, TMEM accumulators) is not used.
//
// Work split: one workgroup (4 waves) per (plan item, KV head).  The item's
// token range is cut into 32-token granules dealt round-robin to the 4 waves,
// so at any time the workgroup streams 4 adjacent granules.  Each wave keeps
// its own online-softmax state; the four are merged through LDS at the end.
//
// Per granule, lane l = 16*j + n holds, for tokens n and n+16 of the granule,
// K and V bytes [32j, 32j+32) of the row (e4m3) or codes [32j, 32j+32) (e2m3,
// 24 bytes): two 16-byte (or three 8-byte) loads per row.  KV bytes are read
// exactly once.  Loads run ahead of use: V one granule ahead (two V buffers),
// K issued right after the current granule's QK^T (one K buffer), and every
// load is unconditional (dead tiles read a few always-valid bytes) so the
// wait counts before each use are static and never drain the queue.
//
// QK^T: v_mfma_f32_16x16x128_f8f6f4 takes the raw K bytes (fp8 or fp6) as the
// B operand, so K is never converted on the VALU.  The A operand holds the
// (at most 4) quantized Q rows replicated four times, so the 16x16 result
// gives every lane the logits of its own token for all 4 rows, and the 4
// lane groups agree.  This spends 4x the MFMA work of the real rows, which is
// < 2 % of the matrix pipe at HBM speed, and saves ~160 VALU operations per
// 16 tokens that a lane-parallel dot product would need.
//
// Softmax: logits in log2 units; the running max per row is raised only when a
// tile exceeds it by more than 8 (output and sum stay consistent with whatever
// reference max is used, so this is exact and rarely rescales).
//
// PV on the VALU: V bytes -> fp32 with the hardware converters, 128 FMAs per
// tile per lane into 4 rows x 32 channels of accumulators.
#include "mj_device.h"
#include "mj_internal.h"

namespace mj {

hipError_t launch_decode_generic(const DecodeParams& p, int kv_format, int row_tiles, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeParams& p, int kv_format, int cache_policy, int tune, hipStream_t s);
bool decode_mfma_supports(int n_q);

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kGran = 32;          // tokens per wave iteration: two 16-token MFMA tiles
constexpr float kLazyMax = 8.0f;   // log2 headroom before the running max is raised
constexpr int kE8m0One = 127;      // MFMA block scale 2^0

template <int FMT>
struct Fmt;
template <>
struct Fmt<0> {  // e4m3
  static constexpr int kDw = 8;    // dwords per lane per row block (32 bytes)
  static constexpr int kLaneOff = 32;
  static constexpr int kMfma = 0;  // MFMA operand format: fp8 e4m3
};
template <>
struct Fmt<1> {  // e2m3, 4 codes per 3 bytes
  static constexpr int kDw = 6;    // 24 bytes = 32 codes
  static constexpr int kLaneOff = 24;
  static constexpr int kMfma = 2;  // MFMA operand format: fp6 e2m3
};

template <int FMT>
struct Rows {  // one lane's slice of the two 16-token tiles of a granule (K or V)
  uint32_t d[2][Fmt<FMT>::kDw];
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// all-reduce over the 16 lanes of a DPP row
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0x124>(x));  // row_ror:4
  x = fmaxf(x, dpp<0x128>(x));  // row_ror:8
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x124>(x);
  x += dpp<0x128>(x);
  return x;
}
__device__ __forceinline__ float uniform_f(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

template <bool NT, typename T>
__device__ __forceinline__ T ld(const T* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

template <int FMT, bool NT>
__device__ __forceinline__ void load_row_block(const uint8_t* src, uint32_t out[Fmt<FMT>::kDw]) {
  if constexpr (FMT == 0) {
    const u32x4* s = reinterpret_cast<const u32x4*>(src);
    const u32x4 a = ld<NT>(s), b = ld<NT>(s + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[i] = a[i];
      out[4 + i] = b[i];
    }
  } else {
    const u32x2* s = reinterpret_cast<const u32x2*>(src);
    const u32x2 a = ld<NT>(s), b = ld<NT>(s + 1), c = ld<NT>(s + 2);
    out[0] = a[0]; out[1] = a[1]; out[2] = b[0]; out[3] = b[1]; out[4] = c[0]; out[5] = c[1];
  }
}

// Per-workgroup constants of one (plan item, KV head).
struct Ctx {
  const int32_t* bt_row;
  const uint8_t* kpool;  // pool + head offset (wave-uniform)
  const uint8_t* vpool;
  const uint8_t* safe;   // always-valid bytes for dead tiles (the workgroup's Q rows)
  int64_t k_sp, v_sp, num_pages;
  uint32_t k_lane, v_lane;  // this lane's byte offset: n * slot_stride + row-block offset
  uint32_t k_ss, v_ss, safe_lane;
  int j0, j1, page_shift, pmask, lim0, causal, n;
  float cscale;
  int row_tok[4];
};

struct State {
  float m[4], l[4], acc[4][32];
};

// Page of the tile starting at token tk (wave-uniform), or -1 if the tile is
// past the range end or its block-table entry is out of range.
__device__ __forceinline__ int64_t tile_page(const Ctx& c, int tk) {
  const int idx = min(tk, c.j1 - 1);  // a granule exists only when j1 > j0
  const int64_t pg = c.bt_row[idx >> c.page_shift];
  return (tk < c.j1 && pg >= 0 && pg < c.num_pages) ? pg : -1;
}

// Issues the loads of one granule's K (IS_V false) or V rows.  Branch-free:
// a dead tile reads this lane's bytes of the Q rows instead.
template <int FMT, bool NT, bool IS_V>
__device__ __forceinline__ Rows<FMT> load_rows(const Ctx& c, int gi) {
  Rows<FMT> R;
  const int t0 = c.j0 + gi * kGran;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int tk = t0 + 16 * k;
    const int64_t pg = tile_page(c, tk);
    const uint32_t slot0 = (uint32_t)(tk & c.pmask);
    const uint8_t* base = pg >= 0 ? (IS_V ? c.vpool + pg * c.v_sp + slot0 * c.v_ss : c.kpool + pg * c.k_sp + slot0 * c.k_ss)
                                  : c.safe;
    const uint32_t off = pg >= 0 ? (IS_V ? c.v_lane : c.k_lane) : c.safe_lane;
    load_row_block<FMT, NT>(base + off, R.d[k]);
  }
  return R;
}

// QK^T and the online-softmax update of one granule; leaves the
// probabilities (pr[k][v]: tile k, row v) for the PV step.
template <int FMT>
__device__ __forceinline__ void qk_softmax(const Ctx& c, const v8i& qa, int gi, const Rows<FMT>& K, State& st,
                                           float pr[2][4]) {
  using F = Fmt<FMT>;
  const int t0 = c.j0 + gi * kGran;
  float s[2][4];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    v8i kb;
#pragma unroll
    for (int i = 0; i < 8; ++i) kb[i] = i < F::kDw ? (int)K.d[k][i] : 0;
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa, kb, zero, 0, F::kMfma, 0, kE8m0One, 0,
                                                                    kE8m0One);
    const int tk = t0 + 16 * k;
    const bool live = tile_page(c, tk) >= 0;  // scalar, re-read from the cached block table
    const int t = tk + c.n;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const bool vis = live && t < c.j1 && (!c.causal || t <= c.lim0 + c.row_tok[v]);
      s[k][v] = vis ? d[v] * c.cscale : -INFINITY;
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float mx = uniform_f(row_max16(fmaxf(s[0][v], s[1][v])));
    if (mx > st.m[v] + kLazyMax) {  // wave-uniform
      const float a = exp2f(st.m[v] - mx);  // m = -inf -> 0
      st.m[v] = mx;
      st.l[v] *= a;
#pragma unroll
      for (int ch = 0; ch < 32; ++ch) st.acc[v][ch] *= a;
    }
    const float ms = st.m[v] == -INFINITY ? 0.0f : st.m[v];
    pr[0][v] = exp2f(s[0][v] - ms);
    pr[1][v] = exp2f(s[1][v] - ms);
    st.l[v] += pr[0][v] + pr[1][v];
  }
}

// Rows past the range end hold whatever the page holds (NaN codes too): a
// tile that crosses the end zeroes this lane's row if its token is past it,
// so that its zero probabilities add exact zeros.
template <int FMT>
__device__ __forceinline__ void pv(const Ctx& c, int gi, Rows<FMT>& V, const float pr[2][4], State& st) {
  const int t0 = c.j0 + gi * kGran;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int tk = t0 + 16 * k;
    if (tk + 16 > c.j1 && tk + c.n >= c.j1) {
#pragma unroll
      for (int i = 0; i < Fmt<FMT>::kDw; ++i) V.d[k][i] = 0u;
    }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if constexpr (FMT == 0) {
      // one dword (4 channels) at a time, consumed at once; a dead tile has
      // p = 0 and finite (Q-row) bytes, so it adds exact zeros
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const v2f lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(V.d[k][i], 1.0f, false);
        const v2f hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(V.d[k][i], 1.0f, true);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          st.acc[v][4 * i + 0] += pr[k][v] * lo[0];
          st.acc[v][4 * i + 1] += pr[k][v] * lo[1];
          st.acc[v][4 * i + 2] += pr[k][v] * hi[0];
          st.acc[v][4 * i + 3] += pr[k][v] * hi[1];
        }
      }
    } else {
      v6i src;
#pragma unroll
      for (int i = 0; i < 6; ++i) src[i] = (int)V.d[k][i];
      const v32f vf = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(src, 1.0f);
#pragma unroll
      for (int ch = 0; ch < 32; ++ch)
#pragma unroll
        for (int v = 0; v < 4; ++v) st.acc[v][ch] += pr[k][v] * vf[ch];
    }
  }
}

template <int FMT, bool NT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
void decode_stream_kernel(DecodeParams p) {
  using F = Fmt<FMT>;
  __shared__ float o_s[kWaves][4][kHeadDim];
  __shared__ float m_s[kWaves][4], l_s[kWaves][4];

  const int w = blockIdx.x;
  const int g = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, j = lane >> 4;
  const int seq = p.work[4 * w];
  if (seq < 0 || seq >= p.num_seqs) return;

  int L = p.seq_lens[seq];
  L = max(0, min(L, p.max_blocks * p.page_size));
  Ctx c;
  c.j0 = p.work[4 * w + 1] * p.kv_tile;
  c.j1 = min(p.work[4 * w + 2] * p.kv_tile, L);
  c.causal = p.causal && p.q_len > 1;
  c.lim0 = L - p.q_len;
  c.n = n;
  c.bt_row = p.bt + (int64_t)seq * p.bt_stride;
  c.kpool = p.k + (int64_t)g * p.k_sh;
  c.vpool = p.v + (int64_t)g * p.v_sh;
  c.safe = p.q8 + ((int64_t)seq * p.h_k + g) * p.n_q * kHeadDim;
  c.k_sp = p.k_sp;
  c.v_sp = p.v_sp;
  c.k_ss = (uint32_t)p.k_ss;
  c.v_ss = (uint32_t)p.v_ss;
  c.k_lane = (uint32_t)(n * p.k_ss + F::kLaneOff * j);
  c.v_lane = (uint32_t)(n * p.v_ss + F::kLaneOff * j);
  c.safe_lane = (uint32_t)(F::kLaneOff * j);
  c.num_pages = p.num_pages;
  c.page_shift = p.page_shift;
  c.pmask = p.page_size - 1;
  c.cscale = p.q_descale[(int64_t)seq * p.h_k + g] * load_descale(p.kd, p.kd_kind, seq, g, p.h_k) * p.scale_log2;
#pragma unroll
  for (int v = 0; v < 4; ++v) c.row_tok[v] = v / p.h_r;
  const bool single = p.n_splits[seq] <= 1;

  // A operand: quantized Q row (n & 3) if it exists, bytes [32j, 32j+32)
  v8i qa;
  {
    const int r = n & 3;
    if (r < p.n_q) {
      const u32x4* src = reinterpret_cast<const u32x4*>(c.safe + r * kHeadDim + 32 * j);
      const u32x4 a = src[0], b = src[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qa[i] = (int)a[i];
        qa[4 + i] = (int)b[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) qa[i] = 0;
    }
  }

  State st;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    st.m[v] = -INFINITY;
    st.l[v] = 0.0f;
#pragma unroll
    for (int ch = 0; ch < 32; ++ch) st.acc[v][ch] = 0.0f;
  }

  const int ngr = (c.j1 - c.j0 + kGran - 1) / kGran;
  int gi = wave;
  if (gi < ngr) {
    // issue order per step: V(next), [QK(cur)], K(next), [softmax, PV(cur)]
    Rows<FMT> K = load_rows<FMT, NT, false>(c, gi);
    Rows<FMT> VA = load_rows<FMT, NT, true>(c, gi);
    float pr[2][4];
    while (true) {
      Rows<FMT> VB = load_rows<FMT, NT, true>(c, gi + kWaves);
      qk_softmax<FMT>(c, qa, gi, K, st, pr);
      K = load_rows<FMT, NT, false>(c, gi + kWaves);
      pv<FMT>(c, gi, VA, pr, st);
      gi += kWaves;
      if (gi >= ngr) break;
      VA = load_rows<FMT, NT, true>(c, gi + kWaves);
      qk_softmax<FMT>(c, qa, gi, K, st, pr);
      K = load_rows<FMT, NT, false>(c, gi + kWaves);
      pv<FMT>(c, gi, VB, pr, st);
      gi += kWaves;
      if (gi >= ngr) break;
    }
  }

  // reduce this wave's per-lane partials over the 16 token lanes
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    st.l[v] = row_sum16(st.l[v]);
#pragma unroll
    for (int ch = 0; ch < 32; ++ch) st.acc[v][ch] = row_sum16(st.acc[v][ch]);
  }
  if (n == 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int ch = 0; ch < 32; ++ch) o_s[wave][v][32 * j + ch] = st.acc[v][ch];
  }
  if (lane == 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      m_s[wave][v] = st.m[v];
      l_s[wave][v] = st.l[v];
    }
  }
  __syncthreads();

  // combine the 4 waves; thread -> (row r, channel ch), r in {tid>>7, (tid>>7)+2}
  const int ch = threadIdx.x & 127;
  const float vd = load_descale(p.vd, p.vd_kind, seq, g, p.h_k);
  for (int r = threadIdx.x >> 7; r < p.n_q; r += 2) {
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, m_s[ww][r]);
    const float Ms = M == -INFINITY ? 0.0f : M;
    float Lsum = 0.0f, O = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float wt = exp2f(m_s[ww][r] - Ms);
      Lsum += wt * l_s[ww][r];
      O += wt * o_s[ww][r][ch];
    }
    const int t = r / p.h_r;
    const int h = g * p.h_r + (r - t * p.h_r);
    const float om = (p.o_mul ? p.o_mul[(int64_t)h * kHeadDim + ch] : 1.0f) * vd;
    if (single) {
      const float o = Lsum > 0.0f ? O / Lsum * om : 0.0f;
      store_out(p.out, p.out_f32, ((int64_t)seq * p.q_len + t) * p.out_ts + (int64_t)h * p.out_hs + ch, o);
      if (ch == 0 && p.lse)
        p.lse[((int64_t)seq * p.q_len + t) * p.h_q + h] = Lsum > 0.0f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
    } else if (w < p.part_items) {
      const int64_t idx = ((int64_t)w * p.h_k + g) * p.nqp + r;
      p.o_part[idx * kHeadDim + ch] = O * om;
      if (ch == 0) {
        p.m_part[idx] = Lsum > 0.0f ? M : -INFINITY;
        p.l_part[idx] = Lsum;
      }
    }
  }
}

}  // namespace

// Kernel choice: 0 = automatic, 1 = always the generic kernel, 2 = the
// VALU-PV streaming kernel wherever it applies, 3 = same as 0, 10..17 = the
// matrix-core kernel with tuning setting (variant - 10): bit 0 two granules
// of prefetch, bit 1 head-major grid, bit 2 XCD-grouped grid.
static int g_variant = 0;
static int g_nontemporal = 1;

void set_decode_variant(int v, int nt) {
  g_variant = v;
  g_nontemporal = nt;
}

// 0 = generic kernel, 1 = matrix-core kernel, 2 = VALU-PV streaming kernel.
// row_tiles (the plan's 64-row tiles) does not enter: the matrix-core kernel
// serves any row count in 32-row tiles of its own.
static int kernel_choice(const DecodeParams& p, int kv_format, int row_tiles) {
  (void)row_tiles;
  // the streaming kernels address a page's rows with 32-bit lane offsets and
  // take whole 16-token tiles inside one page
  const bool small_strides = p.k_ss < (1 << 24) && p.v_ss < (1 << 24) && p.ksb_ss < (1 << 24) && p.vsb_ss < (1 << 24);
  const bool tiles_ok = (p.kv_tile % 16) == 0 && small_strides;
  if (g_variant == 1 || !tiles_ok || !decode_mfma_supports(p.n_q)) return 0;
  if (kv_format != 0 || g_variant != 2 || p.n_q > 4 || p.q_bf16) return 1;
  return 2;
}

bool decode_fuses_step(const DecodeParams& p, int kv_format, int row_tiles) {
  return kernel_choice(p, kv_format, row_tiles) == 1;
}

hipError_t launch_decode(const DecodeParams& p, int kv_format, int row_tiles, hipStream_t s) {
  const int k = kernel_choice(p, kv_format, row_tiles);
  // only the matrix-core kernel fuses the step; bf16 Q is read by it and the generic kernel
  if (k != 1 && ((p.qb && !p.q_bf16) || p.counters)) return hipErrorInvalidValue;
  // the fused merge counts one arrival per (item, KV head): one row tile
  if (p.counters && p.n_q > kMfmaTileRows) return hipErrorInvalidValue;
  if (k == 0) return launch_decode_generic(p, kv_format, row_tiles, s);
  if (k == 1) {
    // debug setting -> matrix-core cache policy bits (K non-temporal, V non-temporal)
    static const int kPolicy[5] = {0, -1, 3, 2, 1};
    return launch_decode_mfma(p, kv_format, kPolicy[g_nontemporal], g_variant >= 10 ? g_variant - 10 : -1, s);
  }
  const dim3 grid(p.num_work, p.h_k);
  if (g_nontemporal)
    hipLaunchKernelGGL((decode_stream_kernel<0, true>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((decode_stream_kernel<0, false>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mj
