// KV-cache write: the step's new key / value rows quantized into the paged
// cache through a slot mapping.
//
// Method (wheel listing mjolnir/backend.py, do_kv_cache_update, _write_kv
// and _install_fp6_scales): an e4m3 cache is written with a per-tensor or
// per-KV-head scale, a packed fp6 cache with per-(KV head, channel) scales
// s_c (any scale kind is taken for any format).  Each value becomes
// round-to-nearest-even(x / s) in the cache format, saturated at its largest
// magnitude (448 e4m3, 7.5 e2m3, 28 e3m2, 6 e2m1), from one correctly rounded
// fp32 division (built with -fhip-fp32-correctly-rounded-divide-sqrt) of
// the exact fp32 value of the bf16 input (computed from the correctly rounded
// reciprocal with one FMA correction), so the bytes are the same as any other
// correct evaluation.  fp6 and fp4 rows are the little-endian 6- and 4-bit
// streams the decode kernels read (code k at stream bits [6k, 6k+6) or
// [4k, 4k+4)).  nvfp4 (the published NVFP4 recipe): per 16-channel block of
// y = x / s, the e4m3 block scale RNE(amax|y| / 6), codes RNE_e2m1(y /
// e4m3(scale)), both divisions correctly rounded, zero codes under a zero
// scale; the scale byte goes to the block-scale row of the same slot.  Slot s is
// page s / page_size, row s % page_size; a negative slot (padding) or one
// past the pool is skipped.
//
// One thread per (KV head, 16 channels) of 1 or 2 tokens: 32 bytes of bf16 in
// per side and token, 16 bytes (e4m3), 12 bytes (fp6) or 8 bytes (fp4;
// nvfp4 also the block's scale byte) of codes out.  The
// write touches every byte once.
#include "mj_device.h"
#include "mj_internal.h"

namespace mj {

namespace {

constexpr int kWThreads = 256;

// The 16 bf16 values of one (token, KV head, channel group) as loaded.
struct Raw16 {
  uint4 a, b;
};

typedef short v2s __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v6i __attribute__((ext_vector_type(6)));

// The encoders are gfx950's converters at unit scale on the correctly
// rounded quotient: round to nearest, ties to even, the sign kept (a
// negative value that rounds to zero gives the negative zero code), e2m3,
// e3m2 and e2m1 saturating at their largest magnitude (all measured against
// the format tables at every grid point, midpoint and its neighbours).  The
// fp8 converter turns values past 448 into the NaN code instead, so e4m3
// inputs are clamped to +-448 first.
// e4m3 codes of a and b in the low and high byte of the low half-word
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  const float lo = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f), hi = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  v2s r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, lo, hi, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r) & 0xFFFFu;
}
// e2m1 codes of v[0..7], code k in bits [4k, 4k + 4)
__device__ __forceinline__ uint32_t e2m1_word(const float* v) {
  uint32_t r = 0u;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[0], v[1], 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2], v[3], 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[4], v[5], 1.0f, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[6], v[7], 1.0f, 3);
  return r;
}

// dst_bs (nvfp4 only): the row's block-scale byte of these 16 channels
template <int FMT>
__device__ __forceinline__ void write_side(const Raw16& in, const float (&sc)[16], const float (&rc)[16], int c0,
                                           uint8_t* dst_row, uint8_t* dst_bs) {
  const uint4 a = in.a, b = in.b;
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float q[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t bits = (i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16);
    q[i] = div_rn(__uint_as_float(bits), sc[i], rc[i]);
  }
  if constexpr (FMT == 4) {
    // nvfp4: the 16 channels are one block; e4m3 scale of amax / 6, codes of
    // q / scale (zero codes under a zero scale)
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(q[i]));
    const uint32_t sc8 = e4m3_pair(div_rn(amax, 6.0f, 1.0f / 6.0f), 0.0f) & 0xFFu;
    const float sv = e4m3_value(sc8);
    const float rv = 1.0f / sv;  // correctly rounded; unused when sv == 0
    float y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = div_rn(q[i], sv, rv);
    uint2 o = {e2m1_word(y), e2m1_word(y + 8)};
    if (!(sv > 0.0f)) o = make_uint2(0u, 0u);
    *reinterpret_cast<uint2*>(dst_row + (c0 / 16) * 8) = o;
    *dst_bs = (uint8_t)sc8;
  } else if constexpr (FMT == 0) {
    uint4 o;
    o.x = e4m3_pair(q[0], q[1]) | (e4m3_pair(q[2], q[3]) << 16);
    o.y = e4m3_pair(q[4], q[5]) | (e4m3_pair(q[6], q[7]) << 16);
    o.z = e4m3_pair(q[8], q[9]) | (e4m3_pair(q[10], q[11]) << 16);
    o.w = e4m3_pair(q[12], q[13]) | (e4m3_pair(q[14], q[15]) << 16);
    *reinterpret_cast<uint4*>(dst_row + c0) = o;
  } else if constexpr (FMT == 3) {
    *reinterpret_cast<uint2*>(dst_row + (c0 / 16) * 8) = make_uint2(e2m1_word(q), e2m1_word(q + 8));
  } else {
    // e2m3 / e3m2: the converter's output slot 2i takes element i of its
    // first operand, slot 2i + 1 element i of its second (measured), so the
    // even channels go first and the odd second; its upper 16 slots are
    // unused here
    v16f ev, od;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ev[i] = q[2 * i];
      od[i] = q[2 * i + 1];
      ev[8 + i] = 0.0f;
      od[8 + i] = 0.0f;
    }
    const v6i pk = FMT == 1 ? __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 1.0f)
                            : __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(ev, od, 1.0f);
    uint32_t* d = reinterpret_cast<uint32_t*>(dst_row + (c0 / 16) * 12);
    d[0] = (uint32_t)pk[0];
    d[1] = (uint32_t)pk[1];
    d[2] = (uint32_t)pk[2];
  }
}

// The 16 divisors of channels [c0, c0 + 16) of KV head g and their
// correctly rounded reciprocals: one of each for a per-tensor or per-head
// scale, sixteen for per-channel scales.
__device__ __forceinline__ void load_divisors(const float* s, int kind, int g, int c0, float (&sc)[16],
                                              float (&rc)[16]) {
  if (kind == 3) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sc[i] = s[g * kHeadDim + c0 + i];
      rc[i] = 1.0f / sc[i];
    }
  } else {
    const float d = kind == 0 ? s[0] : s[g];
    const float r = 1.0f / d;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sc[i] = d;
      rc[i] = r;
    }
  }
}

// Thread -> (KV head g, channel group grp) of TPT consecutive tokens (the
// divisors are set up once per thread); the 8 h_k threads of one token's
// rows are adjacent, so each token's bf16 rows are read with coalesced
// 16-byte loads.  Every slot and every input row of the thread's tokens is
// loaded before any is encoded: the rows do not depend on the slots, so the
// loads are in flight together instead of one token's chain at a time.
template <int FMT, int TPT>
__global__ __launch_bounds__(kWThreads) void write_kv_kernel(WriteParams p) {
  const int64_t gid = (int64_t)blockIdx.x * kWThreads + threadIdx.x;
  const int row_threads = p.h_k * 8;
  const int64_t blocks = ((int64_t)p.num_tokens + TPT - 1) / TPT;
  if (gid >= blocks * row_threads) return;
  const int r = (int)(gid % row_threads);
  const int64_t tb = gid / row_threads;
  const int grp = r & 7, g = r >> 3;
  const int c0 = grp * 16;
  int64_t slot[TPT];
  Raw16 kin[TPT], vin[TPT];
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
    const int64_t t = tb * TPT + u;
    const bool ok = t < p.num_tokens;
    const int64_t tc = ok ? t : tb * TPT;  // past the end: repeat the first token (loaded, never stored)
    slot[u] = ok ? p.slots[tc] : -1;
    const uint16_t* ks = p.key + tc * p.k_ts + (int64_t)g * p.k_hs + c0;
    const uint16_t* vs = p.value + tc * p.v_ts + (int64_t)g * p.v_hs + c0;
    kin[u].a = *reinterpret_cast<const uint4*>(ks);
    kin[u].b = *reinterpret_cast<const uint4*>(ks + 8);
    vin[u].a = *reinterpret_cast<const uint4*>(vs);
    vin[u].b = *reinterpret_cast<const uint4*>(vs + 8);
  }
  float ks[16], kr[16], vs[16], vr[16];
  load_divisors(p.ks, p.ks_kind, g, c0, ks, kr);
  load_divisors(p.vs, p.vs_kind, g, c0, vs, vr);
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
    if (slot[u] < 0) continue;
    const int64_t page = slot[u] >> p.page_shift;
    if (page >= p.num_pages) continue;
    const int64_t row = slot[u] & ((1 << p.page_shift) - 1);
    uint8_t* kb = FMT == 4 ? p.kbs + page * p.kbs_sp + row * p.kbs_ss + (int64_t)g * p.kbs_sh + grp : nullptr;
    uint8_t* vb = FMT == 4 ? p.vbs + page * p.vbs_sp + row * p.vbs_ss + (int64_t)g * p.vbs_sh + grp : nullptr;
    write_side<FMT>(kin[u], ks, kr, c0, p.kc + page * p.kc_sp + row * p.kc_ss + (int64_t)g * p.kc_sh, kb);
    write_side<FMT>(vin[u], vs, vr, c0, p.vc + page * p.vc_sp + row * p.vc_ss + (int64_t)g * p.vc_sh, vb);
  }
}

template <int TPT>
hipError_t launch_tpt(const WriteParams& p, hipStream_t s) {
  const int64_t threads = ((int64_t)p.num_tokens + TPT - 1) / TPT * p.h_k * 8;
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + kWThreads - 1) / kWThreads));
  switch (p.kv_format) {
    case 0: hipLaunchKernelGGL((write_kv_kernel<0, TPT>), grid, dim3(kWThreads), 0, s, p); break;
    case 1: hipLaunchKernelGGL((write_kv_kernel<1, TPT>), grid, dim3(kWThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL((write_kv_kernel<2, TPT>), grid, dim3(kWThreads), 0, s, p); break;
    case 3: hipLaunchKernelGGL((write_kv_kernel<3, TPT>), grid, dim3(kWThreads), 0, s, p); break;
    default: hipLaunchKernelGGL((write_kv_kernel<4, TPT>), grid, dim3(kWThreads), 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_write_kv(const WriteParams& p_in, hipStream_t s) {
  // per-channel scales: two tokens per thread amortize the sixteen
  // reciprocals per side once the grid is large (measured at 16K tokens x 8
  // heads with the hardware encoders: e2m3 24.3 us at one or four tokens per
  // thread, 22.1 at two; e2m1 unchanged); per-tensor or per-head scales (one
  // reciprocal) and small writes (a decode step's new rows) take one token
  // per thread
  WriteParams p = p_in;
  const int64_t rows = (int64_t)p.num_tokens * p.h_k;
  const bool channel = p.ks_kind == 3 || p.vs_kind == 3;
  p.tokens_per_thread = channel && rows >= (1 << 14) ? 2 : 1;
  return p.tokens_per_thread == 2 ? launch_tpt<2>(p, s) : launch_tpt<1>(p, s);
}

}  // namespace mj
