// Device-side helpers shared by the mj kernels (gfx950, wave64).
//
// Formats (the e4m3 / e2m3 / e3m2 / e2m1 codes the mjolnir-kernel pages name;
// bit layouts from the OCP OFP8 and OCP MX specifications):
//   e4m3: s.eeee.mmm, bias 7, subnormal at e == 0, max 448.
//   e2m3: s.ee.mmm (6 bits), bias 1, subnormal at e == 0, max 7.5.
//   e3m2: s.eee.mm (6 bits), bias 3, subnormal at e == 0, max 28.
//   e2m1: s.ee.m (4 bits), bias 1, subnormal at e == 0, max 6.
// All decode by moving the exponent/mantissa bits into an fp32 bit pattern
// with the same mantissa alignment and rescaling by a power of two: an fp32
// with exponent field e and mantissa m/2^k is 2^(e-127)(1+m/2^k), and its
// subnormals (e == 0) are 2^-126 (m/2^k), so one multiply by 2^(127 - bias)
// -- 2^120 (e4m3), 2^126 (e2m3, e2m1), 2^124 (e3m2) -- maps both normal and
// subnormal codes exactly.  Callers fold that power of two into the descale
// they multiply by anyway.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mj {

constexpr int kHeadDim = 128;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kE4m3Rescale = 1.329227995784916e+36f;  // 2^120
constexpr float kE2m3Rescale = 8.507059173023462e+37f;  // 2^126
constexpr float kE3m2Rescale = 2.1267647932558654e+37f;  // 2^124
constexpr float kE2m1Rescale = 8.507059173023462e+37f;  // 2^126

__device__ __forceinline__ float bits_to_float(uint32_t u) { return __uint_as_float(u); }

// e4m3 code (low 8 bits) -> fp32 bit pattern whose value is 2^-120 * value.
__device__ __forceinline__ float e4m3_raw(uint32_t c) {
  return bits_to_float(((c & 0x80u) << 24) | ((c & 0x7Fu) << 20));
}
// e2m3 code (low 6 bits) -> fp32 whose value is 2^-126 * value.
__device__ __forceinline__ float e2m3_raw(uint32_t c) {
  return bits_to_float(((c & 0x20u) << 26) | ((c & 0x1Fu) << 20));
}
// e3m2 code (low 6 bits) -> fp32 whose value is 2^-124 * value.
__device__ __forceinline__ float e3m2_raw(uint32_t c) {
  return bits_to_float(((c & 0x20u) << 26) | ((c & 0x1Fu) << 21));
}
// e2m1 code (low 4 bits) -> fp32 whose value is 2^-126 * value.
__device__ __forceinline__ float e2m1_raw(uint32_t c) {
  return bits_to_float(((c & 0x8u) << 28) | ((c & 0x7u) << 22));
}
__device__ __forceinline__ float e4m3_value(uint32_t c) { return e4m3_raw(c) * kE4m3Rescale; }
__device__ __forceinline__ float e2m3_value(uint32_t c) { return e2m3_raw(c) * kE2m3Rescale; }
__device__ __forceinline__ float e3m2_value(uint32_t c) { return e3m2_raw(c) * kE3m2Rescale; }
__device__ __forceinline__ float e2m1_value(uint32_t c) { return e2m1_raw(c) * kE2m1Rescale; }

// Four e4m3 codes (one word, byte b = code b) -> four bf16 (two words, code
// 2i + h in half h of word i) with gfx950's scaled converter at scale 1.
// Exact: every e4m3 value, subnormals included, is a normal bf16 (8-bit
// significand, exponent range far wider); the two NaN codes give NaN.
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t w, uint32_t out[2]) {
  typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
  out[0] = __builtin_bit_cast(uint32_t, (v2bf_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  out[1] = __builtin_bit_cast(uint32_t, (v2bf_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// Round an fp32 to the nearest e4m3 code, ties to even.  Domain: finite
// |x| <= 464 (the Q quantizer stays within 448 * (1 + 2^-23)).
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  u &= 0x7FFFFFFFu;
  // normal e4m3 (|x| >= 2^-6): keep 3 of 23 mantissa bits, ties to even
  const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
  const uint32_t nrm = min(((r >> 23) << 3) - (120u << 3) + ((r >> 20) & 7u), 0x7Eu);
  // subnormal range: multiples of 2^-9 (8 * 2^-9 is the min normal)
  const uint32_t sub = (uint32_t)__builtin_rintf(__uint_as_float(u) * 512.0f);
  return sign | (u >= 0x3C800000u ? nrm : sub);
}

// Round an fp32 to the nearest e2m3 code (6 bits), ties to even, saturating
// at 7.5 (any magnitude, infinities included).  Normal range (|x| >= 1): keep
// 3 of 23 mantissa bits with the carry running into the exponent; below it,
// multiples of 1/8 (8/8 is the smallest normal, code 8).
__device__ __forceinline__ uint32_t e2m3_rne(float x) {
  uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 26) & 0x20u;
  u &= 0x7FFFFFFFu;
  const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
  const uint32_t nrm = min(((r >> 23) << 3) - (126u << 3) + ((r >> 20) & 7u), 0x1Fu);
  const uint32_t sub = (uint32_t)__builtin_rintf(__uint_as_float(u) * 8.0f);
  return sign | (u >= 0x3F800000u ? nrm : sub);
}

// Round an fp32 to the nearest e3m2 code (6 bits), ties to even, saturating
// at 28.  Normal range (|x| >= 2^-2): keep 2 of 23 mantissa bits with the
// carry running into the exponent; below it, multiples of 2^-4.
__device__ __forceinline__ uint32_t e3m2_rne(float x) {
  uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 26) & 0x20u;
  u &= 0x7FFFFFFFu;
  const uint32_t r = u + 0xFFFFFu + ((u >> 21) & 1u);
  const uint32_t nrm = min(((r >> 23) << 2) - (124u << 2) + ((r >> 21) & 3u), 0x1Fu);
  const uint32_t sub = (uint32_t)__builtin_rintf(__uint_as_float(u) * 16.0f);
  return sign | (u >= 0x3E800000u ? nrm : sub);
}

// Round an fp32 to the nearest e2m1 code (4 bits), ties to even, saturating
// at 6.  Normal range (|x| >= 1): keep 1 of 23 mantissa bits; below it,
// multiples of 1/2.
__device__ __forceinline__ uint32_t e2m1_rne(float x) {
  uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 28) & 0x8u;
  u &= 0x7FFFFFFFu;
  const uint32_t r = u + 0x1FFFFFu + ((u >> 22) & 1u);
  const uint32_t nrm = min(((r >> 23) << 1) - (126u << 1) + ((r >> 22) & 1u), 0x7u);
  const uint32_t sub = (uint32_t)__builtin_rintf(__uint_as_float(u) * 2.0f);
  return sign | (u >= 0x3F800000u ? nrm : sub);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
// One output element: bf16 (round to nearest even), or fp32 when f32 is set
// (the buffer is then fp32 with the same element strides).
__device__ __forceinline__ uint16_t f32_to_bf16(float f);
__device__ __forceinline__ void store_out(uint16_t* out, int f32, int64_t idx, float v) {
  if (f32)
    reinterpret_cast<float*>(out)[idx] = v;
  else
    out[idx] = f32_to_bf16(v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Descale lookup for the three descale shapes (tensor, per KV head, per
// (sequence, KV head)).
__device__ __forceinline__ float load_descale(const float* d, int kind, int seq, int g, int h_k) {
  return kind == 0 ? d[0] : (kind == 1 ? d[g] : d[(int64_t)seq * h_k + g]);
}

// Physical page of token j of a sequence, or -1 if the block-table entry is
// outside [0, num_pages).
__device__ __forceinline__ int64_t page_of(const int32_t* bt_row, int j, int page_shift, int64_t num_pages) {
  const int64_t pg = bt_row[j >> page_shift];
  return (pg >= 0 && pg < num_pages) ? pg : -1;
}

// Byte offset of (page, slot, head) in a pool with byte strides.
__device__ __forceinline__ int64_t kv_offset(int64_t page, int slot, int head, int64_t sp, int64_t ss, int64_t sh) {
  return page * sp + (int64_t)slot * ss + (int64_t)head * sh;
}

// 16 e2m3 codes from 12 packed bytes (three little-endian dwords).
__device__ __forceinline__ void unpack16_6bit(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t out[16]) {
  // stream bit b of the 96-bit group is bit b%32 of word b/32
  const uint64_t lo = (uint64_t)w0 | ((uint64_t)w1 << 32);
  const uint64_t hi = (uint64_t)w1 | ((uint64_t)w2 << 32);  // starts at stream bit 32
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int b = 6 * k;
    out[k] = b + 6 <= 64 ? (uint32_t)((lo >> b) & 63u) : (uint32_t)((hi >> (b - 32)) & 63u);
  }
}

}  // namespace mj

namespace mj {

// x / s rounded to nearest from y = RN(1/s): q = RN(x y) is a faithful
// quotient, the residual x - q s is exact in one FMA, and RN(q + r y) is the
// correctly rounded quotient (Markstein's theorem; Muller et al., Handbook of
// Floating-Point Arithmetic, on division by FMA).  Quotients that underflow
// into fp32 subnormals or overflow lie far below or above every rounding
// boundary of the four formats, so their codes are those of the exact
// quotient.
// Scales are positive and finite; y = 1 / s computed with the (correctly
// rounded) division.
__device__ __forceinline__ float div_rn(float x, float s, float y) {
  const float q = x * y;
  const float r = __builtin_fmaf(-q, s, x);
  // a zero quotient keeps its sign (-0 / s = -0; the correction would give +0)
  return x == 0.0f ? x : __builtin_fmaf(r, y, q);
}

// Dynamic e4m3 quantization of Q per (sequence, KV head), the arithmetic
// both the stand-alone quantize kernel and the fused decode step use, so the
// two produce the same codes and scale bit for bit (mjolnir-kernel wheel page
// mjolnir/runner.py, T5DecodeRunner.run, fp8-Q branch): over the q_len tokens
// and h_r query heads of KV head g, x = fp32(q) [* q_mul], amax = max(max|x|,
// 1e-6), s = amax / 448, code = e4m3(x / s), rows packed t*h_r + r.  The
// division must be the correctly rounded one (the library is built with
// -fhip-fp32-correctly-rounded-divide-sqrt).
constexpr float kQAmaxFloor = 1e-6f;
constexpr float kFp8Max = 448.0f;

// Raw bf16 words and multipliers of channels [c0, c0 + 8) of packed row
// `row` of (seq, g); without q_mul the multiplier words are read from Q
// itself (a valid address) and ignored, so the fetch has no branch.
struct QRaw8 {
  uint4 q;
  float4 m0, m1;
};

__device__ __forceinline__ QRaw8 q_fetch8(const uint16_t* q, int64_t q_ts, int64_t q_hs, const float* q_mul,
                                          int q_len, int h_r, int seq, int g, int row, int c0) {
  const int t = row / h_r;
  const int h = g * h_r + (row - t * h_r);
  const uint16_t* src = q + ((int64_t)seq * q_len + t) * q_ts + (int64_t)h * q_hs + c0;
  QRaw8 r;
  r.q = *reinterpret_cast<const uint4*>(src);
  const float* m = q_mul ? q_mul + (int64_t)h * kHeadDim + c0 : reinterpret_cast<const float*>(src);
  r.m0 = *reinterpret_cast<const float4*>(m);
  r.m1 = *reinterpret_cast<const float4*>(q_mul ? m + 4 : m);
  return r;
}

// The eight values as fp32: x = fp32(q) [* q_mul] (one multiply each).
__device__ __forceinline__ void q_convert8(const QRaw8& r, bool has_mul, float x[8]) {
  const uint32_t w[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(w[e] << 16);
    x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
  }
  if (has_mul) {
    x[0] *= r.m0.x; x[1] *= r.m0.y; x[2] *= r.m0.z; x[3] *= r.m0.w;
    x[4] *= r.m1.x; x[5] *= r.m1.y; x[6] *= r.m1.z; x[7] *= r.m1.w;
  }
}

// Channels [c0, c0 + 8) of packed row `row` of (seq, g) as fp32.
__device__ __forceinline__ void q_load8(const uint16_t* q, int64_t q_ts, int64_t q_hs, const float* q_mul, int q_len,
                                        int h_r, int seq, int g, int row, int c0, float x[8]) {
  q_convert8(q_fetch8(q, q_ts, q_hs, q_mul, q_len, h_r, seq, g, row, c0), q_mul != nullptr, x);
}

__device__ __forceinline__ float q_scale_from_amax(float amax) { return fmaxf(amax, kQAmaxFloor) / kFp8Max; }

// Eight e4m3 codes of x / s, little-endian in two dwords; rs = 1 / s (the
// correctly rounded reciprocal), so each quotient is div_rn's correctly
// rounded one without a division per value.
__device__ __forceinline__ uint2 q_codes8(const float x[8], float s, float rs) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) lo |= e4m3_rne(div_rn(x[e], s, rs)) << (8 * e);
#pragma unroll
  for (int e = 0; e < 4; ++e) hi |= e4m3_rne(div_rn(x[4 + e], s, rs)) << (8 * e);
  return make_uint2(lo, hi);
}

}  // namespace mj
