"""Codecs of the KV-cache and Q formats, from their published definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* e4m3 ("float8_e4m3fn", the dtype the mjolnir-kernel runner maps fp8 Q and
  fp8 KV to; wheel listing mjolnir/runner.py, ``_cutlass_dtype`` and the
  ``FP8_MAX = 448`` constant): OCP 8-bit floating point, E4M3 variant — sign
  bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
  subnormal (m/8 * 2^-6); no infinities; S.1111.111 is NaN; largest finite
  magnitude 448.
* e2m3 (the 6-bit KV format; PyPI project page, "fp6 (e2m3) KV in vLLM";
  ``E2M3_MAX`` = 7.5 in mjolnir/backend.py, ``_install_fp6_scales``): OCP
  Microscaling FP6 E2M3 — sign bit 5, exponent bits 4..3 with bias 1,
  mantissa bits 2..0; exponent field 0 is subnormal (m/8); no NaN or
  infinity; largest magnitude 7.5.
* the packed 6-bit row: "e2m3 codes packed 4 per 3 bytes (little-endian
  bitstream)" (mjolnir/runner.py, the comment above ``RUNNER_KV_FORMATS``).
  Reading taken: code k of a row occupies stream bits [6k, 6k+6) and stream
  bit 8B+j is bit j of byte B.
* e3m2 and e2m1, the other formats the pages' harness reads ("Beyond fp8:
  the harness": fp6 e2m3/e3m2 and fp4 e2m1): OCP Microscaling FP6 E3M2 --
  sign bit 5, exponent bits 4..2 with bias 3, mantissa bits 1..0, exponent
  field 0 subnormal (m/4 * 2^-2), no NaN or infinity, largest magnitude 28 --
  and OCP Microscaling FP4 E2M1 -- sign bit 3, exponent bits 2..1 with bias
  1, mantissa bit 0, exponent field 0 subnormal (m/2), largest magnitude 6.
  Packing (the pages give none for them; the plainest reading, the same
  little-endian bitstream as e2m3): e3m2 rows exactly like e2m3 rows, e2m1
  code k at stream bits [4k, 4k+4), i.e. the low nibble of byte k/2 for even
  k and its high nibble for odd k (64-byte rows).
* nvfp4, the harness's remaining format ("Beyond fp8: the harness"; the
  runner passes the kernel a K and a V "nvfp4 scale pointer", typed
  float8_e4m3fn, mjolnir/runner.py ``dummy_scales``).  The pages give
  neither its block size nor where the scales live; the reading taken is the
  published NVFP4 format: e2m1 codes in blocks of 16 consecutive values that
  share one e4m3 scale, value = e2m1(code) * e4m3(scale), times a per-tensor
  (here also per-head or per-(sequence, head)) fp32 scale.  A 128-channel row
  is then 64 code bytes (the e2m1 row) plus 8 scale bytes, scale b covering
  channels [16b, 16b + 16); the scale rows live in a pool of their own, paged
  like the codes.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M3_MAX = 7.5


def e4m3_value(code: int) -> float:
    """Value of one e4m3 code from its bit fields (NaN for S.1111.111)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e2m3_value(code: int) -> float:
    """Value of one 6-bit e2m3 code from its bit fields."""
    s = -1.0 if code & 0x20 else 1.0
    e = (code >> 3) & 0x3
    m = code & 0x7
    if e == 0:
        return s * (m / 8.0)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 1)


def e3m2_value(code: int) -> float:
    """Value of one 6-bit e3m2 code from its bit fields."""
    s = -1.0 if code & 0x20 else 1.0
    e = (code >> 2) & 0x7
    m = code & 0x3
    if e == 0:
        return s * (m / 4.0) * 2.0 ** -2
    return s * (1.0 + m / 4.0) * 2.0 ** (e - 3)


def e2m1_value(code: int) -> float:
    """Value of one 4-bit e2m1 code from its bit fields."""
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return s * (m / 2.0)
    return s * (1.0 + m / 2.0) * 2.0 ** (e - 1)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M3_TABLE = np.array([e2m3_value(c) for c in range(64)], dtype=np.float64)
E3M2_TABLE = np.array([e3m2_value(c) for c in range(64)], dtype=np.float64)
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E3M2_MAX = 28.0
E2M1_MAX = 6.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e2m3_decode(codes: np.ndarray) -> np.ndarray:
    return E2M3_TABLE[np.asarray(codes, dtype=np.uint8) & 0x3F]


def e3m2_decode(codes: np.ndarray) -> np.ndarray:
    return E3M2_TABLE[np.asarray(codes, dtype=np.uint8) & 0x3F]


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


# finite non-negative e4m3 values in code order 0x00..0x7E (strictly increasing)
_E4M3_POS = E4M3_TABLE[:0x7F]


def e4m3_encode(x) -> np.ndarray:
    """Round fp32 values to the nearest e4m3 code, ties to the even code.

    Round-to-nearest-even over the finite e4m3 values, with the sign kept
    (so -0 and tiny negatives give 0x80).  Domain: |x| <= 464, the midpoint
    above 448 (the quantizer never leaves it: |x/s| <= 448 * (1 + 2^-23)).
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    if np.any(~np.isfinite(a)) or np.any(a > 464.0):
        raise ValueError("e4m3_encode: value outside the rounding domain |x| <= 464")
    # nearest of the candidates below and above a
    hi = np.searchsorted(_E4M3_POS, a, side="left")  # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = _E4M3_POS[hi] - a
    d_lo = a - _E4M3_POS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    # above 448 (hi clamped to 0x7E): 448 is the nearest finite value
    code = np.where(a >= _E4M3_POS[0x7E], 0x7E, np.where(pick_hi, hi, lo))
    sign = np.signbit(x)
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


def e4m3_encode_sat(x) -> np.ndarray:
    """The cache write's e4m3 rounding: saturate to +-448, then round to the
    nearest code, ties to even (finite inputs only)."""
    x = np.asarray(x, dtype=np.float32)
    if np.any(~np.isfinite(x)):
        raise ValueError("e4m3_encode_sat: non-finite input")
    return e4m3_encode(np.clip(x, -E4M3_MAX, E4M3_MAX))


# non-negative e2m3 values in code order 0x00..0x1F (strictly increasing)
_E2M3_POS = E2M3_TABLE[:0x20]


def e2m3_encode(x) -> np.ndarray:
    """Round fp32 values to the nearest e2m3 code (6 bits), ties to the even
    code, saturating at +-7.5; the sign is kept (negative zero gives 0x20)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    if np.any(~np.isfinite(x)):
        raise ValueError("e2m3_encode: non-finite input")
    a = np.minimum(np.abs(x), E2M3_MAX)
    hi = np.minimum(np.searchsorted(_E2M3_POS, a, side="left"), 0x1F)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_hi = _E2M3_POS[hi] - a
    d_lo = a - _E2M3_POS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    return (code | (np.signbit(x).astype(np.int64) << 5)).astype(np.uint8)


def _encode_small(x, table_pos: np.ndarray, vmax: float, sign_bit: int, name: str) -> np.ndarray:
    """Nearest code of a small sign-magnitude format, ties to the even code,
    saturating at +-vmax; table_pos: the non-negative values in code order
    (strictly increasing); the sign is kept (negative zero sets the sign)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    if np.any(~np.isfinite(x)):
        raise ValueError(f"{name}: non-finite input")
    a = np.minimum(np.abs(x), vmax)
    hi = np.minimum(np.searchsorted(table_pos, a, side="left"), len(table_pos) - 1)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_hi = table_pos[hi] - a
    d_lo = a - table_pos[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    return (code | (np.signbit(x).astype(np.int64) << sign_bit)).astype(np.uint8)


def e3m2_encode(x) -> np.ndarray:
    """Round fp32 values to the nearest e3m2 code (6 bits), ties to the even
    code, saturating at +-28."""
    return _encode_small(x, E3M2_TABLE[:0x20], E3M2_MAX, 5, "e3m2_encode")


def e2m1_encode(x) -> np.ndarray:
    """Round fp32 values to the nearest e2m1 code (4 bits), ties to the even
    code, saturating at +-6."""
    return _encode_small(x, E2M1_TABLE[:0x8], E2M1_MAX, 3, "e2m1_encode")


def pack_4bit(codes: np.ndarray) -> np.ndarray:
    """(..., n) 4-bit codes -> (..., n/2) bytes: code k in stream bits
    [4k, 4k+4), written bit by bit like pack_6bit."""
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.shape[-1]
    assert n % 2 == 0
    out = np.zeros(codes.shape[:-1] + (n // 2,), dtype=np.uint8)
    for k in range(n):
        for j in range(4):
            bit = 4 * k + j
            out[..., bit // 8] |= (((codes[..., k] >> j) & 1) << (bit % 8)).astype(np.uint8)
    return out


def unpack_4bit(rows: np.ndarray, n: int) -> np.ndarray:
    """(..., n/2) bytes -> (..., n) codes of the little-endian 4-bit stream."""
    rows = np.asarray(rows, dtype=np.uint8)
    assert rows.shape[-1] * 2 == n
    out = np.zeros(rows.shape[:-1] + (n,), dtype=np.uint8)
    k = np.arange(n)
    for j in range(4):
        bit = 4 * k + j
        v = (rows[..., bit // 8] >> (bit % 8).astype(np.uint8)) & 1
        out |= (v << j).astype(np.uint8)
    return out


# bytes of one 128-value row (codes only; nvfp4 rows also have SCALE_ROW_BYTES
# of block scales in their own pool) and the largest code magnitude
ROW_BYTES = {"e4m3": 128, "e2m3": 96, "e3m2": 96, "e2m1": 64, "nvfp4": 64}
FMT_MAX = {"e4m3": E4M3_MAX, "e2m3": E2M3_MAX, "e3m2": E3M2_MAX, "e2m1": E2M1_MAX}
NVFP4_BLOCK = 16
SCALE_ROW_BYTES = {"nvfp4": 128 // NVFP4_BLOCK}


def nvfp4_decode(code_rows: np.ndarray, scale_rows: np.ndarray, n: int = 128) -> np.ndarray:
    """(..., n/2) e2m1 code bytes and (..., n/16) e4m3 scale bytes -> (..., n)
    values: value c = e2m1(code c) * e4m3(scale c // 16)."""
    vals = e2m1_decode(unpack_4bit(code_rows, n))
    scales = e4m3_decode(np.asarray(scale_rows, dtype=np.uint8))
    assert scales.shape[-1] * NVFP4_BLOCK == n
    return vals * np.repeat(scales, NVFP4_BLOCK, axis=-1)


def decode_row_codes(rows: np.ndarray, kv_format: str, n: int = 128) -> np.ndarray:
    """Packed rows (..., ROW_BYTES) -> (..., n) values of the format."""
    if kv_format == "e4m3":
        return e4m3_decode(rows)
    if kv_format == "e2m3":
        return e2m3_decode(unpack_6bit(rows, n))
    if kv_format == "e3m2":
        return e3m2_decode(unpack_6bit(rows, n))
    if kv_format == "e2m1":
        return e2m1_decode(unpack_4bit(rows, n))
    raise ValueError(kv_format)


def pack_6bit(codes: np.ndarray) -> np.ndarray:
    """(..., n) 6-bit codes -> (..., 3n/4) bytes of the little-endian stream,
    bit by bit: bit j of code k goes to stream bit 6k+j."""
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.shape[-1]
    assert n % 4 == 0
    out = np.zeros(codes.shape[:-1] + (n * 6 // 8,), dtype=np.uint8)
    for k in range(n):
        for j in range(6):
            bit = 6 * k + j
            out[..., bit // 8] |= (((codes[..., k] >> j) & 1) << (bit % 8)).astype(np.uint8)
    return out


def unpack_6bit(rows: np.ndarray, n: int) -> np.ndarray:
    """(..., 3n/4) bytes -> (..., n) codes of the little-endian 6-bit stream.

    Written bit by bit from the stream definition: bit j (0..5) of code k is
    stream bit 6k+j, which is bit (6k+j) % 8 of byte (6k+j) // 8.
    """
    rows = np.asarray(rows, dtype=np.uint8)
    assert rows.shape[-1] * 8 == n * 6
    out = np.zeros(rows.shape[:-1] + (n,), dtype=np.uint8)
    k = np.arange(n)
    for j in range(6):
        bit = 6 * k + j  # stream bit j of every code k
        v = (rows[..., bit // 8] >> (bit % 8).astype(np.uint8)) & 1
        out |= (v << j).astype(np.uint8)
    return out
