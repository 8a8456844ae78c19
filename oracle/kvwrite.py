"""The KV-cache write: new K/V rows quantized into the paged cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: the wheel listing mjolnir/backend.py.  ``do_kv_cache_update`` writes
the step's new key/value rows through ``slot_mapping``: an fp8 cache with the
base backend's write (``reshape_and_cache_flash`` with the layer's per-tensor
or per-head ``_k_scale`` / ``_v_scale``, as ``_write_kv`` calls it), an fp6
cache with the library's own packed write ``kvfp6.write_kv`` and the
per-(KV head, channel) scales that ``_install_fp6_scales`` describes ("Channel
scales s_c (h_k, d) quantize the cache write").  Neither kernel is printed;
the readings taken, the plainest the text supports:

* slot ``s`` of token ``t`` is page ``s // page_size``, row ``s % page_size``;
  a negative slot (a padding token) writes nothing, and neither does a slot
  in a page at or past ``num_pages`` (the pool's size: such a slot addresses
  no row of the cache);
* code = the format's round-to-nearest-even of ``x / scale`` in fp32 (one
  IEEE division, x = fp32 of the bf16 input), saturated at the format's
  largest magnitude (448 for e4m3, 7.5 for e2m3, 28 for e3m2, 6 for e2m1);
* 6-bit rows (e2m3, e3m2) are packed 4 codes per 3 bytes and e2m1 rows 2
  codes per byte, as the decode reads them (the little-endian bitstreams of
  ``formats.pack_6bit`` / ``pack_4bit``).
* nvfp4 (the harness's block-scaled fp4; the pages print no writer): the
  recipe of the published NVFP4 format, on y = x / scale (the fp32 division
  above, scale now the second-level tensor / head / channel divisor).  Per
  block of 16 channels, the e4m3 block scale is the cache write's e4m3
  rounding of amax(|y|) / 6 (one fp32 division), and each code is the e2m1
  rounding of y / e4m3(block scale) (one fp32 division); a block whose scale
  rounds to zero stores zero codes.  Codes go to the e2m1 row, the 8 scale
  bytes to the row of the same slot in the block-scale pool.
"""

from __future__ import annotations

import numpy as np

from .formats import (NVFP4_BLOCK, ROW_BYTES, SCALE_ROW_BYTES, e2m1_encode, e2m3_encode, e3m2_encode, e4m3_decode,
                      e4m3_encode_sat, pack_4bit, pack_6bit)


def scale_of(scale, kind: str, g: int, d: int = 128) -> np.ndarray:
    """The fp32 divisor(s) for KV head g: one value (tensor / head kind) or
    one per channel (channel kind, shape (h_k, d))."""
    scale = np.asarray(scale, dtype=np.float32)
    if kind == "tensor":
        return np.full(d, scale.reshape(-1)[0], dtype=np.float32)
    if kind == "head":
        return np.full(d, scale.reshape(-1)[g], dtype=np.float32)
    if kind == "channel":
        return scale.reshape(-1, d)[g].astype(np.float32)
    raise ValueError(kind)


def nvfp4_encode_row(y: np.ndarray):
    """fp32 values y (n,) -> (e2m1 code bytes (n/2,), e4m3 scale bytes (n/16,))."""
    y = np.asarray(y, dtype=np.float32)
    blocks = y.reshape(-1, NVFP4_BLOCK)
    amax = np.max(np.abs(blocks), axis=1)  # exact
    s_code = e4m3_encode_sat((amax / np.float32(6.0)).astype(np.float32))
    s_val = e4m3_decode(s_code).astype(np.float32)  # exact in fp32; >= 0
    codes = np.zeros(blocks.shape, dtype=np.uint8)
    for b in range(blocks.shape[0]):
        if s_val[b] > 0:
            codes[b] = e2m1_encode((blocks[b] / s_val[b]).astype(np.float32))
    return pack_4bit(codes.reshape(-1)), s_code


def encode_row(x_bf16_as_f32: np.ndarray, divisor: np.ndarray, kv_format: str):
    """One (token, head) row of 128 values -> its cache bytes (nvfp4: the
    pair (code bytes, scale bytes))."""
    q = (np.asarray(x_bf16_as_f32, dtype=np.float32) / divisor).astype(np.float32)
    if kv_format == "nvfp4":
        return nvfp4_encode_row(q)
    if kv_format == "e4m3":
        return e4m3_encode_sat(q)
    if kv_format == "e2m3":
        return pack_6bit(e2m3_encode(q))
    if kv_format == "e3m2":
        return pack_6bit(e3m2_encode(q))
    if kv_format == "e2m1":
        return pack_4bit(e2m1_encode(q))
    raise ValueError(kv_format)


def write_kv(pools, strides, page_size: int, kv_format: str, key, value, slot_mapping, k_scale, v_scale,
             scale_kind: str, bs_pools=None, bs_strides=None, num_pages=None):
    """Apply the write to copies of the two byte pools and return them.

    pools: (k_pool, v_pool) flat uint8 arrays; strides: ((page, slot, head)
    byte strides of K), (same for V)); key/value: float32 arrays
    (num_tokens, h_k, 128) holding the bf16 inputs exactly.  nvfp4 also takes
    the two block-scale pools and their strides, and returns four pools
    (k, v, k block scales, v block scales).  ``num_pages``: pages in each
    pool (None: every page the strides reach).
    """
    k_pool, v_pool = (np.array(p, dtype=np.uint8, copy=True).reshape(-1) for p in pools)
    nv = kv_format == "nvfp4"
    if nv:
        kb_pool, vb_pool = (np.array(p, dtype=np.uint8, copy=True).reshape(-1) for p in bs_pools)
    row = ROW_BYTES[kv_format]
    srow = SCALE_ROW_BYTES.get(kv_format, 0)
    n, h_k, d = key.shape
    for t in range(n):
        s = int(slot_mapping[t])
        if s < 0:
            continue
        page, off = divmod(s, page_size)
        if num_pages is not None and page >= num_pages:
            continue
        for g in range(h_k):
            for side in range(2):
                pool, st, x, sc = ((k_pool, strides[0], key, k_scale), (v_pool, strides[1], value, v_scale))[side]
                base = page * st[0] + off * st[1] + g * st[2]
                enc = encode_row(x[t, g], scale_of(sc, scale_kind, g, d), kv_format)
                if nv:
                    bpool, bst = (kb_pool, vb_pool)[side], bs_strides[side]
                    bbase = page * bst[0] + off * bst[1] + g * bst[2]
                    pool[base:base + row] = enc[0]
                    bpool[bbase:bbase + srow] = enc[1]
                else:
                    pool[base:base + row] = enc
    if nv:
        return k_pool, v_pool, kb_pool, vb_pool
    return k_pool, v_pool
