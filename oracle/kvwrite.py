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
  a negative slot (a padding token) writes nothing;
* code = the format's round-to-nearest-even of ``x / scale`` in fp32 (one
  IEEE division, x = fp32 of the bf16 input), saturated at the format's
  largest magnitude (448 for e4m3, 7.5 for e2m3, 28 for e3m2, 6 for e2m1);
* 6-bit rows (e2m3, e3m2) are packed 4 codes per 3 bytes and e2m1 rows 2
  codes per byte, as the decode reads them (the little-endian bitstreams of
  ``formats.pack_6bit`` / ``pack_4bit``).
"""

from __future__ import annotations

import numpy as np

from .formats import ROW_BYTES, e2m1_encode, e2m3_encode, e3m2_encode, e4m3_encode_sat, pack_4bit, pack_6bit


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


def encode_row(x_bf16_as_f32: np.ndarray, divisor: np.ndarray, kv_format: str) -> np.ndarray:
    """One (token, head) row of 128 values -> its cache bytes."""
    q = (np.asarray(x_bf16_as_f32, dtype=np.float32) / divisor).astype(np.float32)
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
             scale_kind: str):
    """Apply the write to copies of the two byte pools and return them.

    pools: (k_pool, v_pool) flat uint8 arrays; strides: ((page, slot, head)
    byte strides of K), (same for V)); key/value: float32 arrays
    (num_tokens, h_k, 128) holding the bf16 inputs exactly.
    """
    k_pool, v_pool = (np.array(p, dtype=np.uint8, copy=True).reshape(-1) for p in pools)
    row = ROW_BYTES[kv_format]
    n, h_k, d = key.shape
    for t in range(n):
        s = int(slot_mapping[t])
        if s < 0:
            continue
        page, off = divmod(s, page_size)
        for g in range(h_k):
            for pool, st, x, sc in ((k_pool, strides[0], key, k_scale), (v_pool, strides[1], value, v_scale)):
                base = page * st[0] + off * st[1] + g * st[2]
                pool[base:base + row] = encode_row(x[t, g], scale_of(sc, scale_kind, g, d), kv_format)
    return k_pool, v_pool
