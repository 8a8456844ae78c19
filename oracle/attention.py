"""Exact paged decode attention over the dequantized KV cache, in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The method computes exact attention; splitting the KV range and merging the
partials by log-sum-exp only reorders the sums.  So this oracle is the plain
definition (PyPI project page, "What it does", steps 2-4; wheel listing
mjolnir/runner.py, ``T5DecodeRunner.run`` and ``split_kv_cache``):

1. gather each sequence's K/V codes through its block-table row and the
   pool's byte strides (logical view ``(num_pages, page_size, h_k, row)``;
   head-major or token-major pages differ only in the strides);
2. dequantize: ``K = k_descale * dec(k_code)``, ``V = v_descale * dec(v_code)``
   with the descale per tensor, per KV head or per (sequence, KV head)
   (``run``'s ``k_scale`` / ``v_scale`` shapes); for nvfp4, ``dec`` includes
   the row's e4m3 block scale (``formats.nvfp4_decode``);
3. quantize Q exactly as ``qquant.quantize_q`` and dequantize it,
   ``Q = q_descale * dec(q_code)`` (or skip this and use fp32 Q times q_mul);
4. ``S = softmax_scale * Q K^T``; mask; ``P = softmax(S)``; ``O = P V``;
   ``O *= o_mul`` (per query head and channel) when given;
   ``LSE = logsumexp(S)`` in natural log over the keys a row may see.

Masking (readings, stated where the pages leave it open): ``seq_lens``
counts every token including the q_len new ones; query token t of a causal
block sees keys ``0 .. L - q_len + t``; a non-causal ("parallel drafter")
block and every q_len == 1 step see keys ``0 .. L - 1`` (README "What it
does", the decode-only step list; ``plan``: "one query token: the same kernel
either way").  A row that sees no key (L == 0, a graph-padding request)
returns O = 0 and LSE = -inf.

The fp6 channel scales fold into the math around attention
(mjolnir/backend.py, ``_install_fp6_scales``): K's into Q through ``q_mul``
(applied before the Q amax), V's into the output through ``o_mul``, with K/V
descales of 1.  The oracle applies ``o_mul`` to the fp64 output.
"""

from __future__ import annotations

import numpy as np

from .formats import ROW_BYTES, SCALE_ROW_BYTES, decode_row_codes, e4m3_decode, nvfp4_decode
from .qquant import quantize_q


def gather_codes(pool: np.ndarray, strides, page_size: int, bt_row: np.ndarray, L: int, head: int,
                 row_bytes: int) -> np.ndarray:
    """(L, row_bytes) codes of tokens 0..L-1 of one sequence and KV head.

    Token j lives in physical page ``bt_row[j // page_size]`` at slot
    ``j % page_size``; its row starts at byte
    ``page * page_stride + slot * slot_stride + head * head_stride``.
    """
    sp, ss, sh = (int(x) for x in strides)
    j = np.arange(L, dtype=np.int64)
    page = np.asarray(bt_row, dtype=np.int64)[j // page_size]
    start = page * sp + (j % page_size) * ss + head * sh
    return pool[start[:, None] + np.arange(row_bytes, dtype=np.int64)[None, :]]


def dequant_rows(codes: np.ndarray, kv_format: str, d: int) -> np.ndarray:
    return decode_row_codes(codes, kv_format, d)


def descale(values: np.ndarray, kind: str, i: int, g: int) -> float:
    v = np.asarray(values, dtype=np.float64)
    if kind == "tensor":
        return float(v.reshape(-1)[0])
    if kind == "head":
        return float(v.reshape(-1)[g])
    if kind == "seq_head":
        return float(v[i, g])
    raise ValueError(kind)


def visible(L: int, q_len: int, h_r: int, causal: bool) -> np.ndarray:
    """(n_q, L) bool: may packed row ``t*h_r + r`` see key j."""
    n_q = q_len * h_r
    t = np.arange(n_q) // h_r
    j = np.arange(L)
    if causal and q_len > 1:
        return j[None, :] <= (L - q_len + t)[:, None]
    return np.ones((n_q, L), dtype=bool)


def partial(qrows: np.ndarray, K: np.ndarray, V: np.ndarray, allowed: np.ndarray, scale: float,
            lo: int = 0, hi: int | None = None):
    """Unnormalized attention over keys [lo, hi): (O, m, l) per row with
    ``O = sum_j e^{s_j - m} V_j``, ``l = sum_j e^{s_j - m}``, ``m = max_j s_j``
    (m = -inf, l = 0, O = 0 for a row that sees no key in the range)."""
    hi = K.shape[0] if hi is None else hi
    s = scale * (qrows @ K[lo:hi].T)
    ok = allowed[:, lo:hi]
    s = np.where(ok, s, -np.inf)
    m = s.max(axis=1, initial=-np.inf)
    safe = np.where(np.isfinite(m), m, 0.0)
    p = np.where(ok, np.exp(s - safe[:, None]), 0.0)
    return p @ V[lo:hi], m, p.sum(axis=1)


def merge(parts):
    """Log-sum-exp merge of partials: M = max m_s,
    O = sum_s e^{m_s - M} O_s / sum_s e^{m_s - M} l_s, LSE = M + ln sum_s e^{m_s - M} l_s."""
    M = np.max(np.stack([p[1] for p in parts]), axis=0)
    safe = np.where(np.isfinite(M), M, 0.0)
    num = sum(np.exp(np.where(np.isfinite(p[1]), p[1] - safe, -np.inf))[:, None] * p[0] for p in parts)
    den = sum(np.exp(np.where(np.isfinite(p[1]), p[1] - safe, -np.inf)) * p[2] for p in parts)
    empty = den == 0
    O = np.where(empty[:, None], 0.0, num / np.where(empty, 1.0, den)[:, None])
    lse = np.where(empty, -np.inf, safe + np.log(np.where(empty, 1.0, den)))
    return O, lse


def combine(parts):
    """Context-parallel combine of slices given as (O normalized over the
    slice, LSE): the log-sum-exp merge above with m = LSE and l = 1 (l = 0
    for a slice that saw no key of the row)."""
    return merge([(o, lse, np.where(np.isfinite(lse), 1.0, 0.0)) for o, lse in parts])


def attend(qrows, K, V, allowed, scale):
    """Textbook softmax attention for one (sequence, KV head): (O, LSE, P)."""
    s = scale * (qrows @ K.T)
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, initial=-np.inf)
    safe = np.where(np.isfinite(m), m, 0.0)
    e = np.where(allowed, np.exp(s - safe[:, None]), 0.0)
    l = e.sum(axis=1)
    empty = l == 0
    P = e / np.where(empty, 1.0, l)[:, None]
    O = P @ V
    lse = np.where(empty, -np.inf, safe + np.log(np.where(empty, 1.0, l)))
    return O, lse, P


def head_inputs(h: dict, i: int, g: int, *, q_len: int, h_q: int, h_k: int, d: int, page_size: int,
                kv_format: str, q_codes=None, q_descale=None, quantize=True):
    """Dequantized (Q rows, K, V) of sequence i, KV head g, in fp64."""
    h_r = h_q // h_k
    L = int(h["seq_lens"][i])
    row = ROW_BYTES[kv_format] * d // 128
    kc = gather_codes(h["k_pool"], h["k_strides"], page_size, h["block_table"][i], L, g, row)
    vc = gather_codes(h["v_pool"], h["v_strides"], page_size, h["block_table"][i], L, g, row)
    if kv_format == "nvfp4":
        # the block scales of each row, gathered through their own pool's strides
        srow = SCALE_ROW_BYTES[kv_format] * d // 128
        ks = gather_codes(h["k_bs_pool"], h["k_bs_strides"], page_size, h["block_table"][i], L, g, srow)
        vs = gather_codes(h["v_bs_pool"], h["v_bs_strides"], page_size, h["block_table"][i], L, g, srow)
        Kc, Vc = nvfp4_decode(kc, ks, d), nvfp4_decode(vc, vs, d)
    else:
        Kc, Vc = dequant_rows(kc, kv_format, d), dequant_rows(vc, kv_format, d)
    K = Kc * descale(h["k_descale"], h["descale_kind"], i, g)
    V = Vc * descale(h["v_descale"], h["descale_kind"], i, g)
    if quantize:
        qrows = np.float64(q_descale[i, g]) * e4m3_decode(q_codes[i, g])
    else:
        x = h["q"][i * q_len:(i + 1) * q_len, g * h_r:(g + 1) * h_r, :].astype(np.float64)
        if h.get("q_mul") is not None:
            x = x * h["q_mul"][g * h_r:(g + 1) * h_r, :].astype(np.float64)
        qrows = x.reshape(q_len * h_r, d)
    return qrows, K, V


def decode_step(h: dict, *, q_len: int, h_q: int, h_k: int, d: int, page_size: int, kv_format: str,
                causal: bool, quantize: bool = True, pairs=None):
    """The whole step on host inputs ``h`` (see ``synth.Workload.host``).

    Returns O (b*q_len, h_q, d) and LSE (b*q_len, h_q) in fp64 (NaN where a
    (sequence, KV head) pair was not requested in ``pairs``).
    """
    b = len(h["seq_lens"])
    h_r = h_q // h_k
    O = np.full((b * q_len, h_q, d), np.nan)
    LSE = np.full((b * q_len, h_q), np.nan)
    q_codes = q_desc = None
    if quantize:
        q_codes, q_desc = quantize_q(h["q"], b, q_len, h_k, h.get("q_mul"))
    pairs = [(i, g) for i in range(b) for g in range(h_k)] if pairs is None else pairs
    for i, g in pairs:
        qrows, K, V = head_inputs(h, i, g, q_len=q_len, h_q=h_q, h_k=h_k, d=d, page_size=page_size,
                                  kv_format=kv_format, q_codes=q_codes, q_descale=q_desc, quantize=quantize)
        allowed = visible(K.shape[0], q_len, h_r, causal)
        o, lse, _ = attend(qrows, K, V, allowed, h["softmax_scale"])
        o = o.reshape(q_len, h_r, d)
        lse = lse.reshape(q_len, h_r)
        if h.get("o_mul") is not None:
            o = o * h["o_mul"][g * h_r:(g + 1) * h_r, :].astype(np.float64)[None]
        O[i * q_len:(i + 1) * q_len, g * h_r:(g + 1) * h_r] = o
        LSE[i * q_len:(i + 1) * q_len, g * h_r:(g + 1) * h_r] = lse
    return O, LSE
