"""Dynamic e4m3 quantization of Q per (sequence, KV head).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: the mjolnir-kernel 0.1.0 PyPI project page, section "What it does",
step 2 (Q is quantized to e4m3 dynamically, one scale for each sequence and
KV head), and the wheel listing mjolnir/runner.py, the fp8-Q branch of
``T5DecodeRunner.run`` with its ``FP8_MAX`` constant of 448.  For sequence i
and KV head g, over the q_len tokens and the h_r query heads that share g:

    x     = fp32(q)                      (times the fp32 q_mul, if given:
                                          one fp32 multiply, before the amax)
    amax  = max(max |x|, fp32(1e-6))
    scale = amax / 448                   (fp32, IEEE round-to-nearest)
    code  = e4m3(x / scale)              (fp32 IEEE division, then RNE)
    q_descale[i, g] = scale

The codes of one pair form n_q = q_len * h_r rows, token-major: row
t * h_r + r holds token t of query head g * h_r + r (the runner groups the
query heads by KV head and puts the tokens of each group in front of its
heads).  Every step is fp32 as on the pages; the division is a true
division, not a multiply by a reciprocal.
"""

from __future__ import annotations

import numpy as np

from .formats import e4m3_encode

FP8_MAX = np.float32(448.0)
AMAX_FLOOR = np.float32(1e-6)


def quantize_q(q: np.ndarray, b: int, q_len: int, h_k: int, q_mul: np.ndarray | None = None):
    """q: (b*q_len, h_q, d) float32 holding the bf16 values.

    Returns codes (b, h_k, q_len*h_r, d) uint8 and q_descale (b, h_k) float32.
    """
    q = np.asarray(q, dtype=np.float32)
    tokens, h_q, d = q.shape
    assert tokens == b * q_len and h_q % h_k == 0
    h_r = h_q // h_k
    n_q = q_len * h_r
    codes = np.zeros((b, h_k, n_q, d), dtype=np.uint8)
    qd = np.zeros((b, h_k), dtype=np.float32)
    for i in range(b):
        for g in range(h_k):
            x = q[i * q_len:(i + 1) * q_len, g * h_r:(g + 1) * h_r, :]  # (q_len, h_r, d)
            if q_mul is not None:
                x = x * np.asarray(q_mul, dtype=np.float32)[g * h_r:(g + 1) * h_r, :]
            x = x.astype(np.float32)
            amax = np.float32(max(np.float32(np.abs(x).max()), AMAX_FLOOR))
            scale = np.float32(amax / FP8_MAX)
            y = (x / scale).astype(np.float32)
            codes[i, g] = e4m3_encode(y).reshape(n_q, d)  # row = t * h_r + r
            qd[i, g] = scale
    return codes, qd
