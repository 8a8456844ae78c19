"""Pins of the Q-quantization oracle.

* bit-exact against the same definition evaluated with torch's CPU ops (fp32
  amax, clamp, true division and torch's own float8_e4m3fn cast) — the
  library route of the definition on the mjolnir-kernel wheel page
  mjolnir/runner.py, ``T5DecodeRunner.run`` (fp8-Q branch);
* invariants: the amax element of every (sequence, KV head) maps to +-448,
  all-zero Q gives zero codes and descale fp32(1e-6)/448, the row packing
  order puts token t / head g*h_r+r at row t*h_r+r.
"""

import numpy as np
import pytest
import torch

from oracle.qquant import quantize_q
from oracle.formats import e4m3_decode


def torch_route(q: torch.Tensor, b, q_len, h_k, q_mul=None):
    tokens, h_q, d = q.shape
    h_r = h_q // h_k
    x = q.float()
    if q_mul is not None:
        x = x * q_mul
    x = x.view(b, q_len, h_k, h_r, d)
    scale = torch.clamp(torch.amax(torch.abs(x), dim=(1, 3, 4)), min=1e-6) / 448.0
    y = torch.div(x, scale.view(b, 1, h_k, 1, 1))
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    codes = codes.transpose(1, 2).reshape(b, h_k, q_len * h_r, d)
    return codes.numpy(), scale.numpy()


@pytest.mark.parametrize("b,q_len,h_q,h_k,with_mul", [(1, 1, 8, 2, False), (5, 1, 32, 8, False),
                                                      (3, 4, 64, 8, False), (2, 1, 32, 8, True),
                                                      (2, 3, 16, 2, True)])
def test_bit_exact_vs_torch_route(b, q_len, h_q, h_k, with_mul):
    g = torch.Generator().manual_seed(b * 100 + q_len)
    q = torch.randn(b * q_len, h_q, 128, generator=g).to(torch.bfloat16)
    q_mul = torch.rand(h_q, 128, generator=g) * 3.0 + 0.01 if with_mul else None
    ref_c, ref_s = torch_route(q, b, q_len, h_k, q_mul)
    got_c, got_s = quantize_q(q.float().numpy(), b, q_len, h_k, None if q_mul is None else q_mul.numpy())
    assert np.array_equal(got_s, ref_s)
    assert np.array_equal(got_c, ref_c)


def test_amax_maps_to_448_and_packing_order():
    b, q_len, h_q, h_k, d = 2, 3, 12, 3, 128
    h_r = h_q // h_k
    q = np.random.default_rng(1).standard_normal((b * q_len, h_q, d)).astype(np.float32)
    q = torch.from_numpy(q).to(torch.bfloat16).float().numpy()
    codes, qd = quantize_q(q, b, q_len, h_k)
    for i in range(b):
        for g in range(h_k):
            blk = q[i * q_len:(i + 1) * q_len, g * h_r:(g + 1) * h_r]
            t, r, c = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            code = codes[i, g, t * h_r + r, c]
            assert code & 0x7F == 0x7E
            assert (code >> 7) == (blk[t, r, c] < 0)
            # dequantized values track Q within e4m3's half-ulp (2^-4 relative)
            deq = e4m3_decode(codes[i, g]).reshape(q_len, h_r, d) * qd[i, g]
            assert np.all(np.abs(deq - blk) <= 2.0 ** -4 * np.abs(blk) + 2.0 ** -9 * qd[i, g])


def test_all_zero_q():
    q = np.zeros((4, 8, 128), dtype=np.float32)
    codes, qd = quantize_q(q, 4, 1, 2)
    assert np.all(codes == 0)
    assert np.all(qd == np.float32(np.float32(1e-6) / np.float32(448.0)))
