"""Pins of the KV-cache write oracle (oracle/kvwrite.py) and its encoders:
closed forms over every code, tie points and saturation, the hand-worked fp6
packing examples, torch's e4m3 cast, a hand-worked write, and round trips
through the decoders, and the nvfp4 block-scaled write (a hand-worked row,
exact round trips, torch's e4m3 decode of the scales, and brute-force
nearest-value checks)."""

import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import kvwrite as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m3_encode_every_code_maps_to_itself():
    codes = np.arange(64, dtype=np.uint8)
    vals = F.e2m3_decode(codes).astype(np.float32)
    got = F.e2m3_encode(vals)
    # +0 and -0 are distinct codes (0x00, 0x20) and both round-trip
    assert np.array_equal(got, codes)


def test_e2m3_encode_midpoints_tie_to_even_and_neighbours_round_to_nearest():
    pos = F.E2M3_TABLE[:32]
    for k in range(31):
        lo, hi = pos[k], pos[k + 1]
        mid = np.float32((lo + hi) / 2)  # exact in fp32: the grid has 3 mantissa bits
        assert float(mid) == (lo + hi) / 2
        want = k if k % 2 == 0 else k + 1
        assert F.e2m3_encode(mid) == want, (k, lo, hi)
        assert F.e2m3_encode(-mid) == want | 0x20
        assert F.e2m3_encode(np.nextafter(mid, np.float32(0))) == k
        assert F.e2m3_encode(np.nextafter(mid, np.float32(10))) == k + 1


def test_e2m3_encode_saturates():
    x = np.array([7.5, 7.74, 7.75, 8.0, 100.0, 3e38, -7.75, -1e9], dtype=np.float32)
    assert F.e2m3_encode(x).tolist() == [0x1F] * 6 + [0x3F] * 2
    with pytest.raises(ValueError):
        F.e2m3_encode(np.array([np.inf], dtype=np.float32))


def test_e4m3_encode_sat_matches_torch_cast_in_range_and_saturates_above():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-448, 448, 200_000), rng.standard_normal(100_000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode_sat(x), ref)
    big = np.array([449.0, 464.0, 465.0, 1e6, -500.0, -3e38], dtype=np.float32)
    assert F.e4m3_encode_sat(big).tolist() == [0x7E] * 4 + [0xFE] * 2


def _golden_fp6():
    rows = []
    for line in open(os.path.join(GOLDEN, "fp6_pack_example.txt")):
        if line.startswith("#") or "->" not in line:
            continue
        a, b = line.split("->")
        rows.append(([int(x) for x in a.split()], [int(x, 16) for x in b.split()]))
    return rows


@pytest.mark.parametrize("codes,packed", _golden_fp6())
def test_pack_6bit_worked_examples(codes, packed):
    assert F.pack_6bit(np.array(codes, dtype=np.uint8)).tolist() == packed


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 64, size=(33, 128), dtype=np.uint8)
    assert np.array_equal(F.unpack_6bit(F.pack_6bit(codes), 128), codes)


def _pools(kv_format, layout, pages, page_size, h_k):
    row = F.ROW_BYTES[kv_format]
    if layout == "HND":
        st = (h_k * page_size * row, row, page_size * row)
    else:
        st = (page_size * h_k * row, h_k * row, row)
    return pages * page_size * h_k * row, (st, st), row


def test_write_hand_worked_example():
    # one token, two KV heads, page size 16, per-head scales 2 and 0.5, slot
    # 17 = page 1, row 1, HND: head g of row 1 of page 1 starts at byte
    # 1*(2*16*128) + g*(16*128) + 1*128
    size, strides, row = _pools("e4m3", "HND", 2, 16, 2)
    x = np.zeros((1, 2, 128), dtype=np.float32)
    x[0, 0, :4] = [3.0, -1.0, 896.0, 0.0078125]  # / 2 -> 1.5, -0.5, 448, 2^-8
    x[0, 1, :3] = [0.75, 1000.0, -0.001953125]  # / 0.5 -> 1.5, 2000 (saturates), -2^-8
    scale = np.array([2.0, 0.5], dtype=np.float32)
    k, v = W.write_kv((np.full(size, 0xAA, np.uint8), np.zeros(size, np.uint8)), strides, 16, "e4m3",
                      x, x, np.array([17]), scale, scale, "head")
    b0 = 1 * 2 * 16 * 128 + 0 * 16 * 128 + 1 * 128
    b1 = 1 * 2 * 16 * 128 + 1 * 16 * 128 + 1 * 128
    # e4m3: 1.5 = 0x3C, -0.5 = 0xB0, 448 = 0x7E, 2^-8 = subnormal 2/8 * 2^-6 = 0x02
    assert k[b0:b0 + 4].tolist() == [0x3C, 0xB0, 0x7E, 0x02]
    assert k[b1:b1 + 3].tolist() == [0x3C, 0x7E, 0x82]
    assert np.all(k[b0 + 4:b0 + 128] == 0) and np.all(k[b1 + 3:b1 + 128] == 0)
    touched = np.zeros(size, bool)
    touched[b0:b0 + 128] = touched[b1:b1 + 128] = True
    assert np.all(k[~touched] == 0xAA)  # nothing else written
    assert np.array_equal(k, v | (~touched * 0xAA).astype(np.uint8))


def test_padding_slots_write_nothing():
    size, strides, _ = _pools("e2m3", "NHD", 4, 16, 2)
    x = np.ones((3, 2, 128), dtype=np.float32)
    pools = (np.full(size, 7, np.uint8), np.full(size, 9, np.uint8))
    k, v = W.write_kv(pools, strides, 16, "e2m3", x, x, np.array([-1, -1, -1]), np.ones((2, 128), np.float32),
                      np.ones((2, 128), np.float32), "channel")
    assert np.all(k == 7) and np.all(v == 9)


def test_slots_past_num_pages_write_nothing():
    """A 4-page pool of which the cache owns 3 pages: slot 50 (page 3, row 2)
    addresses no row of the cache and leaves every byte alone; slot 33 (page
    2, row 1) is written, by hand at byte 2*(2*16*128) + g*(16*128) + 128."""
    size, strides, _ = _pools("e4m3", "HND", 4, 16, 2)
    x = np.full((2, 2, 128), 1.5, dtype=np.float32)  # e4m3 1.5 = 0x3C at scale 1
    one = np.ones(1, np.float32)
    k, v = W.write_kv((np.zeros(size, np.uint8), np.zeros(size, np.uint8)), strides, 16, "e4m3", x, x,
                      np.array([50, 33]), one, one, "tensor", num_pages=3)
    written = np.zeros(size, bool)
    for g in range(2):
        b = 2 * 2 * 16 * 128 + g * 16 * 128 + 128
        written[b:b + 128] = True
    assert np.all(k[written] == 0x3C) and np.all(k[~written] == 0)
    assert np.array_equal(k, v)
    # without the pool size, page 3 exists and slot 50 is written too
    k2, _ = W.write_kv((np.zeros(size, np.uint8), np.zeros(size, np.uint8)), strides, 16, "e4m3", x, x,
                       np.array([50, 33]), one, one, "tensor")
    assert np.count_nonzero(k2) == 2 * np.count_nonzero(k)


@pytest.mark.parametrize("kv_format,kind", [("e4m3", "tensor"), ("e4m3", "head"), ("e2m3", "channel"),
                                            ("e3m2", "channel"), ("e2m1", "channel"), ("e2m1", "head")])
@pytest.mark.parametrize("layout", ["HND", "NHD"])
def test_write_round_trip_through_decoders(kv_format, kind, layout):
    rng = np.random.default_rng(11)
    h_k, P, pages, n = 2, 16, 8, 40
    size, strides, _ = _pools(kv_format, layout, pages, P, h_k)
    row = F.ROW_BYTES[kv_format]
    x = torch.from_numpy(rng.standard_normal((n, h_k, 128)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    amax = np.abs(x).max()
    if kind == "tensor":
        sc = np.array([amax / F.FMT_MAX[kv_format]], np.float32)
    elif kind == "head":
        sc = (np.abs(x).max(axis=(0, 2)) / F.FMT_MAX[kv_format]).astype(np.float32)
    else:
        sc = (np.abs(x).max(axis=0) / F.FMT_MAX[kv_format]).astype(np.float32)  # (h_k, 128)
    slots = rng.permutation(pages * P)[:n]
    slots[5] = -1
    k, _ = W.write_kv((np.zeros(size, np.uint8), np.zeros(size, np.uint8)), strides, P, kv_format, x, x, slots,
                      sc, sc, kind)
    for t in range(n):
        if slots[t] < 0:
            continue
        page, off = divmod(int(slots[t]), P)
        for g in range(h_k):
            b = page * strides[0][0] + off * strides[0][1] + g * strides[0][2]
            raw = k[b:b + row]
            dec = F.decode_row_codes(raw, kv_format)
            s = W.scale_of(sc, kind, g)
            y = x[t, g] / s
            got = dec
            # nearest-value rounding: the error is at most half the local grid
            # step (m mantissa bits: 2^-(m+1) relative in the normal range,
            # half the subnormal step below it)
            mbits, sub = {"e4m3": (3, 2.0 ** -9), "e2m3": (3, 1.0 / 8), "e3m2": (2, 2.0 ** -4),
                          "e2m1": (1, 0.5)}[kv_format]
            bound = np.maximum(np.abs(y) * 2.0 ** -(mbits + 1), sub / 2)
            assert np.all(np.abs(got - y) <= bound + 1e-12)


def test_write_hand_worked_e2m1_and_e3m2_rows():
    # one token, one KV head, page size 16, per-tensor scale 1, slot 0, HND
    x = np.zeros((1, 1, 128), dtype=np.float32)
    x[0, 0, :4] = [3.0, -1.0, 100.0, 0.25]
    # e2m1: 3 -> 0x5, -1 -> 0x8|0x2 = 0xA, 100 saturates to 6 -> 0x7, 0.25 is the
    # midpoint of 0 and 0.5 -> the even code 0; bytes 0x5|0xA<<4 = 0xA5, 0x7|0<<4 = 0x07
    size = 16 * 64
    k, _ = W.write_kv((np.full(size, 0xEE, np.uint8), np.zeros(size, np.uint8)), ((16 * 64, 64, 16 * 64),) * 2,
                      16, "e2m1", x, x, np.array([0]), np.ones(1, np.float32), np.ones(1, np.float32), "tensor")
    assert k[:2].tolist() == [0xA5, 0x07] and np.all(k[2:64] == 0) and np.all(k[64:] == 0xEE)
    # e3m2: 1 -> 0x0C, 30 saturates to 28 -> 0x1F, -0.0625 -> 0x21, 0.03125 (midpoint of
    # 0 and 2^-4) -> 0; w = 0x0C | 0x1F<<6 | 0x21<<12 = 0x217CC -> bytes CC 17 02
    x[0, 0, :4] = [1.0, 30.0, -0.0625, 0.03125]
    size = 16 * 96
    k, _ = W.write_kv((np.zeros(size, np.uint8), np.zeros(size, np.uint8)), ((16 * 96, 96, 16 * 96),) * 2,
                      16, "e3m2", x, x, np.array([0]), np.ones(1, np.float32), np.ones(1, np.float32), "tensor")
    assert k[:3].tolist() == [0xCC, 0x17, 0x02] and np.all(k[3:96] == 0)


def _nvfp4_golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_row_example.txt")
    x = np.zeros(128, np.float32)
    codes = np.zeros(128, np.uint8)
    dec = {}
    scales = None
    for line in open(path):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        if f[0] == "x":
            x[int(f[1])] = np.float32(float(f[2]))
        elif f[0] == "scales":
            scales = np.array([int(v, 16) for v in f[1:]], np.uint8)
        elif f[0] == "codes":
            c0 = int(f[1])
            codes[c0:c0 + 16] = [int(v, 16) for v in f[2:]]
        elif f[0] == "dec":
            dec[int(f[1])] = float(f[2])
    return x, scales, codes, dec


def test_nvfp4_hand_worked_row():
    x, scales, codes, dec = _nvfp4_golden()
    assert np.array_equal(torch.from_numpy(x).to(torch.bfloat16).float().numpy(), x)  # bf16-exact inputs
    got_codes, got_scales = W.nvfp4_encode_row(x)
    assert got_scales.tolist() == scales.tolist()
    assert np.array_equal(F.unpack_4bit(got_codes, 128), codes)
    vals = F.nvfp4_decode(got_codes, got_scales)
    for c, v in dec.items():
        assert vals[c] == v, c
    # through the slot-mapped write: codes to the e2m1 row, scales to the scale row of the same slot
    size, (st, _), _ = _pools("e2m1", "HND", 2, 16, 1)
    bst = (16 * 8, 8, 16 * 8)
    xx = x.reshape(1, 1, 128)
    k, v, kb, vb = W.write_kv((np.zeros(size, np.uint8), np.zeros(size, np.uint8)), (st, st), 16, "nvfp4", xx, xx,
                              np.array([19]), np.ones(1, np.float32), np.ones(1, np.float32), "tensor",
                              bs_pools=(np.full(2 * 16 * 8, 0xEE, np.uint8), np.zeros(2 * 16 * 8, np.uint8)),
                              bs_strides=(bst, bst))
    b = 1 * st[0] + 3 * st[1]
    assert np.array_equal(k[b:b + 64], got_codes) and np.array_equal(v, k)
    assert kb[8 * 19:8 * 20].tolist() == scales.tolist()
    assert np.all(np.delete(kb, np.arange(8 * 19, 8 * 20)) == 0xEE)


def test_nvfp4_decode_matches_torch_scales():
    """The block-scale half of the decode through torch's float8_e4m3fn."""
    rng = np.random.default_rng(5)
    rows = rng.integers(0, 256, (50, 64), dtype=np.uint8)
    sc = rng.integers(0, 0x7F, (50, 8), dtype=np.uint8)  # finite non-negative scales
    ts = torch.from_numpy(sc).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    lo, hi = rows & 0xF, rows >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(50, 128)
    ref = F.E2M1_TABLE[codes] * np.repeat(ts, 16, axis=1)
    assert np.array_equal(F.nvfp4_decode(rows, sc), ref)


def test_nvfp4_exact_inputs_round_trip():
    """Rows whose every block holds a +-6 code are written back to the same
    codes and scales: amax / 6 is then the block scale exactly."""
    rng = np.random.default_rng(17)
    for _ in range(200):
        codes = rng.integers(0, 16, 128).astype(np.uint8)
        for b in range(8):
            codes[16 * b + rng.integers(0, 16)] = rng.choice([0x7, 0xF])
        scales = rng.integers(0x01, 0x7F, 8).astype(np.uint8)  # positive, finite, incl. subnormals
        packed = F.pack_4bit(codes)
        y = F.nvfp4_decode(packed, scales).astype(np.float32)
        assert np.array_equal(y.astype(np.float64), F.nvfp4_decode(packed, scales))  # exact in fp32
        got_codes, got_scales = W.nvfp4_encode_row(y)
        assert got_scales.tolist() == scales.tolist()
        assert np.array_equal(got_codes, packed)


def test_nvfp4_scale_and_codes_are_nearest_by_brute_force():
    """Random rows: every block scale is the e4m3 value nearest amax / 6 and
    every code the e2m1 value nearest y / scale (saturating), checked by
    search over every value of the two formats."""
    rng = np.random.default_rng(23)
    e4 = F.E4M3_TABLE[:0x7F]  # non-negative finite, code order
    e2 = F.E2M1_TABLE[:8]
    for _ in range(100):
        y = (rng.standard_normal(128) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        packed, scales = W.nvfp4_encode_row(y)
        codes = F.unpack_4bit(packed, 128)
        for b in range(8):
            blk = y[16 * b:16 * b + 16].astype(np.float64)
            t = np.float64(np.float32(np.abs(blk).max() / 6.0))  # the one fp32 division
            best = np.min(np.abs(e4 - min(t, 448.0)))
            assert abs(F.E4M3_TABLE[scales[b]] - min(t, 448.0)) == best
            s = F.E4M3_TABLE[scales[b]]
            if s == 0:
                assert np.all(codes[16 * b:16 * b + 16] == 0)
                continue
            for c in range(16):
                r = np.float64(np.float32(blk[c] / s))
                a = min(abs(r), 6.0)
                val = F.E2M1_TABLE[codes[16 * b + c]]
                assert abs(abs(val) - a) == np.min(np.abs(e2 - a))
                assert (val < 0) == (r < 0) or val == 0
