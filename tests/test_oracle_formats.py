"""Pins of the oracle's codecs against torch's float8 type, the OCP format
tables and hand-worked packing examples (tests/golden/fp6_pack_example.txt)."""

import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from synth.workloads import pack_codes_6bit, e2m3_encode_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_decode_matches_torch_on_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_e4m3_landmarks():
    # OCP OFP8 E4M3: max normal 448 = 1.75 * 2^8, min normal 2^-6, min subnormal 2^-9
    assert F.e4m3_value(0x7E) == 448.0
    assert F.e4m3_value(0x08) == 2.0 ** -6
    assert F.e4m3_value(0x01) == 2.0 ** -9
    assert F.e4m3_value(0x38) == 1.0
    assert F.e4m3_value(0xB8) == -1.0
    assert np.isnan(F.e4m3_value(0x7F)) and np.isnan(F.e4m3_value(0xFF))
    finite = F.E4M3_TABLE[:0x7F]
    assert np.all(np.diff(finite) > 0)


def _torch_e4m3(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encoder_matches_torch_cast_random():
    rng = np.random.default_rng(7)
    parts = [
        rng.standard_normal(1_000_000) * 100.0,
        rng.standard_normal(500_000) * 1e-2,
        rng.uniform(-448.0, 448.0, 500_000),
        np.sign(rng.standard_normal(500_000)) * 2.0 ** rng.uniform(-12, 8.8, 500_000),
    ]
    x = np.clip(np.concatenate(parts), -460.0, 460.0).astype(np.float32)
    assert np.array_equal(F.e4m3_encode(x), _torch_e4m3(x))


def test_e4m3_encoder_matches_torch_cast_at_every_tie():
    v = F.E4M3_TABLE[:0x7F]
    mids = ((v[1:] + v[:-1]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (v[1:] + v[:-1]) / 2)  # exact in fp32
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000))])
    x = np.concatenate([near, -near, v.astype(np.float32), -v.astype(np.float32),
                        np.array([0.0, -0.0, 448.0, 464.0, -464.0, 2.0 ** -10, -(2.0 ** -10)], np.float32)])
    assert np.array_equal(F.e4m3_encode(x), _torch_e4m3(x))


def test_e2m3_table_landmarks_and_subset_of_e4m3():
    # OCP MX FP6 E2M3: max 7.5 = 1.875 * 2^2, min normal 1.0, min subnormal 0.125
    assert F.e2m3_value(0x1F) == 7.5
    assert F.e2m3_value(0x08) == 1.0
    assert F.e2m3_value(0x01) == 0.125
    assert F.e2m3_value(0x07) == 0.875
    assert F.e2m3_value(0x10) == 2.0
    assert F.e2m3_value(0x18) == 4.0
    assert F.e2m3_value(0x3F) == -7.5
    pos = F.E2M3_TABLE[:32]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(F.E2M3_TABLE[32:], -pos)
    # every e2m3 value is an e4m3 value (2 exponent bits fit in 4, 3 mantissa bits in 3)
    e4 = set(F.E4M3_TABLE[~np.isnan(F.E4M3_TABLE)].tolist())
    assert all(v in e4 for v in pos.tolist())
    # the value set the OCP MX table lists for E2M3 (non-negative half)
    listed = [0, .125, .25, .375, .5, .625, .75, .875, 1, 1.125, 1.25, 1.375, 1.5, 1.625, 1.75, 1.875,
              2, 2.25, 2.5, 2.75, 3, 3.25, 3.5, 3.75, 4, 4.5, 5, 5.5, 6, 6.5, 7, 7.5]
    assert pos.tolist() == listed


def _golden_pack():
    rows = []
    with open(os.path.join(GOLDEN, "fp6_pack_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split("->")
            rows.append(([int(x) for x in a.split()], [int(x, 16) for x in b.split()]))
    return rows


@pytest.mark.parametrize("codes,packed", _golden_pack())
def test_unpack_6bit_worked_examples(codes, packed):
    got = F.unpack_6bit(np.array([packed], dtype=np.uint8), 4)[0]
    assert got.tolist() == codes


def test_unpack_6bit_round_trip_random_rows():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 64, size=(257, 128), dtype=np.uint8)
    packed = pack_codes_6bit(torch.from_numpy(codes)).numpy()
    assert packed.shape == (257, 96)
    assert np.array_equal(F.unpack_6bit(packed, 128), codes)


def test_generator_e2m3_encoder_is_nearest_even():
    # the cache-write helper the generator uses: nearest value, ties to even code
    pos = F.E2M3_TABLE[:32]
    mids = (pos[1:] + pos[:-1]) / 2
    x = torch.tensor(np.concatenate([pos, -pos, mids, -mids, [9.0, -9.0]]), dtype=torch.float32)
    c = e2m3_encode_table(x).numpy()
    val = F.e2m3_decode(c)
    xs = np.clip(x.numpy().astype(np.float64), -7.5, 7.5)
    err = np.abs(val - xs)
    best = np.min(np.abs(F.E2M3_TABLE[None, :] - xs[:, None]), axis=1)
    assert np.array_equal(err, best)
    tie = np.isin(np.abs(xs), mids)
    assert np.all((c[tie] & 1) == 0)
