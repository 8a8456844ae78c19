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


# ---- e3m2 / e2m1 (the harness's other formats; OCP MX FP6 E3M2 and FP4 E2M1)

def test_e3m2_landmarks():
    T = F.E3M2_TABLE
    assert T[0x1F] == 28.0                   # largest magnitude
    assert T[0x04] == 0.25                   # smallest normal 2^-2
    assert T[0x01] == 0.0625                 # smallest subnormal 2^-4
    assert T[0x0C] == 1.0 and T[0x2C] == -1.0
    assert T[0x20] == 0.0 and np.signbit(T[0x20])
    assert np.all(np.diff(T[:0x20]) > 0)     # codes 0x00..0x1f increase
    assert np.array_equal(T[0x20:], -T[:0x20])


def test_e2m1_landmarks():
    assert F.E2M1_TABLE[:8].tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.array_equal(F.E2M1_TABLE[8:], -F.E2M1_TABLE[:8])
    assert np.signbit(F.E2M1_TABLE[8])


def test_small_formats_nest_inside_e4m3_per_torch():
    """e2m1 c e3m2 c e4m3 and e2m1 c e2m3 c e4m3 as value sets, e4m3 taken
    from torch's own decode of all 256 codes (independent of the tables)."""
    e4 = set(torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().tolist())
    assert set(F.E3M2_TABLE.tolist()) <= e4
    assert set(F.E2M3_TABLE.tolist()) <= e4
    assert set(F.E2M1_TABLE.tolist()) <= set(F.E3M2_TABLE.tolist())
    assert set(F.E2M1_TABLE.tolist()) <= set(F.E2M3_TABLE.tolist())


@pytest.mark.parametrize("enc,table,n,vmax", [(F.e3m2_encode, F.E3M2_TABLE, 32, 28.0),
                                              (F.e2m1_encode, F.E2M1_TABLE, 8, 6.0)])
def test_small_encoders_nearest_even_and_saturating(enc, table, n, vmax):
    codes = np.arange(2 * n, dtype=np.uint8)
    assert np.array_equal(enc(table.astype(np.float32)), codes)   # every code maps to itself
    pos = table[:n]
    for k in range(n - 1):
        mid = np.float32((pos[k] + pos[k + 1]) / 2)                  # exact: few mantissa bits
        want = k if k % 2 == 0 else k + 1
        assert enc(mid) == want and enc(-mid) == want | n
        assert enc(np.nextafter(mid, np.float32(0))) == k
        assert enc(np.nextafter(mid, np.float32(100))) == k + 1
    big = np.array([vmax, vmax * 1.01, 1e30, -vmax * 3], dtype=np.float32)
    assert enc(big).tolist() == [n - 1, n - 1, n - 1, 2 * n - 1]


def _golden_fp4():
    rows = []
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "fp4_pack_example.txt")):
        if line.startswith("#") or "->" not in line:
            continue
        a, b = line.split("->")
        rows.append(([int(x) for x in a.split()], [int(x, 16) for x in b.split()]))
    return rows


@pytest.mark.parametrize("codes,packed", _golden_fp4())
def test_pack_4bit_worked_examples(codes, packed):
    assert F.pack_4bit(np.array(codes, dtype=np.uint8)).tolist() == packed
    assert F.unpack_4bit(np.array(packed, dtype=np.uint8), len(codes)).tolist() == codes


def test_decode_row_codes_dispatch():
    rng = np.random.default_rng(5)
    c6 = rng.integers(0, 64, (3, 128), dtype=np.uint8)
    c4 = rng.integers(0, 16, (3, 128), dtype=np.uint8)
    assert np.array_equal(F.decode_row_codes(F.pack_6bit(c6), "e3m2"), F.E3M2_TABLE[c6])
    assert np.array_equal(F.decode_row_codes(F.pack_6bit(c6), "e2m3"), F.E2M3_TABLE[c6])
    assert np.array_equal(F.decode_row_codes(F.pack_4bit(c4), "e2m1"), F.E2M1_TABLE[c4])


def test_generator_small_encoders_agree_with_the_oracle():
    """The generator's table encoders (torch, used to fill the caches) give
    the oracle encoders' codes on grid points, midpoints and random values."""
    from synth.workloads import e2m1_encode_table, e3m2_encode_table
    rng = np.random.default_rng(9)
    for enc_t, enc_o, table, n in ((e3m2_encode_table, F.e3m2_encode, F.E3M2_TABLE, 32),
                                   (e2m1_encode_table, F.e2m1_encode, F.E2M1_TABLE, 8)):
        pos = table[:n]
        mids = (pos[1:] + pos[:-1]) / 2
        x = np.concatenate([pos, -pos, mids, -mids, rng.normal(0, pos[-1] / 3, 5000), [1e4, -1e4]])
        x = x.astype(np.float32)
        assert np.array_equal(enc_t(torch.from_numpy(x)).numpy(), enc_o(x))


def test_generator_nvfp4_encoder_agrees_with_the_oracle_write():
    """The generator's nvfp4 block encoder (torch's e4m3 cast, table e2m1
    codes) gives the oracle write's codes and scales, incl. zero blocks,
    saturating blocks and tiny blocks whose scale rounds to zero."""
    from oracle.kvwrite import nvfp4_encode_row
    from synth.workloads import nvfp4_encode_blocks
    rng = np.random.default_rng(29)
    rows = (rng.standard_normal((300, 128)) * 10.0 ** rng.uniform(-4, 3, (300, 1))).astype(np.float32)
    rows[0, :16] = 0.0
    rows[1, 16:32] = 1e-7
    rows[2, :16] *= 1e4
    codes_t, sc_t = nvfp4_encode_blocks(torch.from_numpy(rows))
    for r in range(rows.shape[0]):
        codes_o, sc_o = nvfp4_encode_row(rows[r])
        assert np.array_equal(sc_t[r].numpy(), sc_o), r
        assert np.array_equal(codes_t[r].numpy(), codes_o), r
