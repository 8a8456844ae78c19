"""Pins of the draft-step advance oracle (oracle/draft.py): a hand-worked
example, and the slots it gives composed with the oracle's cache write and
gather (an independent route from a slot to a token position)."""

import numpy as np

from oracle import draft as D
from oracle import kvwrite as W
from oracle.attention import gather_codes


def test_hand_worked_example():
    # page size 16; sequence 0 (length 16) appends positions 16, 17 -> page
    # bt[0][1] = 9, slots 144, 145; sequence 1 is padding (length 0): slots
    # -1, stays 0; sequence 2 (length 47) appends position 47 -> page bt[2][2]
    # = 8, row 15, slot 143, and position 48, past its 3 block-table columns:
    # slot -1, length capped at 48
    bt = np.array([[5, 9, 2], [7, 0, 0], [3, 4, 8]])
    slots, lens = D.draft_advance(bt, [16, 0, 47], q_len=2, page_size=16)
    assert slots.tolist() == [144, 145, -1, -1, 143, -1]
    assert lens.tolist() == [18, 0, 48]


def test_slots_land_at_the_positions_the_gather_reads():
    """Rows written through the advanced slots are the rows the attention
    oracle gathers at positions L .. L + q_len - 1 (HND and NHD strides)."""
    rng = np.random.default_rng(3)
    P, h_k, pages, b, q_len = 16, 2, 40, 5, 3
    perm = rng.permutation(pages)
    bt = perm[:b * 6].reshape(b, 6)
    lens = [0, 1, 15, 16, 70]
    slots, new = D.draft_advance(bt, lens, q_len, P)
    for layout in ("HND", "NHD"):
        row = 128
        st = (h_k * P * row, row, P * row) if layout == "HND" else (P * h_k * row, h_k * row, row)
        x = np.round(rng.standard_normal((b * q_len, h_k, 128)) * 50).astype(np.float32)  # exact in e4m3 range
        x = np.clip(x, -400, 400)
        k, _ = W.write_kv((np.zeros(pages * P * h_k * row, np.uint8),) * 2, (st, st), P, "e4m3", x, x, slots,
                          np.ones(1, np.float32), np.ones(1, np.float32), "tensor")
        for i, L in enumerate(lens):
            if L == 0:
                assert new[i] == 0 and np.all(slots[i * q_len:(i + 1) * q_len] == -1)
                continue
            assert new[i] == L + q_len
            for g in range(h_k):
                got = gather_codes(k, st, P, bt[i], int(new[i]), g, row)[L:]
                for t in range(q_len):
                    assert np.array_equal(got[t], W.encode_row(x[i * q_len + t, g], np.ones(128, np.float32), "e4m3"))
