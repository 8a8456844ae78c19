"""The draft-step advance: cache slots of the tokens a draft step appends,
and the advanced lengths.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: the wheel listing mjolnir/runner.py (``T5DecodeRunner.plan``: a plan
made ``margin`` tokens long stays valid while the device ``seq_lens`` grow by
up to ``margin``, because the kernels mask with the live lengths) and
mjolnir/backend.py (the builder's note on fused multi-step draft decode: the
speculator runs every draft step on one metadata build and advances the
device ``seq_lens`` in place).  Neither prints the advance itself; the
reading taken, the plainest one:

* token position ``p`` of sequence ``i`` lives in slot
  ``block_table[i][p // page_size] * page_size + p % page_size`` (the slot
  mapping the cache write takes, ``kvwrite.write_kv``);
* a draft step appends ``q_len`` tokens at positions ``L .. L + q_len - 1``
  of a sequence of length ``L`` and its length becomes ``L + q_len``;
* a length-0 sequence (a graph-padding request) stays 0 and appends nothing;
  positions past the block table get slot -1 and are not counted.
"""

from __future__ import annotations

import numpy as np


def draft_advance(block_table, seq_lens, q_len: int, page_size: int):
    """Returns (slot_mapping (b * q_len,) int64, new lengths (b,) int64)."""
    bt = np.asarray(block_table, dtype=np.int64)
    lens = [int(x) for x in seq_lens]
    cap = bt.shape[1] * page_size
    slots = np.full((len(lens), q_len), -1, dtype=np.int64)
    new = np.array(lens, dtype=np.int64)
    for i, L in enumerate(lens):
        if L <= 0:
            continue
        for t in range(q_len):
            p = L + t
            if p < cap:
                slots[i, t] = bt[i, p // page_size] * page_size + p % page_size
        new[i] = min(L + q_len, cap)
    return slots.reshape(-1), new
