"""The split-KV plan, written from its definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources (mjolnir-kernel 0.1.0 wheel, mjolnir/runner.py):

* ``tile_width`` / ``T5DecodeRunner.n_tiles``: the n_q = q_len * h_r query
  rows of one KV head are processed in row tiles; ``n_tiles`` tiles per head.
* ``T5DecodeRunner.slots``: the work items that fit one wave,
  ``max(1, floor(CUs * WGs_per_CU / (h_k * n_tiles)))``.
* ``T5DecodeRunner.__init__`` ("Capacity per q_len"): the grid size is
  ``cap = max(slots, max_num_seqs)`` whatever the lengths, so a captured
  graph replays any later plan.
* ``T5DecodeRunner.plan``: lengths are planned ``margin`` tokens long; the
  reduction (merge) launch is decided by batch size, ``max_splits > 1 and
  num_seqs < slots``; the README step 1 (PyPI page, "What it does") calls the
  plan occupancy-pinned and sized to one wave.

The pages give only the planner's signature and outputs.  The rule below is
this project's reading (the plainest one consistent with them):

* ``tiles_i = ceil((L_i + margin) / kv_tile)``; ``S`` = the slot override if
  given, else ``slots``.
* no split (``b >= S`` or ``max_splits == 1``): one item per sequence,
  ``(i, 0, tiles_i, 0)``.
* split: the chunk ``c`` (in KV tiles) is the smallest integer
  ``>= max(1, ceil(max_i tiles_i / max_splits))`` with
  ``sum_i max(1, ceil(tiles_i / c)) <= S``; sequence i gets
  ``n_i = max(1, ceil(tiles_i / c))`` items ``(i, s*c, min((s+1)*c, tiles_i), s)``.
* items are sequence-major, split-minor, padded to ``cap`` with
  ``(-1, 0, 0, 0)``; ``split_begin`` is the exclusive prefix sum of ``n``.

Two parameters of the rule are not on the pages, and the rule takes them as
given rather than choosing them: the chunk floor ``min_chunk_tiles`` (1 is
the rule above) and the workgroups per CU behind ``slots``.  A caller that
compares a library's plans with this rule passes the values that library
reports for the plan.

Block-table width (``max_len``, tokens; ``None`` = unbounded).  A sequence
never holds more tokens than its block-table row can address, and nothing
past that is read, so a plan made ``margin`` tokens long covers at most
``max_len``: ``tiles_i = ceil(min(L_i + margin, max_len) / kv_tile)``.  And
when even a sequence that fills the row is no longer than the chunk floor
(``ceil(max_len / kv_tile) <= min_chunk_tiles``) every sequence is one item
whatever the lengths, so the plan does not split and needs no merge: the
pages' "never split, no merge kernel" case of ``max_splits == 1``, reached
here from the table width instead.  Such a plan has only ``max_num_seqs``
possible items, and its grid (``num_work``) is that; the decision and the
grid depend on the configuration and the table width, never on the lengths.

Row tiles here hold up to 64 query rows (one GQA group of up to 64 rows reads
its KV once); the pages' Thor kernel used at most 32.
"""

from __future__ import annotations

import math

ROW_TILE = 64


def n_tiles(q_len: int, h_q: int, h_k: int, row_tile: int = ROW_TILE) -> int:
    return -(-(q_len * (h_q // h_k)) // row_tile)


def slots(q_len, h_q, h_k, num_cus, wgs_per_cu, row_tile=ROW_TILE) -> int:
    return max(1, (num_cus * wgs_per_cu) // (h_k * n_tiles(q_len, h_q, h_k, row_tile)))


def capacity(q_len, h_q, h_k, num_cus, wgs_per_cu, max_num_seqs, slots_override=0, row_tile=ROW_TILE) -> int:
    s = slots_override if slots_override > 0 else slots(q_len, h_q, h_k, num_cus, wgs_per_cu, row_tile)
    return max(s, max_num_seqs)


def plan_split_kv(
    lens,
    *,
    q_len: int,
    h_q: int,
    h_k: int,
    num_cus: int,
    wgs_per_cu: int,
    kv_tile: int,
    max_splits: int,
    max_num_seqs: int,
    slots_override: int = 0,
    margin: int = 0,
    row_tile: int = ROW_TILE,
    min_chunk_tiles: int = 1,
    max_len: int | None = None,
) -> dict:
    b = len(lens)
    assert 0 < b <= max_num_seqs
    S = slots_override if slots_override > 0 else slots(q_len, h_q, h_k, num_cus, wgs_per_cu, row_tile)
    if max_len is not None:
        assert all(0 <= int(L) <= max_len for L in lens)
    splittable = max_len is None or math.ceil(max_len / kv_tile) > min_chunk_tiles
    cap = max(S, max_num_seqs) if splittable else max_num_seqs
    reach = [int(L) + margin if max_len is None else min(int(L) + margin, max_len) for L in lens]
    tiles = [math.ceil(x / kv_tile) for x in reach]
    split = max_splits > 1 and b < S and splittable
    if split:
        c = max(1, math.ceil(max(tiles) / max_splits), min_chunk_tiles)
        while sum(max(1, math.ceil(t / c)) for t in tiles) > S:
            c += 1
        n = [max(1, math.ceil(t / c)) for t in tiles]
    else:
        c = max(1, max(tiles))
        n = [1] * b
    work = []
    for i in range(b):
        for s in range(n[i]):
            work.append((i, s * c, min((s + 1) * c, tiles[i]), s))
    assert len(work) <= cap
    num_chunks = sum(1 for w in work if w[2] > w[1])
    work += [(-1, 0, 0, 0)] * (cap - len(work))
    split_begin, acc = [], 0
    for x in n:
        split_begin.append(acc)
        acc += x
    return dict(
        work=work,
        n_splits=n,
        split_begin=split_begin,
        chunk_tiles=c,
        num_chunks=num_chunks,
        num_work=cap,
        slots=S,
        with_reduction=bool(split),
    )
