"""Pins of the split-KV plan oracle: hand-worked examples
(tests/golden/plan_examples.txt), brute force on tiny inputs, invariants."""

import itertools
import math
import os

import numpy as np
import pytest

from oracle import plan as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(kind):
    out = []
    with open(os.path.join(GOLDEN, "plan_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if line.startswith(kind + " "):
                a, b = line.split("->")
                out.append((a.split()[1:], [int(x) for x in b.split()]))
    return out


@pytest.mark.parametrize("args,expect", _golden("thor"))
def test_thor_closed_forms(args, expect):
    h_q, h_k, q_len, row_tile, cus, wgs, mns = (int(x) for x in args)
    assert P.n_tiles(q_len, h_q, h_k, row_tile) == expect[0]
    assert P.slots(q_len, h_q, h_k, cus, wgs, row_tile) == expect[1]
    assert P.capacity(q_len, h_q, h_k, cus, wgs, mns, row_tile=row_tile) == expect[2]


@pytest.mark.parametrize("args,expect", _golden("mi355"))
def test_mi355_workload_plans(args, expect):
    name = args[0]
    b, h_q, h_k, q_len, L, ovr = (int(x) for x in args[1:])
    p = P.plan_split_kv([L] * b, q_len=q_len, h_q=h_q, h_k=h_k, num_cus=256, wgs_per_cu=2, kv_tile=128,
                        max_splits=16, max_num_seqs=b, slots_override=ovr)
    assert p["slots"] == expect[0], name
    assert p["chunk_tiles"] == expect[1], name
    assert p["n_splits"] == [expect[2]] * b, name
    assert sum(1 for w in p["work"] if w[0] >= 0) == expect[3], name
    assert int(p["with_reduction"]) == expect[4], name


def _golden_table():
    out = []
    with open(os.path.join(GOLDEN, "plan_examples.txt")) as f:
        for line in f:
            if line.startswith("table "):
                a, b = line.split("->")
                tiles, rest = b.split("|")
                out.append(([int(x) for x in a.split()[2:]], [int(x) for x in tiles.split()],
                            [int(x) for x in rest.split()]))
    return out


@pytest.mark.parametrize("args,tiles,expect", _golden_table())
def test_block_table_width_examples(args, tiles, expect):
    P_, mb, mct, S, mns, margin, *lens = args
    p = P.plan_split_kv(lens, q_len=1, h_q=8, h_k=1, num_cus=1, wgs_per_cu=1, kv_tile=128, max_splits=16,
                        max_num_seqs=mns, slots_override=S, margin=margin, min_chunk_tiles=mct,
                        max_len=mb * P_)
    real = [w for w in p["work"] if w[0] >= 0]
    assert [max(w[2] for w in real if w[0] == i) for i in range(len(lens))] == tiles
    assert [len(real), int(p["with_reduction"]), p["num_work"]] == expect


def test_table_width_clamps_and_unsplittable_loses_nothing():
    """Brute force: with a table width, the plan covers exactly the clamped
    tiles; where the rule declines to split (rows too short for the floor),
    the split rule would have given every sequence one item anyway."""
    rng = np.random.default_rng(17)
    for _ in range(500):
        b = int(rng.integers(1, 6))
        P_ = int(rng.choice([16, 64]))
        mb = int(rng.integers(1, 40))
        T = mb * P_
        lens = [int(x) for x in rng.integers(0, T + 1, size=b)]
        margin = int(rng.integers(0, 300))
        kv = int(rng.choice([16, 64, 128]))
        mct = int(rng.integers(1, 12))
        S = int(rng.integers(b + 1, 30))
        p = P.plan_split_kv(lens, q_len=1, h_q=8, h_k=1, num_cus=1, wgs_per_cu=1, kv_tile=kv, max_splits=8,
                            max_num_seqs=b, slots_override=S, margin=margin, min_chunk_tiles=mct, max_len=T)
        tiles = [math.ceil(min(L + margin, T) / kv) for L in lens]
        real = [w for w in p["work"] if w[0] >= 0]
        for i in range(b):
            assert sorted(t for w in real if w[0] == i for t in range(w[1], w[2])) == list(range(tiles[i]))
        splittable = math.ceil(T / kv) > mct
        assert p["with_reduction"] == splittable
        assert p["num_work"] == (max(S, b) if splittable else b)
        if not splittable:
            # the smallest feasible chunk at or above the floor covers every sequence whole
            c = min(c for c in range(mct, mct + max(tiles) + 2)
                    if sum(max(1, math.ceil(t / c)) for t in tiles) <= S and
                    max(math.ceil(t / c) for t in tiles) <= 8)
            assert all(math.ceil(t / c) <= 1 for t in tiles)
            assert p["n_splits"] == [1] * b


def _check_invariants(p, lens, kv_tile, max_splits, S, cap, margin=0):
    tiles = [math.ceil((L + margin) / kv_tile) for L in lens]
    assert p["num_work"] == cap == len(p["work"])
    real = [w for w in p["work"] if w[0] >= 0]
    pad = p["work"][len(real):]
    assert all(w == (-1, 0, 0, 0) for w in pad)
    # sequence-major, split-minor; chunks tile [0, tiles_i) exactly once
    k = 0
    for i, n in enumerate(p["n_splits"]):
        assert p["split_begin"][i] == k
        items = real[k:k + n]
        assert [w[0] for w in items] == [i] * n
        assert [w[3] for w in items] == list(range(n))
        cover = [t for w in items for t in range(w[1], w[2])]
        assert cover == list(range(tiles[i]))
        assert all(w[2] - w[1] <= p["chunk_tiles"] for w in items)
        k += n
    assert k == len(real)
    if p["with_reduction"]:
        assert len(real) <= S
        assert max(p["n_splits"]) <= max_splits
    else:
        assert p["n_splits"] == [1] * len(lens)


def test_brute_force_minimal_chunk():
    rng = np.random.default_rng(5)
    for _ in range(400):
        b = int(rng.integers(1, 7))
        lens = [int(x) for x in rng.integers(0, 3000, size=b)]
        S = int(rng.integers(b + 1, 40))
        ms = int(rng.integers(2, 9))
        kv = int(rng.choice([16, 64, 128]))
        p = P.plan_split_kv(lens, q_len=1, h_q=8, h_k=1, num_cus=1, wgs_per_cu=1, kv_tile=kv, max_splits=ms,
                            max_num_seqs=b, slots_override=S)
        tiles = [math.ceil(L / kv) for L in lens]
        # enumerate every chunk size: the smallest one that respects both
        # the split cap and the slot budget
        feas = [c for c in range(1, max(1, max(tiles)) + 1)
                if sum(max(1, math.ceil(t / c)) for t in tiles) <= S and max(math.ceil(t / c) for t in tiles) <= ms]
        assert p["chunk_tiles"] == min(feas)
        _check_invariants(p, lens, kv, ms, S, max(S, b))
        # with a floor on the chunk: the smallest feasible chunk at or above it
        floor = int(rng.integers(1, 40))
        q = P.plan_split_kv(lens, q_len=1, h_q=8, h_k=1, num_cus=1, wgs_per_cu=1, kv_tile=kv, max_splits=ms,
                            max_num_seqs=b, slots_override=S, min_chunk_tiles=floor)
        top = max(floor, max(1, max(tiles)))
        feas = [c for c in range(floor, top + 1)
                if sum(max(1, math.ceil(t / c)) for t in tiles) <= S and max(math.ceil(t / c) for t in tiles) <= ms]
        assert q["chunk_tiles"] == min(feas)
        _check_invariants(q, lens, kv, ms, S, max(S, b))


def test_invariants_and_fixed_grid():
    rng = np.random.default_rng(9)
    for q_len, h_q, h_k in itertools.product([1, 2, 4], [8, 32, 64], [1, 2, 8]):
        if h_q % h_k:
            continue
        cap = None
        for trial in range(6):
            b = int(rng.integers(1, 48))
            lens = [int(x) for x in rng.integers(0, 70000, size=b)]
            if trial == 5:
                lens = [0] * b
            margin = int(rng.integers(0, 5))
            p = P.plan_split_kv(lens, q_len=q_len, h_q=h_q, h_k=h_k, num_cus=256, wgs_per_cu=2, kv_tile=128,
                                max_splits=16, max_num_seqs=48, margin=margin)
            S = P.slots(q_len, h_q, h_k, 256, 2)
            _check_invariants(p, lens, 128, 16, S, max(S, 48), margin)
            # the grid size depends on (config, q_len) only, never on the lengths
            cap = p["num_work"] if cap is None else cap
            assert p["num_work"] == cap
            assert p["with_reduction"] == (b < S)


def test_max_splits_one_never_splits():
    p = P.plan_split_kv([100000, 5], q_len=1, h_q=32, h_k=8, num_cus=256, wgs_per_cu=2, kv_tile=128,
                        max_splits=1, max_num_seqs=2)
    assert not p["with_reduction"] and p["n_splits"] == [1, 1]
