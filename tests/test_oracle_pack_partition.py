"""Pins of the pack and ownership oracles: hand-worked literals, the golden
Llama-3.1-8B share, round trips and the LPT makespan bound against a brute
force optimum."""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import pack, partition
from synth import LLAMA31_8B, model_shapes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_pack_literal():
    a = np.array([[1, 2], [3, 4]], dtype=np.uint16)
    b = np.array([[5, 6, 7]], dtype=np.uint16)
    offs, total = partition.pack_offsets([4, 3], 4)
    assert offs == [0, 4] and total == 8
    buf = pack.pack([a, b], offs, total, fill=9)
    assert buf.tolist() == [1, 2, 3, 4, 5, 6, 7, 9]
    offs, total = partition.pack_offsets([3, 4], 4)
    assert offs == [0, 4] and total == 8
    buf = pack.pack([b, a], offs, total, fill=0)
    assert buf.tolist() == [5, 6, 7, 0, 1, 2, 3, 4]


def test_pack_round_trip_and_padding():
    rng = np.random.default_rng(0)
    shapes = [(3, 5), (1, 1), (7, 2), (4, 9)]
    mats = [rng.integers(0, 2 ** 16, size=s, dtype=np.uint16) for s in shapes]
    offs, total = partition.pack_offsets([r * c for r, c in shapes], 8)
    buf = pack.pack(mats, offs, total, fill=0xABCD)
    back = pack.unpack(buf, shapes, offs)
    for m, b in zip(mats, back):
        assert np.array_equal(m, b)
    covered = np.zeros(total, bool)
    for (r, c), o in zip(shapes, offs):
        assert o % 8 == 0
        covered[o:o + r * c] = True
    assert np.all(buf[~covered] == 0xABCD)
    assert covered.sum() == sum(r * c for r, c in shapes)


def test_pack_offsets_literal():
    offs, total = partition.pack_offsets([5, 128, 1, 0, 3], 128)
    assert offs == [0, 128, 256, 384, 384] and total == 512


def test_partition_literal():
    owner, loads = partition.partition_lpt([5, 4, 3, 3, 2], 2)
    assert owner == [0, 1, 1, 0, 1] and loads == [8, 9]
    owner, loads = partition.partition_lpt([1, 1, 1], 4)
    assert owner == [0, 1, 2] and loads == [1, 1, 1, 0]
    assert partition.partition_lpt([], 3) == ([], [0, 0, 0])
    with pytest.raises(ValueError):
        partition.partition_lpt([1], 0)


def brute_force_makespan(numels, n_owners):
    best = None
    for assign in itertools.product(range(n_owners), repeat=len(numels)):
        loads = [0] * n_owners
        for x, r in zip(numels, assign):
            loads[r] += x
        best = max(loads) if best is None else min(best, max(loads))
    return best


@pytest.mark.parametrize("seed", range(12))
def test_partition_lpt_bound(seed):
    rng = np.random.default_rng(seed)
    n_owners = int(rng.integers(2, 4))
    numels = [int(v) for v in rng.integers(1, 50, size=int(rng.integers(3, 8)))]
    owner, loads = partition.partition_lpt(numels, n_owners)
    assert sorted(set(owner)) <= list(range(n_owners)) and len(owner) == len(numels)
    for r in range(n_owners):
        assert loads[r] == sum(x for x, o in zip(numels, owner) if o == r)
    opt = brute_force_makespan(numels, n_owners)
    # Graham's bound for longest-processing-time-first list scheduling
    assert max(loads) <= (4 / 3 - 1 / (3 * n_owners)) * opt + 1e-9


def test_llama31_8b_owner_share_golden():
    g = json.load(open(os.path.join(GOLDEN, "llama31_8b_owner_share.json")))
    shapes = model_shapes(**LLAMA31_8B)
    numels = [r * c for _, r, c in shapes]
    assert sum(numels) == g["total_elements"]
    owner, loads = partition.partition_lpt(numels, g["n_owners"])
    assert loads == [g["load_per_owner"]] * g["n_owners"]
    mine = [shapes[i][0] for i in range(len(shapes)) if owner[i] == 0]
    counts = {k: 0 for k in g["owner0_counts"]}
    layers = {k: [] for k in g["owner0_layers"]}
    for name in mine:
        layer = int(name.split(".")[1])
        kind = name.split(".")[2][:-len("_proj")]
        counts[kind] += 1
        layers.setdefault(kind, []).append(layer)
    assert counts == g["owner0_counts"]
    for k, v in g["owner0_layers"].items():
        assert sorted(layers[k]) == v
