"""Pins of the split-plan oracle: exact cover, split bound, balance, and a
brute-force walk over an explicitly materialised cost line."""

import numpy as np
import pytest

from oracle.plan import plan_pieces_ref, plan_ref, plan_slot_ref


def brute_parts(seqlens, tile, plan):
    """Materialise every cost-line position and read the parts off it."""
    line = []
    for b, L in enumerate(seqlens):
        n = -(-L // tile)
        if plan["mode"] == "whole":
            seg = [None] * plan["c0"] + [(b, k) for k in range(n)]
            seg += [None] * (plan["t"] - len(seg))
        else:
            seg = ([None] * plan["c0"] + [(b, k) for k in range(n)]) if n else []
        line += seg
    t = plan["t"]
    parts = []
    for p in range(plan["parts"]):
        cells = [c for c in line[p * t:(p + 1) * t] if c is not None]
        pieces = []
        for b, k in cells:
            if pieces and pieces[-1][0] == b:
                pieces[-1][2] = k + 1
            else:
                pieces.append([b, k, k + 1])
        parts.append([tuple(x) for x in pieces])
    return parts, len(line)


CASES = [
    ([4096] * 16, 64, 256, 32, 2, 4),
    ([4096] * 16, 64, 256, 2, 2, 4),
    ([300, 0, 5, 1024, 64, 65], 64, 8, 32, 2, 1),
    ([1, 1, 1, 1], 64, 256, 32, 2, 4),
    ([0, 0, 0], 64, 16, 4, 2, 1),
    ([8192, 256, 4000, 777, 0, 2], 64, 5, 3, 1, 1),
    ([100, 200, 300], 16, 4, 1, 2, 1),
    ([0, 70, 0], 64, 4, 1, 2, 1),
]


@pytest.mark.parametrize("seqlens,tile,parts,ns,c0,tmin", CASES)
def test_plan_matches_brute_force_line(seqlens, tile, parts, ns, c0, tmin):
    plan = plan_ref(seqlens, tile, parts, ns, c0, tmin)
    bparts, C = brute_parts(seqlens, tile, plan)
    assert plan["C"] == C
    for p in range(plan["parts"]):
        assert plan_pieces_ref(plan, p) == bparts[p]


def _random_case(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    seqlens = rng.integers(0, 3000, size=B)
    seqlens[rng.random(B) < 0.15] = 0
    return (seqlens.tolist(), int(rng.choice([16, 32, 64])), int(rng.integers(1, 300)),
            int(rng.integers(1, 33)), int(rng.integers(0, 4)), int(rng.integers(1, 6)))


@pytest.mark.parametrize("seed", range(40))
def test_first_piece_slot_from_line_position(seed):
    # The combine finds the slot of a sequence's first piece without reading
    # part_first_seq: sequence b is the first sequence of part first_b exactly
    # when its range on the cost line (c0 positions, then its tiles) begins
    # at or before that part.
    seqlens, tile, parts, ns, c0, tmin = _random_case(seed)
    plan = plan_ref(seqlens, tile, parts, ns, c0, tmin)
    if plan["mode"] != "line":
        return
    for b in range(len(seqlens)):
        if plan["n"][b] == 0:
            continue
        f = plan["first"][b]
        assert (plan["part_first_seq"][f] == b) == (plan["start"][b] - plan["c0"] <= f * plan["t"]), b


@pytest.mark.parametrize("seed", range(40))
def test_plan_invariants_random(seed):
    seqlens, tile, parts, ns, c0, tmin = _random_case(seed)
    plan = plan_ref(seqlens, tile, parts, ns, c0, tmin)
    B = len(seqlens)
    covered = {}
    slots = set()
    for p in range(plan["parts"]):
        pieces = plan_pieces_ref(plan, p)
        load = sum(hi - lo for _, lo, hi in pieces)
        assert load <= plan["t"]                                   # balance bound
        for b, lo, hi in pieces:
            assert 0 <= lo < hi <= plan["n"][b]
            for k in range(lo, hi):
                assert (b, k) not in covered                       # no tile twice
                covered[(b, k)] = p
            if plan["nsplit"][b] > 1:
                assert (b == pieces[0][0]) or (b == pieces[-1][0])  # split => first or last
                s = plan_slot_ref(plan, p, b)
                assert s not in slots and 0 <= s < 2 * plan["parts"]
                slots.add(s)
    for b in range(B):
        n = plan["n"][b]
        assert all((b, k) in covered for k in range(n))          # every tile once
        owners = sorted({covered[(b, k)] for k in range(n)})
        assert len(owners) == plan["nsplit"][b] <= ns              # split bound
        if n:
            assert owners == list(range(plan["first"][b], plan["first"][b] + plan["nsplit"][b]))
    if plan["mode"] == "line":
        assert plan["parts_used"] <= parts
        assert all(p < plan["parts_used"] for p in covered.values())


def test_whole_mode_one_part_per_sequence():
    plan = plan_ref([5, 0, 130, 64], 64, 999, 1, 2, 4)
    assert plan["mode"] == "whole" and plan["parts"] == 4
    assert [plan_pieces_ref(plan, p) for p in range(4)] == [[(0, 0, 1)], [], [(2, 0, 3)], [(3, 0, 1)]]
    assert plan["nsplit"] == [1, 0, 1, 1]


def test_fixed_length_balance_example():
    # 16 sequences x 4096 tokens on 256 parts: 64 tiles + c0 each, 1056 total.
    plan = plan_ref([4096] * 16, 64, 256, 32, 2, 4)
    assert plan["C"] == 16 * 66 and plan["t"] == 5 and plan["parts_used"] == 212
    assert max(plan["nsplit"]) <= 14
