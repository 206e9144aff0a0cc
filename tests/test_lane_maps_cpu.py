"""Lane bookkeeping of the decode kernel's head-distributing row reduction, replayed on the CPU.

Each lane of a 16-lane row holds its slice of the dot products of all G query heads of a group, in
a lane-dependent slot order.  Four DPP exchange steps (row_mirror, row_half_mirror, quad_perm x2;
each lane reads the lane its index pairs with) both finish the sums and leave head h's score on
lanes h*16/G .. h*16/G + 16/G - 1.  The test replays the slot order and the four steps
symbolically -- every slot holds the set of (head, lane) partials it has summed -- and checks that
every lane ends with all 16 partials of its own head, each exactly once.
"""
from collections import Counter

import pytest


def pair_lane(bit, x):
    """Source lane of lane x in the exchange that flips index bit `bit` (row_mirror,
    row_half_mirror, quad_perm [2,3,0,1], quad_perm [1,0,3,2])."""
    return 15 - x if bit == 3 else ((x & 8) | (7 - (x & 7))) if bit == 2 else (x ^ 2) if bit == 1 else (x ^ 1)


def head_of_slot(G, col, k):
    S = G.bit_length() - 1
    y = col
    for s in range(S):
        if k & (G >> (s + 1)):
            y = pair_lane(3 - s, y)
    return 0 if S == 0 else y >> (4 - S)


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_row_reduction_leaves_each_head_whole_on_its_lanes(G):
    S = G.bit_length() - 1
    r = [[Counter({(head_of_slot(G, c, k), c): 1}) for k in range(G)] for c in range(16)]
    n = G
    for bit in (3, 2, 1, 0):
        new = [[slot.copy() for slot in lane] for lane in r]
        if n > 1:
            half = n // 2
            for c in range(16):
                for k in range(half):
                    new[c][k] = r[c][k] + r[pair_lane(bit, c)][half + k]
            n = half
        else:
            for c in range(16):
                new[c][0] = r[c][0] + r[pair_lane(bit, c)][0]
        r = new
    for c in range(16):
        h = c >> (4 - S) if S else 0
        assert r[c][0] == Counter({(h, src): 1 for src in range(16)}), (G, c)
        assert c // (16 // G) == h  # head h sits on lanes h*16/G .. h*16/G + 16/G - 1


def test_every_slot_of_a_lane_holds_a_different_head():
    for G in (2, 4, 8, 16):
        for c in range(16):
            assert sorted(head_of_slot(G, c, k) for k in range(G)) == list(range(G))
