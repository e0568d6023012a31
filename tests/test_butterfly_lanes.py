"""CPU model of the split kernel's wave totals (wave_totals / bfly_index in
csrc/attnres_device.hpp): 64 lanes, each with V per-lane values, halve their
lists at six steps across lane bits 5, 4, ..., 0, whose partners come from
v_permlane32_swap / v_permlane16_swap (lanes l and l ^ 32, l and l ^ 16, each
keeping the two terms of its own half) and DPP row permutations (row_mirror,
row_half_mirror, two quad_perms).

Checked for every value count 1..64 the kernel can use: at each halving step a
lane's partner has the other value of the split bit (so one keeps the lower
half and the other the upper half) and the same bits at every earlier step
(so both hold the same list); every lane ends with the exact total of the value
bfly_index names; and bfly_index names each value 0..NV-1 in exactly one lane
(the lane that publishes it).  Sums are of small integers, so exact.
"""
import random

import pytest


def step_bit(s):
    return 5 - s


def partner(step, lane):
    if step == 0:  # v_permlane32_swap: lanes 0-31 with lanes 32-63
        return lane ^ 32
    if step == 1:  # v_permlane16_swap: even rows with odd rows
        return lane ^ 16
    if step == 2:  # row_mirror: lane i <-> 15 - i within a 16-lane row
        return (lane & ~15) | (15 - (lane & 15))
    if step == 3:  # row_half_mirror: i <-> 7 - i within 8 lanes
        return (lane & ~7) | (7 - (lane & 7))
    if step == 4:  # quad_perm [2,3,0,1]
        return lane ^ 2
    return lane ^ 1  # quad_perm [1,0,3,2]


def pow2_at_least(n):
    return 1 if n <= 1 else 2 * pow2_at_least((n + 1) // 2)


def bfly_index(V, lane):
    return lane // (64 // V) if lane % (64 // V) == 0 else -1


def wave_totals(part):
    nv = len(part[0])
    V = pow2_at_least(nv)
    w = [[row[i] if i < nv else 0 for i in range(V)] for row in part]
    L = V
    for step in range(6):
        b = step_bit(step)
        if L > 1:
            new = []
            for lane in range(64):
                p = partner(step, lane)
                upper = (lane >> b) & 1
                assert (p >> b) & 1 != upper, "partner on the same side of the split bit"
                for s in range(step):
                    assert (p >> step_bit(s)) & 1 == (lane >> step_bit(s)) & 1, "partner holds another list"
                pupper = (p >> b) & 1
                send_of_partner = [w[p][i] if pupper else w[p][i + L // 2] for i in range(L // 2)]
                keep = [w[lane][i + L // 2] if upper else w[lane][i] for i in range(L // 2)]
                new.append([k + r for k, r in zip(keep, send_of_partner)])
            w = new
            L //= 2
        else:
            w = [[w[lane][0] + w[partner(step, lane)][0]] for lane in range(64)]
    return [w[lane][0] for lane in range(64)]


@pytest.mark.parametrize("nv", range(1, 65))
def test_butterfly_totals_and_publishing_lanes(nv):
    rng = random.Random(nv)
    part = [[rng.randrange(-1000, 1000) for _ in range(nv)] for _ in range(64)]
    tot = wave_totals(part)
    V = pow2_at_least(nv)
    publishers = {}
    for lane in range(64):
        # the lane's total is that of the value its bits at the halving steps name
        full = 0
        s = 0
        while (V >> (s + 1)) >= 1:
            full += ((lane >> step_bit(s)) & 1) * (V >> (s + 1))
            s += 1
        exact = sum(part[x][full] for x in range(64)) if full < nv else 0
        assert tot[lane] == exact, (nv, lane, full)
        v = bfly_index(V, lane)
        if 0 <= v < nv:
            assert v == full
            assert v not in publishers, (nv, v)
            publishers[v] = lane
    assert sorted(publishers) == list(range(nv))
