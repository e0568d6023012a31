"""CPU model of the split kernel's first-exchange record layout
(csrc/attnres.hip: split_chunk, fwd_split_long, clear_unread_records).

Per token slot the records are 32 chunk areas of 128 (values 0..63, then
their device-scope copies at 64..127).  A call with C chunks writes and reads:

* one-wave and multi-wave chunks (up to 31 snapshots): area c < C, values
  0 .. NV - 1 (NV = 2(N + 1), or N + 1 + (N + 1)(N + 2) / 2 in the Gram form);
* the two-wave form (32..63 snapshots, C <= 16): wave 0 area c, values
  0..63; wave 1 area c + 16, values 0 .. 2N - 63 (its snapshots, then the
  folded prefix's two values);
* the four-wave form (the same values, four writers per chunk): wave w
  values 32w .. 32w + 31, the prefix's wave also 2N and 2N + 1, so the same
  records as the two-wave form.

Checked for every chunk count and source count each form takes: every
record a reader polls is written by exactly one chunk of the call (its own
chunk index), every index stays inside the slot, and the set the epoch-wrap
clears (everything outside RecordUse{C, nv0, nv1}) is disjoint from what the
call reads and, with it, covers the whole slot: after a wrap no record the
call did not read survives.
"""
import pytest

MAX_CHUNKS = 32
REC_STRIDE = 64
PAGE = MAX_CHUNKS // 2


def one_wave_form(n, C, gram):
    S = n + 1
    nv = S + S * (S + 1) // 2 if gram else 2 * S
    writes = {(c, v): c for c in range(C) for v in range(nv)}
    reads = set(writes)
    return writes, reads, (C, nv, 0)


def two_wave_form(n, C):
    nv = 2 * (n + 1)
    writes = {}
    for c in range(C):
        for wave in (0, 1):
            area = c + PAGE * wave
            # snapshots of the wave: lane l publishes value 64 wave + l if below 2N
            for lane in range(64):
                if 64 * wave + lane < 2 * n:
                    assert (area, lane) not in writes
                    writes[(area, lane)] = c
            if wave == 1:  # the folded prefix: values 2N, 2N + 1
                for wv in (0, 1):
                    assert (area, 2 * n - 64 + wv) not in writes
                    writes[(area, 2 * n - 64 + wv)] = c
    reads = set()
    for wave in (0, 1):
        for lane in range(64):
            if 64 * wave + lane < nv:
                for c in range(C):
                    reads.add((c + PAGE * wave, lane))
    return writes, reads, (C, 64, nv - 64)


def four_wave_form(n, C):
    """Wave w of chunk c publishes value 32w + l of its snapshots (lane l's
    butterfly total) when below 2N, the prefix's wave (N // 16) values 2N and
    2N + 1; value g sits in area c + 16 (g // 64), slot g % 64; wave w gathers
    values 32w .. 32w + 31 below 2(N + 1)."""
    nv = 2 * (n + 1)
    writes = {}
    for c in range(C):
        for wave in range(4):
            vals = [32 * wave + l for l in range(32) if 32 * wave + l < 2 * n]
            if wave == n // 16:
                vals += [2 * n, 2 * n + 1]
            for g in vals:
                key = (c + PAGE * (g // 64), g % 64)
                assert key not in writes
                writes[key] = c
    reads = {(c + PAGE * (g // 64), g % 64) for wave in range(4) for g in range(32 * wave, 32 * wave + 32)
             if g < nv for c in range(C)}
    return writes, reads, (C, 64, nv - 64)


def cleared(use):
    C, nv0, nv1 = use
    out = set()
    for c in range(MAX_CHUNKS):
        page1 = c - PAGE
        used = nv0 if c < C else nv1 if 0 <= page1 < C else 0
        out |= {(c, v) for v in range(used, REC_STRIDE)}
    return out


def check(writes, reads, use):
    slot = {(c, v) for c in range(MAX_CHUNKS) for v in range(REC_STRIDE)}
    assert set(writes) <= slot and reads <= slot
    assert reads <= set(writes), "a reader polls a record no chunk writes"
    clr = cleared(use)
    assert not (clr & reads), "the wrap would clear a record the call still reads"
    assert clr | reads == slot, "a record the call did not read would survive the wrap"


@pytest.mark.parametrize("C", [1, 2, 7, 14, 16, 24, 32])
@pytest.mark.parametrize("n", range(0, 32))
def test_one_wave_forms(n, C):
    S = n + 1
    gram = S <= 6
    nv = S + S * (S + 1) // 2 if gram else 2 * S
    assert nv <= REC_STRIDE
    check(*one_wave_form(n, C, gram))


@pytest.mark.parametrize("C", [1, 2, 7, 14, 16])
@pytest.mark.parametrize("n", range(32, 64))
def test_two_wave_form(n, C):
    check(*two_wave_form(n, C))


@pytest.mark.parametrize("C", [1, 2, 7, 8, 12, 16])
@pytest.mark.parametrize("n", range(32, 64))
def test_four_wave_form(n, C):
    w2, r2, u2 = two_wave_form(n, C)
    w4, r4, u4 = four_wave_form(n, C)
    assert set(w4) == set(w2) and r4 == r2 and u4 == u2, "the two forms share one record layout"
    check(w4, r4, u4)


def test_two_wave_form_stops_at_63():
    # 64 snapshots: 130 values, more than the two pages hold
    with pytest.raises(AssertionError):
        writes, reads, use = two_wave_form(64, 14)
        assert max(v for (_, v) in writes) < REC_STRIDE
