"""Pins of the oracle swizzle (invariants) and ring schedule (brute force
plus the page's stage formulas and hand-derived wait counts)."""
import pytest

from oracle import ring as R
from oracle.swizzle import span_bytes, swizzle, swizzle128


def test_swizzle_involution_and_bijection():
    for base in range(0, 8192, 1024):
        block = [swizzle128(base + o) for o in range(1024)]
        assert sorted(block) == list(range(base, base + 1024))      # bijective on each 1-KiB atom
        for o in range(1024):
            assert swizzle128(swizzle128(base + o)) == base + o      # its own inverse


def test_swizzle_stays_in_row_and_keeps_chunks():
    for o in range(0, 4096, 16):
        p = swizzle128(o)
        assert p // 128 == o // 128                                  # same 128-byte row
        for k in range(16):
            assert swizzle128(o + k) == p + k                        # whole 16-byte chunks move


def test_swizzle_is_latin_square_over_8_rows():
    # each logical chunk column lands in 8 different physical chunk columns
    # over the 8 rows of an atom (column access is bank-conflict free), and
    # row 0 is the identity.
    for c in range(8):
        cols = {(swizzle128(r * 128 + c * 16) % 128) // 16 for r in range(8)}
        assert cols == set(range(8))
    assert [swizzle128(c * 16) for c in range(8)] == [c * 16 for c in range(8)]


def test_swizzle_hand_values():
    # logical chunk 0 of row 1 sits in physical chunk 1; chunk 5 of row 3 in chunk 6;
    # chunk 7 of row 7 in chunk 0 (worked by hand from "chunk XOR row mod 8").
    assert swizzle128(1 * 128 + 0 * 16) == 1 * 128 + 1 * 16
    assert swizzle128(3 * 128 + 5 * 16) == 3 * 128 + 6 * 16
    assert swizzle128(7 * 128 + 7 * 16) == 7 * 128 + 0 * 16
    assert swizzle128(9 * 128 + 2 * 16 + 3) == 9 * 128 + 3 * 16 + 3


@pytest.mark.parametrize("mode", [1, 2, 3])
def test_swizzle_modes_invariants(mode):
    span = span_bytes(mode)
    assert span == {1: 32, 2: 64, 3: 128}[mode]
    block = 128 * (span // 16)                      # one full period of the pattern
    for base in range(0, 4 * block, block):
        img = [swizzle(base + o, mode) for o in range(block)]
        assert sorted(img) == list(range(base, base + block))          # bijective per period
    for o in range(0, 4096):
        p = swizzle(o, mode)
        assert swizzle(p, mode) == o                                   # involution
        assert p // span == o // span                                  # stays in its span
        assert p % 16 == o % 16                                        # whole 16-byte chunks
    # over 2**m consecutive 128-byte rows, each logical chunk of a span takes
    # every physical chunk position of that span once (Latin square)
    n = span // 16
    for c in range(n):
        assert {(swizzle(r * 128 + c * 16, mode) % span) // 16 for r in range(n)} == set(range(n))


def test_swizzle_modes_hand_values():
    # mode 1 (32 B): bit 7 flips bit 4 -- row 1 swaps the two chunks of each span
    assert swizzle(128 + 0, 1) == 128 + 16
    assert swizzle(128 + 48 + 5, 1) == 128 + 32 + 5
    assert swizzle(256 + 16, 1) == 256 + 16            # row 2: bit 7 is 0
    # mode 2 (64 B): bits 7..8 flip bits 4..5 -- row 3, chunk 1 of a span -> chunk 2
    assert swizzle(3 * 128 + 16, 2) == 3 * 128 + 32
    assert swizzle(3 * 128 + 64 + 48, 2) == 3 * 128 + 64 + 0
    assert swizzle(5 * 128 + 16, 2) == 5 * 128 + 0     # row 5 mod 4 = 1
    # mode 0 is the identity; mode 3 is the 128-byte pattern
    assert all(swizzle(o, 0) == o for o in range(2048))
    assert all(swizzle(o, 3) == swizzle128(o) for o in range(4096))


@pytest.mark.parametrize("stages", [2, 3, 4])
def test_ring_bruteforce(stages):
    for n in range(0, 17):
        ev = R.schedule(n, stages, loads=3, stores=2)
        loads = [e for e in ev if e.kind == R.LOAD]
        cons = [e for e in ev if e.kind == R.CONSUME]
        # every iteration loaded exactly once, into stage j % S
        assert [e.iteration for e in loads] == list(range(n))
        assert all(e.stage == e.iteration % stages for e in loads)
        # consumed in order, from the stage it was loaded into
        assert [e.iteration for e in cons] == list(range(n))
        assert all(e.stage == e.iteration % stages for e in cons)
        pos = {(e.kind, e.iteration): k for k, e in enumerate(ev)}
        for i in range(n):
            assert pos[(R.LOAD, i)] < pos[(R.WAIT, i)] < pos[(R.CONSUME, i)]
            # no stage reloaded before its previous occupant is consumed
            if i >= stages:
                assert pos[(R.CONSUME, i - stages)] < pos[(R.LOAD, i)]
        # loads run at most S-1 iterations ahead of consumption
        consumed = 0
        for e in ev:
            if e.kind == R.CONSUME:
                consumed += 1
            if e.kind == R.LOAD:
                assert e.iteration - consumed <= stages - 1


def test_ring_main_loop_slot_order():
    # "Detailed Pseudo-Code" of the circular-buffering page: in the main loop
    # the stage being consumed advances one slot per iteration starting from
    # slot 0, and the stage being loaded runs S - 1 slots ahead of it (mod S).
    # Checked on the schedule's events: the k-th main-loop load goes to the
    # slot that is S - 1 past the slot of the k-th consume.
    for stages in (2, 3, 4):
        for n in range(stages, 20):
            ev = R.schedule(n, stages)
            main_loads = [e for e in ev if e.kind == R.LOAD][stages - 1:]
            cons = [e for e in ev if e.kind == R.CONSUME]
            for k, ld in enumerate(main_loads):
                assert cons[k].stage == k % stages
                assert ld.stage == (cons[k].stage + stages - 1) % stages
                assert ld.iteration == cons[k].iteration + stages - 1


def test_ring_wait_counts_hand_derived():
    # S = 4, 5 load ops and 4 store ops per iteration, N = 10.
    ev = R.schedule(10, 4, loads=5, stores=4)
    waits = {e.iteration: e.count for e in ev if e.kind == R.WAIT}
    # i = 0: loads of iterations 1, 2, 3 were issued after iteration 0's: 15
    assert waits[0] == 15
    # i = 1: loads of 2, 3, 4 and the stores of iteration 0: 15 + 4
    assert waits[1] == 19
    # steady state: loads of i+1..i+3 and stores of i-3..i-1: 15 + 12
    assert waits[5] == 27
    # epilogue: i = 8 has only iteration 9's loads after it, plus 3 stores
    assert waits[8] == 5 + 12
    assert waits[9] == 12
    # tiny trip count below S - 1: N = 2, S = 4
    ev = R.schedule(2, 4, loads=5, stores=4)
    waits = {e.iteration: e.count for e in ev if e.kind == R.WAIT}
    assert waits == {0: 5, 1: 4}


def test_ring_zero_trips():
    assert R.schedule(0, 3) == []
