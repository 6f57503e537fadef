"""The protocol simulator's operations and scheduler, each pinned by a small
hand-worked program whose outcome follows from the GIN page's definitions
(one-sided get, signal methods, counter methods, VA signals), not from the
simulator; and the bf16 AllReduce sum against hand-rounded values."""
import numpy as np
import pytest

from oracle import definitions as D, protocol as pr
from oracle.primitives import (WIN_STRICT_ORDERING, CounterInc, Deadlock, InvalidUsage, SignalAdd, SignalInc,
                               VASignalInc, World)


def _nothing():
    return
    yield


def test_get_copies_the_remote_range_and_counts_at_the_caller():
    # GIN page, one-sided transfers (get): bytes [4, 12) of rank 1's slice land
    # at offset 2 of rank 0's; the local action counts once, at rank 0 only
    w = World(2, counter_count=2)
    src = w.register([np.arange(16, dtype=np.uint8), np.arange(100, 116, dtype=np.uint8)])
    dst = w.register_zeros(16)
    reads = []

    def p0():
        yield pr.Get(peer=1, rwin=src, roff=4, lwin=dst, loff=2, nbytes=8, local=CounterInc(1))
        yield pr.WaitCounter(1, 1)
        reads.append((yield pr.ReadCounter(1)))

    pr.run(w, [p0(), _nothing()])
    want = np.zeros(16, np.uint8)
    want[2:10] = np.arange(104, 112)
    assert np.array_equal(w.buf(dst, 0), want)
    assert not w.buf(dst, 1).any()
    assert reads == [1]
    assert [w.cnt[0][1], w.cnt[1][1], w.cnt[0][0]] == [1, 0, 0]


def test_signal_wait_read_low_bits_and_reset():
    # GIN page, signal methods: a payload-free SignalAdd(5) raises rank 1's
    # signal to 5; reading 2 bits gives 5 mod 4 = 1; a reset reads 0 again
    w = World(2, signal_count=2)
    reads = []

    def p0():
        yield pr.Signal(peer=1, remote=SignalAdd(1, 5))

    def p1():
        yield pr.WaitSignal(1, 5)
        reads.append((yield pr.ReadSignal(1)))
        reads.append((yield pr.ReadSignal(1, bits=2)))
        yield pr.ResetSignal(1)
        reads.append((yield pr.ReadSignal(1)))

    pr.run(w, [p0(), p1()])
    assert reads == [5, 1, 0]
    assert w.sig[0] == [0, 0]


def test_signal_inc_and_add_may_not_mix_without_a_reset():
    # GIN page, signal methods: SignalInc is not mixed with other updates of
    # the same signal unless the signal is reset in between
    w = World(2, signal_count=1)

    def p0():
        yield pr.Signal(peer=1, remote=SignalInc(0))
        yield pr.Signal(peer=1, remote=SignalAdd(0, 2))

    with pytest.raises(InvalidUsage):
        pr.run(w, [p0(), _nothing()])


def test_va_signal_counts_its_increments_in_the_window_word():
    # GIN page, VA signals: the 64-bit word at (window, offset) is the signal;
    # three VASignalIncs make it 3, stored little-endian in rank 1's slice
    w = World(2)
    v = w.register([np.zeros(32, np.uint8) for _ in range(2)], flags=WIN_STRICT_ORDERING)
    reads = []

    def p0():
        for _ in range(3):
            yield pr.Signal(peer=1, remote=VASignalInc(win=v, offset=8))

    def p1():
        yield pr.WaitVASignal(v, 8, 3)
        reads.append((yield pr.ReadVASignal(v, 8)))

    pr.run(w, [p0(), p1()])
    assert reads == [3]
    want = np.zeros(32, np.uint8)
    want[8] = 3
    assert np.array_equal(w.buf(v, 1), want)
    assert not w.buf(v, 0).any()


def test_local_runs_on_the_calling_rank_only():
    w = World(3)
    h = w.register_zeros(4)

    def prog(r):
        def mark(world, rank):
            world.buf(h, rank)[0] = 7 + rank
        yield pr.Local(mark, "mark")

    pr.run(w, [prog(r) for r in range(3)])
    assert [int(w.buf(h, r)[0]) for r in range(3)] == [7, 8, 9]


def test_scheduler_blocks_a_wait_until_its_signal_and_reports_deadlock():
    w = World(2, signal_count=1)

    def sender():
        yield pr.Signal(peer=1, remote=SignalInc(0))

    def waiter():
        yield pr.WaitSignal(0, 1)

    sim = pr.Sim(w, [sender(), waiter()])
    assert sim.runnable() == [0]  # the wait is not ready before the signal
    sim.step(0)
    assert sim.runnable() == [1]
    sim.step(1)
    assert sim.done() and sim.done_ops == [1, 1]
    # a wait that no one will satisfy: every unfinished rank is blocked
    with pytest.raises(Deadlock):
        pr.run(World(2, signal_count=1), [waiter(), _nothing()])


def test_allreduce_sum_bf16_hand_rounded():
    # binary32 sums in rank order, then one round-to-nearest-even to bf16:
    #   1 + 2^-8 + 0: halfway between 1 (0x3F80) and 1 + 2^-7, ties to even -> 0x3F80
    #   (1 + 2^-7) + 2^-8 + 0: halfway, 0x3F81 is odd -> 0x3F82 (1 + 2^-6)
    #   2^8 + 1 - 2^8: exact in binary32 -> 1 (0x3F80); a bf16 running sum would lose the 1
    xs = [np.array([0x3F80, 0x3F81, 0x4380], np.uint16),
          np.array([0x3B80, 0x3B80, 0x3F80], np.uint16),
          np.array([0x0000, 0x0000, 0xC380], np.uint16)]
    assert D.allreduce_sum_bf16(xs).tolist() == [0x3F80, 0x3F82, 0x3F80]
