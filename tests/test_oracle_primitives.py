"""Pins for the oracle's primitives: brute force, wrap-around, usage rules."""
import numpy as np
import pytest

from oracle.primitives import (COUNTER_BITS, CounterInc, InvalidArgument, InvalidUsage,
                               SignalAdd, SignalInc, World, rolling_le)


def test_rolling_le_small_width_brute_force():
    # Against a plain reading on 4-bit integers: b is "at or after" a when
    # stepping forward from a by fewer than 8 increments reaches b.
    bits = 4
    for a in range(16):
        reach = {(a + k) % 16 for k in range(8)}
        for b in range(16):
            assert rolling_le(a, b, bits) == (b in reach), (a, b)


def test_rolling_le_keeps_successor_order_across_wrap():
    for bits in (8, 32, 56, 64):
        top = (1 << bits) - 1
        assert rolling_le(top, 0, bits)          # x <= x + 1 even when x + 1 wraps
        assert not rolling_le(0, top, bits)
        assert rolling_le(5, 5, bits)


def test_put_get_brute_force_tiny_windows():
    # Every (offset, size) pair on an 8-byte window across 2 ranks.
    size = 8
    for soff in range(0, 9):
        for doff in range(0, 9):
            for n in range(0, 9):
                w = World(2)
                src = [np.arange(size, dtype=np.uint8) + 10 * r for r in range(2)]
                s = w.register([x.copy() for x in src])
                d = w.register_zeros(size)
                ok = soff + n <= size and doff + n <= size
                if not ok:
                    with pytest.raises(InvalidArgument):
                        w.put(0, 1, d, doff, s, soff, n)
                    with pytest.raises(InvalidArgument):
                        w.get(1, 0, s, soff, d, doff, n)
                    continue
                w.put(0, 1, d, doff, s, soff, n)
                ref = [0] * size
                ref[doff:doff + n] = list(src[0])[soff:soff + n]
                assert list(w.buf(d, 1)) == ref
                assert list(w.buf(d, 0)) == [0] * size
                w2 = World(2)
                s2 = w2.register([x.copy() for x in src])
                d2 = w2.register_zeros(size)
                w2.get(1, 0, s2, soff, d2, doff, n)
                assert list(w2.buf(d2, 1)) == ref


def test_overlapping_loopback_put_is_memmove():
    w = World(1)
    b = np.arange(16, dtype=np.uint8)
    win = w.register([b.copy()])
    w.put(0, 0, win, 2, win, 0, 10)
    ref = list(range(16))
    ref[2:12] = list(range(10))
    assert list(w.buf(win, 0)) == ref


def test_signal_inc_equals_add_one_and_final_value_counts_puts():
    w1, w2 = World(3), World(3)
    for w, act in ((w1, SignalInc(2)), (w2, SignalAdd(2, 1))):
        s = w.register_zeros(4)
        d = w.register_zeros(12)
        for src in range(3):
            for _ in range(src + 1):
                w.put(src, 1, d, 4 * src, s, 0, 4, remote=act)
    assert w1.sig == w2.sig
    assert w1.read_signal(1, 2) == 6  # 1 + 2 + 3 puts aimed at rank 1
    assert w1.read_signal(0, 2) == 0


def test_signal_wraps_at_64_bits_and_wait_uses_rolling_compare():
    w = World(2, signal_count=1)
    base = (1 << 64) - 3
    w.signal(0, 1, SignalAdd(0, base))
    for _ in range(5):
        w.signal(0, 1, SignalAdd(0, 1))
    assert w.read_signal(1, 0) == 2  # wrapped
    assert w.signal_reached(1, 0, (base + 5) % (1 << 64))
    assert w.signal_reached(1, 0, base)
    assert not w.signal_reached(1, 0, (base + 6) % (1 << 64))


def test_read_signal_low_bits():
    w = World(1, signal_count=1)
    w.signal(0, 0, SignalAdd(0, 0x1_2345_6789))
    assert w.read_signal(0, 0, 16) == 0x6789
    assert w.read_signal(0, 0, 64) == 0x1_2345_6789


def test_counter_is_56_bits():
    w = World(1, counter_count=1)
    w.cnt[0][0] = (1 << COUNTER_BITS) - 2
    s = w.register_zeros(1)
    for _ in range(3):
        w.put(0, 0, s, 0, s, 0, 1, local=CounterInc(0))
    assert w.read_counter(0, 0) == 1
    assert w.counter_reached(0, 0, (1 << COUNTER_BITS) - 1)
    with pytest.raises(InvalidArgument):
        w.read_counter(0, 0, 57)


def test_counter_counts_local_completions_only():
    w = World(2, counter_count=2)
    s = w.register_zeros(8)
    w.put(0, 1, s, 0, s, 0, 4, local=CounterInc(1))
    w.get(1, 0, s, 0, s, 4, 4, local=CounterInc(1))
    assert w.cnt == [[0, 1], [0, 1]]


def test_inc_and_add_mixing_needs_reset():
    w = World(1, signal_count=1)
    w.signal(0, 0, SignalInc(0))
    with pytest.raises(InvalidUsage):
        w.signal(0, 0, SignalAdd(0, 2))
    w.reset_signal(0, 0)
    w.signal(0, 0, SignalAdd(0, 2))
    assert w.read_signal(0, 0) == 2


def test_argument_errors():
    w = World(2, signal_count=2, counter_count=1)
    s = w.register_zeros(8)
    with pytest.raises(InvalidArgument):
        w.put(0, 2, s, 0, s, 0, 1)
    with pytest.raises(InvalidArgument):
        w.put(0, 1, s, 0, s, 0, 1, remote=SignalInc(2))
    with pytest.raises(InvalidArgument):
        w.put(0, 1, s, 0, s, 0, 1, local=CounterInc(1))
    with pytest.raises(InvalidArgument):
        w.put(0, 1, 999, 0, s, 0, 1)
    with pytest.raises(InvalidArgument):
        w.register([np.zeros(4, np.uint8), np.zeros(8, np.uint8)])
    # a failed put changes nothing
    assert w.sig == [[0, 0], [0, 0]] and w.cnt == [[0], [0]]


# -- VA signals (GIN page, VA signals) ------------------------------------------------
from oracle.primitives import VASignalAdd, VASignalInc, WIN_STRICT_ORDERING, InvalidUsage  # noqa: E402


def _va_world(R=2, nbytes=64, flags=WIN_STRICT_ORDERING):
    w = World(R)
    win = w.register([np.zeros(nbytes, np.uint8) for _ in range(R)], flags=flags)
    data = w.register_zeros(nbytes)
    return w, win, data


def test_va_signal_counts_like_an_id_signal():
    # the same sequence of actions on an id signal and on a VA word gives the same values
    w, win, data = _va_world()
    seq = [VASignalInc(win, 16), VASignalInc(win, 16), VASignalInc(win, 16)]
    for a in seq:
        w.signal(0, 1, a)
        w.signal(0, 1, SignalInc(3))
        assert w.read_va_signal(1, win, 16) == w.read_signal(1, 3)
    w2, win2, _ = _va_world()
    for v in (5, 0, (1 << 64) - 1, 7):
        w2.signal(1, 0, VASignalAdd(win2, 8, v))
        w2.signal(1, 0, SignalAdd(2, v))
        assert w2.read_va_signal(0, win2, 8) == w2.read_signal(0, 2)


def test_va_signal_word_is_little_endian_uint64_and_wraps():
    w, win, _ = _va_world()
    w.signal(0, 0, VASignalAdd(win, 24, 0x0102030405060708))
    assert w.buf(win, 0)[24:32].tolist() == [8, 7, 6, 5, 4, 3, 2, 1]
    assert w.buf(win, 0)[:24].tolist() == [0] * 24 and w.buf(win, 1).tolist() == [0] * 64
    w.reset_va_signal(0, win, 24)
    w.signal(0, 0, VASignalAdd(win, 24, (1 << 64) - 3))
    w.signal(0, 0, VASignalAdd(win, 24, 5))
    assert w.read_va_signal(0, win, 24) == 2
    assert w.va_signal_reached(0, win, 24, (1 << 64) - 1)  # rolling compare across the wrap
    assert w.read_va_signal(0, win, 24, bits=1) == 0


def test_va_signal_rules():
    w, win, data = _va_world()
    with pytest.raises(InvalidUsage):
        w2, plain2, _ = _va_world(flags=0)
        w2.signal(0, 1, VASignalInc(plain2, 0))
    with pytest.raises(InvalidArgument):
        w.signal(0, 1, VASignalInc(win, 4))  # not 8-byte aligned
    with pytest.raises(InvalidArgument):
        w.signal(0, 1, VASignalInc(win, 64))  # past the window
    w.signal(0, 1, VASignalInc(win, 32))
    with pytest.raises(InvalidUsage):
        w.signal(0, 1, VASignalAdd(win, 32, 2))  # Inc and Add mixed without a reset
    w.reset_va_signal(1, win, 32)
    w.signal(0, 1, VASignalAdd(win, 32, 2))
    assert w.read_va_signal(1, win, 32) == 2


def test_plain_access_to_a_va_signal_word_is_refused():
    w, win, data = _va_world()
    w.signal(0, 1, VASignalInc(win, 32))
    with pytest.raises(InvalidUsage):
        w.put(0, 1, win, 28, data, 0, 8)       # overlaps the word's first bytes
    with pytest.raises(InvalidUsage):
        w.get(0, 1, win, 36, data, 0, 4)       # reads its last bytes
    with pytest.raises(InvalidUsage):
        w.put(0, 1, win, 25, data, 0, 8)       # only the word's first byte
    with pytest.raises(InvalidUsage):
        w.get(0, 1, win, 39, data, 0, 1)       # only its last byte
    w.put(0, 1, win, 24, data, 0, 8)           # the 8 bytes before it are plain data
    w.put(0, 1, win, 40, data, 0, 24)          # and so is everything after it
    w.put(0, 0, win, 32, data, 0, 8)           # the same offset on another rank is not a signal
    assert w.read_va_signal(1, win, 32) == 1


def test_va_signal_put_then_wait_every_interleaving():
    from oracle import protocol as pr
    payload = np.arange(16, dtype=np.uint8)

    def setup():
        w = World(2)
        win = w.register([np.zeros(16, np.uint8) for _ in range(2)], flags=WIN_STRICT_ORDERING)
        src = w.register([payload.copy(), payload.copy() + 100])
        dst = w.register_zeros(16)
        seen = []

        def prog(r):
            if r == 0:
                yield pr.Put(1, dst, 0, src, 0, 16, VASignalInc(win, 8))
            else:
                yield pr.WaitVASignal(win, 8, 1)
                seen.append(w.buf(dst, 1).copy())
        setup.seen = seen
        return w, [prog(0), prog(1)]

    n = 0
    for w in pr.all_runs(setup):
        n += 1
    assert n >= 1
    assert all(np.array_equal(s, payload) for s in setup.seen)
