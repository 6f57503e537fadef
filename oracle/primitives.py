"""State model and sequential semantics of the one-sided primitives.

State (one simulated job with R virtual ranks):
  * windows: for each registered window, one ``numpy.uint8`` buffer per rank,
    all of the same size (a symmetric window: the same offset names the same
    slot on every rank -- Symmetric-memory page, section on why symmetric
    windows exist, and window registration flags);
  * signals: ``sig[rank][id]``, integers modulo 2**64 (GIN page, signals and
    counters: each signal is a 64-bit atomically updated integer named by a
    32-bit id);
  * counters: ``cnt[rank][id]``, integers modulo 2**56 (GIN page, counter
    methods: counters hold at most 56 bits).

Every operation here takes effect at once ("sequential mode"): a put's bytes
and its signal are visible as soon as it runs. Weaker visibility orders are
modelled separately in ``oracle.ordering``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SIGNAL_BITS = 64
COUNTER_BITS = 56
WINDOW_ALIGNMENT = 4096  # Symmetric-memory page, window registration: required alignment
WIN_STRICT_ORDERING = 0x02  # window flag a VA signal's window must carry (GIN page, VA signals)


class InvalidArgument(ValueError):
    """An argument is out of range (offset, size, rank, id, bits)."""


class InvalidUsage(RuntimeError):
    """A legal-looking call that breaks a usage rule of the primitive."""


class Deadlock(RuntimeError):
    """Every unfinished rank is blocked in a wait that can no longer succeed."""


def rolling_le(a: int, b: int, bits: int) -> bool:
    """``a <= b`` in wrap-around order on ``bits``-bit unsigned integers.

    GIN page, signals and counters: the comparison is "rolling", so that a
    value still counts as smaller than its successor when the successor has
    wrapped past 2**bits. Reading (the page's formula is garbled): b is at or
    past a when the forward distance ``(b - a) mod 2**bits`` is below half the
    range.
    """
    if not 1 <= bits <= 64:
        raise InvalidArgument(f"bits must be in [1, 64], got {bits}")
    m = (1 << bits) - 1
    return ((b - a) & m) < (1 << (bits - 1))


@dataclass(frozen=True)
class SignalInc:
    """Remote action: add 1 to ``sig[peer][id]`` once the payload has landed."""
    id: int
    strong: bool = True


@dataclass(frozen=True)
class SignalAdd:
    """Remote action: add ``value`` to ``sig[peer][id]`` once the payload has landed."""
    id: int
    value: int
    strong: bool = True


@dataclass(frozen=True)
class VASignalInc:
    """Remote action on a VA signal: add 1 to the 64-bit word at byte ``offset``
    of the peer's slice of window ``win`` (GIN page, VA signals: a signal that
    lives at a (window, offset) pair instead of a preallocated signal slot)."""
    win: int
    offset: int
    strong: bool = True


@dataclass(frozen=True)
class VASignalAdd:
    """Remote action on a VA signal: add ``value`` to the word at (win, offset)."""
    win: int
    offset: int
    value: int
    strong: bool = True


@dataclass(frozen=True)
class CounterInc:
    """Local action: add 1 to ``cnt[rank][id]`` once the source has been consumed."""
    id: int


class World:
    """R virtual ranks, their symmetric windows, signals and counters."""

    def __init__(self, nranks: int, signal_count: int = 16, counter_count: int = 16):
        if nranks < 1:
            raise InvalidArgument("nranks must be >= 1")
        self.nranks = nranks
        self.signal_count = signal_count
        self.counter_count = counter_count
        self.windows: dict[int, list[np.ndarray]] = {}
        self._next_win = 1
        self.sig = [[0] * signal_count for _ in range(nranks)]
        self.cnt = [[0] * counter_count for _ in range(nranks)]
        # GIN page, strong and weak signals: SignalInc must not be mixed with
        # other modifications of the same signal unless it is reset in between.
        self._sig_mode = [[None] * signal_count for _ in range(nranks)]
        self.win_flags: dict[int, int] = {}
        # GIN page, VA signals: once a word serves as a signal, every access to
        # it must be a signal operation. (win, rank, offset) -> "inc" / "add"
        self._va_words: dict[tuple[int, int, int], str | None] = {}

    # -- windows -------------------------------------------------------------
    def register(self, buffers, flags: int = 0) -> int:
        """Register one buffer per rank as a symmetric window; returns a handle.

        ``flags``: ``WIN_STRICT_ORDERING`` marks a window that may hold VA
        signals (GIN page, VA signals)."""
        bufs = [np.asarray(b) for b in buffers]
        if len(bufs) != self.nranks:
            raise InvalidArgument("one buffer per rank is required")
        sizes = {b.nbytes for b in bufs}
        if len(sizes) != 1:
            raise InvalidArgument("a symmetric window has the same size on every rank")
        for i in range(len(bufs)):
            for j in range(i):
                if np.shares_memory(bufs[i], bufs[j]):
                    raise InvalidArgument("the ranks' buffers of a window must not overlap")
        views = []
        for b in bufs:
            if not b.flags.c_contiguous:
                raise InvalidArgument("window buffers must be contiguous")
            views.append(b.reshape(-1).view(np.uint8))
        h = self._next_win
        self._next_win += 1
        self.windows[h] = views
        self.win_flags[h] = flags
        return h

    def register_zeros(self, nbytes: int) -> int:
        return self.register([np.zeros(nbytes, dtype=np.uint8) for _ in range(self.nranks)])

    def deregister(self, win: int) -> None:
        if win not in self.windows:
            raise InvalidArgument("unknown window")
        del self.windows[win]
        del self.win_flags[win]
        self._va_words = {k: v for k, v in self._va_words.items() if k[0] != win}

    def buf(self, win: int, rank: int) -> np.ndarray:
        self._check_rank(rank)
        try:
            return self.windows[win][rank]
        except KeyError:
            raise InvalidArgument("unknown window") from None

    def _check_rank(self, r: int) -> None:
        if not 0 <= r < self.nranks:
            raise InvalidArgument(f"rank {r} out of range")

    def _span(self, win: int, rank: int, off: int, n: int) -> np.ndarray:
        b = self.buf(win, rank)
        if off < 0 or n < 0 or off + n > b.size:
            raise InvalidArgument(f"range [{off}, {off + n}) outside window of {b.size} bytes")
        return b[off:off + n]

    # -- actions -------------------------------------------------------------
    def _check_sig(self, rank: int, sid: int) -> None:
        self._check_rank(rank)
        if not 0 <= sid < self.signal_count:
            raise InvalidArgument(f"signal id {sid} out of range")

    def _check_cnt(self, rank: int, cid: int) -> None:
        self._check_rank(rank)
        if not 0 <= cid < self.counter_count:
            raise InvalidArgument(f"counter id {cid} out of range")

    def _validate_remote(self, peer: int, action) -> None:
        if action is None:
            return
        if isinstance(action, (SignalInc, SignalAdd)):
            self._check_sig(peer, action.id)
            if isinstance(action, SignalAdd) and not 0 <= action.value < (1 << 64):
                raise InvalidArgument("SignalAdd value must fit in 64 bits")
            return
        if isinstance(action, (VASignalInc, VASignalAdd)):
            self._check_va(peer, action.win, action.offset)
            if isinstance(action, VASignalAdd) and not 0 <= action.value < (1 << 64):
                raise InvalidArgument("SignalAdd value must fit in 64 bits")
            return
        raise InvalidArgument(f"not a remote action: {action!r}")

    # -- VA signals ----------------------------------------------------------
    def _check_va(self, rank: int, win: int, offset: int) -> None:
        """A VA signal word: 8 bytes, 8-byte aligned, inside a strict-ordering window."""
        self._span(win, rank, offset, 8)
        if offset % 8:
            raise InvalidArgument("a VA signal word must be 8-byte aligned")
        if not self.win_flags[win] & WIN_STRICT_ORDERING:
            raise InvalidUsage("VA signals need a window registered with strict ordering")

    def _va_value(self, rank: int, win: int, offset: int) -> int:
        return int(self.buf(win, rank)[offset:offset + 8].view("<u8")[0])

    def _set_va_value(self, rank: int, win: int, offset: int, v: int) -> None:
        self.buf(win, rank)[offset:offset + 8] = np.array([v], dtype="<u8").view(np.uint8)

    def _check_plain_access(self, win: int, rank: int, off: int, n: int) -> None:
        """Plain data movement must not touch a word in use as a VA signal."""
        for (w, r, o) in self._va_words:
            if w == win and r == rank and n > 0 and o < off + n and off < o + 8:
                raise InvalidUsage("a VA signal word may only be accessed by signal operations")

    def read_va_signal(self, rank: int, win: int, offset: int, bits: int = SIGNAL_BITS) -> int:
        self._check_va(rank, win, offset)
        if not 1 <= bits <= SIGNAL_BITS:
            raise InvalidArgument("bits out of range")
        self._va_words.setdefault((win, rank, offset), None)
        return self._va_value(rank, win, offset) & ((1 << bits) - 1)

    def va_signal_reached(self, rank: int, win: int, offset: int, least: int, bits: int = SIGNAL_BITS) -> bool:
        m = (1 << bits) - 1
        return rolling_le(least & m, self.read_va_signal(rank, win, offset, bits), bits)

    def reset_va_signal(self, rank: int, win: int, offset: int) -> None:
        """Store 0 in the word; it stays a signal, its Inc/Add mode ends."""
        self._check_va(rank, win, offset)
        self._set_va_value(rank, win, offset, 0)
        self._va_words[(win, rank, offset)] = None

    def _validate_local(self, rank: int, action) -> None:
        if action is None:
            return
        if isinstance(action, CounterInc):
            self._check_cnt(rank, action.id)
            return
        raise InvalidArgument(f"not a local action: {action!r}")

    def apply_remote(self, peer: int, action) -> None:
        """Apply a signal action at ``peer`` (modulo 2**64)."""
        if action is None:
            return
        self._validate_remote(peer, action)
        if isinstance(action, (VASignalInc, VASignalAdd)):
            key = (action.win, peer, action.offset)
            mode = "inc" if isinstance(action, VASignalInc) else "add"
            cur = self._va_words.get(key)
            if cur is not None and cur != mode:
                raise InvalidUsage("SignalInc mixed with SignalAdd on one signal without a reset")
            self._va_words[key] = mode
            inc = 1 if mode == "inc" else action.value
            v = self._va_value(peer, action.win, action.offset)
            self._set_va_value(peer, action.win, action.offset, (v + inc) % (1 << SIGNAL_BITS))
            return
        mode = "inc" if isinstance(action, SignalInc) else "add"
        cur = self._sig_mode[peer][action.id]
        if cur is not None and cur != mode:
            raise InvalidUsage("SignalInc mixed with SignalAdd on one signal without a reset")
        self._sig_mode[peer][action.id] = mode
        inc = 1 if mode == "inc" else action.value
        self.sig[peer][action.id] = (self.sig[peer][action.id] + inc) % (1 << SIGNAL_BITS)

    def apply_local(self, rank: int, action) -> None:
        """Apply a counter action at ``rank`` (modulo 2**56)."""
        if action is None:
            return
        self._validate_local(rank, action)
        self.cnt[rank][action.id] = (self.cnt[rank][action.id] + 1) % (1 << COUNTER_BITS)

    # -- one-sided transfers -------------------------------------------------
    def put(self, rank: int, peer: int, dst: int, doff: int, src: int, soff: int,
            nbytes: int, remote=None, local=None) -> None:
        """Copy ``nbytes`` from ``src`` at ``rank`` to ``dst`` at ``peer``.

        GIN page, one-sided transfers: the peer may be the calling rank itself
        (loopback). The remote action runs at the peer once the bytes have
        landed; the local action runs at the caller once the source bytes have
        been read. The source is read in full before any byte is written, so an
        overlapping loopback copy behaves like memmove.
        """
        self._check_rank(rank)
        self._check_rank(peer)
        s = self._span(src, rank, soff, nbytes)
        d = self._span(dst, peer, doff, nbytes)
        self._check_plain_access(src, rank, soff, nbytes)
        self._check_plain_access(dst, peer, doff, nbytes)
        self._validate_remote(peer, remote)
        self._validate_local(rank, local)
        data = s.copy()
        d[...] = data
        self.apply_remote(peer, remote)
        self.apply_local(rank, local)

    def get(self, rank: int, peer: int, remote_win: int, roff: int, local_win: int,
            loff: int, nbytes: int, local=None) -> None:
        """Copy ``nbytes`` from ``remote_win`` at ``peer`` into ``local_win`` at ``rank``.

        GIN page, one-sided transfers (get): the reverse direction of put; the
        data is visible to the caller once the get has been flushed, which in
        sequential mode is at once.
        """
        self._check_rank(rank)
        self._check_rank(peer)
        s = self._span(remote_win, peer, roff, nbytes)
        d = self._span(local_win, rank, loff, nbytes)
        self._check_plain_access(remote_win, peer, roff, nbytes)
        self._check_plain_access(local_win, rank, loff, nbytes)
        self._validate_local(rank, local)
        data = s.copy()
        d[...] = data
        self.apply_local(rank, local)

    def signal(self, rank: int, peer: int, remote) -> None:
        """A remote action with no payload (GIN page, signal methods)."""
        self._check_rank(rank)
        self._check_rank(peer)
        if remote is None:
            raise InvalidArgument("signal needs a remote action")
        self.apply_remote(peer, remote)

    # -- reads, waits, resets ------------------------------------------------
    def read_signal(self, rank: int, sid: int, bits: int = SIGNAL_BITS) -> int:
        """The low ``bits`` bits of the signal (GIN page, signal methods)."""
        self._check_sig(rank, sid)
        if not 1 <= bits <= SIGNAL_BITS:
            raise InvalidArgument("bits out of range")
        return self.sig[rank][sid] & ((1 << bits) - 1)

    def signal_reached(self, rank: int, sid: int, least: int, bits: int = SIGNAL_BITS) -> bool:
        """Whether a wait for ``least`` on this signal would return now."""
        m = (1 << bits) - 1
        return rolling_le(least & m, self.read_signal(rank, sid, bits), bits)

    def reset_signal(self, rank: int, sid: int) -> None:
        """Set the signal to 0; also ends its Inc/Add mode."""
        self._check_sig(rank, sid)
        self.sig[rank][sid] = 0
        self._sig_mode[rank][sid] = None

    def read_counter(self, rank: int, cid: int, bits: int = COUNTER_BITS) -> int:
        """The low ``bits`` (at most 56) bits of the counter (GIN page, counter methods)."""
        self._check_cnt(rank, cid)
        if not 1 <= bits <= COUNTER_BITS:
            raise InvalidArgument("counter bits must be in [1, 56]")
        return self.cnt[rank][cid] & ((1 << bits) - 1)

    def counter_reached(self, rank: int, cid: int, least: int, bits: int = COUNTER_BITS) -> bool:
        m = (1 << bits) - 1
        return rolling_le(least & m, self.read_counter(rank, cid, bits), bits)

    def reset_counter(self, rank: int, cid: int) -> None:
        self._check_cnt(rank, cid)
        self.cnt[rank][cid] = 0
