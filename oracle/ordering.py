"""Relaxed visibility: which states the strong and weak signal rules allow.

GIN page, one-sided transfers and strong/weak signals; GPUDirect Async
survey, section 4: puts are unordered by default. A weak signal being
visible at the peer implies only that the put it is attached to has
landed; a strong signal implies that every earlier put on the same
context to the same peer has landed as well.

Model. A *stream* is the ordered list of puts one issuer sends on one
context to one peer. Put ``k`` of a stream produces two events: ``D_k``
(its bytes are visible at the peer) and ``S_k`` (its signal increment is
visible). The rules are prerequisites:

* always ``D_k`` before ``S_k``;
* strong: also ``D_j`` before ``S_k`` for every ``j < k`` of the stream.

Data events and signal increments of one stream may otherwise land in any
order (increments commute, so only how many have landed is observable).
A *state* is a set of events closed under prerequisites; every prefix of
every legal order is a state and every state is such a prefix, so checking
what an observer may see over all states is the same as checking every
prefix of every legal order. ``linear_extensions`` enumerates the orders
themselves for the smallest cases, to check that equivalence.
"""
from __future__ import annotations

from functools import lru_cache
from itertools import product


def _prereqs(n: int, strong: bool):
    """Prerequisite sets of events ('D', k) and ('S', k) for one stream of n puts."""
    pre = {}
    for k in range(n):
        pre[("D", k)] = frozenset()
        pre[("S", k)] = frozenset(("D", j) for j in (range(k + 1) if strong else [k]))
    return pre


def stream_states(n: int, strong: bool) -> list[frozenset]:
    """All prerequisite-closed event sets of one stream of n puts."""
    pre = _prereqs(n, strong)
    events = list(pre)
    out = []
    for bits in product((0, 1), repeat=len(events)):
        s = frozenset(e for e, b in zip(events, bits) if b)
        if all(pre[e] <= s for e in s):
            out.append(s)
    return out


def observer_ok(state: frozenset, n: int, strong: bool) -> bool:
    """What a reader of the stream's signal value v may conclude.

    strong: the payloads of the first v puts are all visible;
    weak:   only that at least v payloads are visible.
    """
    v = sum(1 for e in state if e[0] == "S")
    landed = {k for (kind, k) in state if kind == "D"}
    if strong:
        return all(k in landed for k in range(v))
    return len(landed) >= v


def prefix_violation_exists(n: int, strong: bool) -> bool:
    """Whether some allowed state shows signal value v without all of the first v payloads."""
    for st in stream_states(n, strong):
        v = sum(1 for e in st if e[0] == "S")
        landed = {k for (kind, k) in st if kind == "D"}
        if not all(k in landed for k in range(v)):
            return True
    return False


def check_streams(sizes: list[int], strong: bool) -> tuple[int, int]:
    """Check the observer rule on every joint state of several independent streams.

    Returns ``(states_checked, violations)``. Streams (different contexts or
    peers) constrain each other in no way, so a joint state is any tuple of
    per-stream states.
    """
    per = [stream_states(n, strong) for n in sizes]
    checked = bad = 0
    for combo in product(*per):
        checked += 1
        if not all(observer_ok(st, n, strong) for st, n in zip(combo, sizes)):
            bad += 1
    return checked, bad


def cross_context_violation_exists(n0: int, n1: int) -> bool:
    """Whether a strong signal on context 0 can be complete while context 1's puts to the same peer are not."""
    for s0, s1 in product(stream_states(n0, True), stream_states(n1, True)):
        v0 = sum(1 for e in s0 if e[0] == "S")
        d1 = sum(1 for e in s1 if e[0] == "D")
        if v0 == n0 and d1 < n1:
            return True
    return False


def linear_extensions(n: int, strong: bool):
    """Every legal order of the 2n events of one stream (small n only)."""
    pre = _prereqs(n, strong)
    events = list(pre)

    def rec(done: frozenset, order: list):
        if len(order) == len(events):
            yield tuple(order)
            return
        for e in events:
            if e not in done and pre[e] <= done:
                order.append(e)
                yield from rec(done | {e}, order)
                order.pop()

    yield from rec(frozenset(), [])


@lru_cache(maxsize=None)
def count_linear_extensions(n: int, strong: bool) -> int:
    """Number of legal orders, by dynamic programming over states."""
    pre = _prereqs(n, strong)
    events = tuple(pre)

    @lru_cache(maxsize=None)
    def ways(done: frozenset) -> int:
        if len(done) == len(events):
            return 1
        return sum(ways(done | {e}) for e in events if e not in done and pre[e] <= done)

    return ways(frozenset())
