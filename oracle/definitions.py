"""Plain definitions of what each collective leaves in the receive windows.

Each function states the result directly, independent of how ranks split
the work or which order puts land in. ``oracle.protocol`` reaches the same
results step by step; tests check that the two agree.

Floating point: IEEE-754 binary32 additions with round-to-nearest-even, one
rank at a time, exactly as numpy's ``float32 + float32`` performs them.
"""
from __future__ import annotations

import numpy as np

BF16_CANONICAL_NAN = 0x7FC0


# -- bf16 -------------------------------------------------------------------
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 exactly: the 16 bits become the high half."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 bit patterns, round-to-nearest-even.

    The high 16 bits are kept after adding ``0x7FFF`` plus the lowest kept
    bit, so that exact halves round to the even neighbour; overflow past the
    largest finite bf16 rounds to infinity. Any NaN becomes the canonical
    quiet NaN 0x7FC0 (reading: the pages fix no NaN rule; this one matches
    torch's CPU conversion and makes the result independent of NaN payloads).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    out[nan] = BF16_CANONICAL_NAN
    return out


# -- AllReduce ----------------------------------------------------------------
def allreduce_sum_f32(xs) -> np.ndarray:
    """Sum of the ranks' vectors in rank order: ``((x0 + x1) + x2) + ... + x_{R-1}``.

    Symmetric-memory page, AllReduce example: every rank ends with the
    element-wise sum over all ranks. Reading of the order (the pages give
    none): start from rank 0's value, then add rank 1, 2, ... in fp32, so
    that the result is one fixed, reproducible rounding of the sum.
    """
    xs = [np.asarray(x, dtype=np.float32) for x in xs]
    if not xs:
        raise ValueError("at least one rank")
    acc = xs[0].copy()
    for x in xs[1:]:
        acc = acc + x  # float32 + float32 -> float32, one IEEE addition per element
    return acc


def allreduce_sum_bf16(xs_bits) -> np.ndarray:
    """bf16 inputs, fp32 accumulation in rank order, bf16 output (RNE)."""
    return f32_to_bf16_bits_rne(allreduce_sum_f32([bf16_bits_to_f32(b) for b in xs_bits]))


def allreduce(xs, dtype: str) -> np.ndarray:
    """The one vector that every rank's receive window holds afterwards."""
    if dtype == "f32":
        return allreduce_sum_f32(xs)
    if dtype == "bf16":
        return allreduce_sum_bf16(xs)
    raise ValueError(dtype)


# -- AlltoAll -----------------------------------------------------------------
def alltoall(sends, block_bytes: int) -> list[np.ndarray]:
    """Block ``d`` of rank ``s``'s send buffer lands as block ``s`` of rank ``d``.

    GIN page, pure-GIN AlltoAll kernel: each rank puts the block at send
    offset ``peer * size`` to each peer at receive offset ``my_rank * size``.
    """
    R = len(sends)
    sends = [np.asarray(s, dtype=np.uint8).reshape(-1) for s in sends]
    out = []
    for d in range(R):
        out.append(np.concatenate([sends[s][d * block_bytes:(d + 1) * block_bytes] for s in range(R)])
                   if R else np.zeros(0, np.uint8))
    return out


# -- AllGather ----------------------------------------------------------------
def allgather(sends) -> list[np.ndarray]:
    """Every rank receives the concatenation of all ranks' contributions in rank order.

    Symmetric-memory page, AllGather example: segment ``k`` of every receive
    buffer holds rank ``k``'s contribution.
    """
    sends = [np.asarray(s, dtype=np.uint8).reshape(-1) for s in sends]
    whole = np.concatenate(sends)
    return [whole.copy() for _ in sends]


def allgather_for_rank(sends, d: int) -> np.ndarray:
    """Receive buffer of rank ``d`` alone (the same for every d)."""
    del d
    return np.concatenate([np.asarray(s, dtype=np.uint8).reshape(-1) for s in sends])


# -- Ring exchange ------------------------------------------------------------
def ring(sends, recv_before, puts_per_rank: int, put_bytes: int) -> list[np.ndarray]:
    """Rank ``r``'s first ``puts_per_rank * put_bytes`` bytes land at rank ``(r+1) mod R``.

    GPUDirect Async survey, section 4 (the paper's ring-exchange example):
    each rank puts to its successor with a SignalInc per put. Bytes of the
    receive windows beyond the exchanged range keep their previous content.
    """
    R = len(sends)
    n = puts_per_rank * put_bytes
    out = [np.array(b, dtype=np.uint8, copy=True).reshape(-1) for b in recv_before]
    for r in range(R):
        out[(r + 1) % R][:n] = np.asarray(sends[r], dtype=np.uint8).reshape(-1)[:n]
    return out


def signal_pingpong(slices, off: int, nbytes: int) -> list[np.ndarray]:
    """Windows after any number (at least one) of ping-pong round trips
    between ranks 0 and 1.

    GIN page, one-sided transfers: a put copies bytes of the caller's slice
    into the peer's slice. Reading (the pages describe the put and the
    signal wait, not this exchange): a round is rank 0's put of
    ``[off, off+nbytes)`` to the same range at rank 1, then rank 1's put of
    that range of its slice to ``[off+nbytes, off+2*nbytes)`` at rank 0.
    Every round moves the same bytes, so the result is that of one round;
    other ranks are untouched.
    """
    out = [np.array(b, dtype=np.uint8, copy=True).reshape(-1) for b in slices]
    out[1][off:off + nbytes] = out[0][off:off + nbytes]
    out[0][off + nbytes:off + 2 * nbytes] = out[1][off:off + nbytes]
    return out


# -- MoE token dispatch --------------------------------------------------------
def dispatch(topk_idx: np.ndarray, x_rows: np.ndarray, num_experts: int,
             capacity_rows: int | None = None):
    """Route every token row to the rank that owns each of its top-k experts.

    GPUDirect Async survey, opening section: an MoE dispatch sends each
    token (hundreds of bytes) to the experts it was routed to. Layout
    (reading; the pages give none): rank ``d`` owns experts
    ``[d*E/R, (d+1)*E/R)``; its receive rows are ordered by expert, then by
    source rank, then by token index -- a stable sort of all routing entries
    ``(s, t, k)`` on the key ``(e, s, t)``. Entries equal to -1 mean "not
    routed" and are skipped.

    Returns ``(rows, src, counts, overflow)`` with, per destination rank d:
    ``rows[d]`` the received rows ``[n_d, row_bytes]`` (uint8), ``src[d]`` the
    int32 tags ``(s << 16) | t`` of each row, ``counts[d]`` the int32 rows per
    local expert, and ``overflow[d]`` whether ``n_d`` exceeded the capacity
    (rows past the capacity are dropped).
    """
    topk_idx = np.asarray(topk_idx)
    R, T, K = topk_idx.shape
    if num_experts % R:
        raise ValueError("num_experts must be a multiple of the rank count")
    epr = num_experts // R
    x_rows = np.asarray(x_rows)
    row_bytes = x_rows[0].reshape(T, -1).view(np.uint8).shape[1] if T else 0
    xb = [x_rows[s].reshape(T, -1).view(np.uint8) for s in range(R)]
    entries = []
    for s in range(R):
        for t in range(T):
            for k in range(K):
                e = int(topk_idx[s, t, k])
                if e == -1:
                    continue
                if not 0 <= e < num_experts:
                    raise ValueError(f"expert id {e} out of range")
                entries.append((e, s, t))
    entries.sort()
    rows, src, counts, overflow = [], [], [], []
    for d in range(R):
        mine = [(e, s, t) for (e, s, t) in entries if e // epr == d]
        c = np.zeros(epr, dtype=np.int32)
        for (e, _, _) in mine:
            c[e - d * epr] += 1
        counts.append(c)
        over = capacity_rows is not None and len(mine) > capacity_rows
        overflow.append(over)
        if capacity_rows is not None:
            mine = mine[:capacity_rows]
        if mine:
            rows.append(np.stack([xb[s][t] for (_, s, t) in mine]))
        else:
            rows.append(np.zeros((0, row_bytes), dtype=np.uint8))
        src.append(np.array([(s << 16) | t for (_, s, t) in mine], dtype=np.int32))
    return rows, src, counts, overflow


def dispatch_rows_per_rank(topk_idx: np.ndarray, num_experts: int) -> np.ndarray:
    """Rows each destination rank receives (the SignalAdd total aimed at it)."""
    topk_idx = np.asarray(topk_idx)
    R = topk_idx.shape[0]
    epr = num_experts // R
    valid = topk_idx[topk_idx >= 0]
    return np.bincount(valid // epr, minlength=R).astype(np.int64)


def dispatch_positions(topk_idx: np.ndarray, num_experts: int,
                       capacity_rows: int | None = None) -> np.ndarray:
    """Receive row of every routing entry: int32 ``[R, T, K]``.

    Same layout as ``dispatch``: entry ``(s, t, k)`` with expert ``e`` lands
    at rank ``e // (E/R)`` in the place the stable sort on ``(e, s, t)``
    gives it (two entries of one token naming the same expert keep their k
    order). -1 marks an entry that is not routed (``e == -1``) or whose row
    fell past the capacity. This is the metadata the combine step needs to
    find each token's rows again (reading: the pages stop at the dispatch;
    the combine is its inverse).
    """
    topk_idx = np.asarray(topk_idx)
    R, T, K = topk_idx.shape
    epr = num_experts // R
    entries = []
    for s in range(R):
        for t in range(T):
            for k in range(K):
                e = int(topk_idx[s, t, k])
                if e == -1:
                    continue
                if not 0 <= e < num_experts:
                    raise ValueError(f"expert id {e} out of range")
                entries.append((e, s, t, k))
    entries.sort()
    pos = np.full((R, T, K), -1, dtype=np.int32)
    filled = [0] * R
    for (e, s, t, k) in entries:
        d = e // epr
        if capacity_rows is None or filled[d] < capacity_rows:
            pos[s, t, k] = filled[d]
        filled[d] += 1
    return pos


def combine(topk_idx: np.ndarray, weights: np.ndarray, pos: np.ndarray, y_rows,
            num_experts: int, dtype: str = "bf16") -> np.ndarray:
    """MoE combine: each token's expert rows brought back and mixed by its weights.

    The inverse step of the dispatch (GPUDirect Async survey, opening
    section, describes the dispatch; the combine that returns the expert
    outputs to the token's rank is the plain reading of its other half).
    For source rank s and token t, with y the expert-output rows of rank
    ``d = topk[s,t,k] // (E/R)`` laid out like the dispatch's receive rows:

        acc = +0.0
        for k = 0 .. K-1 (in this order), if the entry has a row:
            acc = acc + w[s,t,k] * y[d][pos[s,t,k]]

    every product and every sum one IEEE binary32 operation rounded to
    nearest even (no fused multiply-add); bf16 rows are widened exactly and
    the result is rounded to bf16 (RNE, NaN -> 0x7FC0); fp32 rows stay fp32.
    An entry has a row when its expert id is not -1 and its position is not
    -1. Returns ``[R, T, H]`` (uint16 bf16 bits, or float32).
    """
    topk_idx = np.asarray(topk_idx)
    R, T, K = topk_idx.shape
    epr = num_experts // R
    w = np.asarray(weights, dtype=np.float32)
    pos = np.asarray(pos)
    if dtype == "bf16":
        ys = [bf16_bits_to_f32(np.asarray(y, dtype=np.uint16)) for y in y_rows]
    elif dtype == "f32":
        ys = [np.asarray(y, dtype=np.float32) for y in y_rows]
    else:
        raise ValueError(dtype)
    H = ys[0].shape[1]
    out = np.zeros((R, T, H), dtype=np.float32)
    for s in range(R):
        for t in range(T):
            acc = np.zeros(H, dtype=np.float32)
            for k in range(K):
                e = int(topk_idx[s, t, k])
                p = int(pos[s, t, k])
                if e < 0 or p < 0:
                    continue
                prod = w[s, t, k] * ys[e // epr][p]  # float32 * float32 -> float32
                acc = acc + prod
            out[s, t] = acc
    return f32_to_bf16_bits_rne(out) if dtype == "bf16" else out


# -- Signal totals -------------------------------------------------------------
def signal_increment(kind: str, nranks: int) -> int:
    """What one collective adds to every rank's completion signal.

    Each rank receives exactly one SignalInc per contributing rank, its own
    loopback put included (GIN page, pure-GIN AlltoAll kernel: one put per
    peer, each with a SignalInc, and the receiver waits for nRanks of them).
    """
    if kind in ("allreduce", "alltoall", "allgather", "dispatch_counts"):
        return nranks
    raise ValueError(kind)


# -- dispatch with one row per (token, destination rank) --------------------------
def dispatch_dedup(topk_idx: np.ndarray, x_rows: np.ndarray, num_experts: int,
                   capacity_rows: int | None = None):
    """The dispatch in the per-rank layout: each token lands once on every rank
    that owns at least one of its experts.

    Reading (the pages describe the per-expert dispatch; this is the layout
    that sends a token once per destination rank instead of once per
    expert): rank d's rows are ordered by source rank, then token index, one
    row per token of any source routed to d. Each row carries the tag
    ``(s << 16) | t`` and the token's K entries as seen by d: the local
    expert index ``e - d*E/R`` where ``e`` belongs to d, else -1.

    Returns ``(rows, src, experts, counts, overflow)`` per destination rank:
    ``rows[d]`` [n_d, row_bytes] uint8, ``src[d]`` int32 tags, ``experts[d]``
    int32 [n_d, K], ``counts[d]`` int32 rows per local expert (one per routing
    entry naming it, as in ``dispatch``), ``overflow[d]``.
    """
    topk_idx = np.asarray(topk_idx)
    R, T, K = topk_idx.shape
    if num_experts % R:
        raise ValueError("num_experts must be a multiple of the rank count")
    epr = num_experts // R
    x_rows = np.asarray(x_rows)
    row_bytes = x_rows[0].reshape(T, -1).view(np.uint8).shape[1] if T else 0
    xb = [x_rows[s].reshape(T, -1).view(np.uint8) for s in range(R)]
    for e in topk_idx.reshape(-1):
        if e != -1 and not 0 <= e < num_experts:
            raise ValueError(f"expert id {e} out of range")
    rows, src, experts, counts, overflow = [], [], [], [], []
    for d in range(R):
        mine = []  # (s, t), source-major then token
        c = np.zeros(epr, dtype=np.int32)
        for s in range(R):
            for t in range(T):
                local = [int(e) - d * epr if e >= 0 and e // epr == d else -1 for e in topk_idx[s, t]]
                if any(v >= 0 for v in local):
                    mine.append((s, t, local))
                    for v in local:
                        if v >= 0:
                            c[v] += 1
        counts.append(c)
        overflow.append(capacity_rows is not None and len(mine) > capacity_rows)
        if capacity_rows is not None:
            mine = mine[:capacity_rows]
        rows.append(np.stack([xb[s][t] for (s, t, _) in mine]) if mine
                    else np.zeros((0, row_bytes), dtype=np.uint8))
        src.append(np.array([(s << 16) | t for (s, t, _) in mine], dtype=np.int32))
        experts.append(np.array([loc for (_, _, loc) in mine], dtype=np.int32).reshape(len(mine), K))
    return rows, src, experts, counts, overflow


def dispatch_dedup_positions(topk_idx: np.ndarray, num_experts: int,
                             capacity_rows: int | None = None) -> np.ndarray:
    """Row of token (s, t) at each destination rank d, int32 ``[R, T, R]``;
    -1 where the token is not routed to d or its row fell past the capacity."""
    topk_idx = np.asarray(topk_idx)
    R, T, K = topk_idx.shape
    epr = num_experts // R
    pos = np.full((R, T, R), -1, dtype=np.int32)
    for d in range(R):
        n = 0
        for s in range(R):
            for t in range(T):
                if any(e >= 0 and e // epr == d for e in topk_idx[s, t]):
                    if capacity_rows is None or n < capacity_rows:
                        pos[s, t, d] = n
                    n += 1
    return pos


def combine_dedup(pos: np.ndarray, y_rows, dtype: str = "bf16") -> np.ndarray:
    """Combine in the per-rank layout: each destination rank returns one row
    per token (its experts' outputs already mixed there), and the token's
    rank sums them in rank order.

    For source s and token t: ``acc = +0.0``, then for d = 0 .. R-1 with
    ``pos[s,t,d] != -1``, ``acc = acc + y[d][pos[s,t,d]]`` (binary32, nearest
    even); bf16 rows widened exactly and the sum rounded to bf16 (RNE).
    Returns ``[R, T, H]``.
    """
    pos = np.asarray(pos)
    R, T, _ = pos.shape
    if dtype == "bf16":
        ys = [bf16_bits_to_f32(np.asarray(y, dtype=np.uint16)) for y in y_rows]
    elif dtype == "f32":
        ys = [np.asarray(y, dtype=np.float32) for y in y_rows]
    else:
        raise ValueError(dtype)
    H = ys[0].shape[1]
    out = np.zeros((R, T, H), dtype=np.float32)
    for s in range(R):
        for t in range(T):
            acc = np.zeros(H, dtype=np.float32)
            for d in range(R):
                p = int(pos[s, t, d])
                if p >= 0:
                    acc = acc + ys[d][p]
            out[s, t] = acc
    return f32_to_bf16_bits_rne(out) if dtype == "bf16" else out
