"""Pins for the oracle's plain definitions.

Against the pages' worked examples (tests/golden/*.json), hand-worked
binary32 cases, closed forms, library routines (numpy reductions, torch's
bf16 conversion, numpy stable argsort, block transposes) and brute force.
"""
import itertools
import json
import struct

import numpy as np
import pytest

from oracle import definitions as D
import workloads as W

from conftest import golden


def _load(name):
    with open(golden(name)) as f:
        return json.load(f)


# -- AllReduce -------------------------------------------------------------------
def test_allreduce_worked_example_rank_fill():
    g = _load("allreduce_rank_fill.json")
    R, N = g["ranks"], g["count"]
    xs = W.allreduce_f32_inputs(R, N, run="A")
    assert xs[0].nbytes == g["bytes_per_buffer"]
    out = D.allreduce_sum_f32(xs)
    assert out.shape == (N,)
    assert np.all(np.abs(out - g["expected"]) <= g["tolerance"])
    assert np.all(out == np.float32(g["expected"]))  # small integers: the sum is exact


@pytest.mark.parametrize("R", [1, 2, 3, 8, 16])
def test_allreduce_rank_fill_closed_form(R):
    out = D.allreduce_sum_f32(W.allreduce_f32_inputs(R, 4096, run="A"))
    assert np.all(out == np.float32(R * (R - 1) // 2))


def test_allreduce_summation_order_hand_worked():
    g = _load("summation_order.json")
    for case in g["cases"]:
        xs = [np.array([v], dtype=np.float32) for v in case["ranks_values"]]
        out = D.allreduce_sum_f32(xs)
        if "expected" in case:
            assert out[0] == np.float32(case["expected"]), case
        bits = struct.unpack("<I", struct.pack("<f", float(out[0])))[0]
        if "expected_bits_hex" in case:
            assert bits == int(case["expected_bits_hex"], 16), case


def test_allreduce_matches_numpy_axis0_reduction():
    # numpy reduces a C-contiguous [R, N] array over axis 0 row by row
    # (checked here on data where order matters), an independent route to
    # the same fixed-order fp32 sum.
    xs = W.allreduce_f32_inputs(8, 1 << 15, run="B", seed=7)
    xs = [x * np.float32(1e4 ** (r % 3)) for r, x in enumerate(xs)]
    stacked = np.ascontiguousarray(np.stack(xs))
    assert np.array_equal(D.allreduce_sum_f32(xs), np.add.reduce(stacked, axis=0))
    # and a different order really would differ somewhere on this data
    assert not np.array_equal(D.allreduce_sum_f32(xs[::-1]), D.allreduce_sum_f32(xs))


def test_allreduce_matches_exact_sum_rounded_each_step():
    # Rounding each exact partial sum to binary32 with Python's struct (an
    # independent RNE implementation) must reproduce the oracle.
    def r32(v):
        return struct.unpack("<f", struct.pack("<f", v))[0]
    rng = np.random.default_rng(3)
    xs = [(rng.standard_normal(200) * 10.0 ** rng.integers(-3, 6, 200)).astype(np.float32) for _ in range(5)]
    out = D.allreduce_sum_f32(xs)
    for i in range(200):
        acc = float(xs[0][i])
        for r in range(1, 5):
            acc = r32(acc + float(xs[r][i]))  # exact double add of two floats, then one rounding
        assert np.float32(acc) == out[i] or (np.isnan(acc) and np.isnan(out[i]))


def test_allreduce_error_bound_random():
    xs = W.allreduce_f32_inputs(8, 1 << 14, run="B", seed=11)
    out = D.allreduce_sum_f32(xs).astype(np.float64)
    exact = np.sum(np.stack(xs).astype(np.float64), axis=0)
    bound = 7 * 2.0 ** -24 * np.sum(np.abs(np.stack(xs).astype(np.float64)), axis=0) * 1.0001
    assert np.all(np.abs(out - exact) <= bound + 1e-45)


def test_bf16_widening_is_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = D.bf16_bits_to_f32(bits)
    assert np.array_equal(f.view(np.uint32) >> 16, bits.astype(np.uint32))
    assert np.all(f.view(np.uint32) & 0xFFFF == 0)


def test_bf16_rounding_matches_torch_on_non_nan():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    u = rng.integers(0, 1 << 32, 1 << 18, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0x00000000, 0x80000000, 0x3F808000, 0x3F818000, 0x3F807FFF,
                         0x3F808001, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000, 0x7F800000,
                         0xFF800000, 0x00000001, 0x00008000, 0x00018000, 0x807FFFFF],
                        dtype=np.uint32)
    u = np.concatenate([u, specials])
    f = u.view(np.float32)
    keep = ~np.isnan(f)
    f = f[keep]
    ours = D.f32_to_bf16_bits_rne(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rounding_hand_worked_and_nan_reading():
    cases = {0x3F808000: 0x3F80,  # 1 + 2^-8: tie, keep even 0x3F80
             0x3F818000: 0x3F82,  # tie with odd low bit -> round up
             0x3F808001: 0x3F81,  # just above the tie -> up
             0x7F7FFFFF: 0x7F80,  # max finite fp32 overflows bf16 -> +inf
             0x80000000: 0x8000,  # -0 stays -0
             0x7FC00001: 0x7FC0, 0xFFC12345: 0x7FC0, 0x7F800001: 0x7FC0}  # NaN -> canonical
    u = np.array(list(cases), dtype=np.uint32)
    out = D.f32_to_bf16_bits_rne(u.view(np.float32))
    assert [int(v) for v in out] == list(cases.values())


# -- AlltoAll -------------------------------------------------------------------------
def test_alltoall_page_fill_pattern():
    g = _load("alltoall_fill.json")
    R, count = 4, 16
    wr, wd, we = (g["fill"][k] for k in ("rank_weight", "dest_weight", "element_weight"))
    sends = []
    for s in range(R):
        blocks = [np.array([s * wr + d * wd + i * we for i in range(count)], dtype=np.int32)
                  for d in range(R)]
        sends.append(np.concatenate(blocks).view(np.uint8))
    out = D.alltoall(sends, count * 4)
    for d in range(R):
        got = out[d].view(np.int32).reshape(R, count)
        for s in range(R):
            assert list(got[s]) == [s * wr + d * wd + i * we for i in range(count)]


def test_alltoall_is_block_transpose_and_bijection():
    R, B = 5, 24
    sends = W.alltoall_inputs(R, B, seed=1)
    out = D.alltoall(sends, B)
    ref = np.stack(sends).reshape(R, R, B).swapaxes(0, 1).reshape(R, R * B)
    assert all(np.array_equal(out[d], ref[d]) for d in range(R))
    # index-tagged payload: every (source, dest, word) lands exactly once
    tagged = [np.array([(s << 20) | (d << 10) | w for d in range(R) for w in range(B // 4)],
                       dtype=np.uint32).view(np.uint8) for s in range(R)]
    got = np.concatenate([o.view(np.uint32) for o in D.alltoall(tagged, B)])
    assert sorted(got.tolist()) == sorted(np.concatenate([t.view(np.uint32) for t in tagged]).tolist())


# -- AllGather -------------------------------------------------------------------------
def test_allgather_page_segments():
    g = _load("allgather_segments.json")
    R = g["ranks"]
    n = g["send_bytes"] // 4
    sends = [np.full(n, float(r), dtype=np.float32).view(np.uint8) for r in range(R)]
    out = D.allgather(sends)
    for d in range(R):
        assert out[d].nbytes == g["recv_bytes"]
        segs = out[d].view(np.float32).reshape(R, n)
        for k, v in enumerate(g["segment_values"]):
            assert np.all(segs[k] == np.float32(v))


def test_allgather_matches_tile():
    sends = W.allgather_inputs(3, 36, seed=3)
    out = D.allgather(sends)
    ref = np.tile(np.concatenate(sends), (3, 1))
    assert all(np.array_equal(out[d], ref[d]) for d in range(3))


def test_allgather_for_rank_page_segments_and_brute_force():
    # Symmetric-memory page, AllGather example: segment k of every rank's
    # receive buffer holds rank k's contribution (4 ranks, 1 Mi fp32 each)
    g = _load("allgather_segments.json")
    R, n = g["ranks"], g["send_bytes"] // 4
    sends = [np.full(n, float(r), dtype=np.float32).view(np.uint8) for r in range(R)]
    for d in range(R):
        got = D.allgather_for_rank(sends, d)
        assert got.nbytes == g["recv_bytes"]
        segs = got.view(np.float32).reshape(R, n)
        for k, v in enumerate(g["segment_values"]):
            assert np.all(segs[k] == np.float32(v)), (d, k)
    # every destination, every small rank count and size: byte j of segment s
    # at rank d is byte j of rank s's send buffer
    for R in range(1, 5):
        for M in range(0, 7):
            sends = [np.array([(s * 16 + j) & 0xFF for j in range(M)], dtype=np.uint8) for s in range(R)]
            for d in range(R):
                got = D.allgather_for_rank(sends, d)
                assert got.shape == (R * M,)
                for s in range(R):
                    for j in range(M):
                        assert got[s * M + j] == sends[s][j], (R, M, d, s, j)


def _final_signal_of(kind, R):
    """Run one collective's protocol from zeroed signals and return every
    rank's final value of the completion signal it uses."""
    from oracle import protocol as pr
    from oracle.primitives import World
    w = World(R, signal_count=2)
    if kind == "alltoall":
        B = 4
        s = w.register([np.arange(R * B, dtype=np.uint8) for _ in range(R)])
        r = w.register_zeros(R * B)
        progs, sig = pr.alltoall_programs(w, s, r, B, 1), 1
    elif kind == "allgather":
        M = 3
        s = w.register([np.full(M, q, dtype=np.uint8) for q in range(R)])
        r = w.register_zeros(R * M)
        progs, sig = pr.allgather_programs(w, s, r, M, 1), 1
    elif kind == "allreduce":
        N = 2 * R + 1
        s = w.register([np.full(N, q, dtype=np.float32).view(np.uint8) for q in range(R)])
        r = w.register_zeros(N * 4)
        sc = w.register_zeros(pr.allreduce_scratch_bytes(N, R, "f32"))
        progs, sig = pr.allreduce_programs(w, s, r, sc, N, "f32", 1), 1
    elif kind == "dispatch_counts":
        T, H, E, K = 3, 2, 2 * R, 2
        topk, x = W.dispatch_inputs(R, T, H, E, K, seed=R)
        b = pr.DispatchBuffers(w, x, topk, E, R * T * K)
        progs, sig = pr.dispatch_programs(w, b, 0, 1), 0
    else:
        raise ValueError(kind)
    pr.run(w, progs, seed=R)
    return [w.sig[d][sig] for d in range(R)]


@pytest.mark.parametrize("kind", ["alltoall", "allgather", "allreduce", "dispatch_counts"])
def test_signal_increment_equals_protocol_totals(kind):
    # the final signal value is the number of SignalIncs aimed at the rank in
    # the step-by-step protocol, loopback included (GIN page, pure-GIN
    # AlltoAll kernel: the receiver waits for nRanks increments)
    g = _load("alltoall_fill.json")
    assert g["signal_increments_per_receiver"] == "nRanks"
    for R in range(1, 6):
        assert _final_signal_of(kind, R) == [D.signal_increment(kind, R)] * R, (kind, R)
    assert D.signal_increment("alltoall", 7) == 7  # nRanks, the page's rule
    with pytest.raises(ValueError):
        D.signal_increment("ring", 4)


# -- Ring --------------------------------------------------------------------------------
def test_ring_is_cyclic_shift():
    R, P, pb = 5, 6, 8
    sends = W.ring_inputs(R, P, pb, seed=2)
    before = [np.full(P * pb + 5, 0xEE, dtype=np.uint8) for _ in range(R)]
    out = D.ring(sends, before, P, pb)
    ref = np.roll(np.stack(sends), 1, axis=0)
    for d in range(R):
        assert np.array_equal(out[d][:P * pb], ref[d])
        assert np.all(out[d][P * pb:] == 0xEE)


# -- Dispatch ------------------------------------------------------------------------------
def _dispatch_by_loops(topk, x, E):
    """Destination-major loops: for d, for expert e of d, for source s, for
    token t, for entry k -- one row per routing entry naming e, so a token
    whose top-k names e twice sends two rows (in k order)."""
    R, T, K = topk.shape
    epr = E // R
    res = []
    for d in range(R):
        rows, tags = [], []
        for e in range(d * epr, (d + 1) * epr):
            for s in range(R):
                for t in range(T):
                    for k in range(K):
                        if topk[s, t, k] == e:
                            rows.append(x[s, t].view(np.uint8))
                            tags.append((s << 16) | t)
        res.append((rows, tags))
    return res


def test_dispatch_brute_force_all_routings_tiny():
    # Every routing for R=2, T=2, K=2, E=4, a token's two entries allowed to
    # name one expert twice (reading: one row per routing entry).
    R, T, K, E = 2, 2, 2, 4
    pairs = list(itertools.product(range(E), repeat=K))
    x = np.arange(R * T * 2, dtype=np.uint16).reshape(R, T, 2)
    n = 0
    for choice in itertools.product(pairs, repeat=R * T):
        topk = np.array(choice, dtype=np.int32).reshape(R, T, K)
        rows, src, counts, over = D.dispatch(topk, x, E)
        ref = _dispatch_by_loops(topk, x, E)
        for d in range(R):
            rr, tt = ref[d]
            assert rows[d].shape[0] == len(rr)
            if rr:
                assert np.array_equal(rows[d], np.stack(rr))
            assert src[d].tolist() == tt
            assert int(counts[d].sum()) == len(rr)
            assert not over[d]
        n += 1
    assert n == len(pairs) ** (R * T)


def test_dispatch_duplicate_expert_sends_one_row_per_entry():
    # R=2, T=1, K=2, E=4: the token names expert 1 twice -> two rows at rank 0,
    # both tagged (0, 0); counts and the row total count entries
    topk = np.array([[[1, 1]], [[3, -1]]], dtype=np.int32)
    x = np.array([[[7, 8]], [[9, 10]]], dtype=np.uint16)
    rows, src, counts, over = D.dispatch(topk, x, 4)
    assert src[0].tolist() == [0, 0] and src[1].tolist() == [1 << 16]
    assert rows[0].shape == (2, 4) and np.array_equal(rows[0][0], rows[0][1])
    assert counts[0].tolist() == [0, 2] and counts[1].tolist() == [0, 1]
    assert D.dispatch_rows_per_rank(topk, 4).tolist() == [2, 1]
    assert D.dispatch_positions(topk, 4).tolist() == [[[0, 1]], [[0, -1]]]


def test_dispatch_brute_force_three_ranks_one_slot():
    R, T, K, E = 3, 2, 1, 6
    x = (np.arange(R * T * 3, dtype=np.uint16) * 7).reshape(R, T, 3)
    for choice in itertools.product(range(E), repeat=R * T):
        topk = np.array(choice, dtype=np.int32).reshape(R, T, K)
        rows, src, _, _ = D.dispatch(topk, x, E)
        ref = _dispatch_by_loops(topk, x, E)
        for d in range(R):
            assert src[d].tolist() == ref[d][1]


def test_dispatch_matches_numpy_stable_argsort_and_invariants():
    R, T, H, E, K = 4, 300, 8, 32, 4
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=12)
    rows, src, counts, over = D.dispatch(topk, x, E)
    s_idx, t_idx, _ = np.meshgrid(np.arange(R), np.arange(T), np.arange(K), indexing="ij")
    e = topk.reshape(-1).astype(np.int64)
    key = (e * R + s_idx.reshape(-1)) * T + t_idx.reshape(-1)
    order = np.argsort(key, kind="stable")
    epr = E // R
    xb = x.reshape(R, T, -1).view(np.uint8)
    start = 0
    for d in range(R):
        n = int(np.sum(e // epr == d))
        sel = order[start:start + n]
        start += n
        ss, tt = s_idx.reshape(-1)[sel], t_idx.reshape(-1)[sel]
        assert np.array_equal(src[d], ((ss << 16) | tt).astype(np.int32))
        assert np.array_equal(rows[d], xb[ss, tt])
        assert np.array_equal(counts[d], np.bincount(e[e // epr == d] - d * epr, minlength=epr))
    # bijection between routing slots and received rows; totals
    assert sum(r.shape[0] for r in rows) == R * T * K
    got = sorted((int(tag) >> 16, int(tag) & 0xFFFF) for d in range(R) for tag in src[d])
    want = sorted((s, t) for s in range(R) for t in range(T) for _ in range(K))
    assert got == want
    assert np.array_equal(D.dispatch_rows_per_rank(topk, E), [r.shape[0] for r in rows])


def test_dispatch_skips_unrouted_and_flags_capacity():
    topk = np.array([[[0, -1], [1, 0]], [[-1, -1], [0, 3]]], dtype=np.int32)  # R=2,T=2,K=2,E=4
    x = np.arange(2 * 2 * 1, dtype=np.uint16).reshape(2, 2, 1)
    rows, src, counts, over = D.dispatch(topk, x, 4, capacity_rows=2)
    assert counts[0].tolist() == [3, 1] and counts[1].tolist() == [0, 1]
    assert over == [True, False]
    assert src[0].tolist() == [(0 << 16) | 0, (0 << 16) | 1]  # third row dropped
    with pytest.raises(ValueError):
        D.dispatch(np.array([[[4]]], dtype=np.int32), np.zeros((1, 1, 1), np.uint16), 4)


# -- dispatch positions and combine ------------------------------------------------
def _positions_by_loops(topk, E, cap=None):
    """Receive row of every entry by walking rank d's rows in the layout's own
    nesting (expert, then source, then token, then k)."""
    R, T, K = topk.shape
    epr = E // R
    pos = np.full((R, T, K), -1, dtype=np.int32)
    for d in range(R):
        row = 0
        for e in range(d * epr, (d + 1) * epr):
            for s in range(R):
                for t in range(T):
                    for k in range(K):
                        if topk[s, t, k] == e:
                            if cap is None or row < cap:
                                pos[s, t, k] = row
                            row += 1
    return pos


def test_dispatch_positions_brute_force_tiny():
    R, T, K, E = 2, 2, 2, 4
    pairs = list(itertools.product(range(E), repeat=K)) + [(-1, 1), (2, -1)]  # repeats included
    for choice in itertools.product(pairs, repeat=R * T):
        topk = np.array(choice, dtype=np.int32).reshape(R, T, K)
        assert np.array_equal(D.dispatch_positions(topk, E), _positions_by_loops(topk, E))


def test_dispatch_positions_point_at_the_dispatched_rows():
    R, T, H, E, K = 4, 120, 4, 16, 3
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=21)
    topk[np.random.default_rng(2).random(topk.shape) < 0.2] = -1
    rows, src, _, _ = D.dispatch(topk, x, E)
    pos = D.dispatch_positions(topk, E)
    epr = E // R
    xb = x.reshape(R, T, -1).view(np.uint8)
    seen = [np.zeros(r.shape[0], dtype=int) for r in rows]
    for s in range(R):
        for t in range(T):
            for k in range(K):
                e, p = topk[s, t, k], pos[s, t, k]
                if e < 0:
                    assert p == -1
                    continue
                d = e // epr
                assert src[d][p] == (s << 16) | t
                assert np.array_equal(rows[d][p], xb[s, t])
                seen[d][p] += 1
    assert all(np.all(c == 1) for c in seen)  # every received row has exactly one entry


def test_dispatch_positions_capacity():
    topk = np.array([[[0, -1], [1, 0]], [[-1, -1], [0, 3]]], dtype=np.int32)  # R=2,T=2,K=2,E=4
    pos = D.dispatch_positions(topk, 4, capacity_rows=2)
    # rank 0's rows: e0 (s0,t0), e0 (s0,t1), e0 (s1,t1) dropped, e1 (s0,t1) dropped
    assert pos.tolist() == [[[0, -1], [-1, 1]], [[-1, -1], [-1, 0]]]
    assert np.array_equal(pos, _positions_by_loops(topk, 4, cap=2))


def _f32(v):
    return struct.unpack("<f", struct.pack("<f", v))[0]


def _one_token_combine(ws, ys, dtype="f32"):
    """Helper: R=1, T=1, K=len(ws), one expert per k, rows of one element."""
    K = len(ws)
    topk = np.arange(K, dtype=np.int32).reshape(1, 1, K)
    pos = np.zeros((1, 1, K), dtype=np.int32)
    pos[0, 0, :] = np.arange(K)
    y = np.array(ys, dtype=np.float32).reshape(K, 1)
    w = np.array(ws, dtype=np.float32).reshape(1, 1, K)
    # one rank owns all K experts; row p of its y is entry k = p
    return D.combine(topk, w, pos, [y], K, dtype)[0, 0, 0]


def test_combine_hand_worked_rounding_each_product():
    # k0: -1 * (1 + 2^-7); k1: (1 + 2^-20) * (1 + 2^-7) = 1 + 2^-7 + 2^-20 + 2^-27,
    # rounded to binary32 before the add -> 1 + 2^-7 + 2^-20; the sum is 2^-20.
    # A fused multiply-add would keep the 2^-27 and give 2^-20 + 2^-27.
    got = _one_token_combine([1.0, 1.0 + 2.0 ** -20], [-(1.0 + 2.0 ** -7), 1.0 + 2.0 ** -7])
    assert got == 2.0 ** -20


def test_combine_duplicate_expert_mixes_both_rows():
    # R=1, T=1, K=2, both entries name expert 0: the dispatch sent two rows
    # (positions 0 and 1), and the combine mixes each with its own weight:
    # 0.5 * 3 + 0.25 * 3 = 2.25 (reading one row once would give 1.5)
    topk = np.array([[[0, 0]]], dtype=np.int32)
    pos = D.dispatch_positions(topk, 1)
    assert pos.tolist() == [[[0, 1]]]
    y = [np.array([[3.0], [3.0]], dtype=np.float32)]
    w = np.array([[[0.5, 0.25]]], dtype=np.float32)
    assert D.combine(topk, w, pos, y, 1, "f32")[0, 0, 0] == np.float32(2.25)


def test_combine_hand_worked_k_order():
    # 2^24 + 1 rounds (tie to even) back to 2^24, so k order gives 0;
    # the reverse order would give 1.
    assert _one_token_combine([1.0, 1.0, 1.0], [2.0 ** 24, 1.0, -(2.0 ** 24)]) == 0.0
    assert _one_token_combine([1.0, 1.0, 1.0], [-(2.0 ** 24), 1.0, 2.0 ** 24]) == 1.0


def test_combine_hand_worked_weights():
    ws = [0.1, 0.2, 0.7]
    ys = [3.0, -5.0, 0.25]
    acc = 0.0
    for w, y in zip(ws, ys):
        acc = _f32(acc + _f32(_f32(w) * y))  # each product and sum exact in double, then rounded once
    assert _one_token_combine(ws, ys) == np.float32(acc)


def test_combine_round_trip_is_identity_for_one_hot_weights():
    R, T, H, E, K = 4, 60, 8, 16, 4
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=22)
    rows, _, _, _ = D.dispatch(topk, x, E)
    pos = D.dispatch_positions(topk, E)
    pick = np.random.default_rng(3).integers(0, K, (R, T))
    w = np.zeros((R, T, K), dtype=np.float32)
    w[np.arange(R)[:, None], np.arange(T)[None, :], pick] = 1.0
    y = [r.view(np.uint16).reshape(r.shape[0], H) for r in rows]  # identity experts
    out = D.combine(topk, w, pos, y, E)
    assert np.array_equal(out, x)
    # distinct expert outputs: a one-hot weight selects exactly the picked entry's row
    y = W.expert_outputs([r.shape[0] for r in rows], H, seed=5)
    out = D.combine(topk, w, pos, y, E)
    epr = E // R
    for s in range(R):
        for t in range(T):
            k = pick[s, t]
            assert np.array_equal(out[s, t], y[topk[s, t, k] // epr][pos[s, t, k]])


def test_combine_unit_weights_give_k_times_x_rounded_like_torch():
    import torch
    R, T, H, E, K = 2, 40, 16, 8, 3
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=23)
    rows, _, _, _ = D.dispatch(topk, x, E)
    pos = D.dispatch_positions(topk, E)
    y = [r.view(np.uint16).reshape(r.shape[0], H) for r in rows]
    out = D.combine(topk, np.ones((R, T, K), np.float32), pos, y, E)
    # K * x is exact in fp32 for bf16 x; torch rounds it to bf16 independently
    kx = torch.from_numpy(D.bf16_bits_to_f32(x) * np.float32(K)).to(torch.bfloat16)
    assert np.array_equal(out, kx.view(torch.int16).numpy().view(np.uint16))


def test_combine_skips_entries_without_rows():
    topk = np.array([[[0, -1], [1, 1]], [[-1, -1], [2, 3]]], dtype=np.int32)  # R=2,T=2,K=2,E=4
    pos = D.dispatch_positions(topk, 4, capacity_rows=2)
    y = [np.array([[1.0], [2.0]], np.float32), np.array([[4.0], [8.0]], np.float32)]
    w = np.full((2, 2, 2), 0.5, np.float32)
    out = D.combine(topk, w, pos, y, 4, "f32")
    # rank 0 rows: e0 (0,0) -> row0, e1 (0,1,k0) -> row1, e1 (0,1,k1) dropped (capacity 2)
    # rank 1 rows: e2 (1,1) -> row0, e3 (1,1) -> row1
    assert out[:, :, 0].tolist() == [[0.5, 1.0], [0.0, 6.0]]
    assert np.signbit(out[1, 0, 0]) == False  # noqa: E712 -- a token with no rows is +0.0


# -- per-rank (dedup) dispatch and its combine -----------------------------------------
def _dedup_case(R, T, H, E, K, seed, drop=0.0, repeat=0.0):
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=seed)
    rng = np.random.default_rng(seed)
    if repeat:  # entry k names the same expert as entry k-1
        rep = rng.random(topk.shape) < repeat
        rep[:, :, 0] = False
        for k in range(1, K):
            topk[:, :, k] = np.where(rep[:, :, k], topk[:, :, k - 1], topk[:, :, k])
    if drop:
        topk[rng.random(topk.shape) < drop] = -1
    return topk, x


@pytest.mark.parametrize("R,T,H,E,K,seed,drop,repeat", [(2, 30, 4, 4, 2, 1, 0.0, 0.0), (4, 80, 2, 16, 3, 2, 0.25, 0.0),
                                                         (3, 50, 3, 6, 2, 3, 0.1, 0.0), (8, 40, 2, 64, 8, 4, 0.0, 0.0),
                                                         (4, 60, 2, 16, 4, 5, 0.1, 0.4)])
def test_dedup_dispatch_against_the_per_expert_dispatch(R, T, H, E, K, seed, drop, repeat):
    topk, x = _dedup_case(R, T, H, E, K, seed, drop, repeat)
    epr = E // R
    rows, src, experts, counts, over = D.dispatch_dedup(topk, x, E)
    prow, psrc, pcounts, _ = D.dispatch(topk, x, E)
    xb = x.reshape(R, T, -1).view(np.uint8)
    for d in range(R):
        # library form: the unique (s, t) of d's per-expert rows, in (s, t) order
        st = np.unique(psrc[d]) if len(psrc[d]) else np.zeros(0, np.int32)
        assert np.array_equal(src[d], st.astype(np.int32))
        assert np.array_equal(rows[d], xb[src[d] >> 16, src[d] & 0xFFFF])
        # the experts lists hold exactly the per-expert layout's (s, t, e) entries of d
        got = sorted((int(tag) >> 16, int(tag) & 0xFFFF, d * epr + int(v))
                     for tag, loc in zip(src[d], experts[d]) for v in loc if v >= 0)
        want = []
        off = 0
        for j in range(epr):
            for tag in psrc[d][off:off + pcounts[d][j]]:
                want.append((int(tag) >> 16, int(tag) & 0xFFFF, d * epr + j))
            off += pcounts[d][j]
        assert got == sorted(want)
        assert np.array_equal(counts[d], pcounts[d])
        assert not over[d]
    # per token: the ranks it reaches, each once
    for s in range(R):
        for t in range(T):
            dests = {int(e) // epr for e in topk[s, t] if e >= 0}
            seen = {d for d in range(R) if ((s << 16) | t) in set(src[d].tolist())}
            assert seen == dests


def test_dedup_positions_point_at_the_rows_and_capacity():
    R, T, H, E, K = 4, 60, 2, 16, 4
    topk, x = _dedup_case(R, T, H, E, K, 5, 0.2)
    rows, src, _, _, _ = D.dispatch_dedup(topk, x, E)
    pos = D.dispatch_dedup_positions(topk, E)
    for s in range(R):
        for t in range(T):
            for d in range(R):
                p = pos[s, t, d]
                if p >= 0:
                    assert src[d][p] == (s << 16) | t
                else:
                    assert ((s << 16) | t) not in set(src[d].tolist())
    cap = 7
    pc = D.dispatch_dedup_positions(topk, E, capacity_rows=cap)
    assert np.array_equal(pc, np.where(pos < cap, pos, -1))
    rows_c, src_c, _, _, over_c = D.dispatch_dedup(topk, x, E, capacity_rows=cap)
    assert all(len(v) <= cap for v in src_c) and any(over_c)


def test_combine_dedup_unit_rows_give_the_destination_count_times_x():
    import torch
    R, T, H, E, K = 4, 50, 16, 16, 3
    topk, x = _dedup_case(R, T, H, E, K, 6, 0.15)
    rows, _, _, _, _ = D.dispatch_dedup(topk, x, E)
    pos = D.dispatch_dedup_positions(topk, E)
    y = [r.view(np.uint16).reshape(r.shape[0], H) for r in rows]  # identity experts
    out = D.combine_dedup(pos, y)
    n = (pos >= 0).sum(axis=2).astype(np.float32)[:, :, None]
    want = torch.from_numpy(D.bf16_bits_to_f32(x) * n).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, want)


def test_combine_dedup_hand_worked_rank_order():
    # three destinations; 2^24 + 1 ties to even, so rank order 0, 1, 2 gives 0
    pos = np.array([[[0, 0, 0]], [[-1, -1, -1]], [[-1, -1, -1]]], dtype=np.int32)  # R=3, T=1
    y = [np.array([[2.0 ** 24]], np.float32), np.array([[1.0]], np.float32), np.array([[-(2.0 ** 24)]], np.float32)]
    out = D.combine_dedup(pos, y, "f32")
    assert out[0, 0, 0] == 0.0 and out[1, 0, 0] == 0.0 and not np.signbit(out[1, 0, 0])
    y2 = [y[2], y[1], y[0]]
    assert D.combine_dedup(pos, y2, "f32")[0, 0, 0] == 1.0
