"""The protocol simulation reaches the plain definitions under every schedule tried."""
import numpy as np
import pytest

from oracle import definitions as D, protocol as pr
from oracle.primitives import Deadlock, SignalInc, World
import workloads as W


def _alltoall_setup(R, B, sends):
    def setup():
        w = World(R, signal_count=2)
        s = w.register([x.copy() for x in sends])
        r = w.register_zeros(R * B)
        return w, pr.alltoall_programs(w, s, r, B, 1)
    return setup


@pytest.mark.parametrize("R", [3])
def test_alltoall_every_interleaving_state_search(R):
    B = 4
    sends = W.alltoall_inputs(R, B, seed=R)
    exp = D.alltoall(sends, B)
    finals = list(pr.distinct_final_states(_alltoall_setup(R, B, sends)))
    assert len(finals) == 1
    w = finals[0]
    recv = list(w.windows)[1]
    assert all(np.array_equal(w.buf(recv, d), exp[d]) for d in range(R))


@pytest.mark.parametrize("R", [2])
def test_alltoall_every_interleaving(R):
    B = 8
    sends = W.alltoall_inputs(R, B, seed=R)
    exp = D.alltoall(sends, B)
    n = 0
    for w, _ in pr.all_runs(_alltoall_setup(R, B, sends)):
        recv = [h for h in w.windows][1]
        for d in range(R):
            assert np.array_equal(w.buf(recv, d), exp[d])
            assert w.sig[d][1] == R
        n += 1
    assert n > 1


@pytest.mark.parametrize("R", [3, 5, 8])
def test_alltoall_random_interleavings(R):
    B = 12
    sends = W.alltoall_inputs(R, B, seed=R)
    exp = D.alltoall(sends, B)
    for seed in range(20):
        w, progs = _alltoall_setup(R, B, sends)()
        pr.run(w, progs, seed=seed)
        recv = list(w.windows)[1]
        assert all(np.array_equal(w.buf(recv, d), exp[d]) for d in range(R))
        assert [w.sig[d][1] for d in range(R)] == [R] * R


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_allreduce_every_interleaving_two_ranks(dtype):
    R, N = 2, 37
    xs = W.allreduce_f32_inputs(R, N) if dtype == "f32" else W.allreduce_bf16_inputs(R, N)
    exp = D.allreduce(xs, dtype).view(np.uint8)
    es = 4 if dtype == "f32" else 2

    def setup():
        w = World(R)
        s = w.register([x.view(np.uint8).copy() for x in xs])
        r = w.register_zeros(N * es)
        sc = w.register_zeros(pr.allreduce_scratch_bytes(N, R, dtype))
        return w, pr.allreduce_programs(w, s, r, sc, N, dtype, 0)

    n = 0
    for w, _ in pr.all_runs(setup):
        recv = list(w.windows)[1]
        assert all(np.array_equal(w.buf(recv, d), exp) for d in range(R))
        assert [w.sig[d][0] for d in range(R)] == [R] * R
        n += 1
    assert n > 10


@pytest.mark.parametrize("R,N,dtype", [(3, 1001, "f32"), (4, 64, "bf16"), (8, 1000, "bf16"),
                                       (5, 3, "f32"), (1, 17, "f32")])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_allreduce_random_interleavings(R, N, dtype, seed):
    xs = W.allreduce_f32_inputs(R, N, seed=seed) if dtype == "f32" else W.allreduce_bf16_inputs(R, N, seed=seed)
    es = 4 if dtype == "f32" else 2
    w = World(R)
    s = w.register([x.view(np.uint8).copy() for x in xs])
    r = w.register_zeros(N * es)
    sc = w.register_zeros(pr.allreduce_scratch_bytes(N, R, dtype))
    pr.run(w, pr.allreduce_programs(w, s, r, sc, N, dtype, 0), seed=seed)
    exp = D.allreduce(xs, dtype).view(np.uint8)
    assert all(np.array_equal(w.buf(r, d), exp) for d in range(R))
    assert [w.sig[d][0] for d in range(R)] == [R] * R


def test_allreduce_worked_example_through_protocol():
    R, N = 4, 1 << 20
    xs = W.allreduce_f32_inputs(R, N, run="A")
    w = World(R)
    s = w.register([x.view(np.uint8).copy() for x in xs])
    r = w.register_zeros(N * 4)
    sc = w.register_zeros(pr.allreduce_scratch_bytes(N, R, "f32"))
    pr.run(w, pr.allreduce_programs(w, s, r, sc, N, "f32", 0), seed=0)
    for d in range(R):
        assert np.all(w.buf(r, d).view(np.float32) == np.float32(6.0))


@pytest.mark.parametrize("seed", [0, 1])
def test_allgather_protocol(seed):
    R, M = 4, 52
    sends = W.allgather_inputs(R, M, seed=seed)
    w = World(R)
    s = w.register([x.copy() for x in sends])
    r = w.register_zeros(R * M)
    pr.run(w, pr.allgather_programs(w, s, r, M, 3), seed=seed)
    exp = D.allgather(sends)
    assert all(np.array_equal(w.buf(r, d), exp[d]) for d in range(R))
    assert [w.sig[d][3] for d in range(R)] == [R] * R


def test_allgather_every_interleaving_two_ranks():
    R, M = 2, 12
    sends = W.allgather_inputs(R, M, seed=4)
    exp = D.allgather(sends)

    def setup():
        w = World(R)
        s = w.register([x.copy() for x in sends])
        r = w.register_zeros(R * M)
        return w, pr.allgather_programs(w, s, r, M, 0)

    for w, _ in pr.all_runs(setup):
        r = list(w.windows)[1]
        assert all(np.array_equal(w.buf(r, d), exp[d]) for d in range(R))


@pytest.mark.parametrize("seed", [0, 3])
def test_ring_protocol_signals_and_counters(seed):
    R, P, pb, C = 4, 12, 16, 3
    sends = W.ring_inputs(R, P, pb, seed=seed)
    w = World(R, signal_count=C, counter_count=C)
    s = w.register([x.copy() for x in sends])
    r = w.register([np.full(P * pb, 7, np.uint8) for _ in range(R)])
    pr.run(w, pr.ring_programs(w, s, r, P, pb, C, 0, 0), seed=seed)
    exp = D.ring(sends, [np.full(P * pb, 7, np.uint8)] * R, P, pb)
    assert all(np.array_equal(w.buf(r, d), exp[d]) for d in range(R))
    assert w.sig == [[P // C] * C] * R
    assert w.cnt == [[P // C] * C] * R


def test_ring_with_reset_returns_signals_to_zero():
    R, P, pb, C = 3, 4, 8, 2
    sends = W.ring_inputs(R, P, pb, seed=1)
    w = World(R, signal_count=C, counter_count=C)
    s = w.register([x.copy() for x in sends])
    r = w.register_zeros(P * pb)
    pr.run(w, pr.ring_programs(w, s, r, P, pb, C, 0, 0, reset=True), seed=1)
    assert w.sig == [[0] * C] * R
    assert w.cnt == [[P // C] * C] * R


def _with_repeats(topk, frac, seed):
    """Entry k names the same expert as entry k-1 with probability frac."""
    t = topk.copy()
    rep = np.random.default_rng(seed + 1).random(t.shape) < frac
    for k in range(1, t.shape[2]):
        t[:, :, k] = np.where(rep[:, :, k], t[:, :, k - 1], t[:, :, k])
    return t


def _run_dispatch(R, T, H, E, K, seed, cap=None, repeat=0.0):
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=seed)
    if repeat:
        topk = _with_repeats(topk, repeat, seed)
    cap = cap if cap is not None else R * T * min(K, E // R)
    w = World(R)
    b = pr.DispatchBuffers(w, x, topk, E, cap)
    pr.run(w, pr.dispatch_programs(w, b, 0, 1), seed=seed)
    return topk, x, w, b, cap


@pytest.mark.parametrize("R,T,H,E,K,seed", [(4, 37, 8, 16, 3, 0), (2, 50, 4, 8, 2, 1),
                                             (3, 20, 2, 6, 2, 2), (8, 64, 4, 64, 8, 3)])
def test_dispatch_protocol_matches_definition(R, T, H, E, K, seed):
    topk, x, w, b, cap = _run_dispatch(R, T, H, E, K, seed)
    rows, src, counts, over = D.dispatch(topk, x, E, cap)
    for d in range(R):
        n, rb = rows[d].shape
        assert np.array_equal(w.buf(b.recv, d)[:n * rb], rows[d].reshape(-1))
        assert np.array_equal(w.buf(b.recv_src, d)[:n * 4].view(np.int32), src[d])
        assert np.array_equal(b.counts[d], counts[d])
        assert w.sig[d][0] == R            # count exchange: one SignalInc per source
        assert w.sig[d][1] == n            # rows: SignalAdd totals aimed at d
        assert b.overflow[d] == over[d]


def test_dispatch_protocol_capacity_overflow():
    R, T, H, E, K = 2, 40, 2, 4, 2
    topk, x, w, b, cap = _run_dispatch(R, T, H, E, K, 5, cap=30)
    rows, src, counts, over = D.dispatch(topk, x, E, cap)
    assert any(over)
    for d in range(R):
        n, rb = rows[d].shape
        assert np.array_equal(w.buf(b.recv, d)[:n * rb], rows[d].reshape(-1))
        assert b.overflow[d] == over[d]


def test_dispatch_every_interleaving_two_ranks():
    R, T, H, E, K = 2, 3, 1, 4, 2
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=8)
    rows, src, counts, _ = D.dispatch(topk, x, E, R * T * K)
    bufs = []

    def setup():
        w = World(R)
        b = pr.DispatchBuffers(w, x, topk, E, R * T * K)
        bufs.append(b)
        return w, pr.dispatch_programs(w, b, 0, 1)

    n = 0
    for w in pr.distinct_final_states(setup):
        b = bufs[-1]
        for d in range(R):
            k, rb = rows[d].shape
            assert np.array_equal(w.buf(b.recv, d)[:k * rb], rows[d].reshape(-1))
            assert np.array_equal(w.buf(b.recv_src, d)[:k * 4].view(np.int32), src[d])
            assert w.sig[d][1] == k
        n += 1
    assert n == 1  # one outcome, whatever the interleaving


def test_deadlock_is_detected_when_a_put_is_missing():
    R, B = 3, 4
    w = World(R)
    s = w.register_zeros(R * B)
    r = w.register_zeros(R * B)

    def prog(rank):
        base = yield pr.ReadSignal(0)
        yield pr.Barrier()
        for peer in range(R):
            if (rank, peer) == (1, 2):
                continue  # the dropped put
            yield pr.Put(peer, r, rank * B, s, peer * B, B, SignalInc(0))
        yield pr.WaitSignal(0, base + R)

    with pytest.raises(Deadlock):
        pr.run(w, [prog(q) for q in range(R)], seed=0)


def test_dispatch_protocol_positions_match_definition():
    for (R, T, H, E, K, seed, cap) in [(4, 37, 8, 16, 3, 0, None), (2, 40, 2, 4, 2, 5, 30)]:
        topk, x, w, b, cap = _run_dispatch(R, T, H, E, K, seed, cap)
        assert np.array_equal(b.pos, D.dispatch_positions(topk, E, cap))


def _run_combine(R, T, H, E, K, seed, dtype="bf16", every=False):
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=seed)
    topk[np.random.default_rng(seed).random(topk.shape) < 0.15] = -1
    weights = W.router_weights(topk, E)
    pos = D.dispatch_positions(topk, E)
    y = W.expert_outputs(D.dispatch_rows_per_rank(topk, E), H, seed=seed + 7, dtype=dtype)
    want = D.combine(topk, weights, pos, y, E, dtype)
    bufs = []

    def setup():
        w = World(R)
        b = pr.CombineBuffers(w, y, topk, weights, pos, E, dtype)
        bufs.append(b)
        return w, pr.combine_programs(w, b, 3)

    worlds = pr.distinct_final_states(setup) if every else [pr.run(*setup(), seed=seed)]
    n = 0
    for w in worlds:
        b = bufs[-1]
        for s in range(R):
            got = w.buf(b.out, s).view(np.uint16 if dtype == "bf16" else np.float32).reshape(T, H)
            assert np.array_equal(got, want[s])
            assert w.sig[s][3] == R  # one SignalInc from every source once its reads are done
        n += 1
    return n


@pytest.mark.parametrize("R,T,H,E,K,seed,dtype", [(4, 30, 8, 16, 3, 0, "bf16"), (3, 20, 4, 6, 2, 1, "f32"),
                                                  (8, 16, 4, 64, 8, 2, "bf16")])
def test_combine_protocol_matches_definition(R, T, H, E, K, seed, dtype):
    _run_combine(R, T, H, E, K, seed, dtype)


def test_combine_every_interleaving_two_ranks():
    assert _run_combine(2, 2, 2, 4, 2, 9, every=True) == 1


@pytest.mark.parametrize("R,T,H,E,K,seed,cap", [(4, 30, 4, 16, 3, 0, None), (2, 25, 2, 4, 2, 1, 12),
                                                 (3, 20, 2, 6, 2, 2, None)])
def test_dedup_dispatch_and_combine_protocols_match_definitions(R, T, H, E, K, seed, cap):
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=seed)
    topk[np.random.default_rng(seed).random(topk.shape) < 0.2] = -1
    cap = cap if cap is not None else R * T
    w = World(R)
    b = pr.DedupBuffers(w, x, topk, E, cap)
    pr.run(w, pr.dispatch_dedup_programs(w, b, 0, 1), seed=seed)
    rows, src, experts, counts, over = D.dispatch_dedup(topk, x, E, cap)
    for d in range(R):
        n, rb = rows[d].shape
        assert np.array_equal(w.buf(b.recv, d)[:n * rb], rows[d].reshape(-1))
        meta = w.buf(b.recv_meta, d)[:n * 4 * (1 + K)].view(np.int32).reshape(n, 1 + K)
        assert np.array_equal(meta[:, 0], src[d]) and np.array_equal(meta[:, 1:], experts[d])
        assert w.sig[d][0] == R
        assert w.sig[d][1] == sum(1 for s in range(R) for t in range(T)
                                  if any(e >= 0 and e // (E // R) == d for e in topk[s, t]))
        assert b.overflow[d] == over[d]
    assert np.array_equal(b.pos, D.dispatch_dedup_positions(topk, E, cap))
    # combine the dispatched rows back (identity experts) through the protocol
    y_win = b.recv
    out_win = w.register_zeros(max(1, T * b.row_bytes))
    pr.run(w, pr.combine_dedup_programs(w, y_win, out_win, b.pos, b.row_bytes, "bf16", 2), seed=seed)
    y = [w.buf(b.recv, d).reshape(cap, b.row_bytes).view(np.uint16) for d in range(R)]
    want = D.combine_dedup(b.pos, y)
    for s in range(R):
        assert np.array_equal(w.buf(out_win, s)[:T * b.row_bytes].view(np.uint16).reshape(T, -1), want[s])
        assert w.sig[s][2] == R


def test_dedup_dispatch_every_interleaving_two_ranks():
    R, T, H, E, K = 2, 3, 1, 4, 2
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=8)
    rows, src, experts, _, _ = D.dispatch_dedup(topk, x, E)
    bufs = []

    def setup():
        w = World(R)
        b = pr.DedupBuffers(w, x, topk, E, R * T)
        bufs.append(b)
        return w, pr.dispatch_dedup_programs(w, b, 0, 1)

    n = 0
    for w in pr.distinct_final_states(setup):
        b = bufs[-1]
        for d in range(R):
            k, rb = rows[d].shape
            assert np.array_equal(w.buf(b.recv, d)[:k * rb], rows[d].reshape(-1))
        n += 1
    assert n == 1


# -- signal ping-pong --------------------------------------------------------------
def test_pingpong_definition_hand_worked():
    # rank 0 holds 0..7, rank 1 holds 100..107; off 1, 3 bytes: rank 1 gets
    # rank 0's bytes 1..3 in place, rank 0 gets them back at 4..6
    got = D.signal_pingpong([np.arange(8, dtype=np.uint8), np.arange(100, 108, dtype=np.uint8)], 1, 3)
    assert list(got[1]) == [100, 1, 2, 3, 104, 105, 106, 107]
    assert list(got[0]) == [0, 1, 2, 3, 1, 2, 3, 7]


def _pingpong_setup(R, init, off, nbytes, iters):
    def setup():
        w = World(R, signal_count=2)
        h = w.register([a.copy() for a in init])
        return w, pr.pingpong_programs(w, h, off, nbytes, iters, 1)
    return setup


@pytest.mark.parametrize("R,iters,nbytes,seed", [(2, 1, 5, 0), (2, 4, 0, 1), (3, 3, 17, 2), (4, 6, 64, 3)])
def test_pingpong_protocol_matches_definition(R, iters, nbytes, seed):
    rng = np.random.default_rng(seed)
    off = 3
    init = [rng.integers(0, 256, off + 2 * nbytes + 5, dtype=np.uint8) for _ in range(R)]
    w, progs = _pingpong_setup(R, init, off, nbytes, iters)()
    pr.run(w, progs, seed=seed)
    h = list(w.windows)[0]
    exp = D.signal_pingpong(init, off, nbytes)
    assert all(np.array_equal(w.buf(h, r), exp[r]) for r in range(R))
    assert [w.sig[r][1] for r in range(R)] == [iters, iters] + [0] * (R - 2)


def test_pingpong_every_interleaving():
    R, iters, nbytes, off = 3, 2, 3, 1
    init = [np.arange(8, dtype=np.uint8) + 50 * r for r in range(R)]
    exp = D.signal_pingpong(init, off, nbytes)
    n = 0
    for w, _ in pr.all_runs(_pingpong_setup(R, init, off, nbytes, iters)):
        h = list(w.windows)[0]
        assert all(np.array_equal(w.buf(h, r), exp[r]) for r in range(R))
        assert [w.sig[r][1] for r in range(R)] == [iters, iters, 0]
        n += 1
    assert n > 1


def test_pingpong_needs_two_ranks():
    w = World(1, signal_count=1)
    h = w.register([np.zeros(8, np.uint8)])
    with pytest.raises(Exception):
        pr.pingpong_programs(w, h, 0, 1, 1, 0)


# -- the protocol's own element conversions and owner sum --------------------------
def test_protocol_bf16_conversions_match_torch():
    import torch
    # widening: every bf16 pattern, against torch's exact bf16 -> fp32
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    got = pr._bf16_widen(bits)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # rounding: random patterns plus ties and the overflow edge, non-NaN, against
    # torch's round-to-nearest-even fp32 -> bf16
    rng = np.random.default_rng(5)
    u = rng.integers(0, 1 << 32, 1 << 18, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 1 << 16, 4096, dtype=np.uint64).astype(np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    edge = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF, 0xFF7F8000, 0x7F800000, 0x00008000, 0x00018000,
                     0x80000000, 0x00000001], dtype=np.uint32)
    u = np.concatenate([u, ties, edge])
    is_nan = (((u >> np.uint32(23)) & np.uint32(0xFF)) == np.uint32(0xFF)) & ((u & np.uint32(0x7FFFFF)) != 0)
    u = u[~is_nan]
    f = u.view(np.float32)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(pr._bf16_round(f), ref)
    # NaN reading: any NaN becomes the canonical quiet NaN 0x7FC0
    nans = np.array([0x7FC00000, 0xFFC00001, 0x7F800001, 0xFFFFFFFF], dtype=np.uint32).view(np.float32)
    assert pr._bf16_round(nans).tolist() == [0x7FC0] * 4


def test_protocol_owner_sum_is_rank_order():
    # 2^24 + 1 + 1: rank order rounds each +1 away (ties to even), a reversed
    # or pairwise order keeps 2; -0.0 alone stays -0.0 (acc starts at slot 0)
    big = np.float32(2.0 ** 24)
    vals = [np.array([big], np.float32), np.array([1.0], np.float32), np.array([1.0], np.float32)]
    assert pr._owner_sum(vals)[0] == big
    assert np.signbit(pr._owner_sum([np.array([-0.0], np.float32)])[0])


def test_allreduce_protocol_bf16_special_values_match_definition():
    # ties at the bf16 rounding point, overflow to infinity, inf - inf, NaN
    R, N = 3, 8
    f = np.array([[1.0, 3.0e38, np.inf, np.nan, 1.0, -2.0, 0.0, -0.0],
                  [2.0 ** -8, 3.0e38, -np.inf, 1.0, 2.0 ** -8 + 2.0 ** -16, 2.0 ** -7, -0.0, -0.0],
                  [0.0, 0.0, 1.0, 1.0, 0.0, 0.0, 0.0, -0.0]], dtype=np.float32)
    xs = [pr._bf16_round(f[r]) for r in range(R)]
    w = World(R)
    s = w.register([x.view(np.uint8).copy() for x in xs])
    r = w.register_zeros(N * 2)
    sc = w.register_zeros(pr.allreduce_scratch_bytes(N, R, "bf16"))
    with np.errstate(invalid="ignore", over="ignore"):
        pr.run(w, pr.allreduce_programs(w, s, r, sc, N, "bf16", 0), seed=2)
        exp = D.allreduce(xs, "bf16")
    for d in range(R):
        assert np.array_equal(w.buf(r, d).view(np.uint16), exp)



# -- a token naming one expert more than once: one row per routing entry -------------------
@pytest.mark.parametrize("R,T,H,E,K,seed,cap", [(3, 30, 4, 6, 3, 11, None), (4, 25, 2, 16, 4, 12, None),
                                                (2, 40, 2, 4, 2, 13, 30)])
def test_dispatch_protocol_repeated_experts_match_definition(R, T, H, E, K, seed, cap):
    topk, x, w, b, cap = _run_dispatch(R, T, H, E, K, seed, cap, repeat=0.5)
    assert any(len(set(topk[s, t].tolist())) < K for s in range(R) for t in range(T))
    rows, src, counts, over = D.dispatch(topk, x, E, cap)
    for d in range(R):
        n, rb = rows[d].shape
        assert np.array_equal(w.buf(b.recv, d)[:n * rb], rows[d].reshape(-1)), d
        assert np.array_equal(w.buf(b.recv_src, d)[:n * 4].view(np.int32), src[d]), d
        assert np.array_equal(b.counts[d], counts[d])
        assert w.sig[d][1] == D.dispatch_rows_per_rank(topk, E)[d]
        assert b.overflow[d] == over[d]
    assert np.array_equal(b.pos, D.dispatch_positions(topk, E, cap))


def test_dispatch_protocol_repeated_expert_every_interleaving():
    R, T, H, E, K = 2, 2, 1, 4, 2
    topk = np.array([[[1, 1], [2, 1]], [[1, 3], [0, 0]]], dtype=np.int32)
    x = np.arange(R * T * H, dtype=np.uint16).reshape(R, T, H) + 1
    rows, src, counts, _ = D.dispatch(topk, x, E, R * T * K)
    bufs = []

    def setup():
        w = World(R)
        b = pr.DispatchBuffers(w, x, topk, E, R * T * K)
        bufs.append(b)
        return w, pr.dispatch_programs(w, b, 0, 1)

    n = 0
    for w in pr.distinct_final_states(setup):
        b = bufs[-1]
        for d in range(R):
            k, rb = rows[d].shape
            assert np.array_equal(w.buf(b.recv, d)[:k * rb], rows[d].reshape(-1))
            assert np.array_equal(w.buf(b.recv_src, d)[:k * 4].view(np.int32), src[d])
        assert np.array_equal(b.pos, D.dispatch_positions(topk, E))
        n += 1
    assert n == 1


def test_combine_protocol_repeated_experts_match_definition():
    R, T, H, E, K, seed = 3, 20, 4, 6, 3, 21
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=seed)
    topk = _with_repeats(topk, 0.5, seed)
    weights = W.router_weights(topk, E)
    pos = D.dispatch_positions(topk, E)
    y = W.expert_outputs(D.dispatch_rows_per_rank(topk, E), H, seed=seed + 7)
    want = D.combine(topk, weights, pos, y, E)
    w = World(R)
    b = pr.CombineBuffers(w, y, topk, weights, pos, E, "bf16")
    pr.run(w, pr.combine_programs(w, b, 3), seed=seed)
    for s in range(R):
        assert np.array_equal(w.buf(b.out, s).view(np.uint16).reshape(T, H), want[s])


def test_dedup_protocol_repeated_experts_match_definition():
    R, T, H, E, K, seed = 4, 30, 2, 16, 4, 22
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=seed)
    topk = _with_repeats(topk, 0.5, seed)
    w = World(R)
    b = pr.DedupBuffers(w, x, topk, E, R * T)
    pr.run(w, pr.dispatch_dedup_programs(w, b, 0, 1), seed=seed)
    rows, src, experts, counts, over = D.dispatch_dedup(topk, x, E, R * T)
    for d in range(R):
        n, rb = rows[d].shape
        assert np.array_equal(w.buf(b.recv, d)[:n * rb], rows[d].reshape(-1))
        meta = w.buf(b.recv_meta, d)[:n * 4 * (1 + K)].view(np.int32).reshape(n, 1 + K)
        assert np.array_equal(meta[:, 0], src[d]) and np.array_equal(meta[:, 1:], experts[d])
    assert np.array_equal(b.pos, D.dispatch_dedup_positions(topk, E, R * T))
