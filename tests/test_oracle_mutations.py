"""Planted mistakes in the oracle must be caught by its pins (run on the CPU).

Each test swaps one oracle function for a plausible wrong version and
checks that the corresponding pin test fails.
"""
import numpy as np
import pytest

from oracle import definitions as D, ordering as O
import test_oracle_definitions as TD
import test_oracle_ordering as TO
import test_oracle_primitives as TP


def _fails(fn, *a):
    with pytest.raises(AssertionError):
        fn(*a)


def test_sum_started_from_zero_is_caught(monkeypatch):
    def bad(xs):
        acc = np.zeros_like(np.asarray(xs[0], np.float32))
        for x in xs:
            acc = acc + np.asarray(x, np.float32)
        return acc
    monkeypatch.setattr(D, "allreduce_sum_f32", bad)
    _fails(TD.test_allreduce_summation_order_hand_worked)


def test_reversed_rank_order_is_caught(monkeypatch):
    orig = D.allreduce_sum_f32
    monkeypatch.setattr(D, "allreduce_sum_f32", lambda xs: orig(list(xs)[::-1]))
    _fails(TD.test_allreduce_summation_order_hand_worked)
    _fails(TD.test_allreduce_matches_numpy_axis0_reduction)


def test_pairwise_summation_is_caught(monkeypatch):
    def pairwise(xs):
        xs = [np.asarray(x, np.float32) for x in xs]
        while len(xs) > 1:
            xs = [xs[i] + xs[i + 1] if i + 1 < len(xs) else xs[i] for i in range(0, len(xs), 2)]
        return xs[0]
    monkeypatch.setattr(D, "allreduce_sum_f32", pairwise)
    _fails(TD.test_allreduce_matches_numpy_axis0_reduction)


def test_dropped_rank_is_caught(monkeypatch):
    orig = D.allreduce_sum_f32
    monkeypatch.setattr(D, "allreduce_sum_f32", lambda xs: orig(list(xs)[:-1]) if len(xs) > 1 else orig(xs))
    _fails(TD.test_allreduce_worked_example_rank_fill)


def test_bf16_truncation_is_caught(monkeypatch):
    def trunc(x):
        return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    monkeypatch.setattr(D, "f32_to_bf16_bits_rne", trunc)
    _fails(TD.test_bf16_rounding_matches_torch_on_non_nan)
    _fails(TD.test_bf16_rounding_hand_worked_and_nan_reading)


def test_bf16_round_half_up_is_caught(monkeypatch):
    def half_up(x):
        u = np.ascontiguousarray(x, np.float32).view(np.uint32)
        return ((u + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16)
    monkeypatch.setattr(D, "f32_to_bf16_bits_rne", half_up)
    _fails(TD.test_bf16_rounding_hand_worked_and_nan_reading)


def test_alltoall_transposed_index_is_caught(monkeypatch):
    def transposed(sends, B):
        R = len(sends)
        return [np.concatenate([np.asarray(sends[d]).reshape(-1)[s * B:(s + 1) * B] for s in range(R)])
                for d in range(R)]
    monkeypatch.setattr(D, "alltoall", transposed)
    _fails(TD.test_alltoall_page_fill_pattern)
    _fails(TD.test_alltoall_is_block_transpose_and_bijection)


def test_allgather_wrong_segment_is_caught(monkeypatch):
    def shifted(sends):
        R = len(sends)
        return [np.concatenate([np.asarray(sends[(s + 1) % R]).reshape(-1) for s in range(R)]) for _ in range(R)]
    monkeypatch.setattr(D, "allgather", shifted)
    _fails(TD.test_allgather_page_segments)


def test_dispatch_unstable_order_is_caught(monkeypatch):
    orig = D.dispatch

    def token_major(topk, x, E, capacity_rows=None):
        rows, src, counts, over = orig(topk, x, E, capacity_rows)
        # same multiset per destination, but ordered by (source, token) only
        for d in range(len(rows)):
            order = np.argsort(src[d], kind="stable")
            rows[d], src[d] = rows[d][order], src[d][order]
        return rows, src, counts, over
    monkeypatch.setattr(D, "dispatch", token_major)
    _fails(TD.test_dispatch_matches_numpy_stable_argsort_and_invariants)


def test_dispatch_wrong_owner_is_caught(monkeypatch):
    orig = D.dispatch

    def rotated(topk, x, E, capacity_rows=None):
        rows, src, counts, over = orig(topk, x, E, capacity_rows)
        return rows[1:] + rows[:1], src[1:] + src[:1], counts[1:] + counts[:1], over
    monkeypatch.setattr(D, "dispatch", rotated)
    _fails(TD.test_dispatch_brute_force_all_routings_tiny)


def test_rolling_compare_off_by_one_is_caught(monkeypatch):
    def bad(a, b, bits):
        m = (1 << bits) - 1
        return ((b - a) & m) <= (1 << (bits - 1))
    monkeypatch.setattr(TP, "rolling_le", bad)
    _fails(TP.test_rolling_le_small_width_brute_force)


def test_weak_rule_treated_as_strong_is_caught(monkeypatch):
    orig = O._prereqs
    monkeypatch.setattr(O, "_prereqs", lambda n, strong: orig(n, True))
    _fails(TO.test_weak_signal_admits_a_missing_earlier_payload, 3)


def test_strong_rule_treated_as_weak_is_caught(monkeypatch):
    orig = O._prereqs
    monkeypatch.setattr(O, "_prereqs", lambda n, strong: orig(n, False))
    _fails(TO.test_strong_signal_prefix_property_holds_in_every_state, 3)


def test_combine_fused_multiply_add_is_caught(monkeypatch):
    def fused(topk, weights, pos, y_rows, E, dtype="bf16"):
        R, T, K = np.asarray(topk).shape
        epr = E // R
        ys = [np.asarray(y, np.float64) if dtype == "f32" else D.bf16_bits_to_f32(y).astype(np.float64)
              for y in y_rows]
        out = np.zeros((R, T, ys[0].shape[1]), np.float32)
        for s in range(R):
            for t in range(T):
                acc = np.zeros(ys[0].shape[1], np.float32)
                for k in range(K):
                    e, p = int(topk[s, t, k]), int(pos[s, t, k])
                    if e >= 0 and p >= 0:
                        acc = (acc.astype(np.float64) + np.float64(weights[s, t, k]) * ys[e // epr][p]).astype(np.float32)
                out[s, t] = acc
        return D.f32_to_bf16_bits_rne(out) if dtype == "bf16" else out
    monkeypatch.setattr(D, "combine", fused)
    _fails(TD.test_combine_hand_worked_rounding_each_product)


def test_combine_reversed_k_order_is_caught(monkeypatch):
    orig = D.combine

    def reversed_k(topk, weights, pos, y_rows, E, dtype="bf16"):
        return orig(np.asarray(topk)[:, :, ::-1], np.asarray(weights)[:, :, ::-1], np.asarray(pos)[:, :, ::-1],
                    y_rows, E, dtype)
    monkeypatch.setattr(D, "combine", reversed_k)
    _fails(TD.test_combine_hand_worked_k_order)


def test_combine_weights_of_wrong_entry_is_caught(monkeypatch):
    orig = D.combine

    def shifted(topk, weights, pos, y_rows, E, dtype="bf16"):
        return orig(topk, np.roll(np.asarray(weights), 1, axis=2), pos, y_rows, E, dtype)
    monkeypatch.setattr(D, "combine", shifted)
    _fails(TD.test_combine_round_trip_is_identity_for_one_hot_weights)


def test_positions_ignoring_source_order_is_caught(monkeypatch):
    orig = D.dispatch_positions

    def token_first(topk, E, capacity_rows=None):
        # rows of one expert ordered by token before source: a plausible slip
        t = np.asarray(topk)
        return orig(t.transpose(1, 0, 2).copy(), E, capacity_rows).transpose(1, 0, 2) if t.shape[0] == t.shape[1] \
            else orig(t[::-1].copy(), E, capacity_rows)[::-1]
    monkeypatch.setattr(D, "dispatch_positions", token_first)
    _fails(TD.test_dispatch_positions_point_at_the_dispatched_rows)


def test_va_signal_big_endian_word_is_caught(monkeypatch):
    from oracle.primitives import World

    def get_be(self, rank, win, offset):
        return int(self.buf(win, rank)[offset:offset + 8].view(">u8")[0])

    def set_be(self, rank, win, offset, v):
        self.buf(win, rank)[offset:offset + 8] = np.array([v], dtype=">u8").view(np.uint8)
    monkeypatch.setattr(World, "_va_value", get_be)
    monkeypatch.setattr(World, "_set_va_value", set_be)
    _fails(TP.test_va_signal_word_is_little_endian_uint64_and_wraps)


def test_va_word_overlap_off_by_one_is_caught(monkeypatch):
    from oracle.primitives import World, InvalidUsage

    def loose(self, win, rank, off, n):
        for (w, r, o) in self._va_words:
            if w == win and r == rank and n > 0 and o < off + n - 1 and off < o + 7:
                raise InvalidUsage("overlap")
    monkeypatch.setattr(World, "_check_plain_access", loose)
    with pytest.raises(pytest.fail.Exception):
        TP.test_plain_access_to_a_va_signal_word_is_refused()


def test_dedup_token_major_order_is_caught(monkeypatch):
    orig = D.dispatch_dedup

    def token_major(topk, x, E, capacity_rows=None):
        rows, src, experts, counts, over = orig(topk, x, E, capacity_rows)
        for d in range(len(rows)):  # order by token, then source: a plausible slip
            order = np.lexsort((src[d] >> 16, src[d] & 0xFFFF))
            rows[d], src[d], experts[d] = rows[d][order], src[d][order], experts[d][order]
        return rows, src, experts, counts, over
    monkeypatch.setattr(D, "dispatch_dedup", token_major)
    _fails(TD.test_dedup_dispatch_against_the_per_expert_dispatch, 4, 80, 2, 16, 3, 2, 0.25, 0.0)


def test_combine_dedup_reversed_rank_order_is_caught(monkeypatch):
    orig = D.combine_dedup

    def reversed_ranks(pos, y_rows, dtype="bf16"):
        return orig(np.asarray(pos)[:, :, ::-1], list(y_rows)[::-1], dtype)
    monkeypatch.setattr(D, "combine_dedup", reversed_ranks)
    _fails(TD.test_combine_dedup_hand_worked_rank_order)


def test_pingpong_answer_in_place_is_caught(monkeypatch):
    import test_oracle_protocol as TPR

    def in_place(slices, off, nbytes):  # the pong overwrites rank 0's own bytes
        out = [np.array(b, dtype=np.uint8, copy=True).reshape(-1) for b in slices]
        out[1][off:off + nbytes] = out[0][off:off + nbytes]
        return out
    monkeypatch.setattr(D, "signal_pingpong", in_place)
    _fails(TPR.test_pingpong_definition_hand_worked)
    _fails(TPR.test_pingpong_protocol_matches_definition, 3, 3, 17, 2)


def test_allgather_for_rank_rotated_segments_are_caught(monkeypatch):
    def rotated(sends, d):  # segment k of rank d holding rank (k + d) mod R's bytes
        R = len(sends)
        return np.concatenate([np.asarray(sends[(k + d) % R], dtype=np.uint8).reshape(-1) for k in range(R)])
    monkeypatch.setattr(D, "allgather_for_rank", rotated)
    _fails(TD.test_allgather_for_rank_page_segments_and_brute_force)


def test_signal_increment_without_loopback_is_caught(monkeypatch):
    monkeypatch.setattr(D, "signal_increment", lambda kind, R: R - 1)
    _fails(TD.test_signal_increment_equals_protocol_totals, "alltoall")
    _fails(TD.test_signal_increment_equals_protocol_totals, "allreduce")


def test_dispatch_one_row_per_repeated_expert_is_caught(monkeypatch):
    orig = D.dispatch

    def once(topk, x, E, capacity_rows=None):  # a token naming e twice sends one row
        t = np.array(topk, copy=True)
        for k in range(1, t.shape[2]):
            for q in range(k):
                t[:, :, k] = np.where(t[:, :, k] == t[:, :, q], -1, t[:, :, k])
        return orig(t, x, E, capacity_rows)
    monkeypatch.setattr(D, "dispatch", once)
    _fails(TD.test_dispatch_brute_force_all_routings_tiny)
    _fails(TD.test_dispatch_duplicate_expert_sends_one_row_per_entry)


def test_protocol_reversed_owner_sum_is_caught(monkeypatch):
    from oracle import protocol as pr
    import test_oracle_protocol as TPR
    orig = pr._owner_sum
    monkeypatch.setattr(pr, "_owner_sum", lambda vals: orig(list(vals)[::-1]))
    _fails(TPR.test_allreduce_random_interleavings, 8, 257, "f32", 2)
    _fails(TPR.test_protocol_owner_sum_is_rank_order)


def test_protocol_bf16_truncation_is_caught(monkeypatch):
    from oracle import protocol as pr
    import test_oracle_protocol as TPR
    monkeypatch.setattr(pr, "_bf16_round",
                        lambda x: (np.ascontiguousarray(x, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16))
    _fails(TPR.test_protocol_bf16_conversions_match_torch)
    _fails(TPR.test_allreduce_random_interleavings, 4, 300, "bf16", 1)


# -- the remaining definitions, primitives and protocol programs ------------------------
def test_bf16_widening_off_by_one_bit_is_caught(monkeypatch):
    monkeypatch.setattr(D, "bf16_bits_to_f32",
                        lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(15)).view(np.float32))
    _fails(TD.test_bf16_widening_is_exact)


def test_ring_to_the_wrong_successor_is_caught(monkeypatch):
    def two_ahead(sends, recv_before, puts_per_rank, put_bytes):
        R, n = len(sends), puts_per_rank * put_bytes
        out = [np.array(b, dtype=np.uint8, copy=True).reshape(-1) for b in recv_before]
        for r in range(R):
            out[(r + 2) % R][:n] = np.asarray(sends[r], dtype=np.uint8).reshape(-1)[:n]
        return out
    monkeypatch.setattr(D, "ring", two_ahead)
    _fails(TD.test_ring_is_cyclic_shift)


def test_rows_per_rank_counting_tokens_is_caught(monkeypatch):
    def per_token(topk, E):  # one row per (token, rank) instead of per entry
        topk = np.asarray(topk)
        R, T, _ = topk.shape
        epr = E // R
        out = np.zeros(R, np.int64)
        for s in range(R):
            for t in range(T):
                for d in {int(e) // epr for e in topk[s, t] if e >= 0}:
                    out[d] += 1
        return out
    monkeypatch.setattr(D, "dispatch_rows_per_rank", per_token)
    _fails(TD.test_dispatch_duplicate_expert_sends_one_row_per_entry)


def test_dedup_positions_in_token_major_order_are_caught(monkeypatch):
    def token_major(topk, E, capacity_rows=None):
        topk = np.asarray(topk)
        R, T, _ = topk.shape
        epr = E // R
        pos = np.full((R, T, R), -1, dtype=np.int32)
        for d in range(R):
            n = 0
            for t in range(T):  # token before source: a plausible slip
                for s in range(R):
                    if any(e >= 0 and e // epr == d for e in topk[s, t]):
                        if capacity_rows is None or n < capacity_rows:
                            pos[s, t, d] = n
                        n += 1
        return pos
    monkeypatch.setattr(D, "dispatch_dedup_positions", token_major)
    _fails(TD.test_dedup_positions_point_at_the_rows_and_capacity)


def test_put_dropping_its_last_byte_is_caught(monkeypatch):
    from oracle.primitives import World
    orig = World.put

    def short(self, rank, peer, dst, doff, src, soff, nbytes, remote=None, local=None):
        return orig(self, rank, peer, dst, doff, src, soff, max(0, nbytes - 1), remote, local)
    monkeypatch.setattr(World, "put", short)
    _fails(TP.test_put_get_brute_force_tiny_windows)


def test_counter_counting_twice_is_caught(monkeypatch):
    from oracle.primitives import World, COUNTER_BITS

    def twice(self, rank, action):
        if action is None:
            return
        self._validate_local(rank, action)
        self.cnt[rank][action.id] = (self.cnt[rank][action.id] + 2) % (1 << COUNTER_BITS)
    monkeypatch.setattr(World, "apply_local", twice)
    _fails(TP.test_counter_counts_local_completions_only)


def test_protocol_alltoall_at_the_peers_offset_is_caught(monkeypatch):
    from oracle import protocol as pr
    import test_oracle_protocol as TPR

    def transposed(world, send, recv, block, sig, strong=True):
        R = world.nranks

        def prog(rank):
            base = yield pr.ReadSignal(sig)
            yield pr.Barrier()
            for peer in range(R):  # receive offset of the peer instead of the sender's own
                yield pr.Put(peer, recv, peer * block, send, peer * block, block, pr.SignalInc(sig, strong))
            yield pr.WaitSignal(sig, base + R)
            yield pr.Barrier()
        return [prog(r) for r in range(R)]
    monkeypatch.setattr(pr, "alltoall_programs", transposed)
    _fails(TPR.test_alltoall_random_interleavings, 3)


def test_protocol_allgather_wrong_segment_is_caught(monkeypatch):
    from oracle import protocol as pr
    import test_oracle_protocol as TPR

    def wrong(world, send, recv, nbytes, sig):
        R = world.nranks

        def prog(rank):
            base = yield pr.ReadSignal(sig)
            yield pr.Barrier()
            for peer in range(R):  # segment of the destination instead of the source
                yield pr.Put(peer, recv, peer * nbytes, send, 0, nbytes, pr.SignalInc(sig))
            yield pr.WaitSignal(sig, base + R)
            yield pr.Barrier()
        return [prog(r) for r in range(R)]
    monkeypatch.setattr(pr, "allgather_programs", wrong)
    _fails(TPR.test_allgather_protocol, 0)


def test_protocol_allreduce_chunk_bounds_off_by_one_is_caught(monkeypatch):
    from oracle import protocol as pr
    import test_oracle_protocol as TPR
    orig = pr.chunk_bounds
    monkeypatch.setattr(pr, "chunk_bounds", lambda count, R, owner: (lambda a, b: (min(a + 1, b), b))(
        *orig(count, R, owner)))
    _fails(TPR.test_allreduce_random_interleavings, 3, 1001, "f32", 0)


def test_protocol_ring_signalling_one_context_is_caught(monkeypatch):
    from oracle import protocol as pr
    import test_oracle_protocol as TPR
    orig_inc = pr.SignalInc
    # every SignalInc of the exchange lands on the first context's signal: the
    # other contexts' waits can never end, which the scheduler reports
    from oracle.primitives import Deadlock
    monkeypatch.setattr(pr, "SignalInc", lambda sid, strong=True: orig_inc(0, strong))
    with pytest.raises(Deadlock):
        TPR.test_ring_protocol_signals_and_counters(0)
