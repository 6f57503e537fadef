"""Seeded random shapes, offsets and rank counts for every collective, each
checked against the oracle to the same bar as the fixed cases (the shapes are
drawn once from a fixed seed, so every run tests the same cases)."""
import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import definitions as D
import workloads as W
import test_gpu_allgather as TAG
import test_gpu_allreduce as TAR
import test_gpu_alltoall as TAA
import test_gpu_combine as TC
import test_gpu_dispatch as TD
from gpu_util import say

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20251)


def _draw(n, fn):
    return [fn(i) for i in range(n)]


AR_CASES = _draw(8, lambda i: (int(_rng.integers(1, 13)), int(_rng.integers(1, 60000)),
                               ["f32", "bf16"][i % 2], int(_rng.integers(0, 40)), int(_rng.integers(0, 40))))
A2A_CASES = _draw(6, lambda i: (int(_rng.integers(1, 13)), int(_rng.integers(1, 70000)),
                                int(_rng.integers(0, 5000)), int(_rng.integers(0, 5000)), i % 2))
AG_CASES = _draw(6, lambda i: (int(_rng.integers(1, 17)), int(_rng.integers(1, 90000)),
                               int(_rng.integers(0, 5000)), int(_rng.integers(0, 5000)), i % 2))


def _dispatch_case(i):
    R = int(_rng.integers(2, 9))
    E = R * int(_rng.integers(1, 9))
    K = int(_rng.integers(1, min(8, E) + 1))
    return R, int(_rng.integers(1, 400)), int(_rng.integers(1, 48)), E, K, 1000 + i


DISP_CASES = _draw(6, _dispatch_case)


@pytest.mark.parametrize("R,N,dtype,so,ro", AR_CASES)
def test_random_allreduce(R, N, dtype, so, ro):
    es = 4 if dtype == "f32" else 2
    so, ro = so * es, ro * es  # offsets are whole elements
    say(f"random allreduce R={R} N={N} {dtype} send_off={so} recv_off={ro}")
    xs = W.allreduce_f32_inputs(R, N, seed=N) if dtype == "f32" else W.allreduce_bf16_inputs(R, N, seed=N)
    out, sigs = TAR._run(xs, dtype, send_off=so, recv_off=ro)
    want = D.allreduce(xs, dtype).view(np.uint8)
    for d in range(R):
        assert np.array_equal(out[d][ro:ro + N * es], want), d
        assert np.all(out[d][:ro] == 0xCD) and np.all(out[d][ro + N * es:] == 0xCD)
    assert sigs == [R] * R


@pytest.mark.parametrize("R,B,so,ro,ce", A2A_CASES)
def test_random_alltoall(R, B, so, ro, ce):
    say(f"random alltoall R={R} B={B} send_off={so} recv_off={ro} copy_engine={ce}")
    sends = W.alltoall_inputs(R, B, seed=B)
    out, sigs = TAA._run(R, B, sends, send_off=so, recv_off=ro, flags=vr.VR_COLL_COPY_ENGINE if ce else 0)
    want = D.alltoall(sends, B)
    for d in range(R):
        assert np.array_equal(out[d][ro:], want[d]), d
        assert np.all(out[d][:ro] == 0xAB)
    assert sigs == [R] * R


@pytest.mark.parametrize("R,M,so,ro,ce", AG_CASES)
def test_random_allgather(R, M, so, ro, ce):
    say(f"random allgather R={R} M={M} send_off={so} recv_off={ro} copy_engine={ce}")
    sends = W.allgather_inputs(R, M, seed=M)
    out, sigs = TAG._run(sends, M, send_off=so, recv_off=ro, flags=vr.VR_COLL_COPY_ENGINE if ce else 0)
    want = D.allgather(sends)
    for d in range(R):
        assert np.array_equal(out[d][ro:], want[d]), d
        assert np.all(out[d][:ro] == 0x5A)
    assert sigs == [R] * R


@pytest.mark.parametrize("R,T,H,E,K,seed", DISP_CASES)
def test_random_dispatch_and_combine(R, T, H, E, K, seed):
    say(f"random dispatch+combine R={R} T={T} H={H} E={E} K={K}")
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=seed)
    res = TD._run(topk, x, E)
    assert not any(TD._check(res, topk, x, E))
    assert res["err"][0] == vr.VR_OK
    topk, weights, y = TC._inputs(R, T, H, E, K, seed)
    res = TC._run(topk, weights, y, E, H)
    TC._check(res, topk, weights, y, E)
    assert res["err"][0] == vr.VR_OK


DEDUP_CASES = _draw(5, lambda i: _dispatch_case(100 + i) + (["bf16", "f32"][i % 2],))
RING_CASES = _draw(5, lambda i: (lambda R, C: (R, C * int(_rng.integers(1, 300)), 16 * int(_rng.integers(1, 64)), C))(
    int(_rng.integers(2, 17)), int(_rng.integers(1, 9))))
SESS_CASES = _draw(4, lambda i: (int(_rng.integers(2, 13)), int(_rng.integers(1, 80000))))


@pytest.mark.parametrize("R,T,H,E,K,seed,dtype", DEDUP_CASES)
def test_random_dedup_dispatch_and_combine(R, T, H, E, K, seed, dtype):
    import test_gpu_dedup as TDD
    TDD.test_dedup_dispatch_vs_oracle(R, T, H, E, K, seed, 0.1)
    TDD.test_dedup_combine_vs_oracle(R, T, H, E, K, seed, dtype)


@pytest.mark.parametrize("R,P,pb,C", RING_CASES)
def test_random_ring_strong_and_weak(R, P, pb, C):
    import test_gpu_ring as TR
    TR.test_ring_vs_oracle(R, P, pb, C)
    TR.test_ring_weak_vs_oracle(R, P, pb, C)


@pytest.mark.parametrize("R,B", SESS_CASES)
def test_random_alltoall_sessions(R, B):
    import test_gpu_sessions as TS
    TS.test_alltoall_sessions_vs_oracle(R, B)


def _loop_case(i):
    # evenly tiled shapes past the looping form's threshold (at least 8192
    # tiles of 4096 bf16 / 2048 fp32 elements), 16-byte aligned offsets: the
    # rank-split form where R <= 8 and R * tpc is a multiple of 64, else the
    # looping form
    R = [2, 4, 8, 16][int(_rng.integers(0, 4))]
    dtype = ["f32", "bf16"][i % 2]
    tile = 2048 if dtype == "f32" else 4096
    tpc = -(-8192 // R) + int(_rng.integers(0, 1024 // R + 1))
    step = 8 // int(np.gcd(R, 8))  # tiles split evenly over the 8 XCDs
    tpc = -(-tpc // step) * step
    vec = 4 if dtype == "f32" else 8  # elements per 16 bytes
    return R, R * tpc * tile, dtype, vec * int(_rng.integers(0, 64)), vec * int(_rng.integers(0, 64))


LOOP_CASES = _draw(4, _loop_case)


def _split_case(i):
    # evenly tiled shapes of the rank-split form: R <= 8, at least 8192
    # tiles, R * tpc a multiple of 64; 16-byte aligned offsets
    R = [2, 4, 8][int(_rng.integers(0, 3))]
    dtype = ["f32", "bf16"][i % 2]
    tile = 2048 if dtype == "f32" else 4096
    tpc = 8192 // R + (64 // R) * int(_rng.integers(0, 17))
    vec = 4 if dtype == "f32" else 8
    return R, R * tpc * tile, dtype, vec * int(_rng.integers(0, 64)), vec * int(_rng.integers(0, 64))


SPLIT_CASES = _draw(4, _split_case)


@pytest.mark.parametrize("R,N,dtype,so,ro", LOOP_CASES + SPLIT_CASES)
def test_random_allreduce_full_tiles(R, N, dtype, so, ro):
    es = 4 if dtype == "f32" else 2
    so, ro = so * es, ro * es
    say(f"random allreduce full tiles R={R} N={N} {dtype} send_off={so} recv_off={ro}")
    xs = W.allreduce_f32_inputs(R, N, seed=N + R) if dtype == "f32" else W.allreduce_bf16_inputs(R, N, seed=N + R)
    out, sigs = TAR._run(xs, dtype, send_off=so, recv_off=ro, repeats=2)
    want = D.allreduce(xs, dtype).view(np.uint8)
    for d in range(R):
        assert np.array_equal(out[d][ro:ro + N * es], want), d
        assert np.all(out[d][:ro] == 0xCD) and np.all(out[d][ro + N * es:] == 0xCD)
    assert sigs == [2 * R] * R


def _ag_piece_case(i):
    # AllGather sizes of the piece form: 16-byte multiples of at least 64 KiB
    # with 16-byte aligned offsets, any rank count up to 24
    R = int(_rng.integers(1, 25))
    M = 16 * int(_rng.integers(4096, 40000))
    return R, M, 16 * int(_rng.integers(0, 300)), 16 * int(_rng.integers(0, 300))


AG_PIECE_CASES = _draw(5, _ag_piece_case)


@pytest.mark.parametrize("R,M,so,ro", AG_PIECE_CASES)
def test_random_allgather_piece_form(R, M, so, ro):
    say(f"random allgather piece form R={R} M={M} send_off={so} recv_off={ro}")
    sends = W.allgather_inputs(R, M, seed=M + R)
    out, sigs = TAG._run(sends, M, send_off=so, recv_off=ro)
    want = D.allgather(sends)
    for d in range(R):
        assert np.array_equal(out[d][ro:], want[d]), d
        assert np.all(out[d][:ro] == 0x5A)
    assert sigs == [R] * R
