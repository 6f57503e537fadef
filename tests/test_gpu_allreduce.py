"""Sum-AllReduce on the GPU against the oracle: bit-exact in fixed rank order."""
import json

import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import definitions as D
import workloads as W
from conftest import golden
from gpu_util import Job, say

pytestmark = pytest.mark.gpu


def _run(xs, dtype, send_off=0, recv_off=0, sig=2, repeats=1):
    R = len(xs)
    es = 4 if dtype == "f32" else 2
    N = xs[0].size
    dt = vr.VR_DT_F32 if dtype == "f32" else vr.VR_DT_BF16
    with Job(R) as job:
        sw, sv = job.window(send_off + N * es + 16, fill=0)
        rw, rv = job.window(recv_off + N * es + 16, fill=0xCD)
        for r in range(R):
            sv[r][send_off:send_off + N * es].copy_(job.torch.from_numpy(xs[r].view(np.uint8)))
        for _ in range(repeats):
            vr.vr_allreduce(job.comm, sw, send_off, rw, recv_off, N, dt, sig=sig)
        out = job.host(rv)
        sigs = [job.sig(d, sig) for d in range(R)]
        job.assert_no_async_error()
    return out, sigs


def test_allreduce_page_worked_example():
    g = json.load(open(golden("allreduce_rank_fill.json")))
    R, N = g["ranks"], g["count"]
    say("allreduce rank fill R=4 N=1M")
    out, sigs = _run(W.allreduce_f32_inputs(R, N, run="A"), "f32")
    for d in range(R):
        v = out[d][:N * 4].view(np.float32)
        assert np.all(np.abs(v - g["expected"]) <= g["tolerance"])
        assert np.all(v == np.float32(g["expected"]))
        assert np.all(out[d][N * 4:] == 0xCD)
    assert sigs == [R] * R


@pytest.mark.parametrize("R", [1, 2, 3, 8, 16, 64])
def test_allreduce_rank_fill_closed_form(R):
    say(f"allreduce rank fill R={R}")
    out, _ = _run(W.allreduce_f32_inputs(R, 5000, run="A"), "f32")
    for d in range(R):
        assert np.all(out[d][:20000].view(np.float32) == np.float32(R * (R - 1) // 2))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("R,N", [(2, 1), (3, 1001), (4, 4096), (5, 77777), (8, 2048 * 8 + 3), (16, 40000),
                                 (7, 123457), (64, 9000)])
def test_allreduce_random_bit_exact(dtype, R, N):
    say(f"allreduce {dtype} R={R} N={N}")
    xs = W.allreduce_f32_inputs(R, N, seed=R + N) if dtype == "f32" else W.allreduce_bf16_inputs(R, N, seed=R + N)
    out, sigs = _run(xs, dtype)
    es = 4 if dtype == "f32" else 2
    exp = D.allreduce(xs, dtype).view(np.uint8)
    for d in range(R):
        assert np.array_equal(out[d][:N * es], exp), d
    assert sigs == [R] * R


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_allreduce_unaligned_offsets(dtype):
    R, N = 4, 3000
    es = 4 if dtype == "f32" else 2
    say(f"allreduce unaligned {dtype}")
    xs = W.allreduce_f32_inputs(R, N, seed=3) if dtype == "f32" else W.allreduce_bf16_inputs(R, N, seed=3)
    out, _ = _run(xs, dtype, send_off=es * 3, recv_off=es * 5)
    exp = D.allreduce(xs, dtype).view(np.uint8)
    for d in range(R):
        assert np.array_equal(out[d][es * 5:es * 5 + N * es], exp)


@pytest.mark.filterwarnings("ignore:overflow encountered in add:RuntimeWarning")
@pytest.mark.filterwarnings("ignore:invalid value encountered in add:RuntimeWarning")
def test_allreduce_special_values_bf16():
    # ties, overflow to inf, inf + -inf = NaN (canonical 0x7FC0), signed zeros
    R = 3
    vals = np.array([[0x3F80, 0x7F7F, 0x7F80, 0x8000, 0x3F80, 0x0001, 0xFF80, 0x7FC1],
                     [0x3B80, 0x7F7F, 0xFF80, 0x8000, 0xBF80, 0x0001, 0xFF80, 0x0000],
                     [0x0000, 0x7F00, 0x0000, 0x8000, 0x0000, 0x8001, 0x3F80, 0x3F80]], dtype=np.uint16)
    xs = [np.tile(v, 700) for v in vals]
    say("allreduce bf16 special values")
    out, _ = _run(xs, "bf16")
    exp = D.allreduce(xs, "bf16").view(np.uint8)
    for d in range(R):
        assert np.array_equal(out[d][:exp.size], exp)


def test_allreduce_repeated_signal_accumulates():
    say("allreduce repeated x3")
    xs = W.allreduce_f32_inputs(4, 1000, seed=5)
    out, sigs = _run(xs, "f32", repeats=3)
    assert sigs == [12] * 4


def test_allreduce_f32_r4_1Mi_run_b():
    c = W.CONFIGS["allreduce_f32_r4_1Mi"]
    say("allreduce f32 R=4 1 Mi run B")
    xs = W.allreduce_f32_inputs(c["ranks"], c["count"], run="B", seed=c["seed"])
    out, _ = _run(xs, "f32")
    exp = D.allreduce(xs, "f32").view(np.uint8)
    for d in range(c["ranks"]):
        assert np.array_equal(out[d][:exp.size], exp)


def test_allreduce_bf16_r8_64Mi_full_size():
    c = W.CONFIGS["allreduce_bf16_r8_64Mi"]
    R, N = c["ranks"], c["count"]
    say(f"allreduce bf16 full size R={R} N={N}")
    xs = W.allreduce_bf16_inputs(R, N, seed=c["seed"])
    exp = D.allreduce(xs, "bf16").view(np.uint8)
    out, sigs = _run(xs, "bf16")
    for d in range(R):
        assert np.array_equal(out[d][:N * 2], exp), d
    assert sigs == [R] * R


@pytest.mark.parametrize("dtype,R,N", [("f32", 4, 16 << 20), ("bf16", 2, 48 << 20), ("f32", 8, 16 << 20),
                                     ("bf16", 4, 32 << 20), ("f32", 2, 2 * 4096 * 2048), ("bf16", 16, 32 << 20),
                                     ("f32", 16, 16 * 520 * 2048)])
def test_allreduce_rank_split_form(dtype, R, N):
    # Evenly tiled shapes of at least 8192 tiles whose chunk splits into a
    # multiple of 64 pieces run the rank-split form (one piece of
    # max(512/R, 64) vectors per rank per workgroup, three relay levels); a
    # piece is 4 KiB per rank for R=2, R=16 takes four runs per wave, and the
    # fifth shape is the smallest that qualifies. Two calls in a row check
    # that the relay counters come back to 0.
    assert _form(dtype, R, N) == "split"
    say(f"allreduce rank-split form {dtype} R={R} N={N}")
    xs = W.allreduce_f32_inputs(R, N, seed=R + 11) if dtype == "f32" else W.allreduce_bf16_inputs(R, N, seed=R + 11)
    es = 4 if dtype == "f32" else 2
    exp = D.allreduce(xs, dtype).view(np.uint8)
    out, sigs = _run(xs, dtype, repeats=2)
    for d in range(R):
        assert np.array_equal(out[d][:N * es], exp), d
        assert np.all(out[d][N * es:] == 0xCD)
    assert sigs == [2 * R] * R


def _tile(dtype):
    return 2048 if dtype == "f32" else 4096  # elements of a tile (8 KiB per rank)


def _form(dtype, R, N, send_off=0, recv_off=0):
    """The kernel form the library picks (its launch rule, restated)."""
    tile = _tile(dtype)
    per = -(-N // R)
    tpc = max(1, -(-per // tile))
    nwork = R * tpc
    aligned = (send_off | recv_off) % 16 == 0
    if aligned and R in (2, 4, 8, 16) and (tpc * min(R, 8)) % 64 == 0 and nwork >= 8192:
        return "split"
    if aligned and R in (2, 4, 8, 16) and N == R * tpc * tile and nwork % 8 == 0 and nwork >= 8192:
        return "loop"
    return "tile"


@pytest.mark.parametrize("dtype,R,tpc", [("bf16", 2, 32), ("bf16", 4, 16), ("bf16", 8, 8), ("f32", 4, 48),
                                         ("f32", 8, 24), ("bf16", 8, 72), ("f32", 2, 96)])
def test_allreduce_full_tiles_below_the_large_forms(dtype, R, tpc):
    # Whole, aligned tiles but fewer than 8192 of them: one tile per
    # workgroup, the XCD-aware order and the two-level relay; three calls in a
    # row bring every counter back to 0.
    N = R * tpc * _tile(dtype)
    say(f"allreduce full tiles {dtype} R={R} tiles per chunk {tpc} N={N}")
    xs = W.allreduce_f32_inputs(R, N, seed=R + tpc) if dtype == "f32" else W.allreduce_bf16_inputs(R, N, seed=R + tpc)
    es = 4 if dtype == "f32" else 2
    exp = D.allreduce(xs, dtype).view(np.uint8)
    out, sigs = _run(xs, dtype, repeats=3)
    for d in range(R):
        assert np.array_equal(out[d][:N * es], exp), d
        assert np.all(out[d][N * es:] == 0xCD)
    assert sigs == [3 * R] * R


@pytest.mark.parametrize("dtype,R,tpc", [("f32", 16, 514), ("bf16", 16, 513), ("f32", 4, 2050)])
def test_allreduce_looping_form(dtype, R, tpc):
    # Evenly tiled shapes with at least 8192 tiles that split over the 8 XCDs
    # but whose chunks do not split into a multiple of 64 pieces run the
    # looping form (4096 workgroups, each taking several slabs of its XCD's
    # range). R=16 crosses an owner chunk inside a workgroup's loop, R=4
    # spreads one chunk over two XCDs. Two calls in a row check that the
    # relay counters come back to 0.
    N = R * tpc * _tile(dtype)
    assert _form(dtype, R, N) == "loop"
    say(f"allreduce looping form {dtype} R={R} N={N}")
    xs = W.allreduce_f32_inputs(R, N, seed=R + 13) if dtype == "f32" else W.allreduce_bf16_inputs(R, N, seed=R + 13)
    es = 4 if dtype == "f32" else 2
    exp = D.allreduce(xs, dtype).view(np.uint8)
    out, sigs = _run(xs, dtype, repeats=2)
    for d in range(R):
        assert np.array_equal(out[d][:N * es], exp), d
        assert np.all(out[d][N * es:] == 0xCD)
    assert sigs == [2 * R] * R


@pytest.mark.parametrize("dtype,R,N,off", [("bf16", 8, (64 << 20) - 3, 0), ("f32", 4, (16 << 20) - 1000, 16),
                                         ("bf16", 2, 2 * 4096 * 4096 - 3 * 2048 - 7, 4096),
                                         ("f32", 8, (16 << 20) - 4 * 256 - 5, 0),
                                         ("bf16", 16, (32 << 20) - 3 * 512 - 1, 32)])
def test_allreduce_rank_split_form_ragged(dtype, R, N, off):
    # Counts that do not fill the last chunk: the piece holding the end is
    # summed element by element, the pieces past it (up to a few whole tiles'
    # worth) move nothing but still complete the relay. Two calls in a row.
    assert _form(dtype, R, N, off, off) == "split"
    say(f"allreduce rank-split form ragged {dtype} R={R} N={N} off={off}")
    xs = W.allreduce_f32_inputs(R, N, seed=R + N) if dtype == "f32" else W.allreduce_bf16_inputs(R, N, seed=R + N)
    es = 4 if dtype == "f32" else 2
    exp = D.allreduce(xs, dtype).view(np.uint8)
    out, sigs = _run(xs, dtype, send_off=off, recv_off=off, repeats=2)
    for d in range(R):
        assert np.array_equal(out[d][off:off + N * es], exp), d
        assert np.all(out[d][:off] == 0xCD) and np.all(out[d][off + N * es:] == 0xCD)
    assert sigs == [2 * R] * R


def test_allreduce_form_rule_covers_the_tested_shapes():
    # every form is exercised by the shapes above (the rule restated in _form)
    assert _form("bf16", 8, 64 << 20) == "split"
    assert _form("bf16", 16, 16 * 513 * 4096) == "loop"
    assert _form("bf16", 16, 32 << 20) == "split"
    assert _form("f32", 4, 4 * 2050 * 2048) == "loop"
    assert _form("f32", 4, 1 << 20) == "tile"
    assert _form("bf16", 8, 64 << 20, 8, 0) == "tile"
