"""AllGather on the GPU against the oracle."""
import json

import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import definitions as D
import workloads as W
from conftest import golden
from gpu_util import Job, say

pytestmark = pytest.mark.gpu


def _run(sends, M, send_off=0, recv_off=0, sig=1, flags=0):
    R = len(sends)
    with Job(R) as job:
        sw, sv = job.window(send_off + M, fill=0)
        rw, rv = job.window(recv_off + R * M, fill=0x5A)
        for r in range(R):
            sv[r][send_off:].copy_(job.torch.from_numpy(sends[r]))
        vr.vr_allgather(job.comm, sw, send_off, rw, recv_off, M, sig=sig, flags=flags)
        out = job.host(rv)
        sigs = [job.sig(d, sig) for d in range(R)]
        job.assert_no_async_error()
    return out, sigs


def test_allgather_page_segments():
    g = json.load(open(golden("allgather_segments.json")))
    R, n = g["ranks"], g["send_bytes"] // 4
    say("allgather page segments R=4 4MB")
    sends = [np.full(n, float(r), np.float32).view(np.uint8) for r in range(R)]
    out, sigs = _run(sends, g["send_bytes"])
    for d in range(R):
        assert out[d].nbytes == g["recv_bytes"]
        segs = out[d].view(np.float32).reshape(R, n)
        for k, v in enumerate(g["segment_values"]):
            assert np.all(segs[k] == np.float32(v))
    assert sigs == [R] * R


@pytest.mark.parametrize("R,M", [(1, 16), (2, 1), (3, 16385), (4, 16384 * 3), (8, 1000), (16, 32768 + 16), (5, 77),
                                 (64, 5000)])
def test_allgather_random_vs_oracle(R, M):
    say(f"allgather R={R} M={M}")
    sends = W.allgather_inputs(R, M, seed=R * 3 + M)
    out, sigs = _run(sends, M)
    exp = D.allgather(sends)
    for d in range(R):
        assert np.array_equal(out[d], exp[d]), d
    assert sigs == [R] * R


def test_allgather_offsets():
    R, M = 4, 20000
    say("allgather offsets")
    sends = W.allgather_inputs(R, M, seed=2)
    out, _ = _run(sends, M, send_off=7, recv_off=4096 + 3)
    exp = D.allgather(sends)
    for d in range(R):
        assert np.array_equal(out[d][4099:], exp[d])
        assert np.all(out[d][:4099] == 0x5A)


def test_allgather_r16_64MiB_full_size():
    c = W.CONFIGS["allgather_r16_64MiB"]
    R, M = c["ranks"], c["bytes_per_rank"]
    say(f"allgather full size R={R} M={M}")
    sends = W.allgather_inputs(R, M, seed=c["seed"])
    with Job(R) as job:
        sw, sv = job.window(M, fill=None, arrays=sends)
        rw, rv = job.window(R * M, fill=None)
        vr.vr_allgather(job.comm, sw, 0, rw, 0, M, sig=0)
        job.torch.cuda.synchronize()
        for d in range(R):  # one destination at a time: 1 GiB each
            got = rv[d].cpu().numpy()
            assert np.array_equal(got, D.allgather_for_rank(sends, d)), d
            del got
        assert [job.sig(d, 0) for d in range(R)] == [R] * R
        job.assert_no_async_error()


@pytest.mark.parametrize("R,M,send_off,recv_off", [(2, 1, 0, 0), (3, 16385, 7, 3), (8, 1 << 20, 0, 0),
                                                   (16, 32768 + 16, 16, 4096)])
def test_allgather_copy_engine_vs_oracle(R, M, send_off, recv_off):
    say(f"allgather copy engine R={R} M={M}")
    sends = W.allgather_inputs(R, M, seed=R * 5 + M)
    out, sigs = _run(sends, M, send_off, recv_off, flags=vr.VR_COLL_COPY_ENGINE)
    exp = D.allgather(sends)
    for d in range(R):
        assert np.array_equal(out[d][recv_off:], exp[d]), d
        assert np.all(out[d][:recv_off] == 0x5A)
    assert sigs == [R] * R


@pytest.mark.parametrize("R,M", [(16, 2 << 20), (8, (4 << 20) + 3 * 4096), (4, 8 << 20)])
def test_allgather_whole_tiles_twice(R, M):
    # Shapes of whole 4 KiB tiles, 512 to 2051 tiles per source (all of them
    # run the piece form, 1 KiB pieces); two calls in a row check that every
    # relay counter comes back to 0.
    say(f"allgather whole tiles twice R={R} M={M}")
    sends = W.allgather_inputs(R, M, seed=R + M)
    exp = D.allgather(sends)
    with Job(R) as job:
        sw, sv = job.window(M, arrays=sends)
        rw, rv = job.window(R * M, fill=0x5A)
        for _ in range(2):
            vr.vr_allgather(job.comm, sw, 0, rw, 0, M, sig=1)
        out = job.host(rv)
        sigs = [job.sig(d, 1) for d in range(R)]
        job.assert_no_async_error()
    for d in range(R):
        assert np.array_equal(out[d], exp[d]), d
    assert sigs == [2 * R] * R


PIECE_CASES = [(1, 64 << 10, 0, 0), (2, 128 << 10, 16, 4096), (3, 5 * (64 << 10), 0, 16), (5, 3 * (64 << 10), 4096, 0),
               (8, 1 << 20, 0, 0), (16, 64 << 10, 32, 48), (64, 64 << 10, 0, 0), (3, (64 << 10) + 16, 0, 16),
               (16, 100000, 16, 32), (5, (2 << 20) + 1024 + 48, 4096, 0), (7, 200000 - 16 * 3, 0, 0)]


@pytest.mark.parametrize("R,M,send_off,recv_off", PIECE_CASES)
def test_allgather_piece_form(R, M, send_off, recv_off):
    # 16-byte aligned sizes of 64 KiB or more with aligned offsets run the
    # piece form (1 KiB of one source per workgroup, wave w storing to ranks
    # w, w + 4, ...; 64 pieces per source at least, so every first-level relay
    # counter has one); the last four end in a partial piece, so the counters
    # take unequal arrivals. Twice in a row: the counters come back to 0.
    say(f"allgather piece form R={R} M={M} offsets {send_off},{recv_off}")
    sends = W.allgather_inputs(R, M, seed=R * 7 + M)
    exp = D.allgather(sends)
    with Job(R) as job:
        sw, sv = job.window(send_off + M, fill=0)
        rw, rv = job.window(recv_off + R * M + 16, fill=0x5A)
        for r in range(R):
            sv[r][send_off:].copy_(job.torch.from_numpy(sends[r]))
        for _ in range(2):
            vr.vr_allgather(job.comm, sw, send_off, rw, recv_off, M, sig=1)
        out = job.host(rv)
        sigs = [job.sig(d, 1) for d in range(R)]
        job.assert_no_async_error()
    for d in range(R):
        assert np.array_equal(out[d][recv_off:recv_off + R * M], exp[d]), d
        assert np.all(out[d][:recv_off] == 0x5A) and np.all(out[d][recv_off + R * M:] == 0x5A)
    assert sigs == [2 * R] * R
