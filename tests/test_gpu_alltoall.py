"""AlltoAll on the GPU against the oracle: bit-exact bytes, exact signal totals."""
import json

import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import definitions as D
import workloads as W
from conftest import golden
from gpu_util import Job, say

pytestmark = pytest.mark.gpu


def _run(R, B, sends, send_off=0, recv_off=0, repeats=1, sig=3, flags=0):
    with Job(R) as job:
        sw, sv = job.window(send_off + R * B, fill=0)
        rw, rv = job.window(recv_off + R * B, fill=0xAB)
        for r in range(R):
            sv[r][send_off:].copy_(job.torch.from_numpy(sends[r]))
        for rep in range(repeats):
            vr.vr_alltoall(job.comm, sw, send_off, rw, recv_off, B, sig=sig, flags=flags)
        out = job.host(rv)
        sigs = [job.sig(d, sig) for d in range(R)]
        job.assert_no_async_error()
        return out, sigs


def test_alltoall_page_fill_pattern():
    g = json.load(open(golden("alltoall_fill.json")))
    R, count = 4, 1000
    sends = [np.concatenate([np.array([s * 1000 + d * 100 + i for i in range(count)], np.int32)
                             for d in range(R)]).view(np.uint8) for s in range(R)]
    say("alltoall page fill R=4 count=1000")
    out, sigs = _run(R, count * 4, sends)
    for d in range(R):
        got = out[d].view(np.int32).reshape(R, count)
        for s in range(R):
            assert np.array_equal(got[s], s * g["fill"]["rank_weight"] + d * g["fill"]["dest_weight"]
                                  + np.arange(count))
    assert sigs == [R] * R


@pytest.mark.parametrize("R,B", [(1, 64), (2, 1), (3, 17), (4, 4096), (5, 16385), (8, 65536 + 48), (16, 1000),
                                 (64, 300)])
def test_alltoall_random_bytes_vs_oracle(R, B):
    say(f"alltoall R={R} B={B}")
    sends = W.alltoall_inputs(R, B, seed=R * 7 + B)
    out, sigs = _run(R, B, sends)
    exp = D.alltoall(sends, B)
    for d in range(R):
        assert np.array_equal(out[d], exp[d]), d
    assert sigs == [R] * R


@pytest.mark.parametrize("send_off,recv_off", [(16, 32), (3, 5), (4096, 1)])
def test_alltoall_offsets(send_off, recv_off):
    R, B = 4, 5000
    say(f"alltoall offsets {send_off} {recv_off}")
    sends = W.alltoall_inputs(R, B, seed=9)
    out, _ = _run(R, B, sends, send_off, recv_off)
    exp = D.alltoall(sends, B)
    for d in range(R):
        assert np.array_equal(out[d][recv_off:], exp[d])
        assert np.all(out[d][:recv_off] == 0xAB)


def test_alltoall_repeated_signal_accumulates():
    R, B = 3, 256
    say("alltoall repeated x5")
    sends = W.alltoall_inputs(R, B, seed=1)
    out, sigs = _run(R, B, sends, repeats=5)
    assert sigs == [5 * R] * R


def test_alltoall_full_size_config():
    c = W.CONFIGS["alltoall_r8_4MiB"]
    R, B = c["ranks"], c["block_bytes"]
    say(f"alltoall full R={R} B={B}")
    sends = W.alltoall_inputs(R, B, seed=c["seed"])
    out, sigs = _run(R, B, sends)
    exp = D.alltoall(sends, B)
    for d in range(R):
        assert np.array_equal(out[d], exp[d]), d
    assert sigs == [R] * R


@pytest.mark.parametrize("R,B,send_off,recv_off", [(2, 1, 0, 0), (4, 4096, 0, 0), (5, 16385, 3, 7),
                                                   (8, 65536 + 48, 16, 0), (16, 1000, 0, 5)])
def test_alltoall_copy_engine_vs_oracle(R, B, send_off, recv_off):
    say(f"alltoall copy engine R={R} B={B} offsets {send_off},{recv_off}")
    sends = W.alltoall_inputs(R, B, seed=R * 11 + B)
    out, sigs = _run(R, B, sends, send_off, recv_off, repeats=2, flags=vr.VR_COLL_COPY_ENGINE)
    exp = D.alltoall(sends, B)
    for d in range(R):
        assert np.array_equal(out[d][recv_off:], exp[d]), d
        assert np.all(out[d][:recv_off] == 0xAB)
    assert sigs == [2 * R] * R
