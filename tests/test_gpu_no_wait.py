"""Collectives launched with VR_COLL_NO_WAIT: no in-kernel receiver waits.

The signals are still applied, so a stream-ordered vr_signal_wait per rank
afterwards must see each documented total, and the data must equal the
oracle's, exactly as with the in-kernel waits.
"""
import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import definitions as D
import workloads as W
from gpu_util import Job, say

pytestmark = pytest.mark.gpu

TIMEOUT_NS = 2_000_000_000


def _wait_all(job, sig, least):
    for d in range(job.R):
        vr.vr_signal_wait(job.comm, d, sig, least, timeout_ns=TIMEOUT_NS)


@pytest.mark.parametrize("dtype,R,N,send_off,recv_off", [
    ("bf16", 8, 32 << 20, 4096, 16),   # rank-split form, offset windows
    ("f32", 4, 4 * 2050 * 2048, 4096, 16),  # looping form (8200 tiles, not a multiple of 64)
    ("f32", 4, 100003, 0, 0),          # one tile per workgroup, ragged
])
def test_allreduce_no_wait(dtype, R, N, send_off, recv_off):
    say(f"allreduce no-wait {dtype} R={R} N={N} offs={send_off},{recv_off}")
    es = 4 if dtype == "f32" else 2
    xs = W.allreduce_f32_inputs(R, N, seed=R + 5) if dtype == "f32" else W.allreduce_bf16_inputs(R, N, seed=R + 5)
    exp = D.allreduce(xs, dtype).view(np.uint8)
    dt = vr.VR_DT_F32 if dtype == "f32" else vr.VR_DT_BF16
    with Job(R) as job:
        sw, sv = job.window(send_off + N * es, fill=0)
        rw, rv = job.window(recv_off + N * es + 16, fill=0xCD)
        for r in range(R):
            sv[r][send_off:].copy_(job.torch.from_numpy(xs[r].view(np.uint8)))
        vr.vr_allreduce(job.comm, sw, send_off, rw, recv_off, N, dt, sig=3, flags=vr.VR_COLL_NO_WAIT)
        _wait_all(job, 3, R)
        out = job.host(rv)
        sigs = [job.sig(d, 3) for d in range(R)]
        job.assert_no_async_error()
    for d in range(R):
        assert np.array_equal(out[d][recv_off:recv_off + N * es], exp), d
        assert np.all(out[d][:recv_off] == 0xCD) and np.all(out[d][recv_off + N * es:] == 0xCD)
    assert sigs == [R] * R


def test_alltoall_no_wait():
    R, B = 8, (1 << 20) + 48
    say(f"alltoall no-wait R={R} B={B}")
    sends = W.alltoall_inputs(R, B, seed=9)
    exp = D.alltoall(sends, B)
    with Job(R) as job:
        sw, _ = job.window(R * B, arrays=sends)
        rw, rv = job.window(R * B, fill=0)
        vr.vr_alltoall(job.comm, sw, 0, rw, 0, B, sig=2, flags=vr.VR_COLL_NO_WAIT)
        _wait_all(job, 2, R)
        out = job.host(rv)
        sigs = [job.sig(d, 2) for d in range(R)]
        job.assert_no_async_error()
    for d in range(R):
        assert np.array_equal(out[d], exp[d]), d
    assert sigs == [R] * R


@pytest.mark.parametrize("M", [(2 << 20) + 4096 * 3, 2 << 20])  # tile form, piece form
def test_allgather_no_wait(M):
    R = 16
    say(f"allgather no-wait R={R} M={M}")
    sends = W.allgather_inputs(R, M, seed=4)
    exp = D.allgather(sends)
    with Job(R) as job:
        sw, _ = job.window(M, arrays=sends)
        rw, rv = job.window(R * M, fill=0x5A)
        vr.vr_allgather(job.comm, sw, 0, rw, 0, M, sig=1, flags=vr.VR_COLL_NO_WAIT)
        _wait_all(job, 1, R)
        out = job.host(rv)
        sigs = [job.sig(d, 1) for d in range(R)]
        job.assert_no_async_error()
    for d in range(R):
        assert np.array_equal(out[d], exp[d]), d
    assert sigs == [R] * R


def test_dispatch_no_wait():
    import torch
    R, T, H, E, K = 8, 300, 256, 64, 4
    say(f"dispatch no-wait R={R} T={T} E={E} K={K}")
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=12)
    rb = H * 2
    cap = R * T * K
    rows, tags, cnts, _ = D.dispatch(topk, x, E, cap)
    with Job(R) as job:
        xw, _ = job.window(T * rb, arrays=[x[r].reshape(-1).view(np.uint8) for r in range(R)])
        rw, rv = job.window(cap * rb, fill=0xEE)
        tk = torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32)).cuda()
        counts = torch.zeros(R, E // R, dtype=torch.int32, device="cuda")
        src = torch.full((R, cap), -1, dtype=torch.int32, device="cuda")
        vr.vr_dispatch(job.comm, xw, 0, rb, tk, T, K, E, rw, 0, cap, counts, src, None, 4, 5,
                       flags=vr.VR_COLL_NO_WAIT)
        _wait_all(job, 4, R)
        for d in range(R):
            vr.vr_signal_wait(job.comm, d, 5, rows[d].shape[0], timeout_ns=TIMEOUT_NS)
        out = job.host(rv)
        sig_rows = [job.sig(d, 5) for d in range(R)]
        sig_counts = [job.sig(d, 4) for d in range(R)]
        srch, cnth = src.cpu().numpy(), counts.cpu().numpy()
        job.assert_no_async_error()
    for d in range(R):
        n = rows[d].shape[0]
        assert np.array_equal(out[d][:n * rb], rows[d].reshape(-1)), d
        assert np.array_equal(srch[d, :n], tags[d]), d
        assert np.array_equal(cnth[d], cnts[d]), d
        assert sig_rows[d] == n
    assert sig_counts == [R] * R
