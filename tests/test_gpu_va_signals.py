"""VA signals (a signal word at a window offset) on the GPU against the oracle.

GIN page, VA signals: the window must carry strict ordering, Inc and Add
are not mixed without a reset, and a word in use as a signal is accessed by
signal operations only. Strong and weak signals are both published after
every earlier store of the issuing context, so the litmus runs expect the
strong prefix property for both.
"""
import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import definitions as D
from oracle import primitives as P
import workloads as W
from gpu_util import Job, say

pytestmark = pytest.mark.gpu
STRICT = vr.VR_WIN_STRICT_ORDERING


def _code(fn, *a, **k):
    try:
        fn(*a, **k)
    except vr.VrError as e:
        return e.code
    return vr.VR_OK


def test_va_signal_actions_match_the_oracle():
    say("VA signals: put/signal/reset sequence vs oracle")
    rng = np.random.default_rng(1)
    with Job(3, signal_count=2, counter_count=2) as job:
        src = [rng.integers(0, 256, 256, dtype=np.uint8) for _ in range(3)]
        sw, _ = job.window(256, arrays=src)
        dw, dv = job.window(256, fill=0)
        gw, gv = job.window(128, fill=0, flags=STRICT)
        ow = P.World(3, signal_count=2, counter_count=2)
        os_ = ow.register([a.copy() for a in src])
        od = ow.register_zeros(256)
        og = ow.register([np.zeros(128, np.uint8) for _ in range(3)], flags=P.WIN_STRICT_ORDERING)
        ops = [("put", 0, 1, 0, 64, 16, vr.VASignalInc(gw, 8), P.VASignalInc(og, 8)),
               ("put", 2, 1, 64, 0, 40, vr.VASignalInc(gw, 8, strong=False), P.VASignalInc(og, 8, False)),
               ("sig", 1, 0, 0, 0, 0, vr.VASignalAdd(gw, 120, 0xFFFFFFFFFFFFFFFE), P.VASignalAdd(og, 120, (1 << 64) - 2)),
               ("sig", 2, 0, 0, 0, 0, vr.VASignalAdd(gw, 120, 5), P.VASignalAdd(og, 120, 5)),
               ("put", 1, 2, 100, 7, 100, vr.VASignalAdd(gw, 0, 1 << 40), P.VASignalAdd(og, 0, 1 << 40)),
               ("reset", 1, None, 8), ("put", 0, 1, 200, 200, 56, vr.VASignalAdd(gw, 8, 3), P.VASignalAdd(og, 8, 3))]
        for op in ops:
            if op[0] == "put":
                _, r, p, so, do, n, a, oa = op
                vr.vr_put(job.comm, 0, r, p, dw, do, sw, so, n, a)
                ow.put(r, p, od, do, os_, so, n, oa)
            elif op[0] == "sig":
                _, r, p, _, _, _, a, oa = op
                vr.vr_signal(job.comm, 0, r, p, a)
                ow.signal(r, p, oa)
            else:
                _, r, _, off = op
                vr.vr_va_signal_reset(job.comm, gw, r, off)
                ow.reset_va_signal(r, og, off)
        data = job.host(dv)
        words = job.host(gv)
        for r in range(3):
            assert np.array_equal(data[r], ow.buf(od, r)), r
            assert np.array_equal(words[r], ow.buf(og, r)), r  # byte image of every word
            for off in (0, 8, 120):
                assert vr.vr_va_signal_read(job.comm, gw, r, off) == ow.read_va_signal(r, og, off)
        assert vr.vr_va_signal_read(job.comm, gw, 0, 120, bits=8) == 3
        job.assert_no_async_error()


def test_va_signal_usage_rules():
    say("VA signals: usage rules")
    with Job(2, signal_count=2) as job:
        sw, _ = job.window(4096, fill=1)
        plain, _ = job.window(64, fill=0)
        gw, _ = job.window(4096, fill=0, flags=STRICT)
        c = job.comm
        assert _code(vr.vr_signal, c, 0, 0, 1, vr.VASignalInc(plain, 0)) == vr.VR_ERR_INVALID_USAGE
        assert _code(vr.vr_signal, c, 0, 0, 1, vr.VASignalInc(gw, 4)) == vr.VR_ERR_INVALID_ARGUMENT
        assert _code(vr.vr_signal, c, 0, 0, 1, vr.VASignalInc(gw, 4096)) == vr.VR_ERR_INVALID_ARGUMENT
        assert _code(vr.vr_va_signal_wait, c, plain, 0, 0, 0) == vr.VR_ERR_INVALID_USAGE
        vr.vr_signal(c, 0, 0, 1, vr.VASignalInc(gw, 64))
        assert _code(vr.vr_signal, c, 0, 0, 1, vr.VASignalAdd(gw, 64, 2)) == vr.VR_ERR_INVALID_USAGE
        # plain data movement that touches the word (rank 1's slice, bytes 64..71) is refused
        assert _code(vr.vr_put, c, 0, 0, 1, gw, 57, sw, 0, 8) == vr.VR_ERR_INVALID_USAGE
        assert _code(vr.vr_get, c, 0, 0, 1, gw, 71, sw, 0, 1) == vr.VR_ERR_INVALID_USAGE
        assert _code(vr.vr_alltoall, c, gw, 0, sw, 0, 2048, 0) == vr.VR_ERR_INVALID_USAGE
        # a put whose own VA signal lies in its destination range is refused
        assert _code(vr.vr_put, c, 0, 0, 1, gw, 256, sw, 0, 64, vr.VASignalInc(gw, 288)) == vr.VR_ERR_INVALID_USAGE
        # neighbours of the word, and the same offset on another rank, are plain data
        vr.vr_put(c, 0, 0, 1, gw, 56, sw, 0, 8)
        vr.vr_put(c, 0, 0, 1, gw, 72, sw, 0, 8)
        vr.vr_put(c, 0, 1, 0, gw, 64, sw, 0, 8)
        vr.vr_va_signal_reset(c, gw, 1, 64)
        vr.vr_signal(c, 0, 0, 1, vr.VASignalAdd(gw, 64, 2))
        assert vr.vr_va_signal_read(c, gw, 1, 64) == 2
        job.assert_no_async_error()


def test_va_signal_wait_in_stream_and_timeout():
    say("VA signals: stream wait and timeout")
    with Job(2, signal_count=1) as job:
        sw, _ = job.window(1 << 20, fill=7)
        dw, dv = job.window(1 << 20, fill=0)
        gw, _ = job.window(4096, fill=0, flags=STRICT)
        c = job.comm
        vr.vr_put(c, 0, 0, 1, dw, 0, sw, 0, 1 << 20, vr.VASignalInc(gw, 0))
        vr.vr_va_signal_wait(c, gw, 1, 0, 1)
        assert np.all(job.host(dv)[1] == 7)
        job.assert_no_async_error()
        vr.vr_va_signal_wait(c, gw, 1, 0, 2, timeout_ns=2_000_000)  # never reached: times out after 2 ms
        code, bits = job.async_error()
        assert code == vr.VR_ERR_TIMEOUT and bits & vr.VR_ASYNC_TIMEOUT


@pytest.mark.parametrize("R,Pn,pb,C,litmus", [(3, 96, 256, 4, True), (4, 2048, 256, 16, True),
                                              (16, 4096, 256, 64, True), (4, 2048, 256, 16, False),
                                              (2, 400, 64, 100, False)])
def test_ring_with_va_signals_litmus(R, Pn, pb, C, litmus):
    import torch
    say(f"ring with VA signals R={R} P={Pn} pb={pb} C={C} litmus={litmus}")
    sends = W.ring_inputs(R, Pn, pb, seed=R * 7 + Pn)
    off = 4096  # the signal words live after the messages in the receive window
    with Job(R, signal_count=1, counter_count=C, context_count=C) as job:
        sw, _ = job.window(Pn * pb, fill=None, arrays=sends)
        rw, rv = job.window(off + Pn * pb, fill=0, flags=STRICT)
        lit = torch.zeros(2, dtype=torch.int64, device="cuda")
        # messages at [0, Pn*pb) of the receive window would cover the words at `off`: refused
        assert _code(vr.vr_ring_exchange, job.comm, sw, rw, pb, Pn, C, sig_window=rw, sig_window_off=0,
                     litmus=lit) == vr.VR_ERR_INVALID_USAGE
        gw, _ = job.window(8 * C, fill=0, flags=STRICT)
        vr.vr_ring_exchange(job.comm, sw, rw, pb, Pn, C, cnt_base=0, sig_window=gw, sig_window_off=0,
                            litmus=lit if litmus else None)
        out = job.host(rv)
        exp = D.ring(sends, [np.zeros(off + Pn * pb, np.uint8)] * R, Pn, pb)
        for d in range(R):
            assert np.array_equal(out[d], exp[d]), d
            for k in range(C):
                assert vr.vr_va_signal_read(job.comm, gw, d, 8 * k) == Pn // C
                assert vr.vr_counter_read(job.comm, d, k) == Pn // C
        lh = lit.cpu().numpy()
        assert lh[1] == 0 and (lh[0] > 0) == litmus
        job.assert_no_async_error()
