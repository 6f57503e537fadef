"""put / get / signal / wait / counters on the GPU against the oracle's sequential semantics."""
import itertools

import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import primitives as P
from gpu_util import Job, say

pytestmark = pytest.mark.gpu


def test_put_get_brute_force_small_ranges():
    # every (src off, dst off, size) on a 24-byte window, 2 ranks, vs the oracle
    size = 24
    say("put/get brute force 24-byte windows")
    rng = np.random.default_rng(0)
    init = [rng.integers(0, 256, size, dtype=np.uint8) for _ in range(2)]
    cases = [(so, do, n) for so, do, n in itertools.product(range(0, 24, 5), range(0, 24, 3), [0, 1, 7, 16, 17])
             if so + n <= size and do + n <= size]
    with Job(2, signal_count=2, counter_count=2) as job:
        sw, sv = job.window(size, arrays=init)
        dw, dv = job.window(size, fill=0)
        ow = P.World(2, signal_count=2, counter_count=2)
        os_ = ow.register([a.copy() for a in init])
        od = ow.register_zeros(size)
        for i, (so, do, n) in enumerate(cases):
            if i % 2:
                vr.vr_put(job.comm, 0, 0, 1, dw, do, sw, so, n, vr.SignalInc(1), vr.CounterInc(0))
                ow.put(0, 1, od, do, os_, so, n, P.SignalInc(1), P.CounterInc(0))
            else:
                vr.vr_get(job.comm, 0, 1, 0, sw, so, dw, do, n, vr.CounterInc(1))
                ow.get(1, 0, os_, so, od, do, n, P.CounterInc(1))
        out = job.host(dv)
        for r in range(2):
            assert np.array_equal(out[r], ow.buf(od, r)), r
        assert job.sig(1, 1) == ow.read_signal(1, 1)
        assert job.cnt(0, 0) == ow.read_counter(0, 0) and job.cnt(1, 1) == ow.read_counter(1, 1)
        job.assert_no_async_error()


@pytest.mark.parametrize("n", [1, 100, 4096, 4097, 5 * 4096 + 33, 15 * 4096 + 1, 16 * 4096, 21 * 4096 + 5,
                               70 * 4096 - 3, 1 << 22, 16384 * 4096 + 16])
def test_put_multi_workgroup_with_signal(n):
    say(f"put {n} bytes")
    rng = np.random.default_rng(n)
    with Job(3, signal_count=4, counter_count=4) as job:
        src = [rng.integers(0, 256, n + 8, dtype=np.uint8) for _ in range(3)]
        sw, _ = job.window(n + 8, arrays=src)
        dw, dv = job.window(n + 8, fill=0)
        vr.vr_put(job.comm, 0, 2, 0, dw, 8, sw, 3, n, vr.SignalAdd(3, 1000), vr.CounterInc(2))
        out = job.host(dv)
        assert np.array_equal(out[0][8:], src[2][3:3 + n])
        assert np.all(out[1] == 0) and np.all(out[2] == 0)
        assert job.sig(0, 3) == 1000 and job.cnt(2, 2) == 1
        assert vr.vr_signal_expected(job.comm, 0, 3) == 1000
        job.assert_no_async_error()


def test_large_puts_back_to_back_each_signal_once():
    """Puts of 16 tiles (4 KiB each) or more count their tiles in three relay
    levels (per XCD and first-level counter, per XCD, then the XCDs): every
    counter must be back at zero for the next put (sizes 22, 16, 300, 70 and
    1201 tiles, some leaving first-level counters unused)."""
    say("large puts back to back")
    rng = np.random.default_rng(5)
    sizes = [21 * 4096 + 5, 16 * 4096, 300 * 4096 - 7, 70 * 4096, 1201 * 4096 - 1]
    n = max(sizes)
    with Job(2, signal_count=2, counter_count=2) as job:
        src = [rng.integers(0, 256, n, dtype=np.uint8) for _ in range(2)]
        sw, _ = job.window(n, arrays=src)
        dw, dv = job.window(n, fill=0)
        for m in sizes:
            vr.vr_put(job.comm, 0, 0, 1, dw, 0, sw, 0, m, vr.SignalInc(1), vr.CounterInc(0))
            vr.vr_get(job.comm, 0, 0, 1, sw, 0, dw, 0, m, vr.CounterInc(1))
        out = job.host(dv)
        assert np.array_equal(out[1], src[0]) and np.array_equal(out[0], src[1])
        assert job.sig(1, 1) == len(sizes) and job.cnt(0, 0) == len(sizes) and job.cnt(0, 1) == len(sizes)
        job.assert_no_async_error()


@pytest.mark.parametrize("shift", [-1000, -1, 1, 17, 4096, 30000])
def test_overlapping_loopback_put_is_memmove(shift):
    n, size = 20000, 80000
    say(f"loopback overlap shift={shift}")
    rng = np.random.default_rng(abs(shift))
    init = [rng.integers(0, 256, size, dtype=np.uint8)]
    so = 20000
    do = so + shift
    with Job(1) as job:
        w, v = job.window(size, arrays=init)
        vr.vr_put(job.comm, 0, 0, 0, w, do, w, so, n)
        out = job.host(v)[0]
        ow = P.World(1)
        h = ow.register([init[0].copy()])
        ow.put(0, 0, h, do, h, so, n)
        assert np.array_equal(out, ow.buf(h, 0))


def test_signal_wait_and_rolling_wrap():
    say("signal wrap")
    with Job(2, signal_count=2) as job:
        base = (1 << 64) - 3
        vr.vr_signal(job.comm, 0, 0, 1, vr.SignalAdd(1, base))
        for _ in range(5):
            vr.vr_signal(job.comm, 0, 0, 1, vr.SignalAdd(1, 1))
        vr.vr_signal_wait(job.comm, 1, 1, (base + 5) % (1 << 64), timeout_ns=10 ** 9)
        assert job.sig(1, 1) == 2
        assert vr.vr_signal_read(job.comm, 1, 1, bits=1) == 0
        job.assert_no_async_error()
        vr.vr_signal_reset(job.comm, 1, 1)
        assert job.sig(1, 1) == 0
        assert vr.vr_signal_expected(job.comm, 1, 1) == 0


def test_wait_timeout_sets_async_error():
    say("wait timeout (20 ms)")
    with Job(1, signal_count=1, counter_count=1) as job:
        vr.vr_signal_wait(job.comm, 0, 0, 1, timeout_ns=20_000_000)
        code, bits = job.async_error()
        assert code == vr.VR_ERR_TIMEOUT and bits & vr.VR_ASYNC_TIMEOUT
        vr.vr_counter_wait(job.comm, 0, 0, 5, timeout_ns=20_000_000)
        assert job.async_error()[0] == vr.VR_ERR_TIMEOUT
        assert job.async_error()[0] == vr.VR_OK  # reading clears


def test_counter_wraps_at_56_bits_and_waits():
    say("counter 56-bit")
    with Job(1, signal_count=1, counter_count=1) as job:
        w, _ = job.window(64, fill=1)
        for _ in range(3):
            vr.vr_put(job.comm, 0, 0, 0, w, 32, w, 0, 16, None, vr.CounterInc(0))
        vr.vr_counter_wait(job.comm, 0, 0, 3, timeout_ns=10 ** 9)
        assert job.cnt(0, 0) == 3
        vr.vr_counter_reset(job.comm, 0, 0)
        assert job.cnt(0, 0) == 0
        job.assert_no_async_error()


def test_usage_errors():
    say("usage errors")
    with Job(2, signal_count=2, counter_count=1, context_count=2) as job:
        w, _ = job.window(4096, fill=0)
        vr.vr_signal(job.comm, 0, 0, 1, vr.SignalInc(0))
        with pytest.raises(vr.VrError) as e:  # Inc then Add without a reset
            vr.vr_signal(job.comm, 0, 0, 1, vr.SignalAdd(0, 2))
        assert e.value.code == vr.VR_ERR_INVALID_USAGE
        with pytest.raises(vr.VrError) as e:
            vr.vr_put(job.comm, 0, 0, 1, w, 4000, w, 0, 100)
        assert e.value.code == vr.VR_ERR_INVALID_ARGUMENT
        with pytest.raises(vr.VrError) as e:
            vr.vr_put(job.comm, 2, 0, 1, w, 0, w, 0, 1)  # context out of range
        assert e.value.code == vr.VR_ERR_INVALID_ARGUMENT
        with pytest.raises(vr.VrError) as e:
            vr.vr_put(job.comm, 0, 0, 2, w, 0, w, 0, 1)  # peer out of range
        assert e.value.code == vr.VR_ERR_INVALID_ARGUMENT
        with pytest.raises(vr.VrError) as e:
            vr.vr_comm_destroy(job.comm)  # windows still registered
        assert e.value.code == vr.VR_ERR_INVALID_USAGE
        import torch
        t = torch.empty(8192 + 4096, dtype=torch.uint8, device="cuda")
        p = t.data_ptr() + (-t.data_ptr()) % 4096
        with pytest.raises(vr.VrError):  # misaligned base
            vr.vr_window_register(job.comm, [p + 1, p + 4096], 100)
        with pytest.raises(vr.VrError):  # overlapping rank slices
            vr.vr_window_register(job.comm, [p, p], 100)
        with pytest.raises(vr.VrError):  # past the end of the allocation
            vr.vr_window_register(job.comm, [p, p + (1 << 45)], 1 << 45)
        job.assert_no_async_error()


def test_caller_workspace_and_two_communicators_on_two_streams():
    # each communicator owns its signal, counter and relay words (here one in
    # a caller-provided workspace), so two of them can run AlltoAlls on two
    # streams at once without sharing any word
    import torch
    from oracle import definitions as D
    import workloads as W
    say("two communicators, two streams, caller workspace")
    R, B = 4, 1 << 16
    need = vr.vr_comm_workspace_bytes(R, signal_count=2, counter_count=1)
    ws = torch.zeros(need + 256, dtype=torch.uint8, device="cuda")
    off = (-ws.data_ptr()) % 256
    comms = [vr.vr_comm_create(R, 2, 1, 1, workspace=ws.data_ptr() + off, workspace_bytes=need),
             vr.vr_comm_create(R, 2, 1, 1)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    sends = [W.alltoall_inputs(R, B, seed=41), W.alltoall_inputs(R, B, seed=42)]
    slabs, wins = [], []
    try:
        for i, comm in enumerate(comms):
            a = vr.VR_WIN_REQUIRED_ALIGNMENT
            slab = torch.zeros(2 * R * R * B + a, dtype=torch.uint8, device="cuda")
            sh = (-slab.data_ptr()) % a
            sv = [slab[sh + r * R * B: sh + (r + 1) * R * B] for r in range(R)]
            rv = [slab[sh + (R + r) * R * B: sh + (R + r + 1) * R * B] for r in range(R)]
            for v, x in zip(sv, sends[i]):
                v.copy_(torch.from_numpy(x))
            sw = vr.vr_window_register(comm, [v.data_ptr() for v in sv], R * B)
            rw = vr.vr_window_register(comm, [v.data_ptr() for v in rv], R * B)
            slabs.append((slab, rv))
            wins.append((sw, rw))
        torch.cuda.synchronize()
        for rep in range(3):
            for i, comm in enumerate(comms):
                vr.vr_alltoall(comm, wins[i][0], 0, wins[i][1], 0, B, sig=1, stream=streams[i])
        torch.cuda.synchronize()
        for i, comm in enumerate(comms):
            want = D.alltoall(sends[i], B)
            got = [v.cpu().numpy() for v in slabs[i][1]]
            assert all(np.array_equal(got[d], want[d]) for d in range(R)), i
            assert [vr.vr_signal_read(comm, d, 1) for d in range(R)] == [3 * R] * R
            assert vr.vr_comm_get_async_error(comm)[0] == vr.VR_OK
    finally:
        torch.cuda.synchronize()
        for comm, (sw, rw) in zip(comms, wins):
            vr.vr_window_deregister(comm, sw)
            vr.vr_window_deregister(comm, rw)
        for comm in comms:
            vr.vr_comm_destroy(comm)
