"""Array arguments that the kernels would read or write are checked on the host:
a host pointer is refused before any launch (a device fault otherwise)."""
import numpy as np
import pytest

import collective_window_put_amd as vr
import workloads as W
from gpu_util import Job, say

pytestmark = pytest.mark.gpu


def _refused(fn):
    with pytest.raises(vr.VrError) as e:
        fn()
    assert e.value.code == vr.VR_ERR_INVALID_ARGUMENT


def test_dispatch_and_combine_refuse_host_arrays():
    import torch
    R, T, H, E, K = 2, 40, 8, 8, 2
    say("dispatch/combine array checks")
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=3)
    rb, cap = H * 2, R * T * K
    with Job(R, signal_count=4) as job:
        xw, _ = job.window(T * rb, arrays=[x[r] for r in range(R)])
        rw, _ = job.window(cap * rb, fill=0)
        tk = torch.from_numpy(topk).cuda()
        counts = torch.zeros(R, E // R, dtype=torch.int32, device="cuda")
        src = torch.zeros(R, cap, dtype=torch.int32, device="cuda")
        pos = torch.zeros(R, T, K, dtype=torch.int32, device="cuda")
        host_topk = torch.from_numpy(topk.copy())  # pageable host memory
        _refused(lambda: vr.vr_dispatch(job.comm, xw, 0, rb, host_topk, T, K, E, rw, 0, cap, counts, src, pos, 0, 1))
        _refused(lambda: vr.vr_dispatch(job.comm, xw, 0, rb, tk, T, K, E, rw, 0, cap, counts.cpu(), src, pos, 0, 1))
        _refused(lambda: vr.vr_dispatch(job.comm, xw, 0, rb, tk, T, K, E, rw, 0, cap, counts, src, pos.cpu(), 0, 1))
        # a correct call still works after the refusals
        vr.vr_dispatch(job.comm, xw, 0, rb, tk, T, K, E, rw, 0, cap, counts, src, pos, 0, 1)
        ow, _ = job.window(T * rb, fill=0)
        wts = torch.ones(R, T, K, dtype=torch.float32, device="cuda")
        _refused(lambda: vr.vr_combine(job.comm, rw, 0, cap, rb, vr.VR_DT_BF16, tk, torch.ones(R, T, K), pos, T, K,
                                       E, ow, 0, 2))
        _refused(lambda: vr.vr_combine(job.comm, rw, 0, cap, rb, vr.VR_DT_BF16, tk, wts, pos.cpu(), T, K, E, ow, 0, 2))
        vr.vr_combine(job.comm, rw, 0, cap, rb, vr.VR_DT_BF16, tk, wts, pos, T, K, E, ow, 0, 2)
        job.assert_no_async_error()


def test_ring_refuses_host_litmus_words():
    import torch
    R, P, pb, C = 2, 8, 16, 2
    say("ring litmus check")
    sends = W.ring_inputs(R, P, pb, seed=1)
    with Job(R, signal_count=C, counter_count=C, context_count=C) as job:
        sw, _ = job.window(P * pb, arrays=sends)
        rw, rv = job.window(P * pb, fill=0)
        _refused(lambda: vr.vr_ring_exchange(job.comm, sw, rw, pb, P, C, litmus=torch.zeros(2, dtype=torch.int64)))
        vr.vr_ring_exchange(job.comm, sw, rw, pb, P, C, litmus=torch.zeros(2, dtype=torch.int64, device="cuda"))
        out = job.host(rv)
        assert np.array_equal(out[1], sends[0][:P * pb]) and np.array_equal(out[0], sends[1][:P * pb])
        job.assert_no_async_error()


def test_calls_with_another_device_current_are_refused():
    # a communicator belongs to the device current at its creation; with
    # another device current every call but destroy is refused, and destroy
    # selects the device itself and gives the caller's back
    import torch
    if torch.cuda.device_count() < 2:
        pytest.skip("needs a second device to make current")
    say("calls with another device current")
    torch.cuda.set_device(0)
    job = Job(2, signal_count=2)
    w, views = job.window(1024, fill=0)
    try:
        torch.cuda.set_device(1)
        for fn in (lambda: vr.vr_put(job.comm, 0, 0, 1, w, 0, w, 0, 64),
                   lambda: vr.vr_signal_read(job.comm, 0, 0),
                   lambda: vr.vr_comm_get_async_error(job.comm)):
            with pytest.raises(vr.VrError) as e:
                fn()
            assert e.value.code == vr.VR_ERR_INVALID_USAGE
    finally:
        torch.cuda.set_device(0)
    vr.vr_window_deregister(job.comm, w)
    torch.cuda.set_device(1)
    vr.vr_comm_destroy(job.comm)
    assert torch.cuda.current_device() == 1
    torch.cuda.set_device(0)


def test_window_register_needs_one_base_per_rank():
    # the library reads exactly R base pointers; the binding refuses a list
    # of another length before the call
    import torch
    say("window register with a short base list")
    with Job(4) as job:
        slab = torch.empty(4 * 4096, dtype=torch.uint8, device="cuda")
        with pytest.raises(ValueError):
            vr.vr_window_register(job.comm, [slab.data_ptr()] * 3, 4096)
