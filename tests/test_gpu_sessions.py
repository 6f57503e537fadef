"""Barrier sessions and the AlltoAll in the pages' entry/exit-barrier structure, on the GPU.

GIN page, ncclGinBarrierSession: a sync releases its members once all have
arrived; the pure-GIN AlltoAll example enters and leaves through syncs. The
AlltoAll result and signal totals are checked against the oracle's plain
definition; the slot's arrivals against the host's expectation.
"""
import ctypes

import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import definitions as D
import workloads as W
from gpu_util import say

pytestmark = pytest.mark.gpu


def _slot_value(comm, index):
    import torch
    torch.cuda.synchronize()
    view = vr.vr_comm_device_view(comm)
    hip = ctypes.CDLL("libamdhip64.so")
    out = ctypes.c_uint64()
    assert hip.hipMemcpy(ctypes.byref(out), ctypes.c_void_p(view.barriers + 8 * index), ctypes.c_size_t(8), 2) == 0
    return out.value


def test_barrier_syncs_count_arrivals():
    say("barrier sessions: repeated syncs, every fence level")
    import torch
    comm = vr.vr_comm_create(5, 1, 1, 1, barrier_count=3)
    try:
        for fence in (vr.VR_FENCE_NONE, vr.VR_FENCE_PUT, vr.VR_FENCE_GET, vr.VR_FENCE_PUT | vr.VR_FENCE_GET):
            vr.vr_barrier(comm, 2, fence)
        vr.vr_barrier(comm, 0)
        torch.cuda.synchronize()
        assert vr.vr_barrier_expected(comm, 2) == 4 * 5 and _slot_value(comm, 2) == 20
        assert vr.vr_barrier_expected(comm, 0) == 5 and _slot_value(comm, 0) == 5
        assert vr.vr_barrier_expected(comm, 1) == 0 and _slot_value(comm, 1) == 0
        assert vr.vr_comm_get_async_error(comm)[0] == vr.VR_OK
        with pytest.raises(vr.VrError):
            vr.vr_barrier(comm, 3)  # no such slot
        with pytest.raises(vr.VrError):
            vr.vr_barrier(comm, 0, fence=4)
    finally:
        vr.vr_comm_destroy(comm)


def test_barrier_timeout_when_a_member_is_missing():
    # the host expects one arrival more than the R members make: the sync times out (1 ms)
    say("barrier session timeout")
    comm = vr.vr_comm_create(3, 1, 1, 1, barrier_count=1)
    try:
        vr.vr_barrier_advance(comm, 0, 1)
        vr.vr_barrier(comm, 0, vr.VR_FENCE_NONE, timeout_ns=1_000_000)
        code, bits = vr.vr_comm_get_async_error(comm)
        assert code == vr.VR_ERR_TIMEOUT and bits & vr.VR_ASYNC_TIMEOUT
    finally:
        vr.vr_comm_destroy(comm)


def _alltoall_sessions(R, B, seed, repeats=1, extra_barriers=0):
    sends = W.alltoall_inputs(R, B, seed=seed)
    import torch
    comm = vr.vr_comm_create(R, 2, 1, 1, barrier_count=2)
    try:
        a = vr.VR_WIN_REQUIRED_ALIGNMENT
        stride = (R * B + a - 1) // a * a
        slab = torch.empty(2 * R * stride + a, dtype=torch.uint8, device="cuda")
        sh = (-slab.data_ptr()) % a
        sv = [slab[sh + r * stride: sh + r * stride + R * B] for r in range(R)]
        rv = [slab[sh + (R + r) * stride: sh + (R + r) * stride + R * B] for r in range(R)]
        for v, x in zip(sv, sends):
            v.copy_(torch.from_numpy(np.ascontiguousarray(x).reshape(-1).view(np.uint8)))
        for v in rv:
            v.fill_(0xCD)
        sw = vr.vr_window_register(comm, [v.data_ptr() for v in sv], R * B)
        rw = vr.vr_window_register(comm, [v.data_ptr() for v in rv], R * B)
        for i in range(repeats):
            vr.vr_alltoall_sessions(comm, sw, 0, rw, 0, B, sig=1, barrier_index=1)
            for _ in range(extra_barriers):
                vr.vr_barrier(comm, 1)
        torch.cuda.synchronize()
        out = [v.cpu().numpy() for v in rv]
        sigs = [vr.vr_signal_read(comm, d, 1) for d in range(R)]
        res = dict(out=out, sigs=sigs, slot=_slot_value(comm, 1), expected=vr.vr_barrier_expected(comm, 1),
                   err=vr.vr_comm_get_async_error(comm))
        vr.vr_window_deregister(comm, sw)
        vr.vr_window_deregister(comm, rw)
    finally:
        vr.vr_comm_destroy(comm)
    return sends, res


@pytest.mark.parametrize("R,B", [(2, 16), (3, 1000), (4, 32768), (8, 100003), (5, 65536 * 3 + 17), (64, 200)])
def test_alltoall_sessions_vs_oracle(R, B):
    say(f"alltoall with barrier sessions R={R} B={B}")
    sends, res = _alltoall_sessions(R, B, seed=R * 31 + B)
    want = D.alltoall(sends, B)
    for d in range(R):
        assert np.array_equal(res["out"][d], want[d]), d
    assert res["sigs"] == [D.signal_increment("alltoall", R)] * R
    assert res["slot"] == res["expected"] == 2 * R
    assert res["err"][0] == vr.VR_OK


def test_alltoall_sessions_repeated_and_mixed_with_barriers():
    R, B = 4, 4096
    say("alltoall sessions x3 with a barrier after each")
    sends, res = _alltoall_sessions(R, B, seed=7, repeats=3, extra_barriers=1)
    want = D.alltoall(sends, B)
    assert all(np.array_equal(res["out"][d], want[d]) for d in range(R))
    assert res["sigs"] == [3 * R] * R
    assert res["slot"] == res["expected"] == 3 * (2 * R + R)
    assert res["err"][0] == vr.VR_OK


def test_alltoall_sessions_r8_4MiB_full_size():
    c = W.CONFIGS["alltoall_r8_4MiB"]
    say("alltoall sessions full size R=8 4 MiB blocks")
    sends, res = _alltoall_sessions(c["ranks"], c["block_bytes"], seed=c["seed"])
    want = D.alltoall(sends, c["block_bytes"])
    for d in range(c["ranks"]):
        assert np.array_equal(res["out"][d], want[d]), d
    assert res["err"][0] == vr.VR_OK
