"""Zero-size collectives on the GPU: no byte moves, and every rank's signal
still rises by what the oracle says one collective adds."""
import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import definitions as D
from gpu_util import Job, say

pytestmark = pytest.mark.gpu

OPS = ["allreduce_f32", "allreduce_bf16", "alltoall", "alltoall_ce", "allgather", "allgather_ce"]


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("R", [1, 3, 8])
def test_zero_size_collective(R, op):
    say(f"zero-size {op} R={R}")
    with Job(R, signal_count=2) as job:
        sw, sv = job.window(256, fill=0x11)
        rw, rv = job.window(256, fill=0xAB)
        for rep in range(2):  # twice: the relay counters must be back at zero
            if op.startswith("allreduce"):
                dt = vr.VR_DT_F32 if op.endswith("f32") else vr.VR_DT_BF16
                vr.vr_allreduce(job.comm, sw, 16, rw, 32, 0, dt, sig=1)
            elif op.startswith("alltoall"):
                vr.vr_alltoall(job.comm, sw, 16, rw, 32, 0, sig=1,
                               flags=vr.VR_COLL_COPY_ENGINE if op.endswith("_ce") else 0)
            else:
                vr.vr_allgather(job.comm, sw, 16, rw, 32, 0, sig=1,
                                flags=vr.VR_COLL_COPY_ENGINE if op.endswith("_ce") else 0)
        ins, out = job.host(sv), job.host(rv)
        assert all(np.all(a == 0x11) for a in ins) and all(np.all(a == 0xAB) for a in out)
        kind = op.split("_")[0]
        assert [job.sig(d, 1) for d in range(R)] == [2 * D.signal_increment(kind, R)] * R
        job.assert_no_async_error()


@pytest.mark.parametrize("R", [1, 4])
def test_zero_size_alltoall_sessions(R):
    say(f"zero-size alltoall sessions R={R}")
    comm = vr.vr_comm_create(R, signal_count=2, barrier_count=1)
    import torch
    a = vr.VR_WIN_REQUIRED_ALIGNMENT
    slab = torch.full((2 * R * a + a,), 0x5A, dtype=torch.uint8, device="cuda")
    p = slab.data_ptr() + (-slab.data_ptr()) % a
    sw = vr.vr_window_register(comm, [p + r * a for r in range(R)], a)
    rw = vr.vr_window_register(comm, [p + (R + r) * a for r in range(R)], a)
    try:
        vr.vr_alltoall_sessions(comm, sw, 0, rw, 0, 0, sig=1, barrier_index=0)
        torch.cuda.synchronize()
        assert bool((slab == 0x5A).all())
        assert [vr.vr_signal_read(comm, d, 1) for d in range(R)] == [D.signal_increment("alltoall", R)] * R
        assert vr.vr_barrier_expected(comm, 0) == 2 * R
        assert vr.vr_comm_get_async_error(comm)[0] == vr.VR_OK
    finally:
        torch.cuda.synchronize()
        vr.vr_window_deregister(comm, sw)
        vr.vr_window_deregister(comm, rw)
        vr.vr_comm_destroy(comm)
