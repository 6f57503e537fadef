"""Signal ping-pong on the GPU (a kernel written with the device API) against the oracle."""
import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import definitions as D
from gpu_util import Job, say

pytestmark = pytest.mark.gpu


# rank 1 on another XCD, on rank 0's XCD, or the two ranks as the two waves
# of one workgroup (the wave-level put and publish of the device API)
@pytest.mark.parametrize("mode", ["other_xcd", "same_xcd", "waves"])
@pytest.mark.parametrize("R,off,nbytes,iters", [(2, 0, 0, 5), (2, 16, 256, 1000), (3, 5, 100, 7),
                                                (2, 0, 65536 + 3, 20), (4, 4096, 1 << 20, 3)])
def test_pingpong_vs_oracle(R, off, nbytes, iters, mode):
    say(f"ping-pong R={R} off={off} bytes={nbytes} iters={iters} mode={mode}")
    flags = {"other_xcd": 0, "same_xcd": vr.VR_PINGPONG_SAME_XCD, "waves": vr.VR_PINGPONG_WAVES}[mode]
    rng = np.random.default_rng(nbytes + iters)
    size = off + 2 * nbytes + 64
    init = [rng.integers(0, 256, size, dtype=np.uint8) for _ in range(R)]
    with Job(R, signal_count=3) as job:
        w, v = job.window(size, fill=None, arrays=init)
        for rep in range(2):  # the second call starts from the signals the first left
            vr.vr_signal_pingpong(job.comm, w, off, nbytes, iters, sig=2, flags=flags)
        out = job.host(v)
        exp = D.signal_pingpong(init, off, nbytes)
        for r in range(R):
            assert np.array_equal(out[r], exp[r]), r
        assert [job.sig(r, 2) for r in range(R)] == [2 * iters, 2 * iters] + [0] * (R - 2)
        job.assert_no_async_error()


def test_pingpong_argument_and_usage_errors():
    say("ping-pong errors")
    with Job(2, signal_count=2) as job:
        w, _ = job.window(4096, fill=0)
        for args in [(4096 - 10, 8, 1), (0, 0, 0), (0, (1 << 20) + 1, 1)]:  # past the end, no rounds, too big
            with pytest.raises(vr.VrError) as e:
                vr.vr_signal_pingpong(job.comm, w, *args, sig=0)
            assert e.value.code == vr.VR_ERR_INVALID_ARGUMENT
        for bad in (0x1, vr.VR_PINGPONG_SAME_XCD | vr.VR_PINGPONG_WAVES):  # unknown flag; both placements
            with pytest.raises(vr.VrError) as e:
                vr.vr_signal_pingpong(job.comm, w, 0, 8, 1, sig=0, flags=bad)
            assert e.value.code == vr.VR_ERR_INVALID_ARGUMENT
        vr.vr_signal(job.comm, 0, 1, 0, vr.SignalAdd(1, 5))
        with pytest.raises(vr.VrError) as e:  # signal 1 at rank 0 is in Add mode
            vr.vr_signal_pingpong(job.comm, w, 0, 8, 1, sig=1)
        assert e.value.code == vr.VR_ERR_INVALID_USAGE
        job.assert_no_async_error()
    with Job(1, signal_count=1) as job:
        w, _ = job.window(4096, fill=0)
        with pytest.raises(vr.VrError) as e:
            vr.vr_signal_pingpong(job.comm, w, 0, 8, 1, sig=0)
        assert e.value.code == vr.VR_ERR_INVALID_ARGUMENT
