"""Ring exchange on the GPU: cyclic shift, per-context signals and counters, litmus."""
import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import definitions as D
import workloads as W
from gpu_util import Job, say

pytestmark = pytest.mark.gpu


def _run(R, P, pb, C, litmus=True, repeats=1, flags=0):
    import torch
    sends = W.ring_inputs(R, P, pb, seed=R + P)
    with Job(R, signal_count=C + 2, counter_count=C + 1, context_count=C) as job:
        sw, _ = job.window(P * pb, fill=None, arrays=sends)
        rw, rv = job.window(P * pb, fill=0)
        lit = torch.zeros(2, dtype=torch.int64, device="cuda") if litmus else None
        for _ in range(repeats):
            vr.vr_ring_exchange(job.comm, sw, rw, pb, P, C, sig_base=1, cnt_base=1, litmus=lit, flags=flags)
        out = job.host(rv)
        sigs = [[job.sig(d, 1 + k) for k in range(C)] for d in range(R)]
        cnts = [[job.cnt(d, 1 + k) for k in range(C)] for d in range(R)]
        lit_h = lit.cpu().numpy() if litmus else None
        err = job.async_error()
    return sends, out, sigs, cnts, lit_h, err


@pytest.mark.parametrize("R,P,pb,C", [(2, 8, 16, 2), (3, 96, 256, 4), (4, 1000, 48, 10), (16, 4096, 256, 64),
                                      (5, 64, 8192, 2), (64, 256, 16, 4), (2, 520, 16, 1), (3, 12, 32768, 3),
                                      (4, 3000, 64, 3), (2, 4, 65536, 2), (1, 64, 16, 2)])
def test_ring_vs_oracle(R, P, pb, C):
    # each context's workgroup issues rounds of up to 64 KiB (at most 256
    # messages) in order: (2, 520, 16, 1), (3, 12, 32768, 3) and
    # (4, 3000, 64, 3) have 3, 2 and 4 rounds per context, the first and last
    # with a partial last round; 65536-byte messages are the largest allowed
    say(f"ring R={R} P={P} pb={pb} C={C}")
    sends, out, sigs, cnts, lit, err = _run(R, P, pb, C)
    exp = D.ring(sends, [np.zeros(P * pb, np.uint8)] * R, P, pb)
    for d in range(R):
        assert np.array_equal(out[d], exp[d]), d
    assert sigs == [[P // C] * C] * R
    assert cnts == [[P // C] * C] * R
    assert lit[1] == 0 and lit[0] > 0
    assert err[0] == vr.VR_OK


@pytest.mark.parametrize("R,P,pb,C", [(2, 8, 16, 1), (4, 6400, 16, 64), (3, 200, 32, 100), (2, 520, 16, 130),
                                      (1, 300, 32, 3)])
@pytest.mark.parametrize("flags", [0, vr.VR_RING_WEAK])
def test_ring_plain_waits_vs_oracle(R, P, pb, C, flags):
    # without the litmus one wavefront per receiving rank waits, lane j on
    # contexts j, j + 64, ...: 100 and 130 contexts take a second and third pass
    say(f"ring plain waits R={R} P={P} pb={pb} C={C} flags={flags}")
    sends, out, sigs, cnts, lit, err = _run(R, P, pb, C, litmus=False, repeats=2, flags=flags)
    exp = D.ring(sends, [np.zeros(P * pb, np.uint8)] * R, P, pb)
    for d in range(R):
        assert np.array_equal(out[d], exp[d]), d
    assert sigs == [[2 * (P // C)] * C] * R
    assert cnts == [[2 * (P // C)] * C] * R
    assert err[0] == vr.VR_OK, (vr.vr_error_string(err[0]), hex(err[1]))


@pytest.mark.parametrize("flags", [0, vr.VR_RING_WEAK])
def test_ring_repeated_accumulates(flags):
    # two rounds per context, three calls in a row: signals and counters
    # accumulate, the bytes are the last call's
    say(f"ring repeated x3 flags={flags}")
    R, P, pb, C = 4, 1024, 256, 2
    sends, out, sigs, cnts, lit, err = _run(R, P, pb, C, repeats=3, flags=flags)
    exp = D.ring(sends, [np.zeros(P * pb, np.uint8)] * R, P, pb)
    for d in range(R):
        assert np.array_equal(out[d], exp[d]), d
    assert sigs == [[3 * P // C] * C] * R and cnts == [[3 * P // C] * C] * R
    assert err[0] == vr.VR_OK


def test_ring_r16_1Mi_x_256B_full_size():
    c = W.CONFIGS["ring_r16_1Mi_x_256B"]
    say("ring full size R=16 2^20 puts x 256 B")
    R, P, pb, C = c["ranks"], c["puts_per_rank"], c["put_bytes"], c["contexts"]
    sends, out, sigs, cnts, lit, err = _run(R, P, pb, C)
    exp = D.ring(sends, [np.zeros(P * pb, np.uint8)] * R, P, pb)
    for d in range(R):
        assert np.array_equal(out[d], exp[d]), d
    assert sigs == [[P // C] * C] * R and cnts == [[P // C] * C] * R
    assert lit[1] == 0
    assert err[0] == vr.VR_OK


@pytest.mark.parametrize("R,P,pb,C", [(2, 8, 16, 2), (3, 96, 256, 4), (4, 1000, 48, 10), (16, 4096, 256, 64),
                                      (5, 64, 8192, 2), (3, 12, 32768, 3), (2, 520, 16, 1), (2, 4, 65536, 2)])
def test_ring_weak_vs_oracle(R, P, pb, C):
    """Weak SignalIncs: same bytes, signals and counters; the litmus may see
    reorders (allowed), never a missing message at the full count."""
    say(f"ring weak R={R} P={P} pb={pb} C={C}")
    sends, out, sigs, cnts, lit, err = _run(R, P, pb, C, flags=vr.VR_RING_WEAK)
    exp = D.ring(sends, [np.zeros(P * pb, np.uint8)] * R, P, pb)
    for d in range(R):
        assert np.array_equal(out[d], exp[d]), d
    assert sigs == [[P // C] * C] * R
    assert cnts == [[P // C] * C] * R
    assert lit[0] > 0 and 0 <= lit[1] <= lit[0]
    assert err[0] == vr.VR_OK, (vr.vr_error_string(err[0]), hex(err[1]))
    print(f"weak ring: {lit[0]} checks, {lit[1]} observed reorders")


def test_ring_weak_r16_1Mi_x_256B_full_size():
    c = W.CONFIGS["ring_r16_1Mi_x_256B"]
    say("ring weak full size R=16 2^20 puts x 256 B")
    R, P, pb, C = c["ranks"], c["puts_per_rank"], c["put_bytes"], c["contexts"]
    sends, out, sigs, cnts, lit, err = _run(R, P, pb, C, flags=vr.VR_RING_WEAK)
    exp = D.ring(sends, [np.zeros(P * pb, np.uint8)] * R, P, pb)
    for d in range(R):
        assert np.array_equal(out[d], exp[d]), d
    assert sigs == [[P // C] * C] * R and cnts == [[P // C] * C] * R
    assert err[0] == vr.VR_OK
    print(f"weak ring full size: {lit[0]} checks, {lit[1]} observed reorders")
