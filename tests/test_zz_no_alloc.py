"""vr_dispatch_noalloc against vr_dispatch on the GPU: same rows, tags,
counts, positions and signals, bit for bit, on two calls in a row (the second
smaller), with no device memory allocated by either call."""
import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import definitions as D
import workloads as W
from gpu_util import Job, say

pytestmark = pytest.mark.gpu


def _outputs(torch, R, T, K, E, cap):
    return dict(counts=torch.full((R, E // R), -7, dtype=torch.int32, device="cuda"),
                src=torch.full((R, cap), -1, dtype=torch.int32, device="cuda"),
                pos=torch.full((R, T, K), -5, dtype=torch.int32, device="cuda"))


def test_dispatch_noalloc_matches_dispatch_on_two_calls():
    import torch
    R, H = 8, 256
    rb = H * 2
    # first the full dispatch workload (8 ranks x 4096 tokens, top-8 of 256),
    # then a smaller one on the same communicator and the same scratch
    shapes = [(4096, 256, 8, 1.1, 104), (1000, 64, 4, 1.1, 7)]
    capmax = R * 4096 * 8
    with Job(R, signal_count=8) as job:
        xw, xv = job.window(4096 * rb, fill=0)
        rw_a, rv_a = job.window(capmax * rb, fill=0xEE)  # vr_dispatch_noalloc
        rw_b, rv_b = job.window(capmax * rb, fill=0xEE)  # vr_dispatch
        # load the dispatch kernel's code before any memory reading (a tiny
        # dispatch on signals of its own)
        wt, wx = W.dispatch_inputs(R, 8, H, 16, 2, seed=1)
        wk = torch.from_numpy(np.ascontiguousarray(wt, dtype=np.int32)).cuda()
        w = _outputs(torch, R, 8, 2, 16, R * 16)
        vr.vr_dispatch(job.comm, xw, 0, rb, wk, 8, 2, 16, rw_b, 0, R * 16, w["counts"], w["src"], w["pos"], 4, 5)
        rows_seen = [0] * R
        for i, (T, E, K, zs, seed) in enumerate(shapes):
            topk, x = W.dispatch_inputs(R, T, H, E, K, zs, seed=seed)
            for r in range(R):
                xv[r][:T * rb].copy_(torch.from_numpy(np.ascontiguousarray(x[r]).reshape(-1).view(np.uint8)))
            tk = torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32)).cuda()
            cap = R * T * min(K, E // R)
            a = _outputs(torch, R, T, K, E, cap)
            b = _outputs(torch, R, T, K, E, cap)
            torch.cuda.synchronize()
            free0 = torch.cuda.mem_get_info()[0]
            say(f"dispatch_noalloc call {i}: R={R} T={T} E={E} K={K}")
            vr.vr_dispatch_noalloc(job.comm, xw, 0, rb, tk, T, K, E, rw_a, 0, cap, a["counts"], a["src"], a["pos"],
                                   0, 1)
            torch.cuda.synchronize()
            assert torch.cuda.mem_get_info()[0] == free0, "vr_dispatch_noalloc allocated device memory"
            say(f"dispatch call {i}: R={R} T={T} E={E} K={K}")
            vr.vr_dispatch(job.comm, xw, 0, rb, tk, T, K, E, rw_b, 0, cap, b["counts"], b["src"], b["pos"], 2, 3)
            out_a, out_b = job.host(rv_a), job.host(rv_b)
            per = D.dispatch_rows_per_rank(topk, E)
            for d in range(R):
                n = int(per[d])
                assert np.array_equal(out_a[d][:n * rb], out_b[d][:n * rb]), (i, d)
                assert n > 0
            for key in ("counts", "src", "pos"):
                assert torch.equal(a[key], b[key]), (i, key)
            # both equal the oracle too (bit-exact)
            rows, src, counts, _ = D.dispatch(topk, x, E, cap)
            for d in range(R):
                n = rows[d].shape[0]
                assert np.array_equal(out_a[d][:n * rb].reshape(n, rb), rows[d]), (i, d)
                assert np.array_equal(a["src"][d, :n].cpu().numpy(), src[d]), (i, d)
                assert np.array_equal(a["counts"][d].cpu().numpy(), counts[d]), (i, d)
            for d in range(R):
                rows_seen[d] += int(per[d])
            assert [job.sig(d, 0) for d in range(R)] == [(i + 1) * R] * R
            assert [job.sig(d, 1) for d in range(R)] == rows_seen
            assert [job.sig(d, 0) for d in range(R)] == [job.sig(d, 2) for d in range(R)]
            assert [job.sig(d, 1) for d in range(R)] == [job.sig(d, 3) for d in range(R)]
            job.assert_no_async_error()


def test_dispatch_noalloc_rejects_shapes_past_its_scratch():
    import torch
    R, T, E, K, rb = 8, 60000, 1024, 2, 16
    with Job(R) as job:
        xw, _ = job.window(T * rb, fill=0)
        rw, _ = job.window(64 * rb, fill=0)
        tk = torch.zeros((R, T, K), dtype=torch.int32, device="cuda")
        counts = torch.zeros((R, E // R), dtype=torch.int32, device="cuda")
        src = torch.zeros((R, 64), dtype=torch.int32, device="cuda")
        say("dispatch_noalloc past the scratch limit")
        with pytest.raises(vr.VrError) as e:
            vr.vr_dispatch_noalloc(job.comm, xw, 0, rb, tk, T, K, E, rw, 0, 64, counts, src, None, 0, 1)
        assert e.value.code == vr.VR_ERR_INVALID_ARGUMENT
        assert vr.vr_signal_expected(job.comm, 0, 0) == 0  # nothing was enqueued
