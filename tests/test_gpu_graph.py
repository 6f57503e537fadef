"""A collective captured in a HIP graph and replayed.

A call's in-kernel waits take their target from the signal's expected value
when the call is enqueued, so a captured call keeps that target on every
replay. Capturing a vr_signal_reset of the signal at every rank (a kernel
node) before the collective makes each replay start from 0 and wait for
exactly its own R SignalIncs. Each replay is checked against the oracle,
with eager work and synchronizations between the replays.
"""
import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import definitions as D
import workloads as W
from gpu_util import Job, say

pytestmark = pytest.mark.gpu

SIG = 2


@pytest.mark.parametrize("dtype,R,N", [("f32", 4, 70001), ("bf16", 8, 1 << 20)])
def test_allreduce_replayed_from_a_graph_with_signal_resets(dtype, R, N):
    import torch
    say(f"allreduce in a HIP graph {dtype} R={R} N={N}, three replays")
    es = 4 if dtype == "f32" else 2
    dt = vr.VR_DT_F32 if dtype == "f32" else vr.VR_DT_BF16
    with Job(R) as job:
        sw, sv = job.window(N * es, fill=0)
        rw, rv = job.window(N * es, fill=0xCD)
        stream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for d in range(R):
                vr.vr_signal_reset(job.comm, d, SIG)
            vr.vr_allreduce(job.comm, sw, 0, rw, 0, N, dt, sig=SIG)
        for rep in range(3):
            xs = (W.allreduce_f32_inputs(R, N, seed=rep) if dtype == "f32"
                  else W.allreduce_bf16_inputs(R, N, seed=rep))
            for r in range(R):  # eager work between the replays: new inputs, cleared outputs
                sv[r].copy_(torch.from_numpy(xs[r].view(np.uint8)))
                rv[r].fill_(0xCD)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            out = job.host(rv)
            want = D.allreduce(xs, dtype).view(np.uint8)
            for d in range(R):
                assert np.array_equal(out[d], want), (rep, d)
                assert vr.vr_signal_read(job.comm, d, SIG) == R, (rep, d)
            job.assert_no_async_error()
        del graph


def test_dispatch_noalloc_replayed_from_a_graph_with_new_routing():
    # the allocation-free dispatch is for callers such as graph capture: its
    # count target comes from the reset, and its row target is taken on the
    # device from the row signal at kernel start, so every replay may route
    # differently
    import torch
    R, T, H, E, K = 8, 300, 64, 64, 4
    SIGC, SIGR = 4, 5
    rb, cap = H * 2, R * T * K
    say(f"dispatch_noalloc in a HIP graph R={R} T={T} E={E} K={K}, three replays with new routing")
    with Job(R) as job:
        xw, xv = job.window(T * rb, fill=0)
        rw, rv = job.window(cap * rb, fill=0xEE)
        tk = torch.zeros((R, T, K), dtype=torch.int32, device="cuda")
        counts = torch.zeros((R, E // R), dtype=torch.int32, device="cuda")
        src = torch.full((R, cap), -1, dtype=torch.int32, device="cuda")
        pos = torch.full((R, T, K), -5, dtype=torch.int32, device="cuda")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
            for d in range(R):
                vr.vr_signal_reset(job.comm, d, SIGC)
                vr.vr_signal_reset(job.comm, d, SIGR)
            vr.vr_dispatch_noalloc(job.comm, xw, 0, rb, tk, T, K, E, rw, 0, cap, counts, src, pos, SIGC, SIGR)
        for rep in range(3):
            topk, x = W.dispatch_inputs(R, T, H, E, K, seed=50 + rep)
            for r in range(R):  # eager work between the replays: new tokens and routing, cleared outputs
                xv[r].copy_(torch.from_numpy(np.ascontiguousarray(x[r]).reshape(-1).view(np.uint8)))
                rv[r].fill_(0xEE)
            tk.copy_(torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32)))
            src.fill_(-1)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            rows, tags, cnts, _ = D.dispatch(topk, x, E, cap)
            out = job.host(rv)
            src_h, cnt_h, pos_h = src.cpu().numpy(), counts.cpu().numpy(), pos.cpu().numpy()
            assert np.array_equal(pos_h, D.dispatch_positions(topk, E, cap)), rep
            for d in range(R):
                n = rows[d].shape[0]
                assert np.array_equal(out[d][:n * rb], rows[d].reshape(-1)), (rep, d)
                assert np.array_equal(src_h[d, :n], tags[d]) and np.all(src_h[d, n:] == -1), (rep, d)
                assert np.array_equal(cnt_h[d], cnts[d]), (rep, d)
                assert vr.vr_signal_read(job.comm, d, SIGC) == R, (rep, d)
                assert vr.vr_signal_read(job.comm, d, SIGR) == n, (rep, d)
            job.assert_no_async_error()
        del graph
