"""The strong-signal rule checked inside the collectives' kernels (GIN page,
strong and weak signals: a signal seen at the peer means every earlier put of
the context to that peer is visible there).

With vr_comm_set_litmus on, each receiver re-reads, right after its wait and
acquire, the piece that completed every relay aimed at it and a seeded sample
of every tile or row, against the senders' windows. The tests run the full
workloads (AllReduce 8 x 64 Mi bf16, AlltoAll 8 x 4 MiB, dispatch 8 x 4096
tokens top-8 of 256, AllGather 16 x 64 MiB) and ragged or unaligned small
shapes, and require checks > 0 and no mismatch; the small shapes also compare
the results with the oracle, so the litmus leaves them unchanged.
"""
import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import definitions as D
import workloads as W
from gpu_util import Job, say

pytestmark = pytest.mark.gpu


def _litmus(job):
    words = job.torch.zeros(2, dtype=job.torch.int64, device="cuda")
    vr.vr_comm_set_litmus(job.comm, words)
    return words


def _read(job, words):
    job.torch.cuda.synchronize()
    checks, bad = (int(v) for v in words.cpu().tolist())
    return checks, bad


def _device_bf16(torch, n, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(n, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16).view(torch.uint8)


# -- full workloads ------------------------------------------------------------------
def test_litmus_allreduce_bf16_r8_64Mi():
    R, N = 8, 64 << 20
    with Job(R) as job:
        torch = job.torch
        sw, sv = job.window(N * 2, fill=None)
        rw, _ = job.window(N * 2, fill=0xCD)
        for r in range(R):
            sv[r].copy_(_device_bf16(torch, N, 1000 + r))
        words = _litmus(job)
        say("litmus allreduce bf16 R=8 N=64Mi (rank-split form)")
        vr.vr_allreduce(job.comm, sw, 0, rw, 0, N, vr.VR_DT_BF16, sig=1)
        checks, bad = _read(job, words)
        job.assert_no_async_error()
        # per receiver: every one of the 16384 tiles sampled, plus a whole tile per chunk
        assert checks >= R * (N // 4096) and bad == 0, (checks, bad)
        assert [job.sig(d, 1) for d in range(R)] == [R] * R


def test_litmus_alltoall_r8_4MiB():
    R, B = 8, 4 << 20
    sends = W.alltoall_inputs(R, B, seed=103)
    with Job(R) as job:
        sw, _ = job.window(R * B, fill=None, arrays=sends)
        rw, rv = job.window(R * B, fill=0xAB)
        words = _litmus(job)
        say("litmus alltoall R=8 B=4MiB")
        vr.vr_alltoall(job.comm, sw, 0, rw, 0, B, sig=2)
        checks, bad = _read(job, words)
        job.assert_no_async_error()
        assert checks >= R * R * (B // 32768) and bad == 0, (checks, bad)
        out = job.host(rv)
        exp = D.alltoall(sends, B)
        assert all(np.array_equal(out[d], exp[d]) for d in range(R))


def test_litmus_dispatch_r8_t4096_e256_k8():
    import torch
    c = W.CONFIGS["dispatch_r8_t4096_e256_k8"]
    R, T, H, E, K = c["ranks"], c["tokens"], c["hidden"], c["experts"], c["topk"]
    topk, x = W.dispatch_inputs(R, T, H, E, K, c["zipf_s"], seed=c["seed"])
    rb = H * 2
    cap = R * T * min(K, E // R)
    with Job(R) as job:
        xw, _ = job.window(T * rb, fill=None, arrays=[x[r] for r in range(R)])
        rw, rv = job.window(cap * rb, fill=0xEE)
        tk = torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32)).cuda()
        counts = torch.zeros((R, E // R), dtype=torch.int32, device="cuda")
        src = torch.full((R, cap), -1, dtype=torch.int32, device="cuda")
        words = _litmus(job)
        say("litmus dispatch R=8 T=4096 E=256 K=8")
        vr.vr_dispatch(job.comm, xw, 0, rb, tk, T, K, E, rw, 0, cap, counts, src, None, 0, 1)
        checks, bad = _read(job, words)
        job.assert_no_async_error()
        assert checks >= R * T * K and bad == 0, (checks, bad)  # every received row sampled
        out = job.host(rv)
        rows, tags, _, _ = D.dispatch(topk, x, E, cap)
        for d in range(R):
            n = rows[d].shape[0]
            assert np.array_equal(out[d][:n * rb].reshape(n, rb), rows[d]), d


def test_litmus_allgather_r16_64MiB():
    import torch
    R, M = 16, 64 << 20
    with Job(R) as job:
        sw, sv = job.window(M, fill=None)
        rw, _ = job.window(R * M, fill=0x5A)
        g = torch.Generator(device="cuda")
        g.manual_seed(105)
        for r in range(R):
            sv[r].copy_(torch.randint(0, 256, (M,), generator=g, device="cuda", dtype=torch.uint8))
        words = _litmus(job)
        say("litmus allgather R=16 M=64MiB")
        vr.vr_allgather(job.comm, sw, 0, rw, 0, M, sig=3)
        checks, bad = _read(job, words)
        job.assert_no_async_error()
        assert checks >= R * R * (M // 4096) and bad == 0, (checks, bad)
        assert [job.sig(d, 3) for d in range(R)] == [R] * R


# -- small, ragged and unaligned shapes: litmus on, results still the oracle's -------------
@pytest.mark.parametrize("dtype,R,N,off", [("f32", 3, 1001, 0), ("bf16", 8, 2048 * 8 + 3, 0), ("f32", 4, 3000, 12),
                                           ("bf16", 16, 40000, 0), ("bf16", 8, 8 * 4096 * 16, 0), ("f32", 64, 900, 4),
                                           ("bf16", 2, 4 * 4096 + 1, 0), ("f32", 4, (16 << 20) - 1000, 16),
                                           ("bf16", 16, (32 << 20) - 5, 0)])
def test_litmus_allreduce_shapes(dtype, R, N, off):
    es = 4 if dtype == "f32" else 2
    xs = W.allreduce_f32_inputs(R, N, seed=R + N) if dtype == "f32" else W.allreduce_bf16_inputs(R, N, seed=R + N)
    dt = vr.VR_DT_F32 if dtype == "f32" else vr.VR_DT_BF16
    with Job(R) as job:
        sw, sv = job.window(off + N * es, fill=0)
        rw, rv = job.window(off + N * es, fill=0xCD)
        for r in range(R):
            sv[r][off:].copy_(job.torch.from_numpy(xs[r].view(np.uint8)))
        words = _litmus(job)
        say(f"litmus allreduce {dtype} R={R} N={N} off={off}")
        for _ in range(2):
            vr.vr_allreduce(job.comm, sw, off, rw, off, N, dt, sig=0)
        checks, bad = _read(job, words)
        job.assert_no_async_error()
        assert checks > 0 and bad == 0, (checks, bad)
        out = job.host(rv)
        exp = D.allreduce(xs, dtype).view(np.uint8)
        assert all(np.array_equal(out[d][off:], exp) for d in range(R))
        assert [job.sig(d, 0) for d in range(R)] == [2 * R] * R


@pytest.mark.parametrize("R,B,soff,roff", [(3, 17, 0, 0), (5, 16385, 0, 0), (8, 65536 + 48, 3, 5), (2, 1, 0, 0),
                                           (64, 300, 0, 0)])
def test_litmus_alltoall_shapes(R, B, soff, roff):
    sends = W.alltoall_inputs(R, B, seed=R * 7 + B)
    with Job(R) as job:
        sw, sv = job.window(soff + R * B, fill=0)
        rw, rv = job.window(roff + R * B, fill=0xAB)
        for r in range(R):
            sv[r][soff:].copy_(job.torch.from_numpy(sends[r]))
        words = _litmus(job)
        say(f"litmus alltoall R={R} B={B} offsets {soff},{roff}")
        vr.vr_alltoall(job.comm, sw, soff, rw, roff, B, sig=1)
        checks, bad = _read(job, words)
        job.assert_no_async_error()
        assert checks >= R * R and bad == 0, (checks, bad)
        out = job.host(rv)
        exp = D.alltoall(sends, B)
        assert all(np.array_equal(out[d][roff:], exp[d]) for d in range(R))


@pytest.mark.parametrize("R,M,soff,roff", [(3, 16385, 0, 0), (16, 32768 + 16, 0, 0), (4, 20000, 7, 4099),
                                           (2, 1, 0, 0), (64, 5000, 0, 0), (8, 256 << 10, 16, 4096),
                                           (16, 64 << 10, 0, 0), (5, 200000 - 48, 16, 32)])
def test_litmus_allgather_shapes(R, M, soff, roff):
    sends = W.allgather_inputs(R, M, seed=R * 3 + M)
    with Job(R) as job:
        sw, sv = job.window(soff + M, fill=0)
        rw, rv = job.window(roff + R * M, fill=0x5A)
        for r in range(R):
            sv[r][soff:].copy_(job.torch.from_numpy(sends[r]))
        words = _litmus(job)
        say(f"litmus allgather R={R} M={M} offsets {soff},{roff}")
        vr.vr_allgather(job.comm, sw, soff, rw, roff, M, sig=1)
        checks, bad = _read(job, words)
        job.assert_no_async_error()
        assert checks >= R * R and bad == 0, (checks, bad)
        out = job.host(rv)
        exp = D.allgather(sends)
        assert all(np.array_equal(out[d][roff:], exp[d]) for d in range(R))


@pytest.mark.parametrize("layout", ["expert", "noalloc", "rank"])
@pytest.mark.parametrize("R,T,H,E,K,cap", [(4, 300, 8, 16, 4, None), (3, 130, 12, 6, 2, 100), (8, 1537, 64, 32, 4, None)])
def test_litmus_dispatch_shapes(layout, R, T, H, E, K, cap):
    import torch
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=R + T)
    rb = H * 2
    full = R * T * (min(K, E // R) if layout != "rank" else 1)
    cap = cap if cap is not None else full
    with Job(R) as job:
        xw, _ = job.window(T * rb, fill=None, arrays=[x[r] for r in range(R)])
        rw, rv = job.window(cap * rb, fill=0xEE)
        tk = torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32)).cuda()
        counts = torch.zeros((R, E // R), dtype=torch.int32, device="cuda")
        src = torch.full((R, cap), -1, dtype=torch.int32, device="cuda")
        words = _litmus(job)
        say(f"litmus dispatch ({layout}) R={R} T={T} E={E} K={K} cap={cap}")
        if layout == "expert":
            vr.vr_dispatch(job.comm, xw, 0, rb, tk, T, K, E, rw, 0, cap, counts, src, None, 0, 1)
            rows = D.dispatch(topk, x, E, cap)[0]
        elif layout == "noalloc":
            vr.vr_dispatch_noalloc(job.comm, xw, 0, rb, tk, T, K, E, rw, 0, cap, counts, src, None, 0, 1)
            rows = D.dispatch(topk, x, E, cap)[0]
        else:
            ex = torch.zeros((R, cap, K), dtype=torch.int32, device="cuda")
            vr.vr_dispatch_dedup(job.comm, xw, 0, rb, tk, T, K, E, rw, 0, cap, counts, src, ex, None, 0, 1)
            rows = D.dispatch_dedup(topk, x, E, cap)[0]
        checks, bad = _read(job, words)
        code, bits = job.async_error()
        assert bits & ~vr.VR_ASYNC_CAPACITY == 0, hex(bits)  # a small capacity drops rows, nothing else
        assert checks >= sum(r.shape[0] for r in rows) and bad == 0, (checks, bad)
        out = job.host(rv)
        for d in range(R):
            n = rows[d].shape[0]
            assert np.array_equal(out[d][:n * rb].reshape(n, rb), rows[d]), d


def test_litmus_off_again_counts_nothing():
    R, B = 4, 4096
    sends = W.alltoall_inputs(R, B, seed=9)
    with Job(R) as job:
        sw, _ = job.window(R * B, fill=None, arrays=sends)
        rw, _ = job.window(R * B, fill=0)
        words = _litmus(job)
        vr.vr_alltoall(job.comm, sw, 0, rw, 0, B, sig=1)
        first = _read(job, words)
        vr.vr_comm_set_litmus(job.comm, None)
        say("litmus switched off")
        vr.vr_alltoall(job.comm, sw, 0, rw, 0, B, sig=1)
        assert _read(job, words) == first and first[0] > 0 and first[1] == 0
        job.assert_no_async_error()
