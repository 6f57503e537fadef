"""MoE dispatch on the GPU against the oracle: rows, source tags, counts, signals."""
import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import definitions as D
import workloads as W
from gpu_util import Job, say

pytestmark = pytest.mark.gpu

SIG_COUNTS, SIG_ROWS = 4, 5


def _run(topk, x, E, cap=None, repeats=1, x_off=0, recv_off=0):
    import torch
    R, T, K = topk.shape
    rb = x.shape[2] * x.itemsize
    xb = np.ascontiguousarray(x).view(np.uint8).reshape(R, T, rb)
    cap = cap if cap is not None else max(1, R * T * min(K, E // R))
    with Job(R) as job:
        xw, xv = job.window(x_off + T * rb + 1, fill=0)
        for r in range(R):
            xv[r][x_off:x_off + T * rb].copy_(torch.from_numpy(xb[r].reshape(-1)))
        rw, rv = job.window(recv_off + cap * rb, fill=0xEE)
        tk = torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32)).cuda()
        counts = torch.full((R, E // R), -7, dtype=torch.int32, device="cuda")
        src = torch.full((R, cap), -1, dtype=torch.int32, device="cuda")
        pos = torch.full((R, T, K), -5, dtype=torch.int32, device="cuda")
        for _ in range(repeats):
            vr.vr_dispatch(job.comm, xw, x_off, rb, tk, T, K, E, rw, recv_off, cap, counts, src, pos, SIG_COUNTS,
                           SIG_ROWS)
        out = job.host(rv)
        res = dict(rows=[o[recv_off:].reshape(cap, rb) for o in out], src=src.cpu().numpy(),
                   counts=counts.cpu().numpy(), pos=pos.cpu().numpy(), sig_counts=[job.sig(d, SIG_COUNTS) for d in range(R)],
                   sig_rows=[job.sig(d, SIG_ROWS) for d in range(R)], err=job.async_error(), cap=cap)
    return res


def _check(res, topk, x, E, repeats=1):
    R = topk.shape[0]
    rows, src, counts, over = D.dispatch(topk, x, E, res["cap"])
    for d in range(R):
        n = rows[d].shape[0]
        assert np.array_equal(res["rows"][d][:n], rows[d]), d
        assert np.array_equal(res["src"][d][:n], src[d]), d
        assert np.all(res["src"][d][n:] == -1)
        assert np.array_equal(res["counts"][d], counts[d]), d
    assert res["sig_counts"] == [repeats * R] * R
    per = D.dispatch_rows_per_rank(topk, E)
    assert res["sig_rows"] == [int(repeats * v) for v in per]
    assert np.array_equal(res["pos"], D.dispatch_positions(np.where((topk >= -1) & (topk < E), topk, -1), E,
                                                           res["cap"]))
    return over


@pytest.mark.parametrize("R,T,H,E,K,seed", [(2, 5, 4, 4, 2, 0), (4, 37, 8, 16, 3, 1), (3, 130, 12, 6, 2, 2),
                                             (8, 64, 256, 256, 8, 3), (8, 200, 32, 64, 8, 4), (5, 1, 8, 10, 1, 5),
                                             (4, 65, 3, 8, 4, 6), (2, 300, 256, 8, 8, 7),
                                             (4, 1100, 8, 1024, 64, 8), (8, 1537, 64, 32, 4, 9),
                                             (3, 50, 8, 9, 2, 10), (2, 70, 8, 128, 4, 11), (64, 50, 8, 128, 4, 12),
                                             # rows of 528 and 1024 bytes: one row per wave instruction
                                             # on the 16-byte path, eight row vectors per lane
                                             (4, 90, 264, 16, 4, 13), (8, 130, 512, 64, 8, 14)])
def test_dispatch_small_vs_oracle(R, T, H, E, K, seed):
    say(f"dispatch R={R} T={T} H={H} E={E} K={K}")
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=seed)
    res = _run(topk, x, E)
    over = _check(res, topk, x, E)
    assert not any(over)
    assert res["err"][0] == vr.VR_OK


def test_dispatch_maximum_token_count():
    # T = 65535, the largest the source tag's 16-bit token field holds: 256
    # count blocks and 1024 put blocks per source
    R, T, H, E, K = 2, 65535, 8, 4, 2
    say(f"dispatch maximum T R={R} T={T} H={H} E={E} K={K}")
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=21)
    res = _run(topk, x, E)
    over = _check(res, topk, x, E)
    assert not any(over)
    assert res["err"][0] == vr.VR_OK
    assert int(res["src"][0].max()) & 0xFFFF == T - 1 or int(res["src"][1].max()) & 0xFFFF == T - 1


def test_dispatch_unrouted_entries_and_empty_experts():
    R, T, H, E, K = 4, 50, 8, 16, 4
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=11)
    rng = np.random.default_rng(0)
    topk[rng.random(topk.shape) < 0.3] = -1
    say("dispatch with -1 entries")
    res = _run(topk, x, E)
    _check(res, topk, x, E)
    assert res["err"][0] == vr.VR_OK


def test_dispatch_zero_tokens():
    R, E, K = 4, 8, 2
    topk = np.zeros((R, 0, K), np.int32)
    x = np.zeros((R, 0, 4), np.uint16)
    say("dispatch T=0")
    res = _run(topk, x, E, cap=1)
    assert res["sig_counts"] == [R] * R and res["sig_rows"] == [0] * R
    assert np.all(res["counts"] == 0)


def test_dispatch_capacity_overflow_reported():
    R, T, H, E, K = 2, 100, 4, 4, 2
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=12)
    say("dispatch capacity overflow")
    res = _run(topk, x, E, cap=60)
    over = _check(res, topk, x, E)
    assert any(over)
    assert res["err"][0] == vr.VR_ERR_OUT_OF_RESOURCES and res["err"][1] & vr.VR_ASYNC_CAPACITY


def test_dispatch_bad_expert_reported():
    R, T, H, E, K = 2, 10, 4, 4, 2
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=13)
    topk[1, 3, 0] = 99
    say("dispatch bad expert id")
    res = _run(topk, x, E)
    assert res["err"][1] & vr.VR_ASYNC_BAD_EXPERT
    ok = topk.copy()
    ok[1, 3, 0] = -1  # the bad entry is skipped
    _check(res, ok, x, E)


def test_dispatch_unaligned_rows_and_offsets():
    R, T, E, K = 3, 40, 6, 2
    topk, _ = W.dispatch_inputs(R, T, 4, E, K, seed=14)
    x = np.random.default_rng(1).integers(0, 256, (R, T, 13), dtype=np.uint8)
    say("dispatch unaligned 13-byte rows")
    res = _run(topk, x, E, x_off=5, recv_off=3)
    _check(res, topk, x, E)


def test_dispatch_repeated_signals_accumulate():
    R, T, H, E, K = 4, 40, 8, 16, 2
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=15)
    say("dispatch repeated x3")
    res = _run(topk, x, E, repeats=3)
    _check(res, topk, x, E, repeats=3)


def test_dispatch_r8_t4096_e256_k8_full_size():
    c = W.CONFIGS["dispatch_r8_t4096_e256_k8"]
    say("dispatch full size R=8 T=4096 E=256 K=8")
    topk, x = W.dispatch_inputs(c["ranks"], c["tokens"], c["hidden"], c["experts"], c["topk"], c["zipf_s"],
                                seed=c["seed"])
    res = _run(topk, x, c["experts"])
    _check(res, topk, x, c["experts"])
    assert res["err"][0] == vr.VR_OK


def test_dispatch_shapes_interleaved_on_one_comm():
    # One communicator: dispatches of two shapes, a per-rank-layout dispatch
    # and a ring exchange in between, each
    # dispatch checked against the oracle: nothing a dispatch leaves in the
    # scratch may leak into the next one.
    import torch
    R, H, K = 4, 16, 4
    rb = H * 2
    shapes = [(300, 64, 1), (100, 32, 2), (300, 64, 3), (100, 32, 4), (300, 64, 5)]
    with Job(R, signal_count=16, counter_count=16, context_count=2) as job:
        xw, xv = job.window(300 * rb, fill=0)
        cap = R * 300 * K
        rw, rv = job.window(cap * rb, fill=0)
        rs, _ = job.window(4096, fill=3)
        rr, _ = job.window(4096, fill=0)
        steps = []
        for i, (T, E, seed) in enumerate(shapes):
            topk, x = W.dispatch_inputs(R, T, H, E, K, seed=seed)
            for r in range(R):
                xv[r][:T * rb].copy_(torch.from_numpy(np.ascontiguousarray(x[r]).reshape(-1).view(np.uint8)))
            tk = torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32)).cuda()
            counts = torch.zeros(R, E // R, dtype=torch.int32, device="cuda")
            src = torch.full((R, cap), -1, dtype=torch.int32, device="cuda")
            vr.vr_dispatch(job.comm, xw, 0, rb, tk, T, K, E, rw, 0, cap, counts, src, None, 0, 1)
            out = job.host(rv)
            rows, tags, cnts, _ = D.dispatch(topk, x, E, cap)
            for d in range(R):
                n = rows[d].shape[0]
                assert np.array_equal(out[d][:n * rb], rows[d].reshape(-1)), (i, d)
                assert np.array_equal(src[d, :n].cpu().numpy(), tags[d]), (i, d)
                assert np.array_equal(counts[d].cpu().numpy(), cnts[d]), (i, d)
            steps.append(i)
            if i == 1:  # the per-rank layout on the same communicator
                cd = torch.zeros(R, E // R, dtype=torch.int32, device="cuda")
                sd = torch.full((R, cap), -1, dtype=torch.int32, device="cuda")
                ed = torch.full((R, cap, K), -2, dtype=torch.int32, device="cuda")
                vr.vr_dispatch_dedup(job.comm, xw, 0, rb, tk, T, K, E, rw, 0, cap, cd, sd, ed, None, 2, 3)
                out = job.host(rv)
                drows, dtags, _, dcnts, _ = D.dispatch_dedup(topk, x, E, cap)[:5]
                for d in range(R):
                    n = drows[d].shape[0]
                    assert np.array_equal(out[d][:n * rb], drows[d].reshape(-1)), ("dedup", d)
                    assert np.array_equal(sd[d, :n].cpu().numpy(), dtags[d]), ("dedup", d)
            if i == 2:  # a ring exchange on the same communicator
                vr.vr_ring_exchange(job.comm, rs, rr, 256, 8, 2, 4, 0)
                job.torch.cuda.synchronize()
        job.assert_no_async_error()
    assert steps == list(range(len(shapes)))


@pytest.mark.parametrize("zipf_s,seed", [(1.1, 205), (1.1, 306), (0.0, 407)])
def test_dispatch_full_shape_other_routings(zipf_s, seed):
    # the full 8 x 4096 x top-8-of-256 shape under other routing draws: two
    # more Zipf(1.1) seeds and uniform expert popularity (s = 0), where every
    # rank receives about the same number of rows
    c = W.CONFIGS["dispatch_r8_t4096_e256_k8"]
    say(f"dispatch full shape zipf_s={zipf_s} seed={seed}")
    topk, x = W.dispatch_inputs(c["ranks"], c["tokens"], c["hidden"], c["experts"], c["topk"], zipf_s, seed=seed)
    res = _run(topk, x, c["experts"])
    _check(res, topk, x, c["experts"])
    assert res["err"][0] == vr.VR_OK


def _with_repeats(topk, frac, seed):
    """Entry k names the same expert as entry k-1 with probability frac."""
    t = topk.copy()
    rep = np.random.default_rng(seed).random(t.shape) < frac
    for k in range(1, t.shape[2]):
        t[:, :, k] = np.where(rep[:, :, k], t[:, :, k - 1], t[:, :, k])
    return t


@pytest.mark.parametrize("R,T,H,E,K,seed,frac", [(2, 3, 4, 4, 2, 20, 1.0), (4, 100, 8, 16, 4, 21, 0.4),
                                                  (8, 300, 256, 256, 8, 22, 0.3), (3, 70, 8, 6, 3, 23, 0.5)])
def test_dispatch_duplicate_expert_ids_send_one_row_per_entry(R, T, H, E, K, seed, frac):
    # a token whose top-k names one expert more than once sends one row per
    # entry, in k order, and the counts and the row signal count entries
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=seed)
    topk = _with_repeats(topk, frac, seed)
    assert any(len(set(topk[s, t].tolist())) < K for s in range(R) for t in range(T))
    say(f"dispatch with repeated expert ids R={R} T={T} E={E} K={K}")
    res = _run(topk, x, E)
    over = _check(res, topk, x, E)
    assert not any(over)
    assert res["err"][0] == vr.VR_OK


def test_dispatch_trace_records_every_workgroups_phases():
    # vr_comm_set_trace: every workgroup stamps its phases, in order; the
    # result is unchanged
    import torch
    R, T, H, E, K = 4, 600, 16, 32, 4
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=31)
    rb = H * 2
    cap = R * T * K
    nb1 = (T + 255) // 256
    ncount, nput = R * nb1, R * 4 * nb1
    with Job(R) as job:
        xw, _ = job.window(T * rb, fill=None, arrays=[x[r] for r in range(R)])
        rw, rv = job.window(cap * rb, fill=0)
        tk = torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32)).cuda()
        counts = torch.zeros((R, E // R), dtype=torch.int32, device="cuda")
        src = torch.full((R, cap), -1, dtype=torch.int32, device="cuda")
        stamps = torch.zeros((ncount + nput + R) * 8, dtype=torch.int64, device="cuda")
        vr.vr_comm_set_trace(job.comm, stamps)
        say("dispatch with a phase trace")
        vr.vr_dispatch(job.comm, xw, 0, rb, tk, T, K, E, rw, 0, cap, counts, src, None, 0, 1)
        st = stamps.view(-1, 8).cpu().numpy()
        vr.vr_comm_set_trace(job.comm, None)
        out = job.host(rv)
        job.assert_no_async_error()
    cnt, put, rcv = st[:ncount], st[ncount:ncount + nput], st[ncount + nput:]
    assert np.all(cnt[:, :2] > 0) and np.all(cnt[:, 1] >= cnt[:, 0])
    assert (cnt[:, 2] > 0).sum() == R  # one count-row publisher per source
    assert np.all(put[:, :7] > 0) and np.all(np.diff(put[:, :7], axis=1) >= 0)
    assert (put[:, 7] > 0).sum() == R  # one row-signal applier per source
    assert np.all(rcv[:, :3] > 0) and np.all(np.diff(rcv[:, :3], axis=1) >= 0)
    # receiver d's wait ends after every put workgroup of every source sending
    # rows to d has completed its stores (stamped before its relay arrival)
    epr = E // R
    for d in range(R):
        srcs = [s for s in range(R) if np.any(topk[s] // epr == d)]
        last = max(put[b2 * R + s, 6] for s in srcs for b2 in range(4 * nb1))
        assert rcv[d, 2] >= last, d
    rows, tags, _, _ = D.dispatch(topk, x, E, cap)
    for d in range(R):
        n = rows[d].shape[0]
        assert np.array_equal(out[d][:n * rb].reshape(n, rb), rows[d]), d
