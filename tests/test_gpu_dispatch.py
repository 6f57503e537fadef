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
                                             (3, 50, 8, 9, 2, 10), (2, 70, 8, 128, 4, 11), (64, 50, 8, 128, 4, 12)])
def test_dispatch_small_vs_oracle(R, T, H, E, K, seed):
    say(f"dispatch R={R} T={T} H={H} E={E} K={K}")
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=seed)
    res = _run(topk, x, E)
    over = _check(res, topk, x, E)
    assert not any(over)
    assert res["err"][0] == vr.VR_OK


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
