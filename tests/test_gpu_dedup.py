"""Per-rank (dedup) dispatch and combine on the GPU against the oracle.

Each token lands once on every rank that owns one of its experts; the
combine sums each token's per-rank rows in rank order.
"""
import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import definitions as D
import workloads as W
from gpu_util import Job, say

pytestmark = pytest.mark.gpu

SIG_COUNTS, SIG_ROWS, SIG_COMB = 4, 5, 6


def _dispatch(job, topk, x, E, cap, x_off=0, recv_off=0, ids_offset=0):
    torch = job.torch
    R, T, K = topk.shape
    rb = x.shape[2] * x.itemsize
    xb = np.ascontiguousarray(x).view(np.uint8).reshape(R, T, rb)
    xw, xv = job.window(x_off + T * rb + 1, fill=0)
    for r in range(R):
        xv[r][x_off:x_off + T * rb].copy_(torch.from_numpy(xb[r].reshape(-1)))
    rw, rv = job.window(recv_off + cap * rb, fill=0xEE)
    # ids_offset > 0: the routing ids start that many int32 into their buffer
    ids = torch.zeros(ids_offset + topk.size, dtype=torch.int32, device="cuda")
    ids[ids_offset:].copy_(torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32).reshape(-1)))
    tk = ids[ids_offset:].view(R, T, K)
    counts = torch.full((R, E // R), -7, dtype=torch.int32, device="cuda")
    src = torch.full((R, cap), -1, dtype=torch.int32, device="cuda")
    experts = torch.full((R, cap, K), -9, dtype=torch.int32, device="cuda")
    pos = torch.full((R, T, R), -5, dtype=torch.int32, device="cuda")
    vr.vr_dispatch_dedup(job.comm, xw, x_off, rb, tk, T, K, E, rw, recv_off, cap, counts, src, experts, pos,
                         SIG_COUNTS, SIG_ROWS)
    return rw, rv, counts, src, experts, pos


def _check_dispatch(job, topk, x, E, cap, rv, counts, src, experts, pos, recv_off=0, repeats=1):
    R, T, K = topk.shape
    rb = x.shape[2] * x.itemsize
    rows, osrc, oexp, ocounts, over = D.dispatch_dedup(np.where((topk >= -1) & (topk < E), topk, -1), x, E, cap)
    out = job.host(rv)
    src_h, exp_h, counts_h, pos_h = src.cpu().numpy(), experts.cpu().numpy(), counts.cpu().numpy(), pos.cpu().numpy()
    for d in range(R):
        n = rows[d].shape[0]
        assert np.array_equal(out[d][recv_off:recv_off + n * rb].reshape(n, rb), rows[d]), d
        assert np.array_equal(src_h[d][:n], osrc[d]), d
        assert np.all(src_h[d][n:] == -1)
        assert np.array_equal(exp_h[d][:n], oexp[d]), d
        assert np.all(exp_h[d][n:] == -9)
        assert np.array_equal(counts_h[d], ocounts[d]), d
    assert np.array_equal(pos_h, D.dispatch_dedup_positions(np.where((topk >= -1) & (topk < E), topk, -1), E, cap))
    sent = [sum(1 for s in range(R) for t in range(T) if any(0 <= e < E and e // (E // R) == d for e in topk[s, t]))
            for d in range(R)]
    assert [job.sig(d, SIG_ROWS) for d in range(R)] == [repeats * v for v in sent]
    assert [job.sig(d, SIG_COUNTS) for d in range(R)] == [repeats * R] * R
    return over


@pytest.mark.parametrize("R,T,H,E,K,seed,drop", [(2, 5, 4, 4, 2, 0, 0.0), (4, 37, 8, 16, 3, 1, 0.2),
                                                  (3, 130, 12, 6, 2, 2, 0.0), (8, 64, 256, 256, 8, 3, 0.0),
                                                  (8, 200, 32, 64, 8, 4, 0.1), (5, 1, 8, 10, 1, 5, 0.0),
                                                  (4, 1100, 8, 1024, 64, 8, 0.0), (8, 1537, 64, 32, 4, 9, 0.3),
                                                  (64, 50, 8, 128, 4, 12, 0.1),
                                                  # rows of 528 and 1024 bytes (one row per wave instruction)
                                                  (4, 90, 264, 16, 4, 13, 0.1), (8, 130, 512, 64, 8, 14, 0.0)])
def test_dedup_dispatch_vs_oracle(R, T, H, E, K, seed, drop):
    say(f"dedup dispatch R={R} T={T} H={H} E={E} K={K}")
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=seed)
    if drop:
        topk[np.random.default_rng(seed).random(topk.shape) < drop] = -1
    cap = max(1, R * T)
    with Job(R) as job:
        rw, rv, counts, src, experts, pos = _dispatch(job, topk, x, E, cap)
        over = _check_dispatch(job, topk, x, E, cap, rv, counts, src, experts, pos)
        assert not any(over)
        job.assert_no_async_error()


def test_dedup_dispatch_capacity_and_bad_ids():
    R, T, H, E, K = 3, 60, 4, 6, 3
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=12)
    topk[1, 7, 2] = 50
    cap = 25
    say("dedup dispatch capacity and a bad id")
    with Job(R) as job:
        rw, rv, counts, src, experts, pos = _dispatch(job, topk, x, E, cap)
        over = _check_dispatch(job, topk, x, E, cap, rv, counts, src, experts, pos)
        assert any(over)
        code, bits = job.async_error()
        assert bits & vr.VR_ASYNC_CAPACITY and bits & vr.VR_ASYNC_BAD_EXPERT


@pytest.mark.parametrize("ids_offset", [0, 1])
def test_dedup_dispatch_bad_ids_and_id_alignment(ids_offset):
    # K = 8: a token's ids load as two 16-byte vectors when the routing array
    # is 16-byte aligned, one by one when it starts 4 bytes in; an id past E
    # and one below -1 are flagged and skipped either way
    R, T, H, E, K = 4, 70, 8, 16, 8
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=15)
    topk[2, 5, 3] = 99
    topk[0, 69, 7] = -3
    say(f"dedup dispatch bad ids, ids offset {ids_offset} int32")
    with Job(R) as job:
        rw, rv, counts, src, experts, pos = _dispatch(job, topk, x, E, R * T, ids_offset=ids_offset)
        _check_dispatch(job, topk, x, E, R * T, rv, counts, src, experts, pos)
        code, bits = job.async_error()
        assert bits & vr.VR_ASYNC_BAD_EXPERT and not bits & vr.VR_ASYNC_CAPACITY


def test_dedup_dispatch_unaligned_rows():
    R, T, E, K = 3, 40, 6, 2
    topk, _ = W.dispatch_inputs(R, T, 4, E, K, seed=14)
    x = np.random.default_rng(1).integers(0, 256, (R, T, 13), dtype=np.uint8)
    say("dedup dispatch unaligned 13-byte rows")
    with Job(R) as job:
        rw, rv, counts, src, experts, pos = _dispatch(job, topk, x, E, R * T, x_off=5, recv_off=3)
        _check_dispatch(job, topk, x, E, R * T, rv, counts, src, experts, pos, recv_off=3)


@pytest.mark.parametrize("R,T,H,E,K,seed,frac", [(4, 100, 8, 16, 4, 40, 0.4), (8, 300, 256, 256, 8, 41, 0.3),
                                                  (2, 3, 4, 4, 2, 42, 1.0)])
def test_dedup_dispatch_duplicate_expert_ids(R, T, H, E, K, seed, frac):
    # a token naming one expert twice reaches that rank once; its expert list
    # shows the local expert at both entries, and the counts count both
    topk, x = W.dispatch_inputs(R, T, H, E, K, seed=seed)
    rep = np.random.default_rng(seed).random(topk.shape) < frac
    for k in range(1, K):
        topk[:, :, k] = np.where(rep[:, :, k], topk[:, :, k - 1], topk[:, :, k])
    say(f"dedup dispatch with repeated expert ids R={R} T={T} E={E} K={K}")
    cap = max(1, R * T)
    with Job(R) as job:
        rw, rv, counts, src, experts, pos = _dispatch(job, topk, x, E, cap)
        over = _check_dispatch(job, topk, x, E, cap, rv, counts, src, experts, pos)
        assert not any(over)
        job.assert_no_async_error()


def _dedup_combine_case(R, T, H, E, K, seed, dtype, drop=0.15, topk=None):
    import torch
    if topk is None:
        topk, _ = W.dispatch_inputs(R, T, 4, E, K, seed=seed)
        topk[np.random.default_rng(seed).random(topk.shape) < drop] = -1
    es = 2 if dtype == "bf16" else 4
    rb = H * es
    cap = max(1, R * T)
    pos_o = D.dispatch_dedup_positions(topk, E, cap)
    n_d = [int((pos_o[:, :, d] >= 0).sum()) for d in range(R)]
    y = W.expert_outputs(n_d, H, seed=seed + 70, dtype=dtype)
    with Job(R) as job:
        _, _, _, _, _, pos = _dispatch(job, topk, np.zeros((R, T, 4), np.uint16), E, cap)
        pad = [np.concatenate([np.ascontiguousarray(v).view(np.uint8).reshape(v.shape[0], rb),
                               np.zeros((cap - v.shape[0], rb), np.uint8)]) for v in y]
        yw, _ = job.window(cap * rb, fill=None, arrays=pad)
        ow, ov = job.window(T * rb + 64, fill=0xEE)
        dt = vr.VR_DT_BF16 if dtype == "bf16" else vr.VR_DT_F32
        vr.vr_combine_dedup(job.comm, yw, 0, cap, rb, dt, pos, T, ow, 0, SIG_COMB)
        out = job.host(ov)
        assert np.array_equal(pos.cpu().numpy(), pos_o)
        want = D.combine_dedup(pos_o, y, dtype)
        for s in range(R):
            got = out[s][:T * rb].view(np.uint16 if dtype == "bf16" else np.float32).reshape(T, H)
            assert np.array_equal(got, want[s]), s
            assert np.all(out[s][T * rb:] == 0xEE)
        assert [job.sig(d, SIG_COMB) for d in range(R)] == [R] * R
        job.assert_no_async_error()


@pytest.mark.parametrize("R,T,H,E,K,seed,dtype", [(4, 37, 16, 16, 3, 1, "bf16"), (3, 130, 8, 6, 2, 2, "f32"),
                                                  (8, 200, 256, 64, 8, 3, "bf16"), (5, 1, 8, 10, 1, 4, "bf16")])
def test_dedup_combine_vs_oracle(R, T, H, E, K, seed, dtype):
    say(f"dedup combine R={R} T={T} H={H} {dtype}")
    _dedup_combine_case(R, T, H, E, K, seed, dtype)


def test_dedup_combine_r8_t4096_e256_k8_full_size():
    # every token of every rank, at the full dispatch shape and routing
    c = W.CONFIGS["dispatch_r8_t4096_e256_k8"]
    R, T, H, E, K = c["ranks"], c["tokens"], c["hidden"], c["experts"], c["topk"]
    topk, _ = W.dispatch_inputs(R, T, H, E, K, c["zipf_s"], seed=c["seed"])
    say("dedup combine full size R=8 T=4096 E=256 K=8")
    _dedup_combine_case(R, T, H, E, K, c["seed"], "bf16", topk=topk)


def test_dedup_r8_t4096_e256_k8_full_size():
    c = W.CONFIGS["dispatch_r8_t4096_e256_k8"]
    R, T, H, E, K = c["ranks"], c["tokens"], c["hidden"], c["experts"], c["topk"]
    topk, x = W.dispatch_inputs(R, T, H, E, K, c["zipf_s"], seed=c["seed"])
    cap = R * T
    say("dedup dispatch full size R=8 T=4096 E=256 K=8")
    with Job(R) as job:
        rw, rv, counts, src, experts, pos = _dispatch(job, topk, x, E, cap)
        _check_dispatch(job, topk, x, E, cap, rv, counts, src, experts, pos)
        job.assert_no_async_error()
