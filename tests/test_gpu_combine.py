"""MoE combine on the GPU against the oracle: mixed rows, signals, device checks.

The routing's receive positions come from the GPU dispatch for the GPU side
and from the oracle for the oracle side; the dispatch tests check that the
two agree entry by entry.
"""
import numpy as np
import pytest

import collective_window_put_amd as vr
from oracle import definitions as D
import workloads as W
from gpu_util import Job, say

pytestmark = pytest.mark.gpu

SIG = 6


def _inputs(R, T, H, E, K, seed, dtype="bf16", drop=0.0):
    topk, _ = W.dispatch_inputs(R, T, H, E, K, seed=seed)
    if drop:
        topk[np.random.default_rng(seed).random(topk.shape) < drop] = -1
    weights = W.router_weights(topk, E)
    rows = D.dispatch_rows_per_rank(topk, E)
    y = W.expert_outputs(rows, H, seed=seed + 50, dtype=dtype)
    return topk, weights, y


def _run(topk, weights, y, E, H, dtype="bf16", cap=None, repeats=1, y_off=0, out_off=0, pos_override=None):
    """GPU dispatch (for send_pos) on dummy rows, then the combine of y."""
    import torch
    R, T, K = topk.shape
    es = 2 if dtype == "bf16" else 4
    rb = H * es
    cap = cap if cap is not None else max(1, max(int(v.shape[0]) for v in y))
    dt = vr.VR_DT_BF16 if dtype == "bf16" else vr.VR_DT_F32
    with Job(R) as job:
        # positions from the GPU dispatch (rows of 16 zero bytes stand in for tokens)
        xw, _ = job.window(max(1, T * 16), fill=0)
        dw, _ = job.window(max(1, cap * 16), fill=0)
        tk = torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32)).cuda()
        counts = torch.zeros((R, E // R), dtype=torch.int32, device="cuda")
        src = torch.zeros((R, cap), dtype=torch.int32, device="cuda")
        pos = torch.full((R, T, K), -5, dtype=torch.int32, device="cuda")
        vr.vr_dispatch(job.comm, xw, 0, 16, tk, T, K, E, dw, 0, cap, counts, src, pos, 0, 1)
        if pos_override is not None:
            pos = torch.from_numpy(pos_override).cuda()
        pad = [np.concatenate([np.ascontiguousarray(v).view(np.uint8).reshape(v.shape[0], rb),
                               np.zeros((cap - v.shape[0], rb), np.uint8)]) for v in y]
        yw, _ = job.window(y_off + cap * rb, fill=None,
                           arrays=[np.concatenate([np.zeros(y_off, np.uint8), p.reshape(-1)]) for p in pad])
        ow, ov = job.window(out_off + max(1, T * rb), fill=0xEE)
        w = torch.from_numpy(np.ascontiguousarray(weights, dtype=np.float32)).cuda()
        for _ in range(repeats):
            vr.vr_combine(job.comm, yw, y_off, cap, rb, dt, tk, w, pos, T, K, E, ow, out_off, SIG)
        out = job.host(ov)
        res = dict(out=[o[out_off:out_off + T * rb].view(np.uint16 if dtype == "bf16" else np.float32).reshape(T, H)
                        for o in out],
                   tail=[o[out_off + T * rb:] for o in out], pos=pos.cpu().numpy(),
                   sig=[job.sig(d, SIG) for d in range(R)], err=job.async_error(), cap=cap)
    return res


def _check(res, topk, weights, y, E, dtype="bf16", repeats=1, tokens=None):
    R, T, K = topk.shape
    pos = D.dispatch_positions(topk, E, res["cap"])
    assert np.array_equal(res["pos"], pos)
    sel = np.arange(T) if tokens is None else tokens
    want = D.combine(topk[:, sel], weights[:, sel], pos[:, sel], y, E, dtype)
    for s in range(R):
        assert np.array_equal(res["out"][s][sel], want[s]), s
        assert np.all(res["tail"][s][:16] == 0xEE)  # nothing past the last token row
    assert res["sig"] == [repeats * R] * R


@pytest.mark.parametrize("R,T,H,E,K,seed,dtype", [
    (2, 5, 8, 4, 2, 0, "bf16"), (4, 37, 16, 16, 3, 1, "bf16"), (3, 130, 8, 6, 2, 2, "f32"),
    (8, 64, 256, 256, 8, 3, "bf16"), (5, 1, 8, 10, 1, 4, "bf16"), (4, 100, 64, 32, 4, 5, "f32"),
    (8, 200, 136, 64, 8, 6, "bf16"), (4, 70, 1024, 16, 2, 7, "bf16"), (4, 300, 8, 1024, 64, 8, "bf16"),
    (64, 40, 8, 128, 4, 9, "bf16"),
    # K = 12 and 10: a full and a partial batch of row loads; 137 and 68
    # vectors per row: chunks of 64 lanes with a partial last one
    (4, 45, 1096, 16, 12, 12, "bf16"), (3, 70, 272, 12, 10, 13, "f32")])
def test_combine_vs_oracle(R, T, H, E, K, seed, dtype):
    say(f"combine R={R} T={T} H={H} E={E} K={K} {dtype}")
    topk, weights, y = _inputs(R, T, H, E, K, seed, dtype)
    res = _run(topk, weights, y, E, H, dtype)
    _check(res, topk, weights, y, E, dtype)
    assert res["err"][0] == vr.VR_OK


def test_combine_maximum_token_count():
    # T = 65535, the largest token count the dispatch's source tags hold
    R, T, H, E, K = 2, 65535, 8, 4, 2
    say(f"combine maximum T R={R} T={T} H={H} E={E} K={K}")
    topk, weights, y = _inputs(R, T, H, E, K, 23)
    res = _run(topk, weights, y, E, H)
    _check(res, topk, weights, y, E)


def test_combine_unrouted_entries_and_capacity_drops():
    R, T, H, E, K = 4, 80, 16, 16, 4
    topk, weights, y = _inputs(R, T, H, E, K, 9, drop=0.3)
    cap = max(1, int(min(v.shape[0] for v in y)) - 3)  # the busiest ranks drop rows
    say(f"combine with -1 entries, capacity {cap}")
    y = [v[:cap] for v in y]
    res = _run(topk, weights, y, E, H, cap=cap)
    _check(res, topk, weights, y, E)


@pytest.mark.parametrize("H,dtype,y_off,out_off", [(13, "bf16", 6, 2), (5, "f32", 4, 12), (8, "bf16", 2, 0)])
def test_combine_element_path_unaligned(H, dtype, y_off, out_off):
    R, T, E, K = 3, 40, 6, 2
    topk, weights, y = _inputs(R, T, H, E, K, 10, dtype)
    say(f"combine element path H={H} {dtype} offsets {y_off},{out_off}")
    res = _run(topk, weights, y, E, H, dtype, y_off=y_off, out_off=out_off)
    _check(res, topk, weights, y, E, dtype)


def test_combine_rows_too_long_to_stage():
    # rows of 140,000,000 bytes: the 32 rows of a workgroup span more than a
    # 32-bit buffer range, so each lane group stores its own output vectors
    # instead of staging the rows in LDS
    R, T, E, K, H = 2, 2, 2, 1, 70_000_000
    say(f"combine rows of {2 * H} bytes R={R} T={T} E={E} K={K}")
    topk, weights, y = _inputs(R, T, 8, E, K, 11)
    y = W.expert_outputs(D.dispatch_rows_per_rank(topk, E), H, seed=61)
    res = _run(topk, weights, y, E, H)
    _check(res, topk, weights, y, E)
    assert res["err"][0] == vr.VR_OK


def test_combine_zero_tokens():
    R, E, K, H = 4, 8, 2, 8
    topk = np.zeros((R, 0, K), np.int32)
    say("combine T=0")
    res = _run(topk, np.zeros((R, 0, K), np.float32), [np.zeros((0, H), np.uint16)] * R, E, H, cap=1)
    assert res["sig"] == [R] * R
    assert res["err"][0] == vr.VR_OK


def test_combine_repeated_signals_accumulate():
    R, T, H, E, K = 4, 50, 16, 16, 2
    topk, weights, y = _inputs(R, T, H, E, K, 11)
    say("combine repeated x3")
    res = _run(topk, weights, y, E, H, repeats=3)
    _check(res, topk, weights, y, E, repeats=3)


def test_combine_bad_position_and_expert_reported():
    R, T, H, E, K = 2, 12, 8, 4, 2
    topk, weights, y = _inputs(R, T, H, E, K, 12)
    pos = D.dispatch_positions(topk, E)
    bad = pos.copy()
    bad[1, 3, 0] = 1 << 20  # past the capacity: skipped, flagged
    say("combine bad position")
    res = _run(topk, weights, y, E, H, pos_override=bad)
    assert res["err"][1] & vr.VR_ASYNC_CAPACITY
    ok = bad.copy()
    ok[1, 3, 0] = -1
    want = D.combine(topk, weights, ok, y, E)
    assert all(np.array_equal(res["out"][s], want[s]) for s in range(R))
    topk2 = topk.copy()
    topk2[0, 5, 1] = 77
    say("combine bad expert")
    res = _run(topk2, weights, y, E, H, pos_override=pos)
    assert res["err"][1] & vr.VR_ASYNC_BAD_EXPERT
    t3 = topk2.copy()
    t3[0, 5, 1] = -1
    want = D.combine(t3, weights, pos, y, E)
    assert all(np.array_equal(res["out"][s], want[s]) for s in range(R))


def test_combine_r8_t4096_e256_k8_full_size():
    # every token of every rank compared with the oracle
    c = W.CONFIGS["dispatch_r8_t4096_e256_k8"]
    R, T, H, E, K = c["ranks"], c["tokens"], c["hidden"], c["experts"], c["topk"]
    topk, _ = W.dispatch_inputs(R, T, H, E, K, c["zipf_s"], seed=c["seed"])
    weights = W.router_weights(topk, E, c["zipf_s"])
    y = W.expert_outputs(D.dispatch_rows_per_rank(topk, E), H, seed=c["seed"] + 2)
    say("combine full size R=8 T=4096 E=256 K=8")
    res = _run(topk, weights, y, E, H)
    _check(res, topk, weights, y, E)
    assert res["err"][0] == vr.VR_OK


@pytest.mark.parametrize("R,T,H,E,K,seed,dtype", [(4, 90, 16, 16, 4, 30, "bf16"), (8, 200, 256, 256, 8, 31, "bf16"),
                                                  (3, 50, 8, 6, 3, 32, "f32")])
def test_combine_duplicate_expert_ids(R, T, H, E, K, seed, dtype):
    # entries naming one expert twice each have their own row (the dispatch
    # sent one per entry), mixed with their own weights in k order
    topk, weights, y = _inputs(R, T, H, E, K, seed, dtype)
    rep = np.random.default_rng(seed).random(topk.shape) < 0.4
    for k in range(1, K):
        topk[:, :, k] = np.where(rep[:, :, k], topk[:, :, k - 1], topk[:, :, k])
    y = W.expert_outputs(D.dispatch_rows_per_rank(topk, E), H, seed=seed + 50, dtype=dtype)
    say(f"combine with repeated expert ids R={R} T={T} E={E} K={K} {dtype}")
    res = _run(topk, weights, y, E, H, dtype)
    _check(res, topk, weights, y, E, dtype)
    assert res["err"][0] == vr.VR_OK
