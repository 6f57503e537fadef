"""Seeded synthetic inputs for the window put/get collectives.

This module is the one piece shared by the CPU oracle and the GPU path. It
holds no arithmetic of the method itself: it only draws inputs (fills,
uniform and normal values, uniform bytes, Zipf top-k routings) and hands
them out as numpy arrays, one per virtual rank.

Per-rank streams: ``np.random.default_rng(np.random.SeedSequence(seed).spawn(R)[r])``
so that every rank's input is reproducible on its own.

Sizes and value distributions follow the five workloads named on the
symmetric-memory example page (4 ranks x 1,048,576 fp32, each filled with
its rank value) and the GIN/dispatch pages (AlltoAll blocks, MoE dispatch of
hundreds-of-bytes tokens among dozens of experts), at the shapes listed in
``CONFIGS`` below.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "CONFIGS", "rank_rngs", "allreduce_f32_inputs", "allreduce_bf16_inputs",
    "alltoall_inputs", "allgather_inputs", "ring_inputs", "dispatch_inputs",
    "zipf_expert_probs", "f32_to_bf16_bits_torch",
]

# Workload shapes, named by what they are. The large bf16 AllReduce is the headline throughput workload.
CONFIGS = {
    "allreduce_f32_r4_1Mi": dict(kind="allreduce", ranks=4, count=1 << 20, dtype="f32", seed=101),
    "allreduce_bf16_r8_64Mi": dict(kind="allreduce", ranks=8, count=64 << 20, dtype="bf16", seed=102),
    "alltoall_r8_4MiB": dict(kind="alltoall", ranks=8, block_bytes=4 << 20, seed=103),
    "dispatch_r8_t4096_e256_k8": dict(kind="dispatch", ranks=8, tokens=4096, hidden=256, experts=256,
                                      topk=8, zipf_s=1.1, seed=104),
    "allgather_r16_64MiB": dict(kind="allgather", ranks=16, bytes_per_rank=64 << 20, seed=105),
    "ring_r16_1Mi_x_256B": dict(kind="ring", ranks=16, puts_per_rank=1 << 16, put_bytes=256,
                                contexts=64, seed=105),
}


def rank_rngs(seed: int, nranks: int) -> list[np.random.Generator]:
    """One independent generator per virtual rank."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(nranks)]


def f32_to_bf16_bits_torch(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) using torch's CPU conversion.

    Used only to synthesise bf16 inputs; the oracle carries its own rounding.
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def allreduce_f32_inputs(nranks: int, count: int, run: str = "B", seed: int = 101) -> list[np.ndarray]:
    """Run A: rank r holds ``float(r)`` everywhere. Run B: seeded uniform[-1, 1)."""
    if run == "A":
        return [np.full(count, float(r), dtype=np.float32) for r in range(nranks)]
    if run != "B":
        raise ValueError(f"unknown run {run!r}")
    out = []
    for g in rank_rngs(seed, nranks):
        u = g.random(count, dtype=np.float32)
        out.append((u * np.float32(2.0) - np.float32(1.0)).astype(np.float32))
    return out


def allreduce_bf16_inputs(nranks: int, count: int, seed: int = 102) -> list[np.ndarray]:
    """Seeded normal(0, 1) values, stored as bf16 bit patterns (uint16)."""
    return [f32_to_bf16_bits_torch(g.standard_normal(count, dtype=np.float32))
            for g in rank_rngs(seed, nranks)]


def alltoall_inputs(nranks: int, block_bytes: int, seed: int = 103) -> list[np.ndarray]:
    """Each rank's send buffer: ``nranks`` blocks of uniform random bytes."""
    return [g.integers(0, 256, nranks * block_bytes, dtype=np.uint8) for g in rank_rngs(seed, nranks)]


def allgather_inputs(nranks: int, bytes_per_rank: int, seed: int = 105) -> list[np.ndarray]:
    """Each rank's contribution: uniform fp32 in [0,1), handed out as raw bytes."""
    out = []
    for g in rank_rngs(seed, nranks):
        n = bytes_per_rank // 4
        v = g.random(n, dtype=np.float32).view(np.uint8)
        tail = g.integers(0, 256, bytes_per_rank - 4 * n, dtype=np.uint8)
        out.append(np.concatenate([v, tail]) if tail.size else v)
    return out


def ring_inputs(nranks: int, puts_per_rank: int, put_bytes: int, seed: int = 105) -> list[np.ndarray]:
    """Ring payloads: uniform bytes, ``puts_per_rank * put_bytes`` per rank.

    Drawn from a stream separate from the AllGather one (seed + 1000).
    """
    return [g.integers(0, 256, puts_per_rank * put_bytes, dtype=np.uint8)
            for g in rank_rngs(seed + 1000, nranks)]


def zipf_expert_probs(num_experts: int, s: float) -> np.ndarray:
    """Expert popularity ``p(e) proportional to (e + 1) ** -s`` (identity ranking)."""
    w = np.arange(1, num_experts + 1, dtype=np.float64) ** (-s)
    return w / w.sum()


def dispatch_inputs(nranks: int, tokens: int, hidden: int, experts: int, topk: int,
                    zipf_s: float = 1.1, seed: int = 104):
    """MoE routing and token rows.

    Returns ``(topk_idx, x_bits)``: ``topk_idx`` int32 [R][T][K] of distinct
    experts per token, drawn by Gumbel-top-k on ``log p(e)`` (sequential
    weighted sampling without replacement), ordered by perturbed score;
    ``x_bits`` uint16 [R][T][hidden] bf16 bit patterns of normal(0, 1) values.
    """
    if topk > experts:
        raise ValueError("topk > experts")
    logp = np.log(zipf_expert_probs(experts, zipf_s))
    idx = np.empty((nranks, tokens, topk), dtype=np.int32)
    xs = np.empty((nranks, tokens, hidden), dtype=np.uint16)
    for r, g in enumerate(rank_rngs(seed, nranks)):
        score = logp[None, :] + g.gumbel(size=(tokens, experts))
        part = np.argpartition(-score, topk - 1, axis=1)[:, :topk]
        order = np.argsort(-np.take_along_axis(score, part, axis=1), axis=1, kind="stable")
        idx[r] = np.take_along_axis(part, order, axis=1).astype(np.int32)
        xs[r] = f32_to_bf16_bits_torch(g.standard_normal((tokens, hidden), dtype=np.float32))
    return idx, xs


def router_weights(topk_idx: np.ndarray, experts: int, zipf_s: float = 1.1) -> np.ndarray:
    """Router weight of every routing entry, float32 [R][T][K].

    The probability of the chosen expert under the routing distribution,
    renormalised over the token's K chosen experts (the usual top-k gate);
    entries equal to -1 get weight 0.
    """
    p = zipf_expert_probs(experts, zipf_s)
    idx = np.asarray(topk_idx)
    w = np.where(idx >= 0, p[np.clip(idx, 0, experts - 1)], 0.0)
    tot = w.sum(axis=2, keepdims=True)
    return np.divide(w, tot, out=np.zeros_like(w), where=tot > 0).astype(np.float32)


def expert_outputs(rows_per_rank, hidden: int, seed: int = 106, dtype: str = "bf16") -> list[np.ndarray]:
    """Synthetic expert-output rows: rank d holds rows_per_rank[d] rows of
    ``hidden`` normal(0, 1) values, as bf16 bit patterns (uint16) or float32."""
    out = []
    for n, g in zip(rows_per_rank, rank_rngs(seed, len(rows_per_rank))):
        v = g.standard_normal((int(n), hidden), dtype=np.float32)
        out.append(f32_to_bf16_bits_torch(v) if dtype == "bf16" else v)
    return out
