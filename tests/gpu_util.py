"""Helpers for GPU tests: a communicator with windows carved from torch slabs."""
from __future__ import annotations

import sys

import numpy as np

import collective_window_put_amd as vr

ALIGN = vr.VR_WIN_REQUIRED_ALIGNMENT


def say(msg: str) -> None:
    """Name the case before each GPU step, flushed, so a failing run shows it."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


class Job:
    """R virtual ranks on cuda:0 with windows whose memory torch owns."""

    def __init__(self, R: int, signal_count: int = 16, counter_count: int = 16, context_count: int = 1):
        import torch
        self.torch = torch
        self.R = R
        self.comm = vr.vr_comm_create(R, signal_count, counter_count, context_count)
        self._wins = []
        self._slabs = []

    def window(self, nbytes: int, fill: int | None = 0, arrays=None, flags: int = 0):
        """Register a window of nbytes per rank; returns (handle, [per-rank uint8 tensors])."""
        torch = self.torch
        stride = (nbytes + ALIGN - 1) // ALIGN * ALIGN
        slab = torch.empty(self.R * stride + ALIGN, dtype=torch.uint8, device="cuda")
        shift = (-slab.data_ptr()) % ALIGN
        views = [slab[shift + r * stride: shift + r * stride + nbytes] for r in range(self.R)]
        if arrays is not None:
            for v, a in zip(views, arrays):
                v.copy_(torch.from_numpy(np.ascontiguousarray(a).reshape(-1).view(np.uint8)))
        elif fill is not None:
            slab.fill_(fill)
        h = vr.vr_window_register(self.comm, [v.data_ptr() for v in views], nbytes, flags)
        self._wins.append(h)
        self._slabs.append(slab)
        return h, views

    def host(self, views) -> list[np.ndarray]:
        self.torch.cuda.synchronize()
        return [v.cpu().numpy() for v in views]

    def sig(self, rank: int, sid: int) -> int:
        self.torch.cuda.synchronize()
        return vr.vr_signal_read(self.comm, rank, sid)

    def cnt(self, rank: int, cid: int) -> int:
        self.torch.cuda.synchronize()
        return vr.vr_counter_read(self.comm, rank, cid)

    def async_error(self) -> tuple[int, int]:
        self.torch.cuda.synchronize()
        return vr.vr_comm_get_async_error(self.comm)

    def assert_no_async_error(self):
        code, bits = self.async_error()
        assert code == vr.VR_OK, (vr.vr_error_string(code), hex(bits))

    def close(self):
        self.torch.cuda.synchronize()
        for h in self._wins:
            vr.vr_window_deregister(self.comm, h)
        self._wins = []
        vr.vr_comm_destroy(self.comm)
        self._slabs = []

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
