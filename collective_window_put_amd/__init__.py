"""Python binding of libvrcomm: one-sided window put/get with signals and
counters, and the collectives built on them, for R virtual ranks on one
MI355X (gfx950).

Every ``vr_*`` function here marshals its arguments and calls the C function
of the same name in ``libvrcomm.so`` (declared in ``include/vrcomm.h``); all
work runs in the library's HIP kernels. PyTorch is used only to supply
device pointers (``tensor.data_ptr()``) and the current stream. There is no
fallback: if the library is not built, every call raises ``VrLibraryMissing``.

Errors: a non-OK result code raises ``VrError`` carrying the code and its name.
Device-side errors surface through ``vr_comm_get_async_error``.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_int, c_size_t, c_uint32, c_uint64, c_void_p

__all__ = [
    "VrError", "VrLibraryMissing", "LIB_PATH", "lib", "SYMBOLS",
    # result codes, flags and limits (values as in include/vrcomm.h)
    "VR_OK", "VR_ERR_INVALID_ARGUMENT", "VR_ERR_INVALID_USAGE", "VR_ERR_OUT_OF_RESOURCES",
    "VR_ERR_HIP", "VR_ERR_TIMEOUT", "VR_ERR_UNSUPPORTED_DEVICE", "VR_ERR_INTERNAL", "VR_ERR_DEVICE_CHECK",
    "VR_MAX_RANKS", "VR_SIGNAL_BITS", "VR_COUNTER_BITS", "VR_WIN_DEFAULT", "VR_WIN_COLL_SYMMETRIC", "VR_WIN_STRICT_ORDERING", "VR_WIN_REQUIRED_ALIGNMENT",
    "VR_ACTION_NONE", "VR_SIGNAL_INC", "VR_SIGNAL_ADD", "VR_COUNTER_INC", "VR_VA_SIGNAL_INC", "VR_VA_SIGNAL_ADD",
    "VR_DT_F32", "VR_DT_BF16", "VR_OP_SUM", "VR_COLL_NO_WAIT", "VR_COLL_COPY_ENGINE", "VR_CE_STREAMS",
    "VR_RING_WEAK", "VR_PINGPONG_SAME_XCD", "VR_PINGPONG_WAVES", "VR_DISPATCH_NOALLOC_SCRATCH_BYTES",
    "VR_FENCE_NONE", "VR_FENCE_PUT", "VR_FENCE_GET",
    "VR_ASYNC_TIMEOUT", "VR_ASYNC_CAPACITY", "VR_ASYNC_BAD_EXPERT", "VR_ASYNC_LITMUS",
    # argument structures and action helpers
    "vrCommRequirements", "vrRemoteAction", "vrLocalAction", "vrDevComm", "vrDevWindow",
    "SignalInc", "SignalAdd", "CounterInc", "VASignalInc", "VASignalAdd",
    # entry points
    "vr_error_string", "vr_version", "vr_comm_workspace_bytes", "vr_comm_create", "vr_comm_destroy",
    "vr_comm_get_async_error", "vr_comm_query", "vr_comm_set_litmus", "vr_comm_set_trace",
    "vr_comm_device_view", "vr_window_register", "vr_window_deregister", "vr_window_device_view",
    "vr_put", "vr_get", "vr_signal", "vr_signal_wait", "vr_signal_read", "vr_signal_reset", "vr_signal_expected",
    "vr_va_signal_wait", "vr_va_signal_read", "vr_va_signal_reset",
    "vr_counter_wait", "vr_counter_read", "vr_counter_reset",
    "vr_barrier", "vr_barrier_advance", "vr_barrier_expected",
    "vr_allreduce", "vr_alltoall", "vr_alltoall_sessions", "vr_allgather",
    "vr_dispatch", "vr_dispatch_noalloc", "vr_dispatch_dedup", "vr_combine", "vr_combine_dedup",
    "vr_ring_exchange", "vr_signal_pingpong",
]

# The in-tree build; VRCOMM_LIB may name another build of the same library.
LIB_PATH = os.environ.get("VRCOMM_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvrcomm.so")

VR_OK = 0
VR_ERR_INVALID_ARGUMENT = 1
VR_ERR_INVALID_USAGE = 2
VR_ERR_OUT_OF_RESOURCES = 3
VR_ERR_HIP = 4
VR_ERR_TIMEOUT = 5
VR_ERR_UNSUPPORTED_DEVICE = 6
VR_ERR_INTERNAL = 7
VR_ERR_DEVICE_CHECK = 8

VR_MAX_RANKS = 64
VR_SIGNAL_BITS = 64
VR_COUNTER_BITS = 56
VR_WIN_DEFAULT = 0x0
VR_WIN_COLL_SYMMETRIC = 0x1
VR_WIN_STRICT_ORDERING = 0x2
VR_WIN_REQUIRED_ALIGNMENT = 4096
VR_ACTION_NONE, VR_SIGNAL_INC, VR_SIGNAL_ADD, VR_COUNTER_INC = 0, 1, 2, 3
VR_VA_SIGNAL_INC, VR_VA_SIGNAL_ADD = 4, 5
VR_DT_F32, VR_DT_BF16 = 0, 1
VR_OP_SUM = 0
VR_COLL_NO_WAIT = 0x1
VR_COLL_COPY_ENGINE = 0x4
VR_CE_STREAMS = 8
VR_RING_WEAK = 0x8
VR_PINGPONG_SAME_XCD = 0x10
VR_PINGPONG_WAVES = 0x20
VR_DISPATCH_NOALLOC_SCRATCH_BYTES = 4 << 20
VR_FENCE_NONE, VR_FENCE_PUT, VR_FENCE_GET = 0x0, 0x1, 0x2
VR_ASYNC_TIMEOUT, VR_ASYNC_CAPACITY, VR_ASYNC_BAD_EXPERT, VR_ASYNC_LITMUS = 0x1, 0x2, 0x4, 0x8


class VrError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        name = _error_name(code)
        super().__init__(f"{where}: {name} ({code})")
        self.name = name


class VrLibraryMissing(ImportError):
    pass


class vrCommRequirements(Structure):
    _fields_ = [("signal_count", c_uint32), ("counter_count", c_uint32), ("context_count", c_uint32),
                ("barrier_count", c_uint32)]


class vrDevComm(Structure):
    _fields_ = [("nranks", c_int), ("signal_count", c_uint32), ("counter_count", c_uint32),
                ("barrier_count", c_uint32), ("signals", c_void_p), ("counters", c_void_p),
                ("barriers", c_void_p), ("error", c_void_p)]


class vrDevWindow(Structure):
    _fields_ = [("base", c_void_p * 64), ("bytes", c_uint64)]


class vrRemoteAction(Structure):
    _fields_ = [("kind", c_uint32), ("id", c_uint32), ("value", c_uint64), ("strong", c_uint32),
                ("reserved", c_uint32), ("window", c_void_p), ("offset", c_uint64)]


class vrLocalAction(Structure):
    _fields_ = [("kind", c_uint32), ("id", c_uint32)]


def SignalInc(sig_id: int, strong: bool = True) -> vrRemoteAction:
    return vrRemoteAction(VR_SIGNAL_INC, sig_id, 0, int(strong), 0, None, 0)


def SignalAdd(sig_id: int, value: int, strong: bool = True) -> vrRemoteAction:
    return vrRemoteAction(VR_SIGNAL_ADD, sig_id, value, int(strong), 0, None, 0)


def VASignalInc(window, offset: int, strong: bool = True) -> vrRemoteAction:
    return vrRemoteAction(VR_VA_SIGNAL_INC, 0, 0, int(strong), 0, window, offset)


def VASignalAdd(window, offset: int, value: int, strong: bool = True) -> vrRemoteAction:
    return vrRemoteAction(VR_VA_SIGNAL_ADD, 0, value, int(strong), 0, window, offset)


def CounterInc(cnt_id: int) -> vrLocalAction:
    return vrLocalAction(VR_COUNTER_INC, cnt_id)


_R = c_int  # vrResult_t
_P = c_void_p
# name -> (restype, argtypes); the C declarations in include/vrcomm.h
SYMBOLS = {
    "vr_error_string": (c_char_p, [c_int]),
    "vr_version": (c_int, []),
    "vr_comm_workspace_bytes": (c_size_t, [c_int, POINTER(vrCommRequirements)]),
    "vr_comm_create": (_R, [c_int, POINTER(vrCommRequirements), _P, c_size_t, POINTER(_P)]),
    "vr_comm_destroy": (_R, [_P]),
    "vr_comm_get_async_error": (_R, [_P, POINTER(c_int), POINTER(c_uint32)]),
    "vr_comm_query": (_R, [_P, POINTER(c_int), POINTER(vrCommRequirements)]),
    "vr_comm_set_litmus": (_R, [_P, _P]),
    "vr_comm_set_trace": (_R, [_P, _P, c_size_t]),
    "vr_window_register": (_R, [_P, POINTER(_P), c_size_t, c_uint32, POINTER(_P)]),
    "vr_window_deregister": (_R, [_P, _P]),
    "vr_put": (_R, [_P, c_int, c_int, c_int, _P, c_size_t, _P, c_size_t, c_size_t, vrRemoteAction,
                    vrLocalAction, _P]),
    "vr_get": (_R, [_P, c_int, c_int, c_int, _P, c_size_t, _P, c_size_t, c_size_t, vrLocalAction, _P]),
    "vr_signal": (_R, [_P, c_int, c_int, c_int, vrRemoteAction, _P]),
    "vr_signal_wait": (_R, [_P, c_int, c_uint32, c_uint64, c_int, c_uint64, _P]),
    "vr_signal_read": (_R, [_P, c_int, c_uint32, c_int, POINTER(c_uint64)]),
    "vr_signal_reset": (_R, [_P, c_int, c_uint32, _P]),
    "vr_signal_expected": (_R, [_P, c_int, c_uint32, POINTER(c_uint64)]),
    "vr_counter_wait": (_R, [_P, c_int, c_uint32, c_uint64, c_int, c_uint64, _P]),
    "vr_counter_read": (_R, [_P, c_int, c_uint32, c_int, POINTER(c_uint64)]),
    "vr_counter_reset": (_R, [_P, c_int, c_uint32, _P]),
    "vr_allreduce": (_R, [_P, _P, c_size_t, _P, c_size_t, c_size_t, c_int, c_int, c_uint32, c_uint32, _P]),
    "vr_alltoall": (_R, [_P, _P, c_size_t, _P, c_size_t, c_size_t, c_uint32, c_uint32, _P]),
    "vr_allgather": (_R, [_P, _P, c_size_t, _P, c_size_t, c_size_t, c_uint32, c_uint32, _P]),
    "vr_dispatch": (_R, [_P, _P, c_size_t, c_size_t, _P, c_int, c_int, c_int, _P, c_size_t, c_size_t, _P, _P,
                         _P, c_uint32, c_uint32, c_uint32, _P]),
    "vr_dispatch_noalloc": (_R, [_P, _P, c_size_t, c_size_t, _P, c_int, c_int, c_int, _P, c_size_t, c_size_t, _P,
                                 _P, _P, c_uint32, c_uint32, c_uint32, _P]),
    "vr_combine": (_R, [_P, _P, c_size_t, c_size_t, c_size_t, c_int, _P, _P, _P, c_int, c_int, c_int, _P,
                        c_size_t, c_uint32, c_uint32, _P]),
    "vr_dispatch_dedup": (_R, [_P, _P, c_size_t, c_size_t, _P, c_int, c_int, c_int, _P, c_size_t, c_size_t, _P, _P,
                               _P, _P, c_uint32, c_uint32, c_uint32, _P]),
    "vr_combine_dedup": (_R, [_P, _P, c_size_t, c_size_t, c_size_t, c_int, _P, c_int, _P, c_size_t, c_uint32,
                              c_uint32, _P]),
    "vr_ring_exchange": (_R, [_P, _P, _P, c_size_t, c_size_t, c_int, c_uint32, c_uint32, _P, c_size_t, _P,
                              c_uint32, _P]),
    "vr_signal_pingpong": (_R, [_P, _P, c_size_t, c_size_t, c_uint32, c_uint32, c_uint32, _P]),
    "vr_va_signal_wait": (_R, [_P, _P, c_int, c_size_t, c_uint64, c_int, c_uint64, _P]),
    "vr_comm_device_view": (_R, [_P, POINTER(vrDevComm)]),
    "vr_window_device_view": (_R, [_P, _P, POINTER(vrDevWindow)]),
    "vr_barrier_expected": (_R, [_P, c_uint32, POINTER(c_uint64)]),
    "vr_barrier_advance": (_R, [_P, c_uint32, c_uint64]),
    "vr_barrier": (_R, [_P, c_uint32, c_uint32, c_uint64, _P]),
    "vr_alltoall_sessions": (_R, [_P, _P, c_size_t, _P, c_size_t, c_size_t, c_uint32, c_uint32, c_uint32, _P]),
    "vr_va_signal_read": (_R, [_P, _P, c_int, c_size_t, c_int, POINTER(c_uint64)]),
    "vr_va_signal_reset": (_R, [_P, _P, c_int, c_size_t, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise VrLibraryMissing(f"{LIB_PATH} is not built: run collective_window_put_amd.build.build()")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SYMBOLS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def _error_name(code: int) -> str:
    try:
        return lib().vr_error_string(code).decode()
    except Exception:  # noqa: BLE001 - naming an error must never raise
        return f"code {code}"


def _check(code: int, where: str) -> None:
    if code != VR_OK:
        raise VrError(code, where)


def _ptr(x) -> int:
    """Device address of a tensor (data_ptr) or an int; None -> 0."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _remote(a) -> vrRemoteAction:
    return vrRemoteAction(VR_ACTION_NONE, 0, 0, 0, 0) if a is None else a


def _local(a) -> vrLocalAction:
    return vrLocalAction(VR_ACTION_NONE, 0) if a is None else a


# ---- the C ABI, one function each ----------------------------------------------------------
def vr_error_string(code: int) -> str:
    return lib().vr_error_string(code).decode()


def vr_version() -> int:
    return lib().vr_version()


def vr_comm_workspace_bytes(nranks: int, signal_count: int = 16, counter_count: int = 16,
                            context_count: int = 1, barrier_count: int = 0) -> int:
    q = vrCommRequirements(signal_count, counter_count, context_count, barrier_count)
    return lib().vr_comm_workspace_bytes(nranks, ctypes.byref(q))


def vr_comm_create(nranks: int, signal_count: int = 16, counter_count: int = 16, context_count: int = 1,
                   workspace=None, workspace_bytes: int = 0, barrier_count: int = 0) -> int:
    q = vrCommRequirements(signal_count, counter_count, context_count, barrier_count)
    out = c_void_p()
    _check(lib().vr_comm_create(nranks, ctypes.byref(q), _ptr(workspace) or None, workspace_bytes,
                                ctypes.byref(out)), "vr_comm_create")
    return out.value


def vr_comm_destroy(comm: int) -> None:
    _check(lib().vr_comm_destroy(comm), "vr_comm_destroy")


def vr_comm_get_async_error(comm: int) -> tuple[int, int]:
    code, bits = c_int(), c_uint32()
    _check(lib().vr_comm_get_async_error(comm, ctypes.byref(code), ctypes.byref(bits)), "vr_comm_get_async_error")
    return code.value, bits.value


def vr_comm_query(comm: int) -> tuple[int, tuple[int, int, int, int]]:
    n, q = c_int(), vrCommRequirements()
    _check(lib().vr_comm_query(comm, ctypes.byref(n), ctypes.byref(q)), "vr_comm_query")
    return n.value, (q.signal_count, q.counter_count, q.context_count, q.barrier_count)


def vr_comm_device_view(comm: int) -> vrDevComm:
    out = vrDevComm()
    _check(lib().vr_comm_device_view(comm, ctypes.byref(out)), "vr_comm_device_view")
    return out


def vr_window_device_view(comm: int, window) -> vrDevWindow:
    out = vrDevWindow()
    _check(lib().vr_window_device_view(comm, window, ctypes.byref(out)), "vr_window_device_view")
    return out


def vr_barrier_expected(comm: int, index: int) -> int:
    out = c_uint64()
    _check(lib().vr_barrier_expected(comm, index, ctypes.byref(out)), "vr_barrier_expected")
    return out.value


def vr_barrier_advance(comm: int, index: int, arrivals: int) -> None:
    _check(lib().vr_barrier_advance(comm, index, arrivals), "vr_barrier_advance")


def vr_barrier(comm: int, index: int, fence: int = VR_FENCE_PUT | VR_FENCE_GET, timeout_ns: int = 0,
               stream=None) -> None:
    _check(lib().vr_barrier(comm, index, fence, timeout_ns, _stream(stream)), "vr_barrier")


def vr_window_register(comm: int, bases, nbytes: int, flags: int = VR_WIN_DEFAULT) -> int:
    bases = list(bases)
    nranks, _ = vr_comm_query(comm)
    if len(bases) != nranks:  # the library reads exactly nranks pointers
        raise ValueError(f"vr_window_register: {len(bases)} base pointers for {nranks} ranks")
    arr = (c_void_p * len(bases))(*[_ptr(b) for b in bases])
    out = c_void_p()
    _check(lib().vr_window_register(comm, arr, nbytes, flags, ctypes.byref(out)), "vr_window_register")
    return out.value


def vr_window_deregister(comm: int, win: int) -> None:
    _check(lib().vr_window_deregister(comm, win), "vr_window_deregister")


def vr_put(comm, ctx, rank, peer, dst, dst_off, src, src_off, nbytes, remote=None, local=None, stream=None):
    _check(lib().vr_put(comm, ctx, rank, peer, dst, dst_off, src, src_off, nbytes, _remote(remote), _local(local),
                        _stream(stream)), "vr_put")


def vr_get(comm, ctx, rank, peer, remote_win, remote_off, local_win, local_off, nbytes, local=None, stream=None):
    _check(lib().vr_get(comm, ctx, rank, peer, remote_win, remote_off, local_win, local_off, nbytes, _local(local),
                        _stream(stream)), "vr_get")


def vr_signal(comm, ctx, rank, peer, remote, stream=None):
    _check(lib().vr_signal(comm, ctx, rank, peer, remote, _stream(stream)), "vr_signal")


def vr_signal_wait(comm, rank, sig_id, least, bits=64, timeout_ns=0, stream=None):
    _check(lib().vr_signal_wait(comm, rank, sig_id, least, bits, timeout_ns, _stream(stream)), "vr_signal_wait")


def vr_signal_read(comm, rank, sig_id, bits=64) -> int:
    out = c_uint64()
    _check(lib().vr_signal_read(comm, rank, sig_id, bits, ctypes.byref(out)), "vr_signal_read")
    return out.value


def vr_signal_reset(comm, rank, sig_id, stream=None):
    _check(lib().vr_signal_reset(comm, rank, sig_id, _stream(stream)), "vr_signal_reset")


def vr_va_signal_wait(comm, window, rank, offset, least, bits=64, timeout_ns=0, stream=None):
    _check(lib().vr_va_signal_wait(comm, window, rank, offset, least, bits, timeout_ns, _stream(stream)),
           "vr_va_signal_wait")


def vr_va_signal_read(comm, window, rank, offset, bits=64) -> int:
    out = c_uint64()
    _check(lib().vr_va_signal_read(comm, window, rank, offset, bits, ctypes.byref(out)), "vr_va_signal_read")
    return out.value


def vr_va_signal_reset(comm, window, rank, offset, stream=None):
    _check(lib().vr_va_signal_reset(comm, window, rank, offset, _stream(stream)), "vr_va_signal_reset")


def vr_signal_expected(comm, rank, sig_id) -> int:
    out = c_uint64()
    _check(lib().vr_signal_expected(comm, rank, sig_id, ctypes.byref(out)), "vr_signal_expected")
    return out.value


def vr_counter_wait(comm, rank, cnt_id, least, bits=56, timeout_ns=0, stream=None):
    _check(lib().vr_counter_wait(comm, rank, cnt_id, least, bits, timeout_ns, _stream(stream)), "vr_counter_wait")


def vr_counter_read(comm, rank, cnt_id, bits=56) -> int:
    out = c_uint64()
    _check(lib().vr_counter_read(comm, rank, cnt_id, bits, ctypes.byref(out)), "vr_counter_read")
    return out.value


def vr_counter_reset(comm, rank, cnt_id, stream=None):
    _check(lib().vr_counter_reset(comm, rank, cnt_id, _stream(stream)), "vr_counter_reset")


def vr_allreduce(comm, send, send_off, recv, recv_off, count, dtype, op=VR_OP_SUM, sig=0, flags=0, stream=None):
    _check(lib().vr_allreduce(comm, send, send_off, recv, recv_off, count, dtype, op, sig, flags, _stream(stream)),
           "vr_allreduce")


def vr_alltoall(comm, send, send_off, recv, recv_off, block_bytes, sig=0, flags=0, stream=None):
    _check(lib().vr_alltoall(comm, send, send_off, recv, recv_off, block_bytes, sig, flags, _stream(stream)),
           "vr_alltoall")


def vr_alltoall_sessions(comm, send, send_off, recv, recv_off, block_bytes, sig=0, barrier_index=0, flags=0,
                         stream=None):
    _check(lib().vr_alltoall_sessions(comm, send, send_off, recv, recv_off, block_bytes, sig, barrier_index, flags,
                                      _stream(stream)), "vr_alltoall_sessions")


def vr_allgather(comm, send, send_off, recv, recv_off, bytes_per_rank, sig=0, flags=0, stream=None):
    _check(lib().vr_allgather(comm, send, send_off, recv, recv_off, bytes_per_rank, sig, flags, _stream(stream)),
           "vr_allgather")


def vr_dispatch(comm, x, x_off, row_bytes, topk_idx, T, K, num_experts, recv, recv_off, capacity_rows,
                recv_expert_counts, recv_src, send_pos, sig_counts, sig_rows, flags=0, stream=None):
    _check(lib().vr_dispatch(comm, x, x_off, row_bytes, _ptr(topk_idx), T, K, num_experts, recv, recv_off,
                             capacity_rows, _ptr(recv_expert_counts), _ptr(recv_src), _ptr(send_pos), sig_counts,
                             sig_rows, flags, _stream(stream)), "vr_dispatch")


def vr_comm_set_litmus(comm, litmus=None):
    """Turn the collectives' in-kernel strong-signal litmus on (litmus: a device
    uint64 tensor of 2 words: checks, mismatches) or off (None)."""
    _check(lib().vr_comm_set_litmus(comm, _ptr(litmus) or None), "vr_comm_set_litmus")


def vr_comm_set_trace(comm, stamps=None):
    """Record the dispatch's per-workgroup phase timestamps into `stamps` (a
    device uint64/int64 tensor; 8 words per workgroup), or stop (None)."""
    _check(lib().vr_comm_set_trace(comm, _ptr(stamps) or None, 0 if stamps is None else stamps.numel()),
           "vr_comm_set_trace")


def vr_dispatch_noalloc(comm, x, x_off, row_bytes, topk_idx, T, K, num_experts, recv, recv_off, capacity_rows,
                        recv_expert_counts, recv_src, send_pos, sig_counts, sig_rows, flags=0, stream=None):
    _check(lib().vr_dispatch_noalloc(comm, x, x_off, row_bytes, _ptr(topk_idx), T, K, num_experts, recv, recv_off,
                                     capacity_rows, _ptr(recv_expert_counts), _ptr(recv_src), _ptr(send_pos),
                                     sig_counts, sig_rows, flags, _stream(stream)), "vr_dispatch_noalloc")


def vr_dispatch_dedup(comm, x, x_off, row_bytes, topk_idx, T, K, num_experts, recv, recv_off, capacity_rows,
                      recv_expert_counts, recv_src, recv_experts, send_pos, sig_counts, sig_rows, flags=0,
                      stream=None):
    _check(lib().vr_dispatch_dedup(comm, x, x_off, row_bytes, _ptr(topk_idx), T, K, num_experts, recv, recv_off,
                                   capacity_rows, _ptr(recv_expert_counts), _ptr(recv_src), _ptr(recv_experts),
                                   _ptr(send_pos), sig_counts, sig_rows, flags, _stream(stream)), "vr_dispatch_dedup")


def vr_combine_dedup(comm, y, y_off, y_capacity_rows, row_bytes, dtype, send_pos, T, out, out_off, sig, flags=0,
                     stream=None):
    _check(lib().vr_combine_dedup(comm, y, y_off, y_capacity_rows, row_bytes, dtype, _ptr(send_pos), T, out,
                                  out_off, sig, flags, _stream(stream)), "vr_combine_dedup")


def vr_combine(comm, y, y_off, y_capacity_rows, row_bytes, dtype, topk_idx, weights, send_pos, T, K, num_experts,
               out, out_off, sig, flags=0, stream=None):
    _check(lib().vr_combine(comm, y, y_off, y_capacity_rows, row_bytes, dtype, _ptr(topk_idx), _ptr(weights),
                            _ptr(send_pos), T, K, num_experts, out, out_off, sig, flags, _stream(stream)),
           "vr_combine")


def vr_signal_pingpong(comm, win, off, nbytes, iters, sig=0, flags=0, stream=None):
    _check(lib().vr_signal_pingpong(comm, win, off, nbytes, iters, sig, flags, _stream(stream)), "vr_signal_pingpong")


def vr_ring_exchange(comm, send, recv, put_bytes, puts_per_rank, contexts, sig_base=0, cnt_base=0, sig_window=None,
                     sig_window_off=0, litmus=None, flags=0, stream=None):
    _check(lib().vr_ring_exchange(comm, send, recv, put_bytes, puts_per_rank, contexts, sig_base, cnt_base,
                                  sig_window, sig_window_off, _ptr(litmus) or None, flags, _stream(stream)),
           "vr_ring_exchange")
