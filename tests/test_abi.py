"""The C-ABI library loads, exports every function include/vrcomm.h declares,
and rejects bad arguments before touching a GPU (runs without a GPU)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import collective_window_put_amd as vr
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "vrcomm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vr_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(vr.LIB_PATH):
        from collective_window_put_amd.build import build
        build()
    return vr.lib()


def test_header_declares_the_binding_symbols():
    assert _declared_functions() == sorted(vr.SYMBOLS)


def test_binding_exports_every_declared_function_and_constant():
    # each C entry point has a wrapper of the same name that the package exports
    for name in _declared_functions():
        assert callable(getattr(vr, name, None)), name
        assert name in vr.__all__, name
    # each constant the header defines has the same value in the binding, exported
    text = open(HEADER).read()
    defines = re.findall(r"^#define\s+(VR_[A-Z0-9_]+)\s+(\(?[0-9xXa-fA-F]+u?(?:\s*<<\s*[0-9]+)?\)?)", text, flags=re.M)
    assert len(defines) == len(re.findall(r"^#define\s+VR_", text, flags=re.M))  # every one parsed
    for name, expr in defines:
        value = eval(re.sub(r"(?<=[0-9a-fA-F])u", "", expr), {"__builtins__": {}})  # literals and << only
        assert getattr(vr, name) == value, name
        assert name in vr.__all__, name
    for name in vr.__all__:
        assert hasattr(vr, name), name


def test_library_exports_every_declared_function(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", vr.LIB_PATH], capture_output=True, text=True, check=True)
    exported = {line.split()[-1] for line in out.stdout.splitlines() if " T " in line}
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_library_is_built_for_gfx950_only(lib):
    # the offload bundle embedded in our own library names its device targets
    blob = open(vr.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa-[-a-z]*(gfx[0-9a-z]+)", blob))
    assert targets == {b"gfx950"}


def test_error_strings_and_version(lib):
    assert vr.vr_error_string(vr.VR_OK) == "VR_OK"
    assert vr.vr_error_string(vr.VR_ERR_TIMEOUT) == "VR_ERR_TIMEOUT"
    assert vr.vr_error_string(12345) == "VR_ERR_UNKNOWN"
    assert vr.vr_version() >= 100


def test_workspace_bytes_validation(lib):
    assert vr.vr_comm_workspace_bytes(0) == 0
    assert vr.vr_comm_workspace_bytes(65) == 0
    assert vr.vr_comm_workspace_bytes(4, signal_count=0) == 0
    assert vr.vr_comm_workspace_bytes(4, context_count=0) == 0
    n = vr.vr_comm_workspace_bytes(8, signal_count=16, counter_count=16)
    assert n >= 8 * 16 * 8 * 2 and n % 256 == 0


def test_argument_errors_without_gpu(lib):
    for bad in (0, -1, 65):
        with pytest.raises(vr.VrError) as e:
            vr.vr_comm_create(bad)
        assert e.value.code == vr.VR_ERR_INVALID_ARGUMENT
    with pytest.raises(vr.VrError) as e:
        vr.vr_comm_create(4, signal_count=0)
    assert e.value.code == vr.VR_ERR_INVALID_ARGUMENT
    # handles that were never created are rejected, not dereferenced
    for fn, args in ((vr.vr_comm_destroy, (0x1234,)), (vr.vr_comm_query, (0,)),
                     (vr.vr_signal_read, (0x10, 0, 0)), (vr.vr_window_deregister, (0x10, 0x20)),
                     (vr.vr_combine, (0x10, 0x20, 0, 1, 16, vr.VR_DT_BF16, None, None, None, 1, 1, 8, 0x30, 0, 0, 0, 0))):
        with pytest.raises(vr.VrError) as e:
            fn(*args)
        assert e.value.code == vr.VR_ERR_INVALID_ARGUMENT
    rc = lib.vr_allreduce(None, None, 0, None, 0, 0, 0, 0, 0, 0, None)
    assert rc == vr.VR_ERR_INVALID_ARGUMENT
    # the communicator switches and the allocation-free dispatch refuse unknown handles too
    assert lib.vr_comm_set_litmus(0x10, None) == vr.VR_ERR_INVALID_ARGUMENT
    assert lib.vr_comm_set_trace(0x10, None, 0) == vr.VR_ERR_INVALID_ARGUMENT
    assert lib.vr_dispatch_noalloc(0x10, 0x20, 0, 16, None, 0, 1, 8, 0x30, 0, 0, None, None, None, 0, 1, 0,
                                   None) == vr.VR_ERR_INVALID_ARGUMENT


def test_struct_layouts_match_header():
    assert ctypes.sizeof(vr.vrRemoteAction) == 40
    assert ctypes.sizeof(vr.vrLocalAction) == 8
    assert ctypes.sizeof(vr.vrCommRequirements) == 16
    assert ctypes.sizeof(vr.vrDevComm) == 48
    assert ctypes.sizeof(vr.vrDevWindow) == 64 * 8 + 8


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(vr, "_lib", None)
    monkeypatch.setattr(vr, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(vr.VrLibraryMissing):
        vr.vr_version()


USER_KERNEL = r"""
#include "vrcomm_device.hpp"
// a user kernel: each workgroup r puts its block to rank (r+1) % R, signals it,
// then all ranks meet at a barrier session with a Put fence
__global__ void ring_once(vrDevComm c, vrDevWindow w, uint64_t block, uint64_t bar_base) {
  const int r = blockIdx.x, peer = (r + 1) % c.nranks;
  vrdev::put_wg(w, peer, block, w, r, 0, block);
  vrdev::publish_wg();
  if (threadIdx.x == 0) vrdev::signal_add(vrdev::signal_word(c, peer, 0), 1);
  vrdev::barrier_sync_wg(vrdev::barrier_word(c, 0), bar_base + c.nranks, VR_FENCE_PUT, 0, c.error);
  if (threadIdx.x == 0) vrdev::wait_word(vrdev::signal_word(c, r, 0), 1, 64, 0, c.error);
}
// the wave form: each wave of workgroup r puts its own piece and signals it
__global__ void ring_waves(vrDevComm c, vrDevWindow w, uint64_t piece) {
  const int r = blockIdx.x, peer = (r + 1) % c.nranks, wv = threadIdx.x / 64;
  vrdev::put_wave(w, peer, (uint64_t)wv * piece, w, r, (uint64_t)wv * piece, piece);
  vrdev::publish_wave();
  if (threadIdx.x % 64 == 0) vrdev::signal_add(vrdev::signal_word(c, peer, 1), 1);
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_client_compiles_against_the_header():
    # the header is plain C: the C client compiles with gcc in C11 mode
    src = os.path.join(ROOT, "tests", "native", "allreduce_worked_example.c")
    cmd = ["gcc", "-std=c11", "-fsyntax-only", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_device_header_compiles_in_a_user_kernel(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    src = tmp_path / "user.hip"
    src.write_text(USER_KERNEL)
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-I", inc, "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops", "-c", str(src), "-o", str(tmp_path / "user.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
