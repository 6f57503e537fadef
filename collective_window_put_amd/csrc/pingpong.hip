// Signal ping-pong between two ranks, written with the public device API
// (include/vrcomm_device.hpp): the control path of a small put.
//
// GIN page (lpnh.cn/news/2681042): a put with a SignalInc at the peer, and a
// wait for a signal value (signal methods). GDA survey
// (10100.com/article/158785524), opening section: for messages of a few
// hundred bytes the control path, not the data, sets the time.
//
// One kernel, two live workgroups: rank 0's (workgroup 0) and rank 1's
// (workgroup 1, on the next XCD, or workgroup 8, on the same XCD, since
// workgroup b runs on XCD b mod 8; the workgroups between exit at once).
// Round i: rank 0 puts its bytes to rank 1 and signals; rank 1 waits for the
// signal, acquires, puts its (just received) bytes back to rank 0 one message
// further on and signals; rank 0 waits. Both workgroups are resident from the
// start (a grid of at most 9), and every wait has a timeout, so the kernel
// always ends. With VR_PINGPONG_WAVES the two ranks are the two waves of one
// workgroup instead (k_pingpong_waves).
#include <hip/hip_runtime.h>

#include "vr_device.hpp"
#include "vr_internal.hpp"
#include "vrcomm_device.hpp"

namespace vr {
namespace {

struct PPArgs {
  vrDevWindow win;
  vrDevComm comm;
  uint64_t off, bytes, timeout_ns;
  uint64_t base[2];  // the ranks' signal values before the exchange
  uint32_t iters, sig, peer_wg;
};

__global__ __launch_bounds__(64) void k_pingpong(const PPArgs a) {
  const uint32_t b = blockIdx.x;
  if (b != 0 && b != a.peer_wg) return;
  const int rank = b == 0 ? 0 : 1, peer = 1 - rank;
  uint64_t* mine = vrdev::signal_word(a.comm, rank, a.sig);
  uint64_t* theirs = vrdev::signal_word(a.comm, peer, a.sig);
  __shared__ int ok;
  for (uint32_t i = 0; i < a.iters; ++i) {
    if (rank == 1) {  // wait for ping i, then send its bytes back
      if (threadIdx.x == 0) ok = vrdev::wait_word(mine, a.base[1] + i + 1, 64, a.timeout_ns, a.comm.error);
      __syncthreads();
      if (!ok) return;
      vrdev::put_wg(a.win, 0, a.off + a.bytes, a.win, 1, a.off, a.bytes);
    } else {
      vrdev::put_wg(a.win, 1, a.off, a.win, 0, a.off, a.bytes);
    }
    vrdev::publish_wg();
    if (threadIdx.x == 0) vrdev::signal_add(theirs, 1);  // SignalInc at the peer
    if (rank == 0) {  // wait for pong i
      if (threadIdx.x == 0) ok = vrdev::wait_word(mine, a.base[0] + i + 1, 64, a.timeout_ns, a.comm.error, false);
      __syncthreads();
      if (!ok) return;
    }
  }
}

// The same exchange between the two waves of one workgroup (one CU): wave 0
// is rank 0 and wave 1 rank 1, each putting, publishing and signalling with
// the wave-level device API and never meeting the other at a barrier. The
// waiting lane's result reaches its wave through a lane shuffle.
__global__ __launch_bounds__(128) void k_pingpong_waves(const PPArgs a) {
  const int rank = static_cast<int>(threadIdx.x >> 6), peer = 1 - rank;
  const uint32_t lane = threadIdx.x & 63u;
  uint64_t* mine = vrdev::signal_word(a.comm, rank, a.sig);
  uint64_t* theirs = vrdev::signal_word(a.comm, peer, a.sig);
  for (uint32_t i = 0; i < a.iters; ++i) {
    if (rank == 1) {  // wait for ping i, then send its bytes back
      int ok = 0;
      if (lane == 0) ok = vrdev::wait_word(mine, a.base[1] + i + 1, 64, a.timeout_ns, a.comm.error);
      if (!__shfl(ok, 0)) return;
      vrdev::put_wave(a.win, 0, a.off + a.bytes, a.win, 1, a.off, a.bytes);
    } else {
      vrdev::put_wave(a.win, 1, a.off, a.win, 0, a.off, a.bytes);
    }
    vrdev::publish_wave();
    if (lane == 0) vrdev::signal_add(theirs, 1);  // SignalInc at the peer
    if (rank == 0) {  // wait for pong i
      int ok = 0;
      if (lane == 0) ok = vrdev::wait_word(mine, a.base[0] + i + 1, 64, a.timeout_ns, a.comm.error, false);
      if (!__shfl(ok, 0)) return;
    }
  }
}

}  // namespace

vrResult_t launch_pingpong(vrComm* c, const vrWindow* w, size_t off, size_t bytes, uint32_t iters, uint32_t sig,
                           const uint64_t base[2], bool same_xcd, bool waves, hipStream_t st) {
  PPArgs a;
  a.win = device_view(w);
  a.comm = device_view(c);
  a.off = off;
  a.bytes = bytes;
  a.timeout_ns = kDefaultTimeoutNs;
  a.base[0] = base[0];
  a.base[1] = base[1];
  a.iters = iters;
  a.sig = sig;
  a.peer_wg = same_xcd ? 8 : 1;
  if (waves) hipLaunchKernelGGL(k_pingpong_waves, dim3(1), dim3(128), 0, st, a);
  else hipLaunchKernelGGL(k_pingpong, dim3(a.peer_wg + 1), dim3(64), 0, st, a);
  return hipGetLastError() == hipSuccess ? VR_OK : VR_ERR_HIP;
}

}  // namespace vr
