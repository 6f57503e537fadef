// Barrier sessions, and the AlltoAll in the structure of the pages' pure-GIN
// kernel, written with the public device API (include/vrcomm_device.hpp).
//
// GIN page (lpnh.cn/news/2681042), ncclGinBarrierSession: a sync releases
// the members once all have arrived; its fence level selects what must have
// drained (Put: puts aimed at the caller are visible; Get: the caller's gets
// have landed; None: nothing). The AlltoAll example enters through a sync
// with no fence, puts one block per peer with a weak SignalInc, lets one
// receiving group wait for nRanks signals, and leaves through a second sync.
//
// Here every rank is a set of workgroups in one launch. Grid order:
//   [R entry workgroups][R*R*tiles put workgroups][R receiver workgroups]
// Entry workgroup r is rank r's member of the first sync. Put workgroups wait
// until the first sync has completed (the slot reached base + R), put their
// tile, and the workgroup completing block (s, d) applies the weak SignalInc
// at d. Receiver d waits for its signal, then is rank d's member of the second
// sync. Every workgroup that waits is placed after the workgroups it waits
// for, and put workgroups never wait on later ones, so every wait ends.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "vr_device.hpp"
#include "vr_internal.hpp"
#include "vrcomm_device.hpp"

namespace vr {
namespace {

constexpr uint32_t kTile = 32768;

__global__ __launch_bounds__(64) void k_barrier(uint64_t* slot, uint64_t target, uint32_t fence, uint64_t timeout_ns,
                                                uint32_t* err) {
  vrdev::barrier_sync_wg(slot, target, fence, timeout_ns, err);
}

struct SessArgs {
  vrDevWindow send, recv;
  vrDevComm comm;
  U64Tab target;
  uint64_t send_off, recv_off, block;
  uint64_t bar_base;
  uint32_t sig, index, tiles;
  uint32_t* relay;  // [R*R] counters, rstride words apart
  uint32_t rstride;
};

__global__ __launch_bounds__(256) void k_alltoall_sessions(const SessArgs a) {
  const uint32_t R = a.comm.nranks;
  const uint32_t nput = R * R * a.tiles;
  const uint32_t b = blockIdx.x;
  uint64_t* slot = vrdev::barrier_word(a.comm, a.index);
  if (b < R) {  // rank b enters
    vrdev::barrier_sync_wg(slot, a.bar_base + R, VR_FENCE_NONE, 0, a.comm.error);
    return;
  }
  if (b >= R + nput) {  // rank d waits for its R signals, then leaves
    const uint32_t d = b - R - nput;
    if (threadIdx.x == 0)
      vrdev::wait_word(vrdev::signal_word(a.comm, d, a.sig), a.target.v[d], 64, 0, a.comm.error);
    vrdev::barrier_sync_wg(slot, a.bar_base + 2 * R, VR_FENCE_NONE, 0, a.comm.error);
    return;
  }
  const uint32_t w = b - R;
  const uint32_t blk = w % (R * R), tile = w / (R * R);  // consecutive workgroups: different blocks
  const uint32_t s = blk / R, d = blk % R;
  // entry sync done; the sends were written before the kernel, so no acquire
  if (threadIdx.x == 0) vrdev::wait_word(slot, a.bar_base + R, 64, 0, a.comm.error, false);
  __syncthreads();
  const uint64_t t0 = (uint64_t)tile * kTile;
  if (t0 < a.block)
    vrdev::put_wg(a.recv, d, a.recv_off + (uint64_t)s * a.block + t0, a.send, s,
                  a.send_off + (uint64_t)d * a.block + t0, std::min<uint64_t>(kTile, a.block - t0));
  vrdev::publish_wg();
  if (threadIdx.x == 0 && relay_arrive(a.relay + blk * a.rstride, a.tiles, false))
    vrdev::signal_add(vrdev::signal_word(a.comm, d, a.sig), 1);  // weak SignalInc at d
}

}  // namespace

vrResult_t launch_barrier(vrComm* c, uint32_t index, uint64_t target, uint32_t fence, uint64_t timeout_ns,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_barrier, dim3(c->nranks), dim3(64), 0, st, c->bar + index, target, fence, timeout_ns, c->err);
  return hipGetLastError() == hipSuccess ? VR_OK : VR_ERR_HIP;
}

vrResult_t launch_alltoall_sessions(vrComm* c, const vrDevWindow& send, size_t send_off, const vrDevWindow& recv,
                                    size_t recv_off, size_t block, uint32_t sig, const U64Tab& target, uint32_t index,
                                    uint64_t bar_base, hipStream_t st) {
  SessArgs a;
  a.send = send;
  a.recv = recv;
  a.comm = device_view(c);
  a.target = target;
  a.send_off = send_off;
  a.recv_off = recv_off;
  a.block = block;
  a.bar_base = bar_base;
  a.sig = sig;
  a.index = index;
  const uint64_t tiles = std::max<uint64_t>(1, (block + kTile - 1) / kTile);
  const int R = c->nranks;
  if (tiles * R * R + 2 * R > 0x7FFFFFFFull) return VR_ERR_INVALID_ARGUMENT;
  a.tiles = static_cast<uint32_t>(tiles);
  a.relay = c->relay + kRelayColl;
  a.rstride = relay_stride(R * R);
  const uint32_t grid = R + a.tiles * R * R + R;
  hipLaunchKernelGGL(k_alltoall_sessions, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? VR_OK : VR_ERR_HIP;
}

}  // namespace vr
