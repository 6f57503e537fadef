// Equal-block AlltoAll over symmetric windows.
//
// GIN page (lpnh.cn/news/2681042), section "pure-GIN AlltoAll kernel": every
// rank puts the block at send offset peer*size to every peer at receive
// offset my_rank*size, each put carrying a SignalInc, and the receiver waits
// until its signal has grown by nRanks. Here all R ranks run in one launch:
// the put of block (s, d) is split into 16 KiB tiles, one per workgroup; the
// workgroup that completes the block's relay applies its SignalInc at d. The
// last R workgroups of the grid are the receivers' waits; dispatch order puts
// them after every tile workgroup, and tile workgroups never wait, so the
// waits always end.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "vr_device.hpp"
#include "vr_internal.hpp"

namespace vr {
namespace {

constexpr uint32_t kTile = 32768;
constexpr int kU = kTile / (256 * 16);

struct A2AArgs {
  WinTab send, recv;
  U64Tab target;
  uint64_t send_off, recv_off, block;
  uint64_t* sig;         // &sig[0][id]
  uint32_t sig_stride;   // signals per rank
  uint32_t tiles;        // tiles per block
  uint32_t* relay;       // [R*R] counters, rstride words apart
  uint32_t rstride;
  uint32_t* err;
  uint64_t timeout_ns;
  uint64_t* lit;       // litmus words [2], or null
  uint64_t* lit_last;  // [R][R]: tile that completed block (s, d)'s relay
  uint32_t lit_seed;
  int R;
  int wait;
};

// Receiver d, litmus on: the tile that completed each block's relay, whole,
// then one seeded 16-byte sample in every tile of every block aimed at d,
// each against the sender's bytes.
__device__ void a2a_litmus(const A2AArgs& a, uint32_t d) {
  const uint32_t R = a.R, tid = threadIdx.x;
  uint32_t checks = 0, bad = 0;
  auto check = [&](uint32_t s, uint64_t o, uint32_t n) {
    ++checks;
    bad += !equal_upto16(a.recv.p[d] + a.recv_off + (uint64_t)s * a.block + o,
                         a.send.p[s] + a.send_off + (uint64_t)d * a.block + o, n);
  };
  if (a.block) {
    for (uint32_t s = 0; s < R; ++s) {
      const uint64_t t0 = load_relaxed_u64(a.lit_last + (size_t)s * R + d) * kTile;
      if (t0 >= a.block) {  // no record of a relay that must have completed
        if (tid == 0) ++checks, ++bad;
        continue;
      }
      const uint64_t n = std::min<uint64_t>(kTile, a.block - t0);
      for (uint64_t o = (uint64_t)tid * 16; o < n; o += 256 * 16)
        check(s, t0 + o, static_cast<uint32_t>(std::min<uint64_t>(16, n - o)));
    }
    for (uint32_t p = tid; p < R * a.tiles; p += 256) {
      const uint32_t s = p % R;
      const uint64_t t0 = (uint64_t)(p / R) * kTile;
      const uint32_t n = static_cast<uint32_t>(std::min<uint64_t>(kTile, a.block - t0));
      const uint32_t o = (mix32(a.lit_seed + p * 0x9E3779B9u) % n) & ~15u;
      check(s, t0 + o, std::min(16u, n - o));
    }
  }
  litmus_report(a.lit, a.err, checks, bad);
}

__global__ __launch_bounds__(256) void k_alltoall(const A2AArgs a) {
  const uint32_t R = a.R;
  const uint32_t nwork = R * R * a.tiles;
  const uint32_t b = blockIdx.x;
  if (b >= nwork) {  // receiver d waits for R SignalIncs
    const uint32_t d = b - nwork;
    if (!a.lit) {
      if (threadIdx.x == 0)
        wait_reached(a.sig + (size_t)d * a.sig_stride, a.target.v[d], 64, a.timeout_ns, a.err, VR_ASYNC_TIMEOUT);
    } else if (receiver_wait(a.sig + (size_t)d * a.sig_stride, a.target.v[d], a.timeout_ns, a.err)) {
      a2a_litmus(a, d);
    }
    return;
  }
  const uint32_t blk = b % (R * R), tile = b / (R * R);
  const uint32_t s = blk / R, d = blk % R;
  const uint64_t t0 = (uint64_t)tile * kTile;
  if (t0 < a.block) {
    const uint32_t n = static_cast<uint32_t>(std::min<uint64_t>(kTile, a.block - t0));
    const char* src = a.send.p[s] + a.send_off + (uint64_t)d * a.block + t0;
    char* dst = a.recv.p[d] + a.recv_off + (uint64_t)s * a.block + t0;
    copy_any<kU>(dst, src, n, threadIdx.x, 256);
  }
  wg_stores_complete();
  if (threadIdx.x == 0 && relay_arrive(a.relay + blk * a.rstride, a.tiles, false)) {
    if (a.lit) litmus_record(a.lit_last + blk, tile);
    atomic_add_u64(a.sig + (size_t)d * a.sig_stride, 1ull);  // SignalInc at d
  }
}

}  // namespace

vrResult_t launch_alltoall(vrComm* c, const vrWindow* send, size_t send_off, const vrWindow* recv, size_t recv_off,
                           size_t block, uint32_t sig, const U64Tab& target, bool wait, hipStream_t st) {
  A2AArgs a;
  const int R = c->nranks;
  for (int r = 0; r < VR_MAX_RANKS; ++r) {
    a.send.p[r] = send->base[r];
    a.recv.p[r] = recv->base[r];
  }
  a.target = target;
  a.send_off = send_off;
  a.recv_off = recv_off;
  a.block = block;
  a.sig = c->sig + sig;
  a.sig_stride = c->req.signal_count;
  const uint64_t tiles = std::max<uint64_t>(1, (block + kTile - 1) / kTile);
  if (tiles * R * R > 0x7FFFFFFFull) return VR_ERR_INVALID_ARGUMENT;
  a.tiles = static_cast<uint32_t>(tiles);
  a.relay = c->relay + kRelayColl;
  a.rstride = relay_stride(R * R);
  a.err = c->err;
  a.timeout_ns = kDefaultTimeoutNs;
  a.lit = c->litmus;
  a.lit_last = c->lit_last;
  a.lit_seed = c->lit_seed++;
  a.R = R;
  a.wait = wait;
  const uint32_t grid = a.tiles * R * R + (wait ? R : 0);
  hipLaunchKernelGGL(k_alltoall, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? VR_OK : VR_ERR_HIP;
}

}  // namespace vr
