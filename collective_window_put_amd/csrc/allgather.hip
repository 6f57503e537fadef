// AllGather over symmetric windows.
//
// Symmetric page (zwxr.cn/news/250719), AllGather example: every rank's
// receive buffer holds R segments, segment k being rank k's contribution.
// Here the put of source s to each destination d is split into 4 KiB tiles;
// a workgroup reads its tile of s once and stores it into all R receive
// windows (one load, R stores: the operation is write-bound). The workgroup
// completing source s's relay applies one SignalInc at every rank, so each
// rank's signal rises by R. The last R workgroups of the grid are the
// receivers' waits. Measured on 16 ranks x 64 MiB: 4 KiB tiles 3.35 ms,
// 8 KiB 3.43 ms, 16 KiB 3.48 ms.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "vr_device.hpp"
#include "vr_internal.hpp"

namespace vr {
namespace {

constexpr uint32_t kTile = 4096;
constexpr int kU = kTile / (256 * 16);

struct AGArgs {
  WinTab send, recv;
  U64Tab target;
  uint64_t send_off, recv_off, bytes;
  uint64_t* sig;
  uint32_t sig_stride;
  uint32_t tiles;      // tiles per source
  uint32_t* relay;     // [R] counters, rstride words apart
  uint32_t rstride;
  uint32_t* err;
  uint64_t timeout_ns;
  uint64_t* lit;       // litmus words [2], or null
  uint64_t* lit_last;  // [R]: tile that completed source s's relay
  uint32_t lit_seed;
  int R;
};

// Receiver d, litmus on: the tile that completed each source's relay, whole,
// then one seeded 16-byte sample in every tile of every source, each against
// the source's send bytes.
__device__ void ag_litmus(const AGArgs& a, uint32_t R, uint32_t d) {
  const uint32_t tid = threadIdx.x;
  uint32_t checks = 0, bad = 0;
  auto check = [&](uint32_t s, uint64_t o, uint32_t n) {
    ++checks;
    bad += !equal_upto16(a.recv.p[d] + a.recv_off + (uint64_t)s * a.bytes + o, a.send.p[s] + a.send_off + o, n);
  };
  if (a.bytes) {
    for (uint32_t s = 0; s < R; ++s) {
      const uint64_t t0 = load_relaxed_u64(a.lit_last + s) * kTile;
      if (t0 >= a.bytes) {
        if (tid == 0) ++checks, ++bad;
        continue;
      }
      const uint64_t n = std::min<uint64_t>(kTile, a.bytes - t0);
      for (uint64_t o = (uint64_t)tid * 16; o < n; o += 256 * 16)
        check(s, t0 + o, static_cast<uint32_t>(std::min<uint64_t>(16, n - o)));
    }
    for (uint32_t p = tid; p < R * a.tiles; p += 256) {
      const uint32_t s = p % R;
      const uint64_t t0 = (uint64_t)(p / R) * kTile;
      const uint32_t n = static_cast<uint32_t>(std::min<uint64_t>(kTile, a.bytes - t0));
      const uint32_t o = (mix32(a.lit_seed + p * 0x9E3779B9u) % n) & ~15u;
      check(s, t0 + o, std::min(16u, n - o));
    }
  }
  litmus_report(a.lit, a.err, checks, bad);
}

template <int RT, bool ALIGNED>
__global__ __launch_bounds__(256) void k_allgather(const AGArgs a) {
  const uint32_t R = RT ? RT : a.R;
  const uint32_t nwork = R * a.tiles;
  const uint32_t b = blockIdx.x;
  if (b >= nwork) {
    const uint32_t d = b - nwork;
    if (!a.lit) {
      if (threadIdx.x == 0)
        wait_reached(a.sig + (size_t)d * a.sig_stride, a.target.v[d], 64, a.timeout_ns, a.err, VR_ASYNC_TIMEOUT);
    } else if (receiver_wait(a.sig + (size_t)d * a.sig_stride, a.target.v[d], a.timeout_ns, a.err)) {
      ag_litmus(a, R, d);
    }
    return;
  }
  const uint32_t s = b % R, tile = b / R;  // consecutive workgroups: different sources (even relay load)
  const uint64_t t0 = (uint64_t)tile * kTile;
  if (t0 < a.bytes) {
    const uint32_t n = static_cast<uint32_t>(std::min<uint64_t>(kTile, a.bytes - t0));
    const char* src = a.send.p[s] + a.send_off + t0;
    const uint64_t doff = a.recv_off + (uint64_t)s * a.bytes + t0;
    if (ALIGNED && n == kTile) {
      const v4u* sv = reinterpret_cast<const v4u*>(src);
      v4u v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = load16_stream(sv + u * 256 + threadIdx.x);
      for (uint32_t d = 0; d < R; ++d) {
        const __amdgpu_buffer_rsrc_t rd = rsrc(a.recv.p[d] + doff, kTile);
#pragma unroll
        for (int u = 0; u < kU; ++u) store16_agent(rd, (u * 256 + threadIdx.x) * 16, v[u]);
      }
    } else {
      for (uint32_t d = 0; d < R; ++d) copy_any<4>(a.recv.p[d] + doff, src, n, threadIdx.x, 256);
    }
  }
  wg_stores_complete();
  if (threadIdx.x == 0 && relay_arrive(a.relay + s * a.rstride, a.tiles, false)) {
    if (a.lit) litmus_record(a.lit_last + s, tile);
    for (uint32_t d = 0; d < R; ++d) atomic_add_u64(a.sig + (size_t)d * a.sig_stride, 1ull);
  }
}

template <int RT, bool AL>
void launch_t(const AGArgs& a, uint32_t grid, hipStream_t st) {
  hipLaunchKernelGGL((k_allgather<RT, AL>), dim3(grid), dim3(256), 0, st, a);
}

}  // namespace

vrResult_t launch_allgather(vrComm* c, const vrWindow* send, size_t send_off, const vrWindow* recv, size_t recv_off,
                            size_t bytes, uint32_t sig, const U64Tab& target, bool wait, hipStream_t st) {
  AGArgs a;
  const int R = c->nranks;
  for (int r = 0; r < VR_MAX_RANKS; ++r) {
    a.send.p[r] = send->base[r];
    a.recv.p[r] = recv->base[r];
  }
  a.target = target;
  a.send_off = send_off;
  a.recv_off = recv_off;
  a.bytes = bytes;
  a.sig = c->sig + sig;
  a.sig_stride = c->req.signal_count;
  const uint64_t tiles = std::max<uint64_t>(1, (bytes + kTile - 1) / kTile);
  if (tiles * R > 0x7FFFFFFFull) return VR_ERR_INVALID_ARGUMENT;
  a.tiles = static_cast<uint32_t>(tiles);
  a.relay = c->relay + kRelayColl;
  a.rstride = relay_stride(R);
  a.err = c->err;
  a.timeout_ns = kDefaultTimeoutNs;
  a.lit = c->litmus;
  a.lit_last = c->lit_last;
  a.lit_seed = c->lit_seed++;
  a.R = R;
  const bool aligned = ((send_off | recv_off | bytes) & 15) == 0;
  const uint32_t grid = a.tiles * R + (wait ? R : 0);
  if (!aligned) launch_t<0, false>(a, grid, st);
  else if (R == 16) launch_t<16, true>(a, grid, st);
  else if (R == 8) launch_t<8, true>(a, grid, st);
  else if (R == 4) launch_t<4, true>(a, grid, st);
  else launch_t<0, true>(a, grid, st);
  return hipGetLastError() == hipSuccess ? VR_OK : VR_ERR_HIP;
}

}  // namespace vr
