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
// 8 KiB 3.43 ms, 16 KiB 3.48 ms. From 64 KiB per source up (16-byte
// aligned), the piece form below runs instead.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "vr_device.hpp"
#include "vr_internal.hpp"

namespace vr {
namespace {

constexpr uint32_t kTile = 4096;
constexpr int kU = kTile / (256 * 16);
constexpr uint32_t kPiece = 1024;    // piece form: bytes of one source per workgroup
constexpr uint32_t kPieceFan = 8;    // piece form: first-level relay counters per (source, XCD)

struct AGArgs {
  WinTab send, recv;
  U64Tab target;
  uint64_t send_off, recv_off, bytes;
  uint64_t* sig;
  uint32_t sig_stride;
  uint32_t tiles;      // tiles per source
  uint32_t pieces;     // piece form: pieces per source (0: tile form)
  uint32_t nwg;        // work workgroups (R * tiles, or R * pieces)
  uint32_t* relay;     // [R] counters, rstride words apart
  uint32_t rstride;
  uint32_t* err;
  uint64_t timeout_ns;
  uint64_t* lit;       // litmus words [2], or null
  uint64_t* lit_last;  // [R]: byte offset of the tile or piece that completed source s's relay
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
      const uint64_t t0 = load_relaxed_u64(a.lit_last + s);
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

// Piece form, used when the offsets and the size are 16-byte aligned and
// each source holds at least 64 pieces of kPiece bytes (the last may be
// partial). Workgroup b takes piece b mod (pieces per source) of source
// b div (pieces per source), so a source's pieces are consecutive in the
// grid and at any time the chip writes one narrow band of each receive
// window. Wave 0 loads the piece
// (64 lanes x 16 bytes) into LDS; after a barrier wave w stores it to ranks
// w, w + 4, ...: four stores per thread for R = 16, and 16 KiB written per
// workgroup. Measured stand-alone at 16 ranks x 64 MiB, back to back on one
// machine: 3.08-3.10 ms against 3.48 ms for the tile form's data path. Every
// wave loading the piece itself was as fast without a relay (3.07 ms) but
// 3.27-3.28 ms with one. The relay has three levels: (source, XCD, k) with
// k = (b / 8) mod kPieceFan, then (source, XCD), then source; one counter
// per source took 6.4 ms (arrivals from every XCD).
template <int RT>
__device__ void ag_piece(const AGArgs& a, uint32_t R, uint32_t b) {
  constexpr int kPer = RT ? (RT + 3) / 4 : VR_MAX_RANKS / 4;  // ranks per wave
  const uint32_t pps = a.pieces;
  const uint32_t s = b / pps;
  const uint64_t off = (uint64_t)(b % pps) * kPiece;
  const uint32_t n = static_cast<uint32_t>(std::min<uint64_t>(kPiece, a.bytes - off));  // a multiple of 16
  __shared__ v4u buf[kPiece / 16];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // this wave's store addresses, computed before the barrier: with the
  // pointer (or offset) loads inside the store loop, each store waited for
  // one (measured 3.16 against 3.06 ms at 16 x 64 MiB)
  const uint64_t doff = a.recv_off + (uint64_t)s * a.bytes + off;
  char* dst[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    dst[j] = w + 4 * j < R ? a.recv.p[w + 4 * j] + doff : nullptr;
    asm volatile("" : "+s"(dst[j]));  // keeps the address computed here, above the barrier
  }
  if (w == 0 && lane * 16u < n)
    buf[lane] = load16_stream(reinterpret_cast<const v4u*>(a.send.p[s] + a.send_off + off) + lane);
  __syncthreads();
  const v4u v = buf[lane];
#pragma unroll
  for (int j = 0; j < kPer; ++j)  // lanes past a partial last piece fall outside the descriptor: dropped
    if (w + 4 * j < R) store16_agent(rsrc(dst[j], n), lane * 16u, v);
  wg_stores_complete();
  if (threadIdx.x == 0) {
    // counters of one source sit R apart, so those hit together are spread.
    // First level: the source's pieces b with b mod 8F = 8k + x (F =
    // kPieceFan); with 64 pieces or more every (x, k) has at least one.
    const uint32_t x = b & 7u, k = (b >> 3) & (kPieceFan - 1), r = 8 * k + x, m = 8 * kPieceFan;
    const uint32_t lo = s * pps, hi = lo + pps;
    auto upto = [&](uint32_t e) { return e > r ? (e - 1 - r) / m + 1 : 0u; };  // b < e with b mod m = r
    const bool last = relay_arrive(a.relay + (9 * R + (x * kPieceFan + k) * R + s) * a.rstride, upto(hi) - upto(lo),
                                   false) &&
                      relay_arrive(a.relay + (R + x * R + s) * a.rstride, kPieceFan, false) &&
                      relay_arrive(a.relay + s * a.rstride, 8, false);
    if (last) {
      if (a.lit) litmus_record(a.lit_last + s, off);
      for (uint32_t d = 0; d < R; ++d) atomic_add_u64(a.sig + (size_t)d * a.sig_stride, 1ull);
    }
  }
}

template <int RT, bool ALIGNED, bool PIECE>
__global__ __launch_bounds__(256) void k_allgather(const AGArgs a) {
  const uint32_t R = RT ? RT : a.R;
  const uint32_t nwork = a.nwg;
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
  if constexpr (PIECE) {
    static_assert(ALIGNED, "the piece form needs aligned offsets");
    ag_piece<RT>(a, R, b);
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
    if (a.lit) litmus_record(a.lit_last + s, t0);
    for (uint32_t d = 0; d < R; ++d) atomic_add_u64(a.sig + (size_t)d * a.sig_stride, 1ull);
  }
}

template <int RT, bool AL, bool PIECE = false>
void launch_t(const AGArgs& a, uint32_t grid, hipStream_t st) {
  hipLaunchKernelGGL((k_allgather<RT, AL, PIECE>), dim3(grid), dim3(256), 0, st, a);
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
  a.err = c->err;
  a.timeout_ns = kDefaultTimeoutNs;
  a.lit = c->litmus;
  a.lit_last = c->lit_last;
  a.lit_seed = c->lit_seed++;
  a.R = R;
  const bool aligned = ((send_off | recv_off | bytes) & 15) == 0;
  const uint64_t pieces = (bytes + kPiece - 1) / kPiece;
  // at least 64 pieces per source, so every first-level relay counter has one
  const bool piece = aligned && pieces >= 64 && pieces * R <= 0x7FFFFFFFull;
  a.pieces = piece ? static_cast<uint32_t>(pieces) : 0;
  a.nwg = piece ? a.pieces * R : a.tiles * R;
  // [R] per source, then (piece form) [8][R] per (XCD, source) and
  // [8][kPieceFan][R] per (XCD, k, source)
  a.rstride = relay_stride(piece ? (9 + 8 * kPieceFan) * R : R);
  const uint32_t grid = a.nwg + (wait ? R : 0);
  if (piece) {
    if (R == 16) launch_t<16, true, true>(a, grid, st);
    else if (R == 8) launch_t<8, true, true>(a, grid, st);
    else if (R == 4) launch_t<4, true, true>(a, grid, st);
    else launch_t<0, true, true>(a, grid, st);
  } else if (!aligned) launch_t<0, false>(a, grid, st);
  else if (R == 16) launch_t<16, true>(a, grid, st);
  else if (R == 8) launch_t<8, true>(a, grid, st);
  else if (R == 4) launch_t<4, true>(a, grid, st);
  else launch_t<0, true>(a, grid, st);
  return hipGetLastError() == hipSuccess ? VR_OK : VR_ERR_HIP;
}

}  // namespace vr
