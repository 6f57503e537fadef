// Host-side state of a communicator and the launch entry points each kernel
// file provides. Shared by the .hip files of libvrcomm; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <set>
#include <utility>
#include <vector>

#include "vrcomm.h"  // include/ is on the include path

namespace vr {

// Relay counters: one region per kind of operation, so that a collective and
// a single put enqueued back to back never share a counter. Counters that
// many workgroups hit sit kRelaySpread words (256 bytes) apart: measured on
// gfx950, returning atomics on one 256-byte span serialize at ~12 ns each,
// while separate spans proceed in parallel.
constexpr uint32_t kRelaySpread = 64;
constexpr uint32_t kRelaySingle = 0;  // vr_put / vr_get: a total, 8 per XCD, 64 first-level, spread
constexpr uint32_t kRelayColl = 73 * kRelaySpread;  // collectives: up to R*R counters
// (and the AllReduce's rank-split and the AllGather's piece forms: 73
// counters per rank, spread 256 bytes apart up to R = 16)
constexpr uint32_t kRelayCollWords =
    VR_MAX_RANKS * VR_MAX_RANKS > 73 * 16 * kRelaySpread ? VR_MAX_RANKS * VR_MAX_RANKS : 73 * 16 * kRelaySpread;
constexpr uint32_t kRelayDispatch = kRelayColl + kRelayCollWords;  // 18 counters per source rank
constexpr uint32_t kRelayDispatchWords = 18 * VR_MAX_RANKS * 8;
constexpr uint32_t kRelaySlots = kRelayDispatch + kRelayDispatchWords;
// Stride between n counters in a region of `words`: as wide as the region
// allows, up to kRelaySpread.
inline uint32_t relay_stride(uint32_t n, uint32_t words = kRelayCollWords) {
  uint32_t st = kRelaySpread;
  while (st > 1 && (uint64_t)st * n > words) st >>= 1;
  return st;
}

constexpr uint64_t kDefaultTimeoutNs = 5ull * 1000 * 1000 * 1000;

struct WinTab {
  char* p[VR_MAX_RANKS];
};
struct U64Tab {
  uint64_t v[VR_MAX_RANKS];
};

}  // namespace vr

struct vrWindow {
  vrComm* comm;
  size_t bytes;
  uint32_t flags;
  int nranks;
  char* base[VR_MAX_RANKS];
  // words in use as VA signals: (rank, offset) -> 0 (no Inc/Add yet), 1 Inc, 2 Add
  std::map<std::pair<int, uint64_t>, uint8_t> va_words;
};

struct vrComm {
  int device;
  int nranks;
  vrCommRequirements req;
  // device words (one allocation, or the caller's workspace)
  char* ws;
  size_t ws_bytes;
  bool owns_ws;
  uint64_t* sig;    // [R][signal_count]
  uint64_t* cnt;    // [R][counter_count]
  uint32_t* err;    // error bits
  uint32_t* relay;  // [kRelaySlots]
  uint64_t* bar;    // [barrier_count] barrier-session slots
  uint64_t* lit_last;  // [R][R] litmus records: the piece that completed each relay
  uint64_t* litmus;    // caller's litmus words [2] (checks, mismatches), or null: litmus off
  uint32_t lit_seed;   // per-launch seed of the litmus samples
  uint64_t* ring_bases;  // [R][context_count] ring signal values published by the producers
  uint64_t* ring_gens;   // [R][context_count] exchange generation of each published value
  uint64_t ring_gen;     // generation of the last ring exchange enqueued
  uint64_t* trace;     // caller's dispatch phase timestamps, or null: tracing off
  uint64_t trace_words;
  // growable scratch for dispatch (histograms, count exchange)
  char* scratch;
  size_t scratch_bytes;
  // host view of the signals: the value each will hold once all enqueued work has run
  std::vector<uint64_t> expect;      // [R][S]
  std::vector<uint8_t> expect_known; // 0 when a device-computed amount was added
  std::vector<uint8_t> sig_mode;     // 0 none, 1 SignalInc, 2 SignalAdd (since the last reset)
  std::vector<uint64_t> bar_expect;  // [barrier_count] slot values once enqueued work has run
  // copy-engine path: internal streams and fork/join events, created on first use
  std::vector<hipStream_t> ce_streams;
  std::vector<hipEvent_t> ce_events;  // [0] fork, [1 + i] join of stream i
  std::set<vrWindow*> windows;
};

namespace vr {

// launch entry points (each returns VR_OK or VR_ERR_HIP)
vrResult_t launch_alltoall(vrComm* c, const vrWindow* send, size_t send_off, const vrWindow* recv,
                           size_t recv_off, size_t block, uint32_t sig, const U64Tab& target,
                           bool wait, hipStream_t st);
vrResult_t launch_allreduce(vrComm* c, const vrWindow* send, size_t send_off, const vrWindow* recv,
                            size_t recv_off, size_t count, int dtype, uint32_t sig,
                            const U64Tab& target, bool wait, hipStream_t st);
vrResult_t launch_allgather(vrComm* c, const vrWindow* send, size_t send_off, const vrWindow* recv,
                            size_t recv_off, size_t bytes, uint32_t sig, const U64Tab& target,
                            bool wait, hipStream_t st);
// scratch: device memory of at least dispatch_scratch_bytes() bytes, 256-byte aligned
vrResult_t launch_dispatch(vrComm* c, const vrWindow* x, size_t x_off, size_t row_bytes,
                           const int32_t* topk, int T, int K, int E, const vrWindow* recv,
                           size_t recv_off, size_t cap, int32_t* counts_out, int32_t* src_out,
                           int32_t* pos_out, int32_t* experts_out, bool dedup, uint32_t sig_counts,
                           uint32_t sig_rows, const U64Tab& target_counts, bool wait, char* scratch,
                           hipStream_t st);
// dedup: pos is [R][T][R] (a row per destination rank), weights are 1, topk unused
vrResult_t launch_combine(vrComm* c, const vrWindow* y, size_t y_off, size_t cap, size_t row_bytes, int dtype,
                          const int32_t* topk, const float* weights, const int32_t* pos, int T, int K, int E,
                          bool dedup, const vrWindow* out, size_t out_off, uint32_t sig, const U64Tab& target,
                          bool wait, hipStream_t st);
size_t dispatch_scratch_bytes(int R, int T, int E, int Eo);
vrResult_t launch_ring(vrComm* c, const vrWindow* send, const vrWindow* recv, size_t put_bytes,
                       size_t puts_per_rank, int contexts, uint64_t* const* sig_ctx0, uint32_t cnt_base,
                       bool wait, bool weak, uint64_t* litmus, hipStream_t st);

vrResult_t launch_barrier(vrComm* c, uint32_t index, uint64_t target, uint32_t fence, uint64_t timeout_ns,
                          hipStream_t st);
vrResult_t launch_alltoall_sessions(vrComm* c, const vrDevWindow& send, size_t send_off, const vrDevWindow& recv,
                                    size_t recv_off, size_t block, uint32_t sig, const U64Tab& target, uint32_t index,
                                    uint64_t bar_base, hipStream_t st);

// helpers in comm.hip
vrResult_t ensure_scratch(vrComm* c, size_t bytes);
vrResult_t launch_pingpong(vrComm* c, const vrWindow* w, size_t off, size_t bytes, uint32_t iters, uint32_t sig,
                           const uint64_t base[2], bool same_xcd, bool waves, hipStream_t st);
vrDevComm device_view(const vrComm* c);
vrDevWindow device_view(const vrWindow* w);

}  // namespace vr
