// Fine-grained ring exchange with strong signals, counters and a litmus check.
//
// GDA survey (10100.com/article/158785524), section 4: the GIN paper's ring
// exchange is put (with SignalInc), waitSignal, resetSignal; signals and
// counters are addressed by integer ids; a strong signal on a context makes
// every earlier put of that context to the peer visible. GIN page
// (lpnh.cn/news/2681042), counter methods: a counter counts puts whose source
// has been consumed.
//
// Rank r sends puts_per_rank messages to rank (r+1) mod R, split into
// `contexts` contiguous ranges. One workgroup owns each (rank, context) and
// issues its messages in order, in rounds of up to 64 KiB (at most 256
// messages, one signalling thread each): it loads the round's messages,
// stores them with agent-coherent stores, waits for every wave's stores,
// then applies one SignalInc per message at the receiver and one CounterInc
// per message at itself. Every signal is therefore applied after the
// payloads of all earlier messages of its context are visible (strong).
// Measured on 16 ranks x 65536 puts of 256 B, 64 contexts: rounds of 16 KiB
// by one wave took 225 us, 64 KiB rounds by one wave 119 us, 64 KiB rounds
// by a 256-thread workgroup 98 us (32 KiB: 155 us; 128 KiB: 97 us): the time
// follows the number of serial rounds per issuer and the loads in flight.
// Before its first signal, the producer of (rank, context) -- the only writer
// of that signal during the exchange -- reads the signal's value and
// publishes it, followed by the call's generation number, in the
// communicator's workspace; the receiver waits for the generation, reads the
// value and from it the target (replacing a separate snapshot kernel before
// the exchange: one launch less per call). One waiting wavefront per
// receiving rank then polls the signals of all its contexts, lane j those of
// contexts j, j + 64, ..., until each has grown by its context's message
// count. One wavefront per (rank, context), 1024 of them on 16 x 64, polled
// often enough to slow the exchange: 86.3-86.7 us against 82.6-82.9 us
// (flushed, alternating on one machine; no waits at all: 81.7 us), and one
// wavefront per context walked in turn by each rank's four waves 92 us. With
// the litmus on, one wavefront still watches each (rank, context): each time
// it sees a new value v it acquires and checks that message v-1 and one
// earlier message of the context are present, counting violations.
//
// Weak signals (GIN page, strong and weak signals: a weak signal is ordered
// after its own put only) need no workgroup-wide completion: each wavefront
// takes every fourth 16 KiB chunk of the context's messages, stores it, waits
// for its own stores and applies the chunk's signals, never meeting the other
// waves. A reader that sees v may then miss one of the first v messages (a
// later chunk's wave finished first); the litmus counts those observations,
// and only a missing message once the signal reads the full count is an
// error.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "vr_device.hpp"
#include "vr_internal.hpp"

namespace vr {
namespace {

constexpr int kThreads = 256;          // one workgroup issues each (rank, context)
constexpr int kWaves = kThreads / 64;
constexpr uint32_t kRoundBytes = 65536;  // bytes per round (per chunk with weak signals: a quarter)
constexpr uint32_t kSigPerThread = 1;    // signals (and counter increments) each thread applies per round

struct RingArgs {
  WinTab send, recv;
  uint64_t put_bytes, per_ctx;
  uint64_t* sigp[VR_MAX_RANKS];  // rank d's signal of context 0; context k at sigp[d] + k
  uint64_t* cnt;        // &cnt[0][cnt_base]
  uint32_t cnt_stride;
  uint64_t* bases;      // [R][C] signal values before this exchange, published by the producers
  uint64_t* gens;       // [R][C] generation of the exchange whose base bases[] holds
  uint64_t gen;
  uint64_t* litmus;     // [2] checks, violations; or null
  uint32_t* err;
  uint64_t timeout_ns;
  int R, C, waiters;   // receiving workgroups: R * C with the litmus, R without, 0 with no waits
};

// Compare message m at receiver d with its source at sender; true if equal.
__device__ bool message_present(const RingArgs& a, int d, int sender, uint64_t m) {
  const v4u* got = reinterpret_cast<const v4u*>(a.recv.p[d] + m * a.put_bytes);
  const v4u* want = reinterpret_cast<const v4u*>(a.send.p[sender] + m * a.put_bytes);
  bool same = true;
  for (uint64_t i = threadIdx.x; i < a.put_bytes / 16; i += 64) {
    const v4u x = got[i], y = want[i];
    same &= (x[0] == y[0]) & (x[1] == y[1]) & (x[2] == y[2]) & (x[3] == y[3]);
  }
  return ballot(!same) == 0;
}

// Receiver d, context k, one wave (lane = its lane): waits for the
// context's signal to reach this exchange's total, checking prefixes when the
// litmus is on; false after a timeout (reported in the error word).
template <bool WEAK>
__device__ bool receive_ctx(const RingArgs& a, int d, int k, int lane, uint64_t t0) {
  const int R = a.R, C = a.C;
  const int sender = (d + R - 1) % R;
  // this exchange's base, once the producer has published it
  while (load_relaxed_u64(a.gens + (size_t)d * C + k) != a.gen) {
    if (now_ns() - t0 > a.timeout_ns) {
      if (lane == 0) atomic_or_u32(a.err, VR_ASYNC_TIMEOUT);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  const uint64_t base = load_relaxed_u64(a.bases + (size_t)d * C + k);
  const uint64_t* sig = a.sigp[d] + k;
  const uint64_t m0 = (uint64_t)k * a.per_ctx;
  uint64_t seen = 0;
  for (;;) {
    const uint64_t v = load_relaxed_u64(sig);
    const uint64_t n = static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v - base))) |
                       (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>((v - base) >> 32))) << 32);
    // n: messages of this context the signal vouches for
    if (a.litmus && n > seen && n <= a.per_ctx) {
      acquire_agent();
      const uint64_t earlier = ((n * 2654435761ull) >> 7) % n;
      const bool ok = message_present(a, d, sender, m0 + n - 1) && message_present(a, d, sender, m0 + earlier);
      if (lane == 0) {
        atomic_add_u64(a.litmus, 2ull);
        if (!ok) {
          atomic_add_u64(a.litmus + 1, 1ull);
          // strong: every observation must see its prefix; weak: only the full count
          if (!WEAK || n == a.per_ctx) atomic_or_u32(a.err, VR_ASYNC_LITMUS);
        }
      }
      seen = n;
    }
    if (rolling_le(base + a.per_ctx, base + n, 64)) break;
    if (now_ns() - t0 > a.timeout_ns) {
      if (lane == 0) atomic_or_u32(a.err, VR_ASYNC_TIMEOUT);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  acquire_agent();
  return true;
}

template <bool WEAK>
__global__ __launch_bounds__(kThreads) void k_ring(const RingArgs a) {
  const int R = a.R, C = a.C;
  const int w = blockIdx.x;
  const int tid = threadIdx.x;
  if (w < R * C) {  // producer: rank r, context k
    const int r = w / C, k = w % C, peer = (r + 1) % R;
    const uint64_t P = a.put_bytes;
    // thread t applies the signals of messages t, t + kThreads, ...
    const uint64_t per_round =
        std::min<uint64_t>(kThreads * kSigPerThread, std::max<uint64_t>(1, kRoundBytes / P));
    const uint64_t m0 = (uint64_t)k * a.per_ctx, m1 = m0 + a.per_ctx;
    uint64_t* sig = a.sigp[peer] + k;
    uint64_t* cnt = a.cnt + (size_t)r * a.cnt_stride + k;
    if (a.waiters) {  // publish the signal's value before any of this exchange's signals
      if (tid == 0) {
        const size_t i = (size_t)peer * C + k;
        store8_agent(a.bases + i, load_relaxed_u64(sig));
        wait_vmem();  // the value has landed before the generation that announces it
        store8_agent(a.gens + i, a.gen);
      }
      __syncthreads();  // no wave signals before the value has been read
    }
    if (WEAK) {  // wave v: chunks v, v + 4, ... of the context; lane j signals message j of a chunk
      const uint32_t lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar addresses
      const uint64_t per_chunk = std::min<uint64_t>(64, std::max<uint64_t>(1, kRoundBytes / kWaves / P));
      for (uint64_t m = m0 + wave * per_chunk; m < m1; m += kWaves * per_chunk) {
        const uint64_t nm = std::min<uint64_t>(per_chunk, m1 - m);
        copy16<16>(a.recv.p[peer] + m * P, a.send.p[r] + m * P, static_cast<uint32_t>(nm * P), lane, 64);
        wait_vmem();  // this wave's stores (and loads) of the chunk have completed
        if (lane < nm) {
          atomic_add_u64(sig, 1ull);  // weak SignalInc of message m + lane
          atomic_add_u64(cnt, 1ull);  // CounterInc: its source has been read
        }
      }
      return;
    }
    for (uint64_t m = m0; m < m1; m += per_round) {
      const uint64_t nm = std::min<uint64_t>(per_round, m1 - m);
      const uint32_t bytes = static_cast<uint32_t>(nm * P);
      copy16<16>(a.recv.p[peer] + m * P, a.send.p[r] + m * P, bytes, tid, kThreads);
      wg_stores_complete();  // this round's payloads, from every wave, are visible at agent scope
      for (uint64_t j = tid; j < nm; j += kThreads) {
        atomic_add_u64(sig, 1ull);  // strong SignalInc of message m + j
        atomic_add_u64(cnt, 1ull);  // CounterInc: its source has been read
      }
    }
    return;
  }
  const int i = w - R * C;
  if (i >= a.waiters) return;
  if (a.litmus) {  // one wave watches each receiving (rank, context)
    if (tid < 64) receive_ctx<WEAK>(a, i / C, i % C, tid, now_ns());
    return;
  }
  // plain waits: one wave per receiving rank; lane j watches contexts j,
  // j + 64, ... (one vector load polls 64 contexts)
  if (tid >= 64) return;
  const int d = i, lane = tid;
  const uint64_t t0 = now_ns();
  for (int k0 = 0; k0 < C; k0 += 64) {
    const int k = k0 + lane;
    const bool mine = k < C;
    for (;;) {  // every watched context's producer has published this exchange's base
      const bool ok = !mine || load_relaxed_u64(a.gens + (size_t)d * C + k) == a.gen;
      if (ballot(!ok) == 0) break;
      if (now_ns() - t0 > a.timeout_ns) {
        if (lane == 0) atomic_or_u32(a.err, VR_ASYNC_TIMEOUT);
        return;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    const uint64_t target = mine ? load_relaxed_u64(a.bases + (size_t)d * C + k) + a.per_ctx : 0;
    for (;;) {
      const bool done = !mine || rolling_le(target, load_relaxed_u64(a.sigp[d] + k), 64);
      if (ballot(!done) == 0) break;
      if (now_ns() - t0 > a.timeout_ns) {
        if (lane == 0) atomic_or_u32(a.err, VR_ASYNC_TIMEOUT);
        return;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  acquire_agent();
}

}  // namespace

vrResult_t launch_ring(vrComm* c, const vrWindow* send, const vrWindow* recv, size_t put_bytes, size_t puts_per_rank,
                       int contexts, uint64_t* const* sig_ctx0, uint32_t cnt_base, bool wait, bool weak,
                       uint64_t* litmus, hipStream_t st) {
  const int R = c->nranks;
  RingArgs a;
  for (int q = 0; q < VR_MAX_RANKS; ++q) {
    a.send.p[q] = send->base[q];
    a.recv.p[q] = recv->base[q];
  }
  a.put_bytes = put_bytes;
  a.per_ctx = puts_per_rank / contexts;
  for (int q = 0; q < VR_MAX_RANKS; ++q) a.sigp[q] = q < R ? sig_ctx0[q] : nullptr;
  a.cnt = c->cnt + cnt_base;
  a.cnt_stride = c->req.counter_count;
  a.bases = c->ring_bases;
  a.gens = c->ring_gens;
  a.gen = ++c->ring_gen;
  a.litmus = litmus;
  a.err = c->err;
  a.timeout_ns = kDefaultTimeoutNs;
  a.R = R;
  a.C = contexts;
  a.waiters = wait ? (litmus ? R * contexts : R) : 0;
  if (weak) hipLaunchKernelGGL(k_ring<true>, dim3(R * contexts + a.waiters), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL(k_ring<false>, dim3(R * contexts + a.waiters), dim3(kThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? VR_OK : VR_ERR_HIP;
}

}  // namespace vr
