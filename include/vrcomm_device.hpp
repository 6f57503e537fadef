/* vrcomm_device.hpp -- device-side one-sided primitives for HIP kernels on gfx950.
 *
 * The kernel-side counterpart of vrcomm.h (GIN page, lpnh.cn/news/2681042:
 * the device API puts, signals, counters and barrier sessions in the user's
 * own kernel). Views of a communicator and of a window come from
 * vr_comm_device_view() and vr_window_device_view() on the host and are
 * passed to the kernel by value; everything here is header-only.
 *
 * Visibility protocol (the same one the library's own kernels use): payload
 * bytes are stored with agent-coherent stores; before a signal, counter or
 * barrier arrival the issuing workgroup waits for its stores and meets at a
 * workgroup barrier (publish_wg), or the issuing wave waits for its own
 * stores (publish_wave); the signal is then a relaxed agent-scope
 * atomic, and a waiter that sees the value it needs issues one agent-scope
 * acquire. Every signal is therefore published after all earlier stores of
 * its workgroup: strong and weak signals (GIN page, strong and weak
 * signals) get the same, strong, guarantee.
 *
 * Unit of cooperation: the workgroup, or a single wave (put_wave and
 * publish_wave). Functions marked "all threads" must be reached by every
 * thread of the workgroup, "all lanes of one wave" by the 64 lanes of the
 * wave that issues them, and "one thread" functions by a single thread (any).
 */
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vrcomm.h"

namespace vrdev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

/* ---- addressing ------------------------------------------------------------------- */
/* Signal `id` of `rank`, counter `id` of `rank`, barrier slot `index`. */
__device__ inline uint64_t* signal_word(const vrDevComm& c, int rank, uint32_t id) {
  return c.signals + (size_t)rank * c.signal_count + id;
}
__device__ inline uint64_t* counter_word(const vrDevComm& c, int rank, uint32_t id) {
  return c.counters + (size_t)rank * c.counter_count + id;
}
__device__ inline uint64_t* barrier_word(const vrDevComm& c, uint32_t index) { return c.barriers + index; }
/* A VA signal (GIN page, VA signals): the 8-byte word at `offset` of rank's
 * slice of a window registered with VR_WIN_STRICT_ORDERING. */
__device__ inline uint64_t* va_signal_word(const vrDevWindow& w, int rank, uint64_t offset) {
  return reinterpret_cast<uint64_t*>(w.base[rank] + offset);
}

/* ---- stores and publication ---------------------------------------------------------- */
/* A buffer resource over [base, base + nbytes) (nbytes < 2^32; base uniform
 * across the wave) whose stores use cache policy sc1: coherent at agent
 * scope. */
__device__ inline __amdgpu_buffer_rsrc_t agent_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nbytes, 0x00020000);
}
constexpr int kSc1 = 16;

/* All threads: wait until this workgroup's loads and stores have completed,
 * then meet at a workgroup barrier. After it, the workgroup's stores are
 * visible at agent scope and may be announced. */
__device__ inline void publish_wg() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

/* The body of a put, shared by the workgroup and the wave forms: thread t of
 * the nthr cooperating threads copies its share of [s, s + bytes) to d with
 * agent-coherent stores. */
__device__ inline void put_span(char* d, const char* s, uint64_t bytes, uint32_t t, uint32_t nthr) {
  const bool vec = ((reinterpret_cast<uintptr_t>(d) | reinterpret_cast<uintptr_t>(s)) & 15) == 0;
  constexpr uint64_t kChunk = 1ull << 30;  // one buffer resource per GiB
  for (uint64_t c0 = 0; c0 < bytes; c0 += kChunk) {
    const uint32_t n = static_cast<uint32_t>(bytes - c0 < kChunk ? bytes - c0 : kChunk);
    const __amdgpu_buffer_rsrc_t r = agent_rsrc(d + c0, n);
    const char* sc = s + c0;
    uint32_t i = 0;
    if (vec) {
      const uint32_t nv = n >> 4;
      const u32x4* sv = reinterpret_cast<const u32x4*>(sc);
      uint32_t v = t;
      for (; v + 7 * nthr < nv; v += 8 * nthr) {  // eight loads in flight, then their stores
        u32x4 x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = __builtin_nontemporal_load(sv + v + u * nthr);
#pragma unroll
        for (int u = 0; u < 8; ++u) __builtin_amdgcn_raw_buffer_store_b128(x[u], r, (v + u * nthr) << 4, 0, kSc1);
      }
      for (; v < nv; v += nthr) __builtin_amdgcn_raw_buffer_store_b128(__builtin_nontemporal_load(sv + v), r, v << 4, 0, kSc1);
      i = nv << 4;
    }
    for (uint32_t b = i + t; b < n; b += nthr)
      __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(sc[b]), r, b, 0, kSc1);
  }
}

/* All threads: put -- copy `bytes` from src (rank's slice, src_off) to dst
 * (peer's slice, dst_off) with agent-coherent stores (GIN page, one-sided
 * transfers: put, with a workgroup as the cooperating group). peer, rank and
 * the offsets must be the same in every thread. Call publish_wg() before
 * announcing it. */
__device__ inline void put_wg(const vrDevWindow& dst, int peer, uint64_t dst_off, const vrDevWindow& src,
                              int rank, uint64_t src_off, uint64_t bytes) {
  const uint32_t t = threadIdx.x + blockDim.x * (threadIdx.y + blockDim.y * threadIdx.z);
  const uint32_t nthr = blockDim.x * blockDim.y * blockDim.z;
  put_span(dst.base[peer] + dst_off, src.base[rank] + src_off, bytes, t, nthr);
}

/* All 64 lanes of one wave: the same put with the wave as the cooperating
 * group, so that each wave of a workgroup can issue, publish and announce
 * its own puts without meeting the others at a workgroup barrier. The
 * arguments must be the same in every lane. Call publish_wave() before
 * announcing it. */
__device__ inline void put_wave(const vrDevWindow& dst, int peer, uint64_t dst_off, const vrDevWindow& src,
                                int rank, uint64_t src_off, uint64_t bytes) {
  put_span(dst.base[peer] + dst_off, src.base[rank] + src_off, bytes, __lane_id(), 64);
}

/* All lanes of one wave: wait until this wave's loads and stores have
 * completed (the wave's memory counter covers every lane). After it, the
 * wave's stores are visible at agent scope and one lane may announce them. */
__device__ inline void publish_wave() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

/* ---- signals and counters ------------------------------------------------------------ */
/* One thread, after publish_wg() or publish_wave(): SignalAdd (SignalInc is value 1) on a
 * signal word, or CounterInc on a counter word (GIN page, signals and
 * counters). */
__device__ inline void signal_add(uint64_t* word, uint64_t value) {
  __hip_atomic_fetch_add(word, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void counter_inc(uint64_t* word) { signal_add(word, 1); }

/* `a` at or before `b` in rolling order on `bits` bits (GIN page, signals and
 * counters: the rolling comparison). */
__device__ inline bool rolling_le(uint64_t a, uint64_t b, int bits) {
  const uint64_t m = bits >= 64 ? ~0ull : ((1ull << bits) - 1);
  return ((b - a) & m) < (1ull << (bits - 1));
}

/* One thread: wait until the low `bits` bits of *word reach `least` in
 * rolling order, then acquire (unless `acquire` is false: the caller then
 * reads nothing that the signalling side wrote in this kernel; an agent
 * acquire invalidates this XCD's L2 lines, which costs when many workgroups
 * do it). Gives up after timeout_ns (0: 5 s), sets VR_ASYNC_TIMEOUT in *err
 * and returns false. */
__device__ inline bool wait_word(const uint64_t* word, uint64_t least, int bits, uint64_t timeout_ns, uint32_t* err,
                                 bool acquire = true) {
  const uint64_t mask = bits >= 64 ? ~0ull : ((1ull << bits) - 1);
  if (!timeout_ns) timeout_ns = 5000000000ull;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime() * 10ull;  // 100 MHz counter, in ns
  for (;;) {
    const uint64_t v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & mask;
    if (rolling_le(least & mask, v, bits)) break;
    if (__builtin_amdgcn_s_memrealtime() * 10ull - t0 > timeout_ns) {
      __hip_atomic_fetch_or(err, VR_ASYNC_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  if (acquire) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return true;
}

/* ---- barrier sessions ---------------------------------------------------------------- */
/* All threads: one sync of a barrier session (GIN page, ncclGinBarrierSession
 * and its fence levels) among `members` workgroups that use slot `word`.
 * `target` is the slot value once every member has arrived at this sync:
 * the slot's base (vr_barrier_expected on the host, before the kernel) plus
 * members times the number of this sync (1 for the first).
 *   VR_FENCE_PUT  before arriving, this workgroup's stores (its puts) have
 *                 completed; after the sync, the puts other members issued
 *                 before it are visible here.
 *   VR_FENCE_GET  before arriving, this workgroup's loads (its gets) have
 *                 landed.
 *   VR_FENCE_NONE pure synchronization: no drain, no acquire.
 * Every member must reach the sync, so the members must be resident at the
 * same time (in a grid, place them before any workgroup that waits on
 * them). Returns false in every thread on timeout (VR_ASYNC_TIMEOUT set). */
__device__ inline bool barrier_sync_wg(uint64_t* word, uint64_t target, uint32_t fence, uint64_t timeout_ns,
                                       uint32_t* err) {
  __shared__ int ok;
  if (fence & (VR_FENCE_PUT | VR_FENCE_GET)) publish_wg();
  else __syncthreads();
  const uint32_t t = threadIdx.x + blockDim.x * (threadIdx.y + blockDim.y * threadIdx.z);
  if (t == 0) {
    signal_add(word, 1);
    if (!timeout_ns) timeout_ns = 5000000000ull;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime() * 10ull;
    int good = 1;
    while (!rolling_le(target, __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), 64)) {
      if (__builtin_amdgcn_s_memrealtime() * 10ull - t0 > timeout_ns) {
        __hip_atomic_fetch_or(err, VR_ASYNC_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        good = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (fence & (VR_FENCE_PUT | VR_FENCE_GET)) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    ok = good;
  }
  __syncthreads();
  return ok != 0;
}

}  // namespace vrdev
