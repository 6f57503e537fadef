// Device-side primitives of the window put/get library for gfx950 (CDNA4).
//
// Visibility protocol (GIN page, one-sided transfers and strong/weak signals:
// a signal seen at the peer implies the payload of its put -- and, for a
// strong signal, of every earlier put of the context to that peer -- is
// visible there).
//
// gfx950 has one L2 per XCD; the L2s are not coherent with each other for
// ordinary stores. The compiler's generic agent-scope release writes back the
// whole XCD L2 (buffer_wbl2) before the flag, which costs roughly ten times
// the copy itself when every workgroup publishes its tile. Instead:
//   * every byte a put delivers is written with an agent-scope-coherent store
//     (cache policy sc1: the same instruction the compiler emits for a relaxed
//     atomic store at agent scope), so no dirty payload stays behind in an
//     XCD-private L2;
//   * the issuer waits until its own stores have completed (s_waitcnt
//     vmcnt(0)), the workgroup meets at a barrier, and one thread then applies
//     the signal with a relaxed agent-scope atomic add;
//   * a waiter polls the signal with relaxed agent-scope loads and, once the
//     value suffices, issues one agent-scope acquire fence (buffer_inv sc1) so
//     its following loads miss in any stale L2 line.
// A multi-workgroup put (one logical put split into tiles) adds a relay: each
// tile's workgroup publishes as above but increments a relay counter instead
// of the signal; the workgroup that brings the counter to the tile count is
// last, resets the counter for the next use, and applies the put's actions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vrcomm.h"  // VR_ASYNC_* bits

namespace vr {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr uint32_t kRelaxed = __ATOMIC_RELAXED;
constexpr int kLoadStream = 2;    // buffer/global cache policy: nt (streaming)
constexpr int kStoreAgent = 16;   // cache policy: sc1 (coherent at agent scope)
constexpr int kStoreAgentStream = 18;  // sc1 + nt: coherent at agent scope, streaming
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer descriptor, gfx9 family

// Buffer resource over [base, base + nbytes); accesses outside are dropped by
// the hardware (loads return 0), which bounds every buffer access below.
__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nbytes, kRsrcWord3);
}

__device__ inline v4u load16_stream(const v4u* p) { return __builtin_nontemporal_load(p); }

// Loads through a pointer the compiler cannot place (read from LDS, say)
// would be emitted as flat loads, which also count against lgkmcnt and so
// serialize behind every LDS wait; these name the global address space.
typedef __attribute__((address_space(1))) const v4u g_v4u;
typedef __attribute__((address_space(1))) const uint16_t g_u16;
typedef __attribute__((address_space(1))) const float g_f32;
__device__ inline v4u load16_stream_global(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<g_v4u*>(reinterpret_cast<uintptr_t>(p)));
}
__device__ inline uint16_t load2_global(const void* p) {
  return *reinterpret_cast<g_u16*>(reinterpret_cast<uintptr_t>(p));
}
__device__ inline float load4f_global(const void* p) {
  return *reinterpret_cast<g_f32*>(reinterpret_cast<uintptr_t>(p));
}

__device__ inline void store16_agent(__amdgpu_buffer_rsrc_t r, uint32_t off, v4u v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kStoreAgent);
}
__device__ inline void store16_agent_stream(__amdgpu_buffer_rsrc_t r, uint32_t off, v4u v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kStoreAgentStream);
}
__device__ inline void store4_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void store8_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void store1_agent(__amdgpu_buffer_rsrc_t r, uint32_t off, uint8_t v) {
  __builtin_amdgcn_raw_buffer_store_b8(v, r, off, 0, kStoreAgent);
}

// All vector memory operations this wave issued have completed.
__device__ inline void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Every wave of the workgroup has completed its stores (see the protocol above).
__device__ inline void wg_stores_complete() {
  wait_vmem();
  __syncthreads();
}

__device__ inline uint64_t atomic_add_u64(uint64_t* p, uint64_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint32_t atomic_add_u32(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void atomic_or_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t load_relaxed_u64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint32_t load_relaxed_u32(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
// Coherent 32-bit read at agent scope (sc1: never satisfied by a stale line of
// an XCD-private L2). Used for small data published earlier in the same kernel
// by other workgroups, read after the signal that announced it has been seen.
__device__ inline int32_t load_coherent_i32(const int32_t* p) {
  return static_cast<int32_t>(load_relaxed_u32(reinterpret_cast<const uint32_t*>(p)));
}
__device__ inline void compiler_fence() { asm volatile("" ::: "memory"); }

// Rolling comparison on `bits`-bit values (GIN page, signals and counters):
// b has reached a when (b - a) mod 2^bits < 2^(bits-1).
__device__ inline bool rolling_le(uint64_t a, uint64_t b, int bits) {
  const uint64_t mask = bits >= 64 ? ~0ull : ((1ull << bits) - 1);
  const uint64_t half = 1ull << (bits - 1);
  return ((b - a) & mask) < half;
}

__device__ inline uint64_t now_ns() { return __builtin_amdgcn_s_memrealtime() * 10ull; }  // 100 MHz counter

// Poll a 64-bit word until its low `bits` bits reach `least` (rolling order),
// then acquire (unless `acquire` is false: the caller only reads data that an
// earlier kernel on the stream wrote, which the kernel boundary already made
// visible). On timeout sets the error bit and returns false.
__device__ inline bool wait_reached(const uint64_t* word, uint64_t least, int bits,
                                    uint64_t timeout_ns, uint32_t* err, uint32_t err_bit,
                                    bool acquire = true) {
  const uint64_t mask = bits >= 64 ? ~0ull : ((1ull << bits) - 1);
  const uint64_t t0 = now_ns();
  for (;;) {
    uint64_t v = load_relaxed_u64(word) & mask;
    if (rolling_le(least & mask, v, bits)) break;
    if (now_ns() - t0 > timeout_ns) {
      atomic_or_u32(err, err_bit);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  if (acquire) acquire_agent();
  return true;
}

// Relay of a multi-workgroup put: call from one thread after
// wg_stores_complete(). Returns true in the workgroup that completes the set
// of `parts`; that workgroup has acquired the other parts' publications
// (unless `acquire` is false: the caller then reads what the other parts
// wrote only with agent-coherent loads, or not at all).
// Measured on gfx950: returning atomics on one counter are cheap while every
// arrival comes from the same XCD, and cost ~0.7 us each when consecutive
// arrivals come from different XCDs, so callers keep a counter's parts on one
// XCD or spread them over several counters.
__device__ inline bool relay_arrive(uint32_t* counter, uint32_t parts, bool acquire = true) {
  if (parts <= 1) return true;
  uint32_t prev = atomic_add_u32(counter, 1u);
  if (prev + 1u != parts) return false;
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next use
  if (acquire) acquire_agent();
  return true;
}

// ---- copies -------------------------------------------------------------------
// Cooperative copy of n bytes by threads [tid, nthr): destination written with
// agent-coherent stores. Both pointers 16-byte aligned, n a multiple of 16,
// n < 2^31. U vectors in flight per thread.
template <int U>
__device__ inline void copy16(char* __restrict__ dst, const char* __restrict__ src, uint32_t n,
                              uint32_t tid, uint32_t nthr) {
  const uint32_t nv = n >> 4;
  const v4u* s = reinterpret_cast<const v4u*>(src);
  const __amdgpu_buffer_rsrc_t rd = rsrc(dst, n);
  uint32_t i = tid;
  for (; i + (U - 1) * nthr < nv; i += U * nthr) {
    v4u v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load16_stream(s + i + u * nthr);
#pragma unroll
    for (int u = 0; u < U; ++u) store16_agent(rd, (i + u * nthr) << 4, v[u]);
  }
  for (; i < nv; i += nthr) store16_agent(rd, i << 4, load16_stream(s + i));
}

// Byte-granular cooperative copy for unaligned or ragged ranges (n < 2^31).
__device__ inline void copy_bytes(char* __restrict__ dst, const char* __restrict__ src, uint32_t n,
                                  uint32_t tid, uint32_t nthr) {
  const __amdgpu_buffer_rsrc_t rd = rsrc(dst, n);
  for (uint32_t i = tid; i < n; i += nthr) store1_agent(rd, i, static_cast<uint8_t>(src[i]));
}

// General cooperative copy (non-overlapping ranges, n < 2^31): vector path
// for the part where source and destination share 16-byte alignment.
template <int U>
__device__ inline void copy_any(char* __restrict__ dst, const char* __restrict__ src, uint32_t n,
                                uint32_t tid, uint32_t nthr) {
  const uintptr_t d = reinterpret_cast<uintptr_t>(dst), s = reinterpret_cast<uintptr_t>(src);
  if (((d ^ s) & 15u) != 0 || n < 64) {
    copy_bytes(dst, src, n, tid, nthr);
    return;
  }
  uint32_t head = static_cast<uint32_t>((16u - (d & 15u)) & 15u);
  if (head > n) head = n;
  const uint32_t body = (n - head) & ~15u;
  const uint32_t tail = n - head - body;
  if (head) copy_bytes(dst, src, head, tid, nthr);
  if (body) copy16<U>(dst + head, src + head, body, tid, nthr);
  if (tail) copy_bytes(dst + head + body, src + head + body, tail, tid, nthr);
}

// ---- bf16 ------------------------------------------------------------------------
__device__ inline float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// fp32 -> bf16 bits, round to nearest even; any NaN -> 0x7FC0.
__device__ inline uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7FC0u : r;
}

// ---- strong-signal litmus of the collectives' receivers ---------------------------
// GIN page, strong and weak signals: a signal seen at the peer means the
// payload of every earlier put of the context to that peer is visible there.
// With a communicator's litmus on, the workgroup that completes a relay
// records the piece it stored last (a tile, a slab, a row) before applying
// the signal; each receiver, once its wait has ended and it has acquired,
// checks those pieces in full first, then one seeded sample in every piece
// aimed at it. A signal applied before its pieces were visible would show up
// as a mismatch.

__device__ inline uint32_t mix32(uint32_t x) {  // an integer hash (xorshift-multiply rounds)
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// The n <= 16 bytes at `got` equal those at `want`.
__device__ inline bool equal_upto16(const char* got, const char* want, uint32_t n) {
  if (n == 16 && ((reinterpret_cast<uintptr_t>(got) | reinterpret_cast<uintptr_t>(want)) & 15) == 0) {
    const v4u x = *reinterpret_cast<const v4u*>(got), y = *reinterpret_cast<const v4u*>(want);
    return x[0] == y[0] && x[1] == y[1] && x[2] == y[2] && x[3] == y[3];
  }
  bool eq = true;
  for (uint32_t i = 0; i < n; ++i) eq &= got[i] == want[i];
  return eq;
}

// From the thread that completed a relay: record the piece it stored last;
// the record has landed before the signal the caller applies next.
__device__ inline void litmus_record(uint64_t* slot, uint64_t piece) {
  store8_agent(slot, piece);
  wait_vmem();
}

// Adds the workgroup's counts to words[0] (checks) and words[1] (mismatches);
// a mismatch also sets VR_ASYNC_LITMUS. Every thread of the workgroup calls it.
__device__ inline void litmus_report(uint64_t* words, uint32_t* err, uint32_t checks, uint32_t bad) {
  __shared__ uint32_t tot[2];
  if (threadIdx.x == 0) tot[0] = tot[1] = 0;
  __syncthreads();
  if (checks) atomicAdd(&tot[0], checks);
  if (bad) atomicAdd(&tot[1], bad);
  __syncthreads();
  if (threadIdx.x == 0) {
    atomic_add_u64(words, tot[0]);
    if (tot[1]) {
      atomic_add_u64(words + 1, tot[1]);
      atomic_or_u32(err, VR_ASYNC_LITMUS);
    }
  }
}

// A receiver's wait, then (litmus on) an acquire by every thread: true when
// the wait ended before its timeout. Every thread of the workgroup calls it.
__device__ inline bool receiver_wait(const uint64_t* word, uint64_t least, uint64_t timeout_ns, uint32_t* err) {
  __shared__ int ok;
  if (threadIdx.x == 0) ok = wait_reached(word, least, 64, timeout_ns, err, VR_ASYNC_TIMEOUT);
  __syncthreads();
  if (!ok) return false;
  acquire_agent();
  return true;
}

// ---- wave helpers -------------------------------------------------------------------
__device__ inline uint32_t lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }
__device__ inline uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Lanes of the wave holding the same key (key < 2^nbits), from nbits ballots:
// a lane matches when it agrees with this lane on every bit. Inactive lanes
// never match.
__device__ inline uint64_t match_any(uint32_t key, int nbits) {
  uint64_t m = __builtin_amdgcn_read_exec();
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t set = ballot(bit);
    m &= bit ? set : ~set;
  }
  return m;
}

}  // namespace vr
