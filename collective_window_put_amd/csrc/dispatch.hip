// MoE token dispatch over symmetric windows: count exchange, offsets, puts.
//
// GDA survey (10100.com/article/158785524), opening section: an MoE dispatch
// routes tokens of a few hundred bytes among dozens of experts, with sizes
// and targets known only at run time; section 4: a batch of puts closed by
// one signal orders them cheaply. Layout of rank d's receive rows: by expert
// (rank d owns experts [d*E/R, (d+1)*E/R)), then source rank, then token.
//
// One kernel, three kinds of workgroup, in grid order:
// * count (s, b): histograms the routing entries of its 256 tokens in LDS, per
//   64-token sub-block (in the per-rank layout, a wave per sub-block and one
//   ballot per rank over its tokens' destination masks), and stores the
//   sub-blocks' exclusive prefixes within the block plus the block's totals. The last block of source s (relay)
//   sums the block totals into the count row C[s][.] (turning each block's
//   total into the prefix of the earlier blocks' on the way), puts the row
//   into every rank's count window and applies a SignalInc there (the count
//   exchange). Block (s, 0) first records rank s's row signal as the base its
//   receiver will wait from.
// * put (s, b) of 64 tokens: ranks its routing entries within the block
//   (wave ballots, token order), loads its token rows, waits for rank s's
//   count signal, derives each expert's receive offset from the full count
//   matrix
//     off(s, e) = sum_{e' < e owned by the same rank} sum_s' C[s'][e]
//               + sum_{s' < s} C[s'][e],
//   adds the rows of earlier blocks and sub-blocks of source s (two loads:
//   both prefixes are stored), records each
//   row's source, and copies each token row once per routed expert. The last
//   block of source s applies one SignalAdd(rows sent to d) at every rank d.
// * receiver d (the last R workgroups): waits until its row signal has grown
//   by the rows aimed at it.
// Count workgroups never wait, and every workgroup that waits comes later in
// the grid than all the workgroups it waits for, so the waits always end.
// Data published inside the kernel (prefixes, count rows, bases) is read with
// agent-coherent loads after the announcing signal has been seen.
//
// Row copies use 16-byte lanes (two 512-byte rows per wave instruction) when
// every rank's receive slice lies within one 4 GiB span, so that one buffer
// resource addresses them all; otherwise 8-byte agent-coherent stores.
// Measured on the 8 x 4096 x 512 B, E=256, K=8 shape: 16-byte lanes with 8
// tokens per wave copy the rows in 29 us, 8-byte lanes in 55 us.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "vr_device.hpp"
#include "vr_internal.hpp"

namespace vr {
namespace {

constexpr int kThreads = 512;     // threads per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kTokPerWave = 8;    // tokens per wave in a put workgroup
constexpr int kSub = kWaves * kTokPerWave;  // tokens per put workgroup (sub-block): 64
constexpr int kCountBlock = 256;  // tokens per count workgroup
constexpr int kSubs = kCountBlock / kSub;
constexpr int kRelayFan = 16;     // first-level relay counters per source (put blocks)

struct DispArgs {
  WinTab x, recv;
  U64Tab target_counts;
  uint64_t x_off, recv_off, row_bytes, cap;
  const int32_t* topk;   // [R][T][K]
  int32_t* counts_out;   // [R][E/R]
  int32_t* src_out;      // [R][cap]
  int32_t* pos_out;      // [R][T][K] receive row of each routing entry ([R][T][R] per rank when dedup), or nullptr
  int32_t* experts_out;  // dedup: [R][cap][K] local expert of each entry of a received row
  int32_t* ecounts_out;  // dedup: [R][Eo/R] rows per local expert
  int32_t* eblk;         // dedup: [R][NB1][Eo] entries per expert of each count block
  int32_t* ecw;          // dedup: [R][Eo] entries per expert of each source
  int Eo, epro;          // dedup: keys are destination ranks (E = R); Eo experts, epro per rank
  uint64_t epro_mul;     // ceil(2^32 / epro): e / epro as a multiply (see div_by)
  uint64_t epr_mul;      // ceil(2^32 / (E / R)), for the keys' rank
  int kbits;             // bits holding every key value up to E (dedup: rank or the non-key E)
  int ids_vec;           // K % 4 == 0 and topk 16-byte aligned: a token's ids load as 16-byte vectors
  int gbits;             // bits naming a token within a wave: 2^gbits >= ceil(64 / K)
  int nbits_o;           // dedup: bits of an expert id
  int xo_vec;            // dedup: K % 4 == 0 and experts_out 16-byte aligned: 16-byte stores
  int32_t* subpfx;       // [R][NB1*kSubs][E]: sub-block prefix within its count block
  int32_t* blktot;       // [R][NB1][E]: rows per expert of each count block
  int32_t* cwin;         // [R][R][E]: rank d's copy of every source's count row
  uint64_t* base_rows;   // [R]
  uint64_t* sig_counts;  // &sig[0][id]
  uint64_t* sig_rows;
  uint32_t sig_stride;
  uint32_t* relay;       // [19R + 2] counters (see launch_dispatch), rstride words apart
  uint32_t rstride;
  uint32_t* err;
  uint64_t timeout_ns;
  uint64_t* trace;       // phase timestamps [grid][kTracePhases] (ns), or null
  uint64_t trace_n;      // words of trace
  uint64_t* lit;         // litmus words [2], or null
  uint64_t* lit_last;    // [R][R]: a row the block completing source s's relay sent to d (~0: none)
  uint32_t lit_seed;
  char* span_base;       // lowest receive address, when the span path is on
  uint32_t span_bytes;
  uint32_t dspan[VR_MAX_RANKS];  // recv.p[d] + recv_off - span_base
  int R, T, K, E, NB1, NB2, nbits;
  int mode;              // 2: 16-byte lanes via the span; 1: 8-byte lanes; 0: bytes
  int rowbuf;            // count rows loaded with 16-byte lanes through LDS
};

// Phase timestamps of this workgroup, for the timeline a traced call records:
// word blockIdx.x * kTracePhases + phase receives the real-time clock in ns.
constexpr int kTracePhases = 8;
__device__ inline void stamp(const DispArgs& a, int phase) {
  if (a.trace && threadIdx.x == 0) {
    const uint64_t i = (uint64_t)blockIdx.x * kTracePhases + phase;
    if (i < a.trace_n) a.trace[i] = now_ns();
  }
}

// n / d for 0 <= n < 2^16 and 1 <= d <= 2^16, with mul = ceil(2^32 / d)
// computed on the host: exact, since n * (mul * d - 2^32) < n * d <= 2^32.
// (A 32-bit division by a runtime value expands to some twenty instructions.)
__device__ inline int32_t div_by(int32_t n, uint64_t mul) {
  return static_cast<int32_t>((static_cast<uint64_t>(static_cast<uint32_t>(n)) * mul) >> 32);
}

__device__ inline int32_t load_topk(const DispArgs& a, int s, int t, int k) {
  return a.topk[((size_t)s * a.T + t) * a.K + k];
}

// Dedup key of an entry whose token's K entries sit in lanes [group*K,
// group*K + K) of this wave: the destination rank if no lower lane of the
// same token names that rank, -1 for such a later entry and for unrouted
// ones; ids outside [-1, E) map to the out-of-range key a.E, which the
// callers flag and skip. The rank is matched over the wave (kbits ballots)
// and the match then kept to the token's lanes; matching (token, rank) over
// the wave took gbits + 8 ballots. All lanes of the wave call it.
__device__ inline int32_t dedup_rep(const DispArgs& a, int32_t e, int group, bool active) {
  const int32_t d = (e >= 0 && e < a.Eo) ? div_by(e, a.epro_mul) : (e == -1 ? -1 : a.E);
  const bool cand = active && d >= 0 && d < a.E;
  const uint32_t key = cand ? static_cast<uint32_t>(d) : static_cast<uint32_t>(a.E);  // non-candidates: no rank
  const uint64_t token = a.K >= 64 ? ~0ull : (((1ull << a.K) - 1ull) << (group * a.K));
  const uint64_t m = match_any(key, a.kbits) & token;
  const uint64_t lt = (1ull << lane_id()) - 1ull;
  if (!active) return -1;
  return cand ? ((m & lt) == 0 ? d : -1) : d;
}

// Last count block of source s: C[s][e] = sum of the block totals (16
// independent loads in flight per expert), each block's total replaced in
// place by the exclusive prefix of the earlier blocks' totals; then the count
// row to every rank and a SignalInc there (the count exchange).
__device__ void count_exchange(const DispArgs& a, int s) {
  const int R = a.R, E = a.E;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kThreads) {
    int32_t* col = a.blktot + (size_t)s * a.NB1 * E + e;
    int32_t run = 0;
    for (int b0 = 0; b0 < a.NB1; b0 += 16) {
      int32_t v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = b0 + q < a.NB1 ? load_coherent_i32(col + (size_t)(b0 + q) * E) : 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if (b0 + q < a.NB1) store4_agent(reinterpret_cast<uint32_t*>(col + (size_t)(b0 + q) * E), run);
        run += v[q];
      }
    }
    for (int d = 0; d < R; ++d)
      store4_agent(reinterpret_cast<uint32_t*>(a.cwin + ((size_t)d * R + s) * E + e), run);
  }
  wg_stores_complete();
  if (tid < R) atomic_add_u64(a.sig_counts + (size_t)tid * a.sig_stride, 1ull);  // SignalInc at each rank
}

// Dedup layout, off the count exchange's critical path: the entries of
// count block (s, blk) per expert (any entry of a token counts, whichever
// entry carries its row), then -- in the block completing source s's second
// relay -- source s's entries per expert over its count blocks, announced on
// a counter that the put blocks writing the per-expert counts wait for.
__device__ void expert_counts(const DispArgs& a, int32_t* lds, int* last_flag, int s, int blk) {
  const int tid = threadIdx.x;
  int32_t* hist_o = lds;  // [Eo]
  __syncthreads();  // the key histogram is no longer needed
  for (int i = tid; i < a.Eo; i += kThreads) hist_o[i] = 0;
  __syncthreads();
  const int t0 = blk * kCountBlock;
  const int n = max(0, min(a.T - t0, kCountBlock)) * a.K;
  for (int i0 = 0; i0 < n; i0 += 8 * kThreads) {  // 8 loads in flight per thread
    int32_t f[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kThreads + tid;
      f[u] = i < n ? a.topk[((size_t)s * a.T + t0) * a.K + i] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (f[u] >= 0 && f[u] < a.Eo) atomicAdd(&hist_o[f[u]], 1);
  }
  __syncthreads();
  for (int e = tid; e < a.Eo; e += kThreads)
    store4_agent(reinterpret_cast<uint32_t*>(a.eblk + ((size_t)s * a.NB1 + blk) * a.Eo + e), hist_o[e]);
  wg_stores_complete();
  if (tid == 0) *last_flag = relay_arrive(a.relay + (18 * a.R + s) * a.rstride, a.NB1, false);
  __syncthreads();
  if (!*last_flag) return;
  for (int e = tid; e < a.Eo; e += kThreads) {  // 16 loads in flight
    const int32_t* col = a.eblk + (size_t)s * a.NB1 * a.Eo + e;
    int32_t run = 0;
    for (int b0 = 0; b0 < a.NB1; b0 += 16) {
      int32_t v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = b0 + q < a.NB1 ? load_coherent_i32(col + (size_t)(b0 + q) * a.Eo) : 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) run += v[q];
    }
    store4_agent(reinterpret_cast<uint32_t*>(a.ecw + (size_t)s * a.Eo + e), run);
  }
  wg_stores_complete();
  if (tid == 0) atomic_add_u32(a.relay + (19 * a.R) * a.rstride, 1u);  // source s's expert counts are out
}

template <bool DEDUP>
__device__ void count_block(const DispArgs& a, int32_t* lds, int* last_flag, int wg) {
  const int R = a.R, E = a.E;
  const int s = wg % R, blk = wg / R;  // interleaved: sources' relays hit in parallel
  const int tid = threadIdx.x;
  int32_t* hist = lds;  // [kSubs][E]
  stamp(a, 0);
  for (int i = tid; i < kSubs * E; i += kThreads) hist[i] = 0;
  if (blk == 0 && tid == 0)
    store8_agent(a.base_rows + s, load_relaxed_u64(a.sig_rows + (size_t)s * a.sig_stride));
  __syncthreads();
  const int t0 = blk * kCountBlock;
  const int ntok = max(0, min(a.T - t0, kCountBlock));
  const int lane = tid & 63;
  if constexpr (DEDUP) {
    // per-rank layout: wave q < kSubs takes sub-block q, one token per lane.
    // The token's destination ranks form a bit mask (a rank named twice still
    // gets one row), and the sub-block's row count for rank r is the popcount
    // of one ballot: no LDS atomics. (Matching each entry's rank within its
    // token's lanes and adding per entry took 1.65 us from the routing loads
    // to the counts, against 0.64 us for the per-expert histogram; this way
    // the per-rank dispatch measured 31.0-31.4 against 32.0-32.1 us flushed,
    // 26.1 against 27.4 us back to back.)
    static_assert(kSub == 64, "a sub-block is one wave");
    const int q = tid >> 6;
    if (q < kSubs) {
      const int tl = q * kSub + lane;
      uint64_t mask = 0;
      bool bad = false;
      auto note = [&](int32_t e) {
        if (e == -1) return;
        if (e < 0 || e >= a.Eo) bad = true;
        else mask |= 1ull << div_by(e, a.epro_mul);
      };
      if (tl < ntok) {
        const int32_t* ids = a.topk + ((size_t)s * a.T + t0 + tl) * a.K;
        if (a.ids_vec) {  // 16-byte loads of the token's ids, four in flight
          const v4u* ids4 = reinterpret_cast<const v4u*>(ids);
          for (int k0 = 0; k0 < a.K / 4; k0 += 4) {
            v4u f[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) f[u] = k0 + u < a.K / 4 ? ids4[k0 + u] : v4u{~0u, ~0u, ~0u, ~0u};
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
              for (int j = 0; j < 4; ++j) note(static_cast<int32_t>(f[u][j]));
          }
        } else {
          for (int k0 = 0; k0 < a.K; k0 += 8) {
            int32_t f[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) f[u] = k0 + u < a.K ? ids[k0 + u] : -1;
#pragma unroll
            for (int u = 0; u < 8; ++u) note(f[u]);
          }
        }
      }
      if (bad) atomic_or_u32(a.err, VR_ASYNC_BAD_EXPERT);
      for (int r = 0; r < R; ++r) {  // keys are ranks: E == R
        const uint64_t b = ballot((mask >> r) & 1ull);
        if (lane == 0) hist[q * E + r] = static_cast<int32_t>(__popcll(b));
      }
    }
  } else {
    // plain LDS atomics (measured faster than first grouping equal keys of a
    // wave instruction with ballots)
    const int iters = (ntok * a.K + kThreads - 1) / kThreads;
    // entry i = step * kThreads + tid is (token i / K, k = i % K); both advance
    // by a fixed amount per step, so no division by K inside the loop
    const int sq = kThreads / a.K, sr = kThreads - sq * a.K;
    int cq = tid / a.K, cr = tid - cq * a.K;  // for step 0
    for (int it0 = 0; it0 < iters; it0 += 8) {  // 8 loads in flight per thread, then the adds
      int ev[8], tq[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = (it0 + u) * kThreads + tid;
        const bool in = it0 + u < iters && i < ntok * a.K;
        tq[u] = cq;
        ev[u] = in ? load_topk(a, s, t0 + cq, cr) : -1;
        cq += sq;
        cr += sr;
        if (cr >= a.K) {
          cr -= a.K;
          ++cq;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (it0 + u >= iters) break;
        const int e = ev[u];
        if (e != -1 && (e < 0 || e >= E)) atomic_or_u32(a.err, VR_ASYNC_BAD_EXPERT);
        if (e >= 0 && e < E) atomicAdd(&hist[(tq[u] / kSub) * E + e], 1);
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    int32_t run = 0;
    for (int q = 0; q < kSubs; ++q) {
      store4_agent(reinterpret_cast<uint32_t*>(a.subpfx + ((size_t)s * a.NB1 * kSubs + blk * kSubs + q) * E + e), run);
      run += hist[q * E + e];
    }
    store4_agent(reinterpret_cast<uint32_t*>(a.blktot + ((size_t)s * a.NB1 + blk) * E + e), run);
  }
  wg_stores_complete();
  stamp(a, 1);
  if (tid == 0) *last_flag = relay_arrive(a.relay + s * a.rstride, a.NB1, false);
  __syncthreads();
  if (*last_flag) {
    count_exchange(a, s);
    stamp(a, 2);
  }
  if (DEDUP) expert_counts(a, lds, last_flag, s, blk);
}

// Dedup layout, put block (s, 0): rank s's entries per local expert over
// every source, once every source's counts are out; the last of the R
// readers resets the announcement counter for the next launch.
__device__ void put_expert_counts(const DispArgs& a, int s) {
  const int R = a.R, tid = threadIdx.x;
  __shared__ int ok;
  uint32_t* ready = a.relay + (19 * R) * a.rstride;
  uint32_t* readers = a.relay + (19 * R + 1) * a.rstride;
  if (tid == 0) {
    const uint64_t t0 = now_ns();
    ok = 1;
    while (load_relaxed_u32(ready) < static_cast<uint32_t>(R)) {
      if (now_ns() - t0 > a.timeout_ns) {
        atomic_or_u32(a.err, VR_ASYNC_TIMEOUT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
  if (ok)
    for (int j = tid; j < a.epro; j += kThreads) {
      int32_t run = 0;
      for (int q0 = 0; q0 < R; q0 += 16) {  // 16 loads in flight
        int32_t v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q)
          v[q] = q0 + q < R ? load_coherent_i32(a.ecw + (size_t)(q0 + q) * a.Eo + s * a.epro + j) : 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) run += v[q];
      }
      store4_agent(reinterpret_cast<uint32_t*>(a.ecounts_out + (size_t)s * a.epro + j), static_cast<uint32_t>(run));
    }
  wait_vmem();  // this thread's loads of the counts are done
  __syncthreads();
  if (tid == 0 && relay_arrive(readers, R, false))
    __hip_atomic_store(ready, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool DEDUP, int G>
__device__ void put_block(const DispArgs& a, int32_t* lds, int* last_flag, int wg) {
  // LDS: tot[E] (rows of expert e over all sources), base[E] (receive row of
  // this block's first row of expert e), hw[kWaves][E] (per-wave counts, then
  // exclusive per-wave prefixes), dpos/dexp[64*K] (destination row and expert
  // of each routing entry of the block), crow[E] (this source's count row)
  const int R = a.R, E = a.E, epr = a.E / a.R, K = a.K;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int32_t* tot = lds;
  int32_t* base = tot + E;
  int32_t* hwf = base + E;
  int32_t* dpos = hwf + kWaves * E;
  int32_t* dexp = dpos + kSub * K;
  int32_t* crow = dexp + kSub * K;
  int32_t* dorig = crow + E;  // dedup: [kSub*K] each entry's expert id
  const int s = wg % R, b2 = wg / R;  // interleaved sources
  const int b1 = b2 / kSubs;
  stamp(a, 0);
  const int tpr = 64 / K;  // tokens per ballot round
  const int tw0 = b2 * kSub + wave * kTokPerWave;
  const int rounds = (kTokPerWave + tpr - 1) / tpr;
  const int ntw = max(0, min(kTokPerWave, a.T - tw0));
  const uint64_t rb = a.row_bytes;
  // Loads that depend on no count are issued first: this wave's routing
  // entries, one register per ballot round.
  int lpr = 1;
  const int nv = static_cast<int>(rb >> 4);
  while (lpr < nv) lpr <<= 1;
  const int rpi = a.mode == 2 ? 64 / lpr : 1;
  const int l = lane & (lpr - 1), sub = lane / lpr;
  const int groups = (kTokPerWave + rpi - 1) / rpi;
  int ent[kTokPerWave];  // routing entry of this lane in each ballot round (-1: none)
#pragma unroll
  for (int rd = 0; rd < kTokPerWave; ++rd) {
    const int tl = rd * tpr + lane / K;
    ent[rd] = (rd < rounds && lane < tpr * K && tl < ntw) ? load_topk(a, s, tw0 + tl, lane % K) : -1;
  }
  // This wave's token rows (16-byte path, at most G vectors per lane) stay
  // in registers until the copy. They are loaded here, before the ranking,
  // so that the row loads are done before the count exchange's round trips
  // instead of queueing in front of them (per-expert layout: 40.0 against
  // 41.1 us flushed, 33.5 against 34.4 us back to back, three alternations
  // on one box) -- except in the per-rank layout with G = kTokPerWave, where
  // the longer live range takes the kernel to 92 VGPRs and 5 waves per SIMD:
  // there they are loaded after the ranking.
  v4u v[G];
  auto load_rows = [&]() {
    if (a.mode != 2) return;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int tl = g * rpi + sub;
      v[g] = (g < groups && tl < ntw && l < nv)
                 ? load16_stream(reinterpret_cast<const v4u*>(a.x.p[s] + a.x_off + (uint64_t)(tw0 + tl) * rb + l * 16))
                 : v4u{0, 0, 0, 0};
    }
  };
  constexpr bool kEarly = !DEDUP || G < kTokPerWave;
  if (kEarly) load_rows();
  // Ranking within the block needs no counts: per-wave counts, their
  // exclusive prefix over the waves, then each entry's rank among the
  // block's entries of its expert (token order). dpos holds that local rank.
  for (int e = tid; e < E; e += kThreads)
    for (int w = 0; w < kWaves; ++w) hwf[w * E + e] = 0;
  const uint64_t lt = (1ull << lane) - 1ull;
  __syncthreads();
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int rd = 0; rd < kTokPerWave; ++rd) {
      if (rd >= rounds) break;
      const int tl = rd * tpr + lane / K;  // token index within the wave
      const int k = lane % K;
      const bool valid = lane < tpr * K && tl < ntw;
      // a round holds whole tokens, so the dedup key comes from the neighbouring lanes
      const int e = DEDUP ? dedup_rep(a, ent[rd], lane / K, valid) : ent[rd];
      const bool ok = valid && e >= 0 && e < E;
      if (pass == 0 && valid && e != -1 && !ok) atomic_or_u32(a.err, VR_ASYNC_BAD_EXPERT);
      int32_t lpos = -1;
      if (ok && pass == 0) atomicAdd(&hwf[wave * E + e], 1);  // counts only
      if (ok && pass == 1) {  // rank among the wave's entries of expert e, in lane (token) order
        const uint64_t m = match_any(static_cast<uint32_t>(e), a.nbits);
        const bool leader = (m & lt) == 0;
        const int cnt = __popcll(m);
        lpos = hwf[wave * E + e] + __popcll(m & lt);
        if (leader) hwf[wave * E + e] += cnt;
      }
      if (pass == 1 && valid) {
        const int slot = (wave * kTokPerWave + tl) * K + k;
        dpos[slot] = lpos;
        dexp[slot] = ok ? e : -1;
        if (DEDUP) dorig[slot] = ent[rd];
      }
    }
    __syncthreads();
    if (pass == 0)
      for (int e = tid; e < E; e += kThreads) {
        int32_t run = 0;
        for (int w = 0; w < kWaves; ++w) {
          const int32_t c = hwf[w * E + e];
          hwf[w * E + e] = run;
          run += c;
        }
      }
    __syncthreads();
  }
  if (!kEarly) load_rows();  // loaded while the counts are awaited
  // count exchange: rank s waits until every source's count row has arrived;
  // the rows and prefixes are then read with agent-coherent loads.
  stamp(a, 1);
  if (tid == 0)
    wait_reached(a.sig_counts + (size_t)s * a.sig_stride, a.target_counts.v[s], 64, a.timeout_ns, a.err,
                 VR_ASYNC_TIMEOUT, false);
  stamp(a, 2);
  __syncthreads();
  compiler_fence();
  const int32_t* cw = a.cwin + (size_t)s * R * E;  // rank s's copy: cw[s'][e]
  const int32_t* pb = a.blktot + ((size_t)s * a.NB1 + b1) * E;  // rows of source s's earlier count blocks
  const int32_t* ps = a.subpfx + ((size_t)s * a.NB1 * kSubs + b2) * E;
  if (a.rowbuf) {
    // the R count rows and the two prefix rows, 16-byte agent-coherent loads
    // (one or two per thread, all in flight together), staged in LDS
    int32_t* rb4 = dorig + (DEDUP ? kSub * K : 0);  // [(R + 2)][E]
    const int n4 = E >> 2;
    const __amdgpu_buffer_rsrc_t rcw = rsrc(cw, (uint32_t)(R * E * 4));
    const __amdgpu_buffer_rsrc_t rps = rsrc(ps, (uint32_t)(E * 4)), rpb = rsrc(pb, (uint32_t)(E * 4));
    for (int i = tid; i < (R + 2) * n4; i += kThreads) {
      const int q = i / n4, e4 = i - q * n4;
      const v4u v = q < R ? __builtin_amdgcn_raw_buffer_load_b128(rcw, (uint32_t)(i * 16), 0, kStoreAgent)
                          : __builtin_amdgcn_raw_buffer_load_b128(q == R ? rps : rpb, (uint32_t)(e4 * 16), 0,
                                                                  kStoreAgent);
      *reinterpret_cast<v4u*>(rb4 + i * 4) = v;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) {
      int32_t t = 0, pre = 0, own = 0;
      for (int j = 0; j < R; ++j) {
        const int32_t x = rb4[j * E + e];
        t += x;
        if (j < s) pre += x;
        if (j == s) own = x;
      }
      tot[e] = t;
      crow[e] = own;
      base[e] = pre + rb4[R * E + e] + rb4[(R + 1) * E + e];
    }
  } else
  for (int e = tid; e < E; e += kThreads) {
    // count rows of every source, the prefix over this source's earlier count
    // blocks and over the earlier sub-blocks of this one: independent loads
    // issued in batches of 16, one round trip each
    int32_t t = 0, pre = 0, own = 0;
    int32_t before = load_coherent_i32(ps + e) + load_coherent_i32(pb + e);
    for (int q0 = 0; q0 < R; q0 += 16) {
      int32_t v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = q0 + q < R ? load_coherent_i32(cw + (size_t)(q0 + q) * E + e) : 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int j = q0 + q;
        if (j < R) {
          t += v[q];
          if (j < s) pre += v[q];
          if (j == s) own = v[q];
        }
      }
    }
    tot[e] = t;
    crow[e] = own;  // C[s][e], for the trailing signals
    base[e] = pre + before;
  }
  __syncthreads();
  stamp(a, 3);
  // seg[e]: rows of the experts before e on the same rank. When the rank's
  // experts tile the waves (epr a power of two up to 64), a shuffle scan
  // within each group of epr lanes; otherwise a loop over LDS.
  const bool scan = epr <= 64 && (epr & (epr - 1)) == 0;
  for (int e = tid; e < E; e += kThreads) {
    int32_t seg = 0;
    if (scan) {
      const int32_t v = tot[e];
      const int pos = e & (epr - 1);  // = lane mod epr: kThreads is a multiple of 64
      int32_t x = v;
      for (int d = 1; d < epr; d <<= 1) {
        const int32_t y = __shfl_up(x, d, 64);
        if (pos >= d) x += y;
      }
      seg = x - v;
    } else {
      for (int q = (e / epr) * epr; q < e; ++q) seg += tot[q];
    }
    base[e] += seg;
  }
  if (b2 == 0)
    for (int j = tid; j < epr; j += kThreads)
      store4_agent(reinterpret_cast<uint32_t*>(a.counts_out + (size_t)s * epr + j), tot[s * epr + j]);
  __syncthreads();
  // final receive rows; each row's source tag
  for (int slot = tid; slot < kSub * K; slot += kThreads) {
    const int tlb = slot / K;  // token within the block
    if (tlb >= kSub || b2 * kSub + tlb >= a.T) continue;
    const int e = dexp[slot];
    const int tg = b2 * kSub + tlb;
    uint32_t* po = nullptr;  // dedup positions are written below, one per (token, rank)
    if (a.pos_out && !DEDUP) po = reinterpret_cast<uint32_t*>(a.pos_out + ((size_t)s * a.T + b2 * kSub) * K + slot);
    if (DEDUP && e < 0) continue;  // not a key entry
    if (e < 0) {
      if (po) store4_agent(po, 0xFFFFFFFFu);
      continue;
    }
    const int32_t pos = base[e] + dpos[slot];
    dpos[slot] = pos;
    const int d = div_by(e, a.epr_mul);
    const bool kept = (uint64_t)pos < a.cap;
    if (DEDUP && kept) {  // the row's entries as rank d sees them (an output: plain stores)
      int32_t* xo = a.experts_out + ((size_t)d * a.cap + pos) * K;
      auto local = [&](int k) {
        const int32_t f = dorig[tlb * K + k];
        return (f >= 0 && f < a.Eo && div_by(f, a.epro_mul) == d) ? f - d * a.epro : -1;
      };
      if (a.xo_vec) {
        for (int k = 0; k < K; k += 4)
          *reinterpret_cast<v4u*>(xo + k) = v4u{static_cast<uint32_t>(local(k)), static_cast<uint32_t>(local(k + 1)),
                                                static_cast<uint32_t>(local(k + 2)), static_cast<uint32_t>(local(k + 3))};
      } else {
        for (int k = 0; k < K; ++k) xo[k] = local(k);
      }
    }
    if (kept) {
      store4_agent(reinterpret_cast<uint32_t*>(a.src_out + (size_t)d * a.cap + pos),
                   static_cast<uint32_t>((s << 16) | (b2 * kSub + tlb)));
      if (po) store4_agent(po, static_cast<uint32_t>(pos));
    } else {
      atomic_or_u32(a.err, VR_ASYNC_CAPACITY);
      if (po) store4_agent(po, 0xFFFFFFFFu);
    }
  }
  __syncthreads();
  if (DEDUP && a.pos_out)  // each token's row at every rank, -1 where it is not sent (contiguous per token)
    for (int i = tid; i < kSub * R; i += kThreads) {
      const int tlb = i / R, d = i % R;
      if (b2 * kSub + tlb >= a.T) continue;
      int32_t pos = -1;
      for (int k = 0; k < K; ++k)
        if (dexp[tlb * K + k] == d) pos = dpos[tlb * K + k];
      a.pos_out[((size_t)s * a.T + b2 * kSub) * R + i] = (uint64_t)pos < a.cap ? pos : -1;
    }
  stamp(a, 4);
  // copy: the wave's 8 token rows, each once per routed expert
  if (a.mode == 2) {
    const __amdgpu_buffer_rsrc_t rd = rsrc(a.span_base, a.span_bytes);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (g >= groups) break;
      const int tl = g * rpi + sub;
      if (tl < ntw && l < nv) {
        const int slot0 = (wave * kTokPerWave + tl) * K;
        for (int k = 0; k < K; ++k) {
          const int32_t pos = dpos[slot0 + k];
          if (pos < 0 || (uint64_t)pos >= a.cap) continue;
          const int d = dexp[slot0 + k] / epr;
          store16_agent(rd, a.dspan[d] + static_cast<uint32_t>(pos) * static_cast<uint32_t>(rb) + l * 16, v[g]);
        }
      }
    }
  } else {
    for (int tl = 0; tl < ntw; ++tl) {
      const char* src = a.x.p[s] + a.x_off + (uint64_t)(tw0 + tl) * rb;
      const int slot0 = (wave * kTokPerWave + tl) * K;
      for (int k = 0; k < K; ++k) {
        const int32_t pos = dpos[slot0 + k];
        if (pos < 0 || (uint64_t)pos >= a.cap) continue;
        char* dst = a.recv.p[dexp[slot0 + k] / epr] + a.recv_off + (uint64_t)pos * rb;
        if (a.mode == 1) {
          for (uint64_t o = (uint64_t)lane * 8; o < rb; o += 512)
            store8_agent(reinterpret_cast<uint64_t*>(dst + o),
                         __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(src + o)));
        } else {
          copy_bytes(dst, src, static_cast<uint32_t>(rb), lane, 64);
        }
      }
    }
  }
  stamp(a, 5);
  if (DEDUP && b2 == 0) put_expert_counts(a, s);
  wg_stores_complete();
  stamp(a, 6);
  if (tid == 0) {
    // two-level relay: 16 first-level counters per source, then one per source
    const int g = b2 % kRelayFan;
    const int in_g = (a.NB2 - g + kRelayFan - 1) / kRelayFan;
    bool lastp = relay_arrive(a.relay + (R + s * kRelayFan + g) * a.rstride, in_g, false);
    if (lastp) lastp = relay_arrive(a.relay + (R + R * kRelayFan + s) * a.rstride, min(a.NB2, kRelayFan), false);
    *last_flag = lastp;
  }
  __syncthreads();
  if (*last_flag && tid < R) {  // one trailing SignalAdd(rows from s) per destination
    const int d = tid;
    uint64_t rows = 0;
    for (int e = d * epr; e < (d + 1) * epr; ++e) rows += crow[e];
    if (a.lit) {  // the last receive row this block wrote at d, for the receiver's litmus
      uint64_t last = ~0ull;
      for (int slot = 0; slot < kSub * K; ++slot) {
        if (b2 * kSub + slot / K >= a.T || dexp[slot] < 0 || dexp[slot] / epr != d) continue;
        const int32_t pos = dpos[slot];
        if (pos >= 0 && (uint64_t)pos < a.cap && (last == ~0ull || (uint64_t)pos > last)) last = (uint64_t)pos;
      }
      litmus_record(a.lit_last + (size_t)s * R + d, last);
    }
    if (rows) atomic_add_u64(a.sig_rows + (size_t)d * a.sig_stride, rows);
  }
  if (*last_flag) stamp(a, 7);
}

// Receiver d, litmus on, after its row signal has reached its target: the
// row each source's completing block wrote last at d, whole, then one
// seeded 16-byte sample of every received row, each against the token row
// its source tag names (and the tag itself checked).
__device__ void dispatch_litmus(const DispArgs& a, int d, int32_t rows) {
  const int R = a.R, tid = threadIdx.x;
  const uint64_t rb = a.row_bytes;
  const uint64_t n = std::min<uint64_t>(static_cast<uint64_t>(rows), a.cap);
  const char* rbase = a.recv.p[d] + a.recv_off;
  const int32_t* tags = a.src_out + (size_t)d * a.cap;
  uint32_t checks = 0, bad = 0;
  for (int s = 0; s < R; ++s) {
    const uint64_t i = load_relaxed_u64(a.lit_last + (size_t)s * R + d);
    if (i == ~0ull) continue;  // source s's completing block sent nothing to d
    const int32_t tag = i < n ? tags[i] : -1;
    const int ts = tag >> 16, tt = tag & 0xFFFF;
    if (i >= n || ts != s || tt >= a.T) {
      if (tid == 0) ++checks, ++bad;
      continue;
    }
    for (uint64_t o = (uint64_t)tid * 16; o < rb; o += kThreads * 16) {
      ++checks;
      bad += !equal_upto16(rbase + i * rb + o, a.x.p[ts] + a.x_off + (uint64_t)tt * rb + o,
                           static_cast<uint32_t>(std::min<uint64_t>(16, rb - o)));
    }
  }
  for (uint64_t i = tid; i < n; i += kThreads) {
    const int32_t tag = tags[i];
    const int ts = tag >> 16, tt = tag & 0xFFFF;
    ++checks;
    if (ts < 0 || ts >= R || tt >= a.T) {
      ++bad;
      continue;
    }
    const uint32_t o = (mix32(a.lit_seed + static_cast<uint32_t>(i) * 0x9E3779B9u) % static_cast<uint32_t>(rb)) & ~15u;
    bad += !equal_upto16(rbase + i * rb + o, a.x.p[ts] + a.x_off + (uint64_t)tt * rb + o,
                         std::min(16u, static_cast<uint32_t>(rb) - o));
  }
  litmus_report(a.lit, a.err, checks, bad);
}

// Receiver d: waits for the count exchange (which fixes how many rows are
// aimed at d and the base recorded before any row signal moved), then for
// the row signal to grow by that many rows.
__device__ void receiver_block(const DispArgs& a, int32_t* lds, int d) {
  const int R = a.R, E = a.E, epr = a.E / a.R;
  const int tid = threadIdx.x;
  stamp(a, 0);
  if (tid == 0)
    wait_reached(a.sig_counts + (size_t)d * a.sig_stride, a.target_counts.v[d], 64, a.timeout_ns, a.err,
                 VR_ASYNC_TIMEOUT, false);
  stamp(a, 1);
  __syncthreads();
  compiler_fence();
  int32_t part = 0;
  for (int i = tid; i < R * epr; i += kThreads)
    part += load_coherent_i32(a.cwin + ((size_t)d * R + i / epr) * E + d * epr + i % epr);
  lds[tid] = part;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) lds[tid] += lds[tid + w];
    __syncthreads();
  }
  const int32_t rows = lds[0];
  if (!a.lit) {
    if (tid == 0) {
      const uint64_t base = load_relaxed_u64(a.base_rows + d);
      wait_reached(a.sig_rows + (size_t)d * a.sig_stride, base + static_cast<uint64_t>(rows), 64, a.timeout_ns,
                   a.err, VR_ASYNC_TIMEOUT);
    }
    stamp(a, 2);
  } else if (receiver_wait(a.sig_rows + (size_t)d * a.sig_stride,
                           load_relaxed_u64(a.base_rows + d) + static_cast<uint64_t>(rows), a.timeout_ns, a.err)) {
    dispatch_litmus(a, d, rows);
  }
}

template <bool DEDUP, int G>
__global__ __launch_bounds__(kThreads) void k_dispatch(const DispArgs a) {
  extern __shared__ int32_t lds[];
  __shared__ int last;
  const int ncount = a.R * a.NB1, nput = a.R * a.NB2;
  const int b = blockIdx.x;
  if (b < ncount) count_block<DEDUP>(a, lds, &last, b);
  else if (b < ncount + nput) put_block<DEDUP, G>(a, lds, &last, b - ncount);
  else receiver_block(a, lds, b - ncount - nput);
}


size_t al256(size_t v) { return (v + 255) / 256 * 256; }

struct Layout {
  size_t subpfx, blktot, cwin, base_rows, rows, eblk, ecw, total;
};
Layout scratch_layout(int R, int T, int E, int Eo) {
  const size_t NB1 = std::max(1, (T + kCountBlock - 1) / kCountBlock);
  Layout l;
  l.subpfx = 0;
  l.blktot = al256((size_t)R * NB1 * kSubs * E * 4);
  l.cwin = l.blktot + al256((size_t)R * NB1 * E * 4);
  l.base_rows = l.cwin + al256((size_t)R * R * E * 4);
  l.rows = l.base_rows + al256((size_t)R * 8);  // dedup: rows per destination rank
  l.eblk = l.rows + al256((size_t)R * 4);
  l.ecw = l.eblk + al256((size_t)R * NB1 * Eo * 4);
  l.total = l.ecw + al256((size_t)R * Eo * 4);
  return l;
}

}  // namespace

size_t dispatch_scratch_bytes(int R, int T, int E, int Eo) { return scratch_layout(R, T, E, Eo).total; }

vrResult_t launch_dispatch(vrComm* c, const vrWindow* x, size_t x_off, size_t row_bytes, const int32_t* topk, int T,
                           int K, int E, const vrWindow* recv, size_t recv_off, size_t cap, int32_t* counts_out,
                           int32_t* src_out, int32_t* pos_out, int32_t* experts_out, bool dedup, uint32_t sig_counts,
                           uint32_t sig_rows, const U64Tab& target_counts, bool wait, char* scratch,
                           hipStream_t st) {
  DispArgs a;
  const int R = c->nranks;
  // dedup: the layout's keys are the destination ranks (E = R, one per rank)
  a.Eo = E;
  a.epro = E / R;
  a.epro_mul = ((1ull << 32) + a.epro - 1) / a.epro;
  a.experts_out = experts_out;
  a.ecounts_out = dedup ? counts_out : nullptr;
  a.gbits = 0;  // tokens within a wave: lane / K < ceil(64 / K)
  while ((1 << a.gbits) < (64 + K - 1) / K) ++a.gbits;
  a.xo_vec = K % 4 == 0 && (reinterpret_cast<uintptr_t>(experts_out) & 15) == 0;
  a.ids_vec = K % 4 == 0 && (reinterpret_cast<uintptr_t>(topk) & 15) == 0;
  const int Eo = E;
  if (dedup) E = R;
  for (int r = 0; r < VR_MAX_RANKS; ++r) {
    a.x.p[r] = x->base[r];
    a.recv.p[r] = recv->base[r];
    a.dspan[r] = 0;
  }
  a.target_counts = target_counts;
  a.x_off = x_off;
  a.recv_off = recv_off;
  a.row_bytes = row_bytes;
  a.cap = cap;
  a.topk = topk;
  a.counts_out = counts_out;
  a.src_out = src_out;
  a.pos_out = pos_out;
  a.NB1 = std::max(1, (T + kCountBlock - 1) / kCountBlock);
  a.NB2 = a.NB1 * kSubs;
  const Layout l = scratch_layout(R, T, E, dedup ? Eo : 0);
  if (dedup) a.counts_out = reinterpret_cast<int32_t*>(scratch + l.rows);
  a.eblk = reinterpret_cast<int32_t*>(scratch + l.eblk);
  a.ecw = reinterpret_cast<int32_t*>(scratch + l.ecw);
  int nbo = 1;
  while ((1 << nbo) < Eo) ++nbo;
  a.nbits_o = nbo;
  a.subpfx = reinterpret_cast<int32_t*>(scratch + l.subpfx);
  a.blktot = reinterpret_cast<int32_t*>(scratch + l.blktot);
  a.cwin = reinterpret_cast<int32_t*>(scratch + l.cwin);
  a.base_rows = reinterpret_cast<uint64_t*>(scratch + l.base_rows);
  a.sig_counts = c->sig + sig_counts;
  a.sig_rows = c->sig + sig_rows;
  a.sig_stride = c->req.signal_count;
  a.relay = c->relay + kRelayDispatch;
  // counters: [R) count blocks, [R, 17R) and [17R, 18R) put blocks, [18R, 19R)
  // dedup expert counts, then the dedup counts' announcement and its readers
  a.rstride = relay_stride(19 * R + 2, kRelayDispatchWords);
  a.err = c->err;
  a.timeout_ns = kDefaultTimeoutNs;
  a.lit = c->litmus;
  a.lit_last = c->lit_last;
  a.lit_seed = c->lit_seed++;
  a.trace = c->trace;
  a.trace_n = c->trace_words;
  a.R = R;
  a.T = T;
  a.K = K;
  a.E = E;
  int nb = 1;
  while ((1 << nb) < E) ++nb;
  a.nbits = nb;
  int kb = 1;
  while ((1 << kb) <= E) ++kb;
  a.kbits = kb;  // values 0..E
  a.epr_mul = ((1ull << 32) + E / R - 1) / (E / R);
  // copy path: one buffer resource over all receive slices when they fit a 4 GiB span
  char* lo = recv->base[0] + recv_off;
  char* hi = lo + cap * row_bytes;
  for (int r = 1; r < R; ++r) {
    lo = std::min(lo, recv->base[r] + recv_off);
    hi = std::max(hi, recv->base[r] + recv_off + cap * row_bytes);
  }
  const bool al16 = row_bytes % 16 == 0 && x_off % 16 == 0 && recv_off % 16 == 0 && row_bytes <= 1024;
  a.span_base = lo;
  a.span_bytes = 0;
  if (al16 && (uint64_t)(hi - lo) < (1ull << 32)) {
    a.mode = 2;
    a.span_bytes = static_cast<uint32_t>(hi - lo);
    for (int r = 0; r < R; ++r) a.dspan[r] = static_cast<uint32_t>(recv->base[r] + recv_off - lo);
  } else {
    a.mode = (row_bytes % 8 == 0 && x_off % 8 == 0 && recv_off % 8 == 0) ? 1 : 0;
  }
  // count rows through LDS when E splits into 16-byte lanes and the rows fit 16 KiB
  a.rowbuf = (E % 4) == 0 && (size_t)(R + 2) * E * 4 <= 16384;
  const size_t lds = sizeof(int32_t) * std::max<size_t>({(size_t)kSubs * E + (dedup ? (size_t)Eo : 0),
                                                         (3 + kWaves) * (size_t)E + 2 * (size_t)kSub * K +
                                                             (dedup ? (size_t)kSub * K : 0) +
                                                             (a.rowbuf ? (size_t)(R + 2) * E : 0),
                                                         (size_t)kThreads});
  const int grid = R * a.NB1 + R * a.NB2 + (wait ? R : 0);
  // Per-rank layout with rows of up to 512 bytes: two or more rows per wave
  // instruction, so at most kTokPerWave / 2 row vectors per lane, which lets
  // its row loads go out before its ranking at 76 VGPRs (30.5-31.0 against
  // 31.2-31.4 us flushed, three alternations on one box). The per-expert
  // layout keeps the full bound: with it (58 VGPRs, 7 waves per SIMD) it
  // measured 0.3 us slower.
  if (dedup && a.mode == 2 && row_bytes <= 512)
    hipLaunchKernelGGL((k_dispatch<true, kTokPerWave / 2>), dim3(grid), dim3(kThreads), lds, st, a);
  else if (dedup)
    hipLaunchKernelGGL((k_dispatch<true, kTokPerWave>), dim3(grid), dim3(kThreads), lds, st, a);
  else
    hipLaunchKernelGGL((k_dispatch<false, kTokPerWave>), dim3(grid), dim3(kThreads), lds, st, a);
  return hipGetLastError() == hipSuccess ? VR_OK : VR_ERR_HIP;
}

}  // namespace vr
