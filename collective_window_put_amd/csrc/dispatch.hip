// MoE token dispatch over symmetric windows: count exchange, offsets, puts.
//
// GDA survey (10100.com/article/158785524), opening section: an MoE dispatch
// routes tokens of a few hundred bytes among dozens of experts, with sizes
// and targets known only at run time; section 4: a batch of puts closed by
// one signal orders them cheaply. Layout of rank d's receive rows: by expert
// (rank d owns experts [d*E/R, (d+1)*E/R)), then source rank, then token.
//
// Kernel 1 (count): workgroup (s, b) histograms the routing entries of its 64
// tokens in LDS and stores the block histogram. The last block of source s
// (relay) turns source s's block histograms into exclusive prefixes (the
// stable position of each block's first row per expert), then puts the count
// row C[s][.] into every rank's count window and applies a SignalInc at each
// (count exchange). Block (s, 0) also records rank s's row signal as the base
// its receiver will wait from.
// Kernel 2 (put): workgroup (s, b) waits for rank s's count signal, derives
// every expert's receive offset from the full count matrix
//   off(s, e) = sum_{e' < e owned by the same rank} sum_s' C[s'][e]
//             + sum_{s' < s} C[s'][e],
// ranks its routing entries stably (token order) with wave ballots, and copies
// each token row once per routed expert. The last block of source s applies
// one SignalAdd(rows sent to d) at every rank d. The last R workgroups wait
// until each rank's row signal has grown by the rows aimed at it.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "vr_device.hpp"
#include "vr_internal.hpp"

namespace vr {
namespace {

constexpr int kTokPerBlock = 64;   // tokens per workgroup
constexpr int kTokPerWave = 16;    // 4 waves
constexpr int kMaxE = 1024;
constexpr int kMaxK = 64;

struct DispArgs {
  WinTab x, recv;
  U64Tab target_counts;
  uint64_t x_off, recv_off, row_bytes, cap;
  const int32_t* topk;  // [R][T][K]
  int32_t* counts_out;  // [R][E/R]
  int32_t* src_out;     // [R][cap]
  int32_t* hblk;        // [R][NB][E]
  int32_t* cwin;        // [R][R][E]: rank d's copy of every source's count row
  uint64_t* base_rows;  // [R]
  uint64_t* sig_counts; // &sig[0][id]
  uint64_t* sig_rows;
  uint32_t sig_stride;
  uint32_t* relay;      // [2R]: count kernel, put kernel
  uint32_t* err;
  uint64_t timeout_ns;
  int R, T, K, E, NB, nbits;
  int fast;             // rows and bases 8-byte aligned
};

__device__ inline int32_t load_topk(const DispArgs& a, int s, int t, int k) {
  return a.topk[((size_t)s * a.T + t) * a.K + k];
}

__global__ __launch_bounds__(256) void k_dispatch_count(const DispArgs a) {
  __shared__ int32_t hist[kMaxE];
  __shared__ int last;
  const int s = blockIdx.x / a.NB, blk = blockIdx.x % a.NB;
  const int tid = threadIdx.x;
  for (int e = tid; e < a.E; e += 256) hist[e] = 0;
  if (blk == 0 && tid == 0)
    store8_agent(a.base_rows + s, load_relaxed_u64(a.sig_rows + (size_t)s * a.sig_stride));
  __syncthreads();
  const int t0 = blk * kTokPerBlock;
  const int ntok = max(0, min(a.T - t0, kTokPerBlock));
  for (int i = tid; i < ntok * a.K; i += 256) {
    const int e = load_topk(a, s, t0 + i / a.K, i % a.K);
    if (e == -1) continue;
    if (e < 0 || e >= a.E) {
      atomic_or_u32(a.err, VR_ASYNC_BAD_EXPERT);
      continue;
    }
    atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  int32_t* hb = a.hblk + ((size_t)s * a.NB + blk) * a.E;
  for (int e = tid; e < a.E; e += 256) store4_agent(reinterpret_cast<uint32_t*>(hb + e), hist[e]);
  wg_stores_complete();
  if (tid == 0) last = relay_arrive(a.relay + s, a.NB);
  __syncthreads();
  if (!last) return;
  // last block of source s: exclusive prefix over blocks, count row to every rank
  for (int e = tid; e < a.E; e += 256) {
    int32_t run = 0;
    for (int b = 0; b < a.NB; ++b) {
      int32_t* p = a.hblk + ((size_t)s * a.NB + b) * a.E + e;
      const int32_t v = *p;
      store4_agent(reinterpret_cast<uint32_t*>(p), run);
      run += v;
    }
    for (int d = 0; d < a.R; ++d)
      store4_agent(reinterpret_cast<uint32_t*>(a.cwin + ((size_t)d * a.R + s) * a.E + e), run);
  }
  wg_stores_complete();
  if (tid < a.R) atomic_add_u64(a.sig_counts + (size_t)tid * a.sig_stride, 1ull);  // SignalInc at each rank
}

__global__ __launch_bounds__(256) void k_dispatch_put(const DispArgs a) {
  // dynamic LDS: tot[E] (rows of expert e over all sources), base[E] (receive
  // row of this block's first row of expert e), hw[4][E] (per-wave counts, then
  // exclusive per-wave prefixes), dpos/dexp[64*K] (destination row and expert
  // of each routing entry of the block)
  extern __shared__ int32_t lds[];
  __shared__ int last;
  const int R = a.R, E = a.E, epr = a.E / a.R;
  int32_t* tot = lds;
  int32_t* base = tot + E;
  int32_t* hwf = base + E;
  int32_t* dpos = hwf + 4 * E;
  int32_t* dexp = dpos + kTokPerBlock * a.K;
#define hw(w, e) hwf[(w) * E + (e)]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nwork = R * a.NB;
  if ((int)blockIdx.x >= nwork) {  // receiver d waits for the rows aimed at it
    const int d = blockIdx.x - nwork;
    if (tid == 0) {
      uint64_t rows = 0;
      for (int sp = 0; sp < R; ++sp)
        for (int e = d * epr; e < (d + 1) * epr; ++e) rows += a.cwin[((size_t)d * R + sp) * E + e];
      wait_reached(a.sig_rows + (size_t)d * a.sig_stride, a.base_rows[d] + rows, 64, a.timeout_ns, a.err,
                   VR_ASYNC_TIMEOUT);
    }
    return;
  }
  const int s = blockIdx.x / a.NB, blk = blockIdx.x % a.NB;
  // count exchange: rank s waits for every source's count row
  if (tid == 0)
    wait_reached(a.sig_counts + (size_t)s * a.sig_stride, a.target_counts.v[s], 64, a.timeout_ns, a.err,
                 VR_ASYNC_TIMEOUT);
  __syncthreads();
  const int32_t* cw = a.cwin + (size_t)s * R * E;  // rank s's copy: cw[s'][e]
  const int32_t* pb = a.hblk + ((size_t)s * a.NB + blk) * E;
  for (int e = tid; e < E; e += 256) {
    int32_t t = 0, pre = 0;
    for (int sp = 0; sp < R; ++sp) {
      const int32_t v = cw[(size_t)sp * E + e];
      t += v;
      if (sp < s) pre += v;
    }
    tot[e] = t;
    base[e] = pre + pb[e];
    for (int w = 0; w < 4; ++w) hw(w, e) = 0;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    int32_t seg = 0;
    for (int q = (e / epr) * epr; q < e; ++q) seg += tot[q];
    base[e] += seg;
  }
  if (blk == 0)
    for (int j = tid; j < epr; j += 256)
      store4_agent(reinterpret_cast<uint32_t*>(a.counts_out + (size_t)s * epr + j), tot[s * epr + j]);
  // pass 1: per-wave counts; pass 2: stable positions
  const int K = a.K;
  const int tpr = 64 / K;  // tokens per round
  const int tw0 = blk * kTokPerBlock + wave * kTokPerWave;
  const int rounds = (kTokPerWave + tpr - 1) / tpr;
  const uint64_t lt = (1ull << lane) - 1ull;
  __syncthreads();
  for (int pass = 0; pass < 2; ++pass) {
    for (int rd = 0; rd < rounds; ++rd) {
      const int tl = rd * tpr + lane / K;  // token index within the wave
      const int k = lane % K;
      const int t = tw0 + tl;
      const bool valid = lane < tpr * K && tl < kTokPerWave && t < a.T;
      int e = valid ? load_topk(a, s, t, k) : -1;
      const bool ok = valid && e >= 0 && e < E;
      if (pass == 0 && valid && e != -1 && !ok) atomic_or_u32(a.err, VR_ASYNC_BAD_EXPERT);
      int32_t pos = -1;
      if (ok) {
        const uint64_t m = match_any(static_cast<uint32_t>(e), a.nbits);
        const bool leader = (m & lt) == 0;
        const int cnt = __popcll(m);
        if (pass == 1) pos = base[e] + hw(wave, e) + __popcll(m & lt);
        if (leader) hw(wave, e) += cnt;
      }
      if (pass == 1 && valid) {
        const int slot = (wave * kTokPerWave + tl) * K + k;
        dpos[slot] = pos;
        dexp[slot] = ok ? e : -1;
        if (ok) {
          const int d = e / epr;
          if ((uint64_t)pos < a.cap)
            store4_agent(reinterpret_cast<uint32_t*>(a.src_out + (size_t)d * a.cap + pos),
                         static_cast<uint32_t>((s << 16) | t));
          else
            atomic_or_u32(a.err, VR_ASYNC_CAPACITY);
        }
      }
    }
    __syncthreads();
    if (pass == 0)
      for (int e = tid; e < E; e += 256) {
        int32_t run = 0;
        for (int w = 0; w < 4; ++w) {
          const int32_t v = hw(w, e);
          hw(w, e) = run;
          run += v;
        }
      }
    __syncthreads();
  }
  // copy: each wave moves its 16 tokens' rows, 512 bytes per wave instruction;
  // all 16 rows' pieces are loaded before any is stored.
  const uint64_t rb = a.row_bytes;
  const int ntw = max(0, min(kTokPerWave, a.T - tw0));
  if (a.fast) {
    for (uint64_t c0 = 0; c0 < rb; c0 += 512) {
      const uint64_t o = c0 + (uint64_t)lane * 8;
      const bool in = o < rb;
      uint64_t v[kTokPerWave];
#pragma unroll
      for (int tl = 0; tl < kTokPerWave; ++tl)
        v[tl] = (in && tl < ntw)
                    ? __builtin_nontemporal_load(
                          reinterpret_cast<const uint64_t*>(a.x.p[s] + a.x_off + (uint64_t)(tw0 + tl) * rb + o))
                    : 0;
#pragma unroll
      for (int tl = 0; tl < kTokPerWave; ++tl) {
        if (tl >= ntw) break;
        const int slot0 = (wave * kTokPerWave + tl) * K;
        for (int k = 0; k < K; ++k) {
          const int32_t pos = dpos[slot0 + k];
          if (pos < 0 || (uint64_t)pos >= a.cap) continue;
          const int d = dexp[slot0 + k] / epr;
          if (in)
            store8_agent(reinterpret_cast<uint64_t*>(a.recv.p[d] + a.recv_off + (uint64_t)pos * rb + o), v[tl]);
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
        const int d = dexp[slot0 + k] / epr;
        copy_bytes(a.recv.p[d] + a.recv_off + (uint64_t)pos * rb, src, static_cast<uint32_t>(rb), lane, 64);
      }
    }
  }
  wg_stores_complete();
  if (tid == 0) last = relay_arrive(a.relay + R + s, a.NB);
  __syncthreads();
  if (last && tid < R) {  // one trailing SignalAdd(rows from s) per destination
    const int d = tid;
    uint64_t rows = 0;
    for (int e = d * epr; e < (d + 1) * epr; ++e) rows += cw[(size_t)s * E + e];
    if (rows) atomic_add_u64(a.sig_rows + (size_t)d * a.sig_stride, rows);
  }
#undef hw
}

size_t al256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

size_t dispatch_scratch_bytes(int R, int T, int E) {
  const size_t NB = std::max(1, (T + kTokPerBlock - 1) / kTokPerBlock);
  return al256((size_t)R * NB * E * 4) + al256((size_t)R * R * E * 4) + al256((size_t)R * 8);
}

vrResult_t launch_dispatch(vrComm* c, const vrWindow* x, size_t x_off, size_t row_bytes, const int32_t* topk, int T,
                           int K, int E, const vrWindow* recv, size_t recv_off, size_t cap, int32_t* counts_out,
                           int32_t* src_out, uint32_t sig_counts, uint32_t sig_rows, const U64Tab& target_counts,
                           bool wait, hipStream_t st) {
  DispArgs a;
  const int R = c->nranks;
  for (int r = 0; r < VR_MAX_RANKS; ++r) {
    a.x.p[r] = x->base[r];
    a.recv.p[r] = recv->base[r];
  }
  a.target_counts = target_counts;
  a.x_off = x_off;
  a.recv_off = recv_off;
  a.row_bytes = row_bytes;
  a.cap = cap;
  a.topk = topk;
  a.counts_out = counts_out;
  a.src_out = src_out;
  a.NB = std::max(1, (T + kTokPerBlock - 1) / kTokPerBlock);
  a.hblk = reinterpret_cast<int32_t*>(c->scratch);
  a.cwin = reinterpret_cast<int32_t*>(c->scratch + al256((size_t)R * a.NB * E * 4));
  a.base_rows = reinterpret_cast<uint64_t*>(c->scratch + al256((size_t)R * a.NB * E * 4) + al256((size_t)R * R * E * 4));
  a.sig_counts = c->sig + sig_counts;
  a.sig_rows = c->sig + sig_rows;
  a.sig_stride = c->req.signal_count;
  a.relay = c->relay + kRelayDispatch;
  a.err = c->err;
  a.timeout_ns = kDefaultTimeoutNs;
  a.R = R;
  a.T = T;
  a.K = K;
  a.E = E;
  int nb = 1;
  while ((1 << nb) < E) ++nb;
  a.nbits = nb;
  a.fast = (row_bytes % 8 == 0) && (x_off % 8 == 0) && (recv_off % 8 == 0);
  hipLaunchKernelGGL(k_dispatch_count, dim3(R * a.NB), dim3(256), 0, st, a);
  if (hipGetLastError() != hipSuccess) return VR_ERR_HIP;
  const size_t lds = sizeof(int32_t) * (6 * (size_t)E + 2 * (size_t)kTokPerBlock * K);
  hipLaunchKernelGGL(k_dispatch_put, dim3(R * a.NB + (wait ? R : 0)), dim3(256), lds, st, a);
  return hipGetLastError() == hipSuccess ? VR_OK : VR_ERR_HIP;
}

}  // namespace vr
