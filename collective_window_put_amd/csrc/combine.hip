// MoE combine over symmetric windows: the inverse of the dispatch.
//
// GDA survey (10100.com/article/158785524), opening section: the dispatch
// sends each token to the ranks owning its top-k experts; the combine brings
// the expert outputs back. Source rank s gets, for each of its tokens t and
// each k in order, the row the dispatch placed at send_pos[s][t][k] on rank
// d = topk[s][t][k] / (E/R), and mixes them with the router weights:
//   acc = +0.0;  acc = acc + w[s][t][k] * y   (k = 0..K-1, entries with a row)
// each product and sum one binary32 operation rounded to nearest even (the
// library is built with -ffp-contract=off, so no fused multiply-add), bf16
// rows widened exactly and the result rounded to bf16 (RNE).
//
// A get (GIN page, one-sided transfers: get) of each row straight into
// registers, so every routed row is read once and every output row written
// once. Workgroup (s, b) takes 32 tokens of source s; the grid interleaves
// sources (b mod R) so that for R = 8 each source's workgroups, and its
// relay counter, stay on one XCD. The workgroup completing source s's relay
// applies one SignalInc at every rank d: s has read all the rows it needs,
// so d's signal rises by R. The last R workgroups are the expert ranks'
// waits for that.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "vr_device.hpp"
#include "vr_internal.hpp"

namespace vr {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTokPerWave = 8;
constexpr int kTok = kWaves * kTokPerWave;  // tokens per workgroup
// Row loads per batch (two batches in flight per lane). 4: 70 VGPRs, 6
// waves per SIMD; 8: 105 VGPRs, 4 waves. Measured flushed, alternating on
// one machine: combine 34.1-34.4 us against 34.5-34.9 us, per-rank combine
// 22.1-22.2 us against 22.7 us.
constexpr int kBatch = 4;

struct CombArgs {
  WinTab y;
  U64Tab target;
  uint64_t y_off, out_off, row_bytes, cap;
  char* out_base[VR_MAX_RANKS];
  const int32_t* topk;   // [R][T][K]
  const float* weights;  // [R][T][K]
  const int32_t* pos;    // [R][T][K]
  uint64_t* sig;
  uint32_t sig_stride;
  uint32_t* relay;       // [R] counters, rstride words apart
  uint32_t rstride;
  uint32_t* err;
  uint64_t timeout_ns;
  int R, T, K, E, nblk;
  int dedup;  // entries are destination ranks (k = d), weight 1, no topk or weights
};

template <int DT> struct CElem;
template <> struct CElem<VR_DT_F32> {
  static constexpr int kSize = 4, kPerVec = 4;
  __device__ static void widen(v4u w, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j] = __uint_as_float(w[j]);
  }
  __device__ static v4u narrow(const float* f) {
    v4u w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = __float_as_uint(f[j]);
    return w;
  }
  __device__ static float load1(const char* p) { return load4f_global(p); }
  __device__ static void store1(__amdgpu_buffer_rsrc_t r, uint32_t off, float f) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f), r, off, 0, kStoreAgent);
  }
};
template <> struct CElem<VR_DT_BF16> {
  static constexpr int kSize = 2, kPerVec = 8;
  __device__ static void widen(v4u w, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = bf16lo(w[j]);
      f[2 * j + 1] = bf16hi(w[j]);
    }
  }
  __device__ static v4u narrow(const float* f) {
    v4u w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = bf16_rne(f[2 * j]) | (bf16_rne(f[2 * j + 1]) << 16);
    return w;
  }
  __device__ static float load1(const char* p) {
    return __uint_as_float(static_cast<uint32_t>(load2_global(p)) << 16);
  }
  __device__ static void store1(__amdgpu_buffer_rsrc_t r, uint32_t off, float f) {
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(bf16_rne(f)), r, off, 0, kStoreAgent);
  }
};

// One lane group's walk over (token, batch-of-kBatch-entries) items for one
// 16-byte column: load() issues an item's row loads, mix() folds them into
// the accumulator in k order and, after a token's last batch, stores the
// token's output column and clears the accumulator.
template <int DT>
struct Mixer {
  const char* const* src;
  const float* wt;
  char* out;
  int t0, tl0, rpi, K, nb, col;
  uint64_t rb;
  __device__ __forceinline__ int token(int it) const { return tl0 + (it / nb) * rpi; }
  __device__ __forceinline__ void reset(float (&acc)[CElem<DT>::kPerVec]) const {
#pragma unroll
    for (int j = 0; j < CElem<DT>::kPerVec; ++j) acc[j] = 0.0f;
  }
  // returns the mask of entries that have a row
  __device__ __forceinline__ uint32_t load(int it, v4u (&v)[kBatch]) const {
    const int tl = token(it), k0 = (it % nb) * kBatch;
    // entries without a row issue no load (the lanes are masked off);
    // mix() drops them by a select
    const char* p[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) p[q] = k0 + q < K ? src[tl * K + k0 + q] : nullptr;
    uint32_t m = 0;
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      m |= p[q] ? 1u << q : 0u;
      v[q] = p[q] ? load16_stream_global(p[q] + col * 16) : v4u{0, 0, 0, 0};
    }
    return m;
  }
  __device__ __forceinline__ void mix(int it, const v4u (&v)[kBatch], uint32_t m,
                                      float (&acc)[CElem<DT>::kPerVec]) const {
    using EL = CElem<DT>;
    const int tl = token(it), kb = it % nb, k0 = kb * kBatch;
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const float w = k0 + q < K ? wt[tl * K + k0 + q] : 0.0f;
      float f[EL::kPerVec];
      EL::widen(v[q], f);
#pragma unroll
      for (int j = 0; j < EL::kPerVec; ++j) {
        const float sum = acc[j] + w * f[j];
        acc[j] = (m >> q) & 1u ? sum : acc[j];
      }
    }
    if (kb == nb - 1) {
      store16_agent_stream(rsrc(out + (uint64_t)(t0 + tl) * rb, static_cast<uint32_t>(rb)), col * 16,
                           EL::narrow(acc));
      reset(acc);
    }
  }
};

// VEC: 16-byte lanes (row_bytes and both offsets multiples of 16); otherwise
// one element per lane.
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_combine(const CombArgs a) {
  using EL = CElem<DT>;
  __shared__ const char* src[kTok * 64];  // row address of each entry (nullptr: no row)
  __shared__ float wt[kTok * 64];
  __shared__ int last;
  const int R = a.R, K = a.K;
  const int nwork = R * a.nblk;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  if (b >= nwork) {  // expert rank d waits until every source has read its rows
    const int d = b - nwork;
    if (tid == 0)
      wait_reached(a.sig + (size_t)d * a.sig_stride, a.target.v[d], 64, a.timeout_ns, a.err, VR_ASYNC_TIMEOUT);
    return;
  }
  const int s = b % R, blk = b / R;
  const int t0 = blk * kTok;
  const int ntok = max(0, min(kTok, a.T - t0));
  const int epr = a.E / R;
  const uint64_t rb = a.row_bytes;
  // entries of this workgroup's tokens: one per thread, coalesced
  for (int i = tid; i < ntok * K; i += kThreads) {
    const size_t g = ((size_t)s * a.T + t0) * K + i;
    const int e = a.dedup ? i % K : a.topk[g];
    const int p = a.pos[g];
    const float w = a.dedup ? 1.0f : a.weights[g];
    const char* addr = nullptr;
    if (e != -1 && (e < 0 || e >= a.E)) {
      atomic_or_u32(a.err, VR_ASYNC_BAD_EXPERT);
    } else if (e >= 0 && p != -1) {
      if (p < 0 || (uint64_t)p >= a.cap) atomic_or_u32(a.err, VR_ASYNC_CAPACITY);
      else addr = a.y.p[e / epr] + a.y_off + (uint64_t)p * rb;
    }
    src[i] = addr;
    wt[i] = w;
  }
  __syncthreads();
  // per-rank layout: most of a token's R entries have no row; move the rows
  // to the front, in rank order, so that the tail of a batch issues no loads
  // (measured 24.9 -> 22.8 us on the dedup combine workload)
  if (a.dedup) {
    for (int t = tid; t < ntok; t += kThreads) {
      int n = 0;
      for (int k = 0; k < K; ++k) {
        const char* q = src[t * K + k];
        if (q) {
          src[t * K + n] = q;
          wt[t * K + n] = wt[t * K + k];
          ++n;
        }
      }
      for (int k = n; k < K; ++k) src[t * K + k] = nullptr;
    }
    __syncthreads();
  }
  const int wave = tid >> 6, lane = tid & 63;
  char* out = a.out_base[s] + a.out_off;
  if (VEC) {
    const int nv = static_cast<int>(rb >> 4);
    int lpr = 1;
    while (lpr < nv && lpr < 64) lpr <<= 1;
    const int rpi = 64 / lpr;
    const int l = lane & (lpr - 1), grp = lane / lpr;
    const int nb = (K + kBatch - 1) / kBatch;  // load batches per token
    for (int c0 = 0; c0 < nv; c0 += lpr) {
      const int col = c0 + l;
      // this lane group's tokens: ti = grp, grp + rpi, ... (within the wave's share)
      int ntl = 0;
      for (int ti = grp; ti < kTokPerWave && wave * kTokPerWave + ti < ntok; ti += rpi) ++ntl;
      const int items = col < nv ? ntl * nb : 0;  // (token, batch) pairs, in order
      // two register buffers: the loads of item i+1 are in flight while item i is mixed
      float acc[CElem<DT>::kPerVec];
      v4u va[kBatch], vb[kBatch];
      uint32_t ma = 0, mb = 0;
      Mixer<DT> mx{src, wt, out, t0, wave * kTokPerWave + grp, rpi, K, nb, col, rb};
      mx.reset(acc);
      if (items > 0) ma = mx.load(0, va);
      for (int it = 0; it < items; it += 2) {
        if (it + 1 < items) mb = mx.load(it + 1, vb);
        mx.mix(it, va, ma, acc);
        if (it + 1 >= items) break;
        if (it + 2 < items) ma = mx.load(it + 2, va);
        mx.mix(it + 1, vb, mb, acc);
      }
    }
  } else {
    const int H = static_cast<int>(rb / EL::kSize);
    for (int tl = wave; tl < ntok; tl += kWaves) {
      const __amdgpu_buffer_rsrc_t ro = rsrc(out + (uint64_t)(t0 + tl) * rb, static_cast<uint32_t>(rb));
      for (int h = lane; h < H; h += 64) {
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) {
          const char* p = src[tl * K + k];
          if (p) acc = acc + wt[tl * K + k] * EL::load1(p + (uint64_t)h * EL::kSize);
        }
        EL::store1(ro, static_cast<uint32_t>(h * EL::kSize), acc);
      }
    }
  }
  wg_stores_complete();
  if (tid == 0) last = relay_arrive(a.relay + s * a.rstride, a.nblk, false);
  __syncthreads();
  if (last && tid < R) atomic_add_u64(a.sig + (size_t)tid * a.sig_stride, 1ull);  // SignalInc at each rank
}

template <int DT>
void launch_dt(const CombArgs& a, bool vec, int grid, hipStream_t st) {
  if (vec) hipLaunchKernelGGL((k_combine<DT, true>), dim3(grid), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL((k_combine<DT, false>), dim3(grid), dim3(kThreads), 0, st, a);
}

}  // namespace

vrResult_t launch_combine(vrComm* c, const vrWindow* y, size_t y_off, size_t cap, size_t row_bytes, int dtype,
                          const int32_t* topk, const float* weights, const int32_t* pos, int T, int K, int E,
                          bool dedup, const vrWindow* out, size_t out_off, uint32_t sig, const U64Tab& target,
                          bool wait, hipStream_t st) {
  CombArgs a;
  const int R = c->nranks;
  for (int r = 0; r < VR_MAX_RANKS; ++r) {
    a.y.p[r] = y->base[r];
    a.out_base[r] = out->base[r];
  }
  a.target = target;
  a.y_off = y_off;
  a.out_off = out_off;
  a.row_bytes = row_bytes;
  a.cap = cap;
  a.topk = topk;
  a.weights = weights;
  a.pos = pos;
  a.sig = c->sig + sig;
  a.sig_stride = c->req.signal_count;
  a.relay = c->relay + kRelayColl;
  a.rstride = relay_stride(R);
  a.err = c->err;
  a.timeout_ns = kDefaultTimeoutNs;
  a.R = R;
  a.T = T;
  a.K = K;
  a.E = E;
  a.dedup = dedup ? 1 : 0;
  a.nblk = std::max(1, (T + kTok - 1) / kTok);
  const bool vec = row_bytes % 16 == 0 && y_off % 16 == 0 && out_off % 16 == 0;
  const int grid = R * a.nblk + (wait ? R : 0);
  if (dtype == VR_DT_F32) launch_dt<VR_DT_F32>(a, vec, grid, st);
  else launch_dt<VR_DT_BF16>(a, vec, grid, st);
  return hipGetLastError() == hipSuccess ? VR_OK : VR_ERR_HIP;
}

}  // namespace vr
