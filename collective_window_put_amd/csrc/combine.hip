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
constexpr int kLoads = 8;                   // row loads in flight per lane: one batch of a token's entries

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
  int lpr;        // 16-byte path: lanes per row (a power of two, at most 64)
  int staged;     // 16-byte path: output rows staged in LDS, stored per column chunk
  uint32_t wt_off, stage_off;  // byte offsets of the weights and the staging rows in dynamic LDS
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

// VEC: 16-byte lanes (row_bytes and both offsets multiples of 16); otherwise
// one element per lane.
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_combine(const CombArgs a) {
  using EL = CElem<DT>;
  extern __shared__ __align__(16) char smem[];
  const char** src = reinterpret_cast<const char**>(smem);  // [kTok][K] row address of each entry (nullptr: no row)
  float* wt = reinterpret_cast<float*>(smem + a.wt_off);    // [kTok][K]
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
    // A lane group of lpr lanes takes one column chunk (lpr 16-byte vectors)
    // of a token's row; the wave's rpi = 64 / lpr groups take its tokens in
    // turn. Per token: its entries' rows in batches of kLoads loads in flight,
    // mixed in k order, the output vector staged in LDS; after each chunk the
    // workgroup stores the staged rows together (contiguous runs of the
    // output), or, where a buffer descriptor cannot span the workgroup's rows,
    // each group stores its own vector. Measured at 8 ranks x 4096 tokens,
    // 512-byte rows, K = 8 (flushed, alternating on one machine): 31.2-31.3
    // us against 34.6-34.8 us with two batches of four loads in flight and
    // each vector stored as soon as it was mixed; per-rank combine 20.7-20.8
    // against 22.1-22.2 us. A stand-alone probe put the gather alone at
    // 25.4 us and its stores, unstaged, at +5 us.
    const int nv = static_cast<int>(rb >> 4);
    const int lpr = a.lpr, rpi = 64 / lpr;
    const int l = lane & (lpr - 1), grp = lane / lpr;
    v4u* stage = reinterpret_cast<v4u*>(smem + a.stage_off);  // [kTok][lpr]
    for (int c0 = 0; c0 < nv; c0 += lpr) {
      const int col = c0 + l;
      for (int ti = grp; ti < kTokPerWave && col < nv; ti += rpi) {
        const int tl = wave * kTokPerWave + ti;
        if (tl >= ntok) break;
        float acc[EL::kPerVec];
#pragma unroll
        for (int j = 0; j < EL::kPerVec; ++j) acc[j] = 0.0f;
        for (int k0 = 0; k0 < K; k0 += kLoads) {
          v4u v[kLoads];
#pragma unroll
          for (int q = 0; q < kLoads; ++q) {
            const char* p = k0 + q < K ? src[tl * K + k0 + q] : nullptr;
            v[q] = p ? load16_stream_global(p + col * 16) : v4u{0, 0, 0, 0};
          }
#pragma unroll
          for (int q = 0; q < kLoads; ++q) {
            if (k0 + q < K && src[tl * K + k0 + q]) {  // entries without a row are skipped
              const float w = wt[tl * K + k0 + q];
              float f[EL::kPerVec];
              EL::widen(v[q], f);
#pragma unroll
              for (int j = 0; j < EL::kPerVec; ++j) acc[j] = acc[j] + w * f[j];
            }
          }
        }
        if (a.staged) stage[tl * lpr + l] = EL::narrow(acc);
        else store16_agent(rsrc(out + (uint64_t)(t0 + tl) * rb, static_cast<uint32_t>(rb)), col * 16, EL::narrow(acc));
      }
      if (a.staged) {
        __syncthreads();
        if (ntok > 0) {
          const int w16 = min(lpr, nv - c0);  // vectors of this chunk
          const __amdgpu_buffer_rsrc_t ro =
              rsrc(out + (uint64_t)t0 * rb + (uint64_t)c0 * 16, static_cast<uint32_t>((ntok - 1) * rb + w16 * 16));
          for (int i = tid; i < ntok * lpr; i += kThreads) {
            const int tl = i / lpr, l2 = i & (lpr - 1);
            if (l2 < w16) store16_agent(ro, static_cast<uint32_t>(tl * rb + l2 * 16), stage[i]);
          }
        }
        __syncthreads();  // the stage is rewritten by the next chunk
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
  // the signal says that the rows have been read: every row load has
  // returned (its value is in the output), so no wait for the stores
  __syncthreads();
  if (tid == 0) last = relay_arrive(a.relay + s * a.rstride, a.nblk, false);
  __syncthreads();
  if (last && tid < R) atomic_add_u64(a.sig + (size_t)tid * a.sig_stride, 1ull);  // SignalInc at each rank
}

template <int DT>
void launch_dt(const CombArgs& a, bool vec, int grid, uint32_t lds, hipStream_t st) {
  if (vec) hipLaunchKernelGGL((k_combine<DT, true>), dim3(grid), dim3(kThreads), lds, st, a);
  else hipLaunchKernelGGL((k_combine<DT, false>), dim3(grid), dim3(kThreads), lds, st, a);
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
  const uint64_t nv = row_bytes / 16;
  a.lpr = 1;
  while (a.lpr < 64 && (uint64_t)a.lpr < nv) a.lpr <<= 1;
  // staging: one descriptor spans the workgroup's kTok rows of a chunk
  a.staged = vec && (uint64_t)(kTok - 1) * row_bytes + 16ull * a.lpr <= 0xFFFFFFFFull;
  a.wt_off = static_cast<uint32_t>(kTok * K * sizeof(const char*));
  a.stage_off = (a.wt_off + kTok * K * sizeof(float) + 15) & ~15u;
  const uint32_t lds = a.stage_off + (a.staged ? kTok * a.lpr * 16u : 0u);  // at most 56 KiB (K <= 64)
  const int grid = R * a.nblk + (wait ? R : 0);
  if (dtype == VR_DT_F32) launch_dt<VR_DT_F32>(a, vec, grid, lds, st);
  else launch_dt<VR_DT_BF16>(a, vec, grid, lds, st);
  return hipGetLastError() == hipSuccess ? VR_OK : VR_ERR_HIP;
}

}  // namespace vr
