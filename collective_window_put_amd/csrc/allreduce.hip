// Sum-AllReduce over symmetric windows: reduce-scatter by gets, all-gather by
// puts, fused in one kernel so a reduced chunk never round-trips through HBM.
//
// Symmetric page (zwxr.cn/news/250719), AllReduce example: every rank ends
// with the element-wise sum over all ranks. GIN page (lpnh.cn/news/2681042):
// get pulls a peer's window bytes, put pushes them with a SignalInc.
//
// Owner c reduces elements [c*csz, (c+1)*csz) (csz = ceil(N/R) rounded up to
// a whole number of tiles). A workgroup reads a tile from every rank's send
// window (the gets of the reduce-scatter), sums in rank order in fp32 --
// acc = x_0, then acc += x_r for r = 1..R-1, each an IEEE binary32 addition
// rounded to nearest even -- converts, and stores the tile into every rank's
// receive window (the puts of the all-gather). Ragged or unaligned shapes
// run one tile per workgroup; large aligned ones with R = 2, 4, 8 or 16 run
// the rank-split form below (one piece per workgroup, ranks split across its
// waves, the sum through LDS), and the remaining large evenly tiled ones the
// looping form (a fixed grid striding over slabs, loads two slabs ahead).
// The workgroup completing a chunk's relay applies one SignalInc at every
// rank, so each rank's signal rises by R (one per owner). Output stores are
// agent-coherent and streaming (sc1 nt): measured back to back 0.7 % faster
// than sc1 alone in the looping form.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "vr_device.hpp"
#include "vr_internal.hpp"

namespace vr {
namespace {

constexpr int kU = 2;  // 16-byte vectors per thread per tile

// Kernel forms (see the comments at each): one tile per workgroup, a fixed
// grid looping over slabs, and one rank-split piece per workgroup.
enum Form { kOneTile = 0, kLoop = 1, kSplit = 2 };
constexpr uint32_t kSplitFan = 8;  // first-level relay counters per (chunk, XCD) in the rank-split form

struct ARArgs {
  WinTab send, recv;
  U64Tab target;
  uint64_t send_off, recv_off;
  uint64_t count;   // elements
  uint64_t csz;     // elements per owner chunk (multiple of the tile)
  uint32_t tpc;     // tiles per chunk
  uint32_t nwg;     // work workgroups: R * tpc (one tile each), fewer looping over tiles, or R * ppc pieces
  uint32_t ppc;     // rank-split form: pieces per chunk
  uint64_t* sig;
  uint32_t sig_stride;
  uint32_t* relay;  // [R] per chunk, then [R][8] per (chunk, XCD); rstride words apart
  uint32_t rstride;
  uint32_t* err;
  uint64_t timeout_ns;
  uint64_t* lit;       // litmus words [2], or null
  uint64_t* lit_last;  // [R]: first element of the piece that completed chunk c's relay
  uint32_t lit_seed;
  int R;
  int wait;
};

template <int DT> struct Elem;
template <> struct Elem<VR_DT_F32> {
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
  __device__ static float load1(const char* p) { return *reinterpret_cast<const float*>(p); }
  __device__ static void store1(__amdgpu_buffer_rsrc_t r, uint32_t off, float f) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f), r, off, 0, kStoreAgent);
  }
};
template <> struct Elem<VR_DT_BF16> {
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
    return __uint_as_float(static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(p)) << 16);
  }
  __device__ static void store1(__amdgpu_buffer_rsrc_t r, uint32_t off, float f) {
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(bf16_rne(f)), r, off, 0, kStoreAgent);
  }
};

// One tile [start, end) of the owner's chunk. RT: compile-time rank count, or
// 0 for any R. ALIGNED: every rank's (base + offset) is 16-byte aligned.
template <int DT, int RT, bool ALIGNED>
__device__ void reduce_tile(const ARArgs& a, uint64_t start, uint64_t end) {
  using E = Elem<DT>;
  constexpr int V = E::kPerVec;
  const int R = RT ? RT : a.R;
  const uint32_t tid = threadIdx.x;
  const uint32_t nbytes = static_cast<uint32_t>((end - start) * E::kSize);
  if (ALIGNED) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint64_t i = start + (uint64_t)(u * 256 + tid) * V;
      if (i + V <= end) {
        float acc[V];
        const uint64_t sb = a.send_off + i * E::kSize;
        if (RT) {
          v4u x[RT ? RT : 1];
#pragma unroll
          for (int r = 0; r < (RT ? RT : 1); ++r)
            x[r] = load16_stream(reinterpret_cast<const v4u*>(a.send.p[r] + sb));
          E::widen(x[0], acc);
#pragma unroll
          for (int r = 1; r < (RT ? RT : 1); ++r) {
            float f[V];
            E::widen(x[r], f);
#pragma unroll
            for (int j = 0; j < V; ++j) acc[j] = acc[j] + f[j];
          }
        } else {
          E::widen(load16_stream(reinterpret_cast<const v4u*>(a.send.p[0] + sb)), acc);
          for (int r0 = 1; r0 < R; r0 += 4) {
            v4u x[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (r0 + q < R) x[q] = load16_stream(reinterpret_cast<const v4u*>(a.send.p[r0 + q] + sb));
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (r0 + q < R) {
                float f[V];
                E::widen(x[q], f);
#pragma unroll
                for (int j = 0; j < V; ++j) acc[j] = acc[j] + f[j];
              }
          }
        }
        const v4u out = E::narrow(acc);
        const uint32_t off = static_cast<uint32_t>((i - start) * E::kSize);
        for (int d = 0; d < R; ++d)
          store16_agent_stream(rsrc(a.recv.p[d] + a.recv_off + start * E::kSize, nbytes), off, out);
      } else if (i < end) {  // ragged tail of the whole vector: element by element
        for (uint64_t k = i; k < end; ++k) {
          const uint64_t sb = a.send_off + k * E::kSize;
          float acc = E::load1(a.send.p[0] + sb);
          for (int r = 1; r < R; ++r) acc = acc + E::load1(a.send.p[r] + sb);
          const uint32_t off = static_cast<uint32_t>((k - start) * E::kSize);
          for (int d = 0; d < R; ++d)
            E::store1(rsrc(a.recv.p[d] + a.recv_off + start * E::kSize, nbytes), off, acc);
        }
      }
    }
  } else {
    for (uint64_t k = start + tid; k < end; k += 256) {
      const uint64_t sb = a.send_off + k * E::kSize;
      float acc = E::load1(a.send.p[0] + sb);
      for (int r = 1; r < R; ++r) acc = acc + E::load1(a.send.p[r] + sb);
      const uint32_t off = static_cast<uint32_t>((k - start) * E::kSize);
      for (int d = 0; d < R; ++d) E::store1(rsrc(a.recv.p[d] + a.recv_off + start * E::kSize, nbytes), off, acc);
    }
  }
}

// relay_arrive for a workgroup that brings `n` of the `parts` at once: true
// in the one that completes the set (which resets the counter); a
// workgroup holding every part touches no counter.
__device__ inline bool relay_arrive_n(uint32_t* counter, uint32_t n, uint32_t parts, bool acquire) {
  if (n >= parts) return true;
  const uint32_t prev = atomic_add_u32(counter, n);
  if (prev + n != parts) return false;
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (acquire) acquire_agent();
  return true;
}

// Thread 0 of a workgroup whose stores have completed: `n` units of chunk c
// done on XCD x, `per_tile` units to a tile. Two-level relay when the tiles
// split evenly over the XCDs: first the tiles of chunk c on this XCD
// (arrivals from one XCD only), then the XCDs that hold part of chunk c (one
// for R = 8); the workgroup that completes the chunk applies one SignalInc
// at every rank.
__device__ void chunk_done(const ARArgs& a, uint32_t R, uint32_t c, uint32_t x, uint32_t n, uint32_t per_tile,
                           uint64_t piece) {
  const uint32_t nwork = R * a.tpc;
  bool last;
  if ((nwork & 7u) == 0) {
    const uint32_t per = nwork >> 3;
    const uint32_t lo = std::max(x * per, c * a.tpc), hi = std::min((x + 1) * per, (c + 1) * a.tpc);
    const uint32_t nx = ((c + 1) * a.tpc - 1) / per - (c * a.tpc) / per + 1;
    last = relay_arrive_n(a.relay + (R + c * 8 + x) * a.rstride, n, (hi - lo) * per_tile, false) &&
           relay_arrive(a.relay + c * a.rstride, nx, false);
  } else {
    last = relay_arrive_n(a.relay + c * a.rstride, n, a.tpc * per_tile, false);
  }
  if (last) {
    if (a.lit) litmus_record(a.lit_last + c, piece);
    for (uint32_t d = 0; d < R; ++d) atomic_add_u64(a.sig + (size_t)d * a.sig_stride, 1ull);
  }
}

// Element k of rank d's receive slice equals the rank-order sum of element k
// of every send slice, recomputed here (binary32 adds, then the element type).
template <int DT>
__device__ bool elem_ok(const ARArgs& a, uint32_t R, uint32_t d, uint64_t k) {
  using E = Elem<DT>;
  const uint64_t sb = a.send_off + k * E::kSize;
  float acc = E::load1(a.send.p[0] + sb);
  for (uint32_t r = 1; r < R; ++r) acc = acc + E::load1(a.send.p[r] + sb);
  const char* got = a.recv.p[d] + a.recv_off + k * E::kSize;
  if (DT == VR_DT_F32) return *reinterpret_cast<const uint32_t*>(got) == __float_as_uint(acc);
  return *reinterpret_cast<const uint16_t*>(got) == static_cast<uint16_t>(bf16_rne(acc));
}

// Receiver d, litmus on: from the piece that completed each chunk's relay,
// a whole tile's elements, then one seeded element in every tile.
template <int DT>
__device__ void ar_litmus(const ARArgs& a, uint32_t R, uint32_t d) {
  constexpr uint64_t tile = 256ull * kU * Elem<DT>::kPerVec;
  const uint32_t tid = threadIdx.x;
  uint32_t checks = 0, bad = 0;
  for (uint32_t c = 0; c < R; ++c) {
    const uint64_t cbeg = (uint64_t)c * a.csz, cend = std::min<uint64_t>(a.count, cbeg + a.csz);
    if (cbeg >= cend) continue;  // an empty chunk
    uint64_t p0 = load_relaxed_u64(a.lit_last + c);
    // an empty tile or piece past the data may complete the relay: check the chunk's last tile then
    if (p0 >= cend && p0 < cbeg + a.csz) p0 = std::max<uint64_t>(cbeg, cend >= tile ? cend - tile : 0);
    if (p0 < cbeg || p0 >= cend) {
      if (tid == 0) ++checks, ++bad;
      continue;
    }
    for (uint64_t k = p0 + tid; k < std::min<uint64_t>(cend, p0 + tile); k += 256) {
      ++checks;
      bad += !elem_ok<DT>(a, R, d, k);
    }
  }
  for (uint32_t w = tid; w < R * a.tpc; w += 256) {
    const uint32_t c = w / a.tpc, j = w % a.tpc;
    const uint64_t cend = std::min<uint64_t>(a.count, (uint64_t)c * a.csz + a.csz);
    const uint64_t start = (uint64_t)c * a.csz + (uint64_t)j * tile;
    const uint64_t end = std::min<uint64_t>(cend, start + tile);
    if (start >= end) continue;
    ++checks;
    bad += !elem_ok<DT>(a, R, d, start + mix32(a.lit_seed + w * 0x9E3779B9u) % (end - start));
  }
  litmus_report(a.lit, a.err, checks, bad);
}

// Sum of one 256-vector slab in rank order, stored to every rank.
template <int DT, int RT>
__device__ inline void sum_store_slab(const ARArgs& a, uint64_t start, const v4u (&x)[RT]) {
  using E = Elem<DT>;
  float acc[E::kPerVec];
  E::widen(x[0], acc);
#pragma unroll
  for (int r = 1; r < RT; ++r) {
    float f[E::kPerVec];
    E::widen(x[r], f);
#pragma unroll
    for (int j = 0; j < E::kPerVec; ++j) acc[j] = acc[j] + f[j];
  }
  const v4u out = E::narrow(acc);
  constexpr uint32_t nbytes = 256u * 16u;
#pragma unroll
  for (int d = 0; d < RT; ++d)
    store16_agent_stream(rsrc(a.recv.p[d] + a.recv_off + start * E::kSize, nbytes), threadIdx.x * 16u, out);
}

template <int DT, int RT>
__device__ inline void load_slab(const ARArgs& a, uint64_t start, v4u (&x)[RT]) {
  const uint64_t sb = a.send_off + (start + threadIdx.x * Elem<DT>::kPerVec) * Elem<DT>::kSize;
#pragma unroll
  for (int r = 0; r < RT; ++r) x[r] = load16_stream(reinterpret_cast<const v4u*>(a.send.p[r] + sb));
}

// Looping form, used when every tile is full and 16-byte aligned and the
// tiles split evenly over the XCDs. A tile is kU slabs of 256 vectors per
// rank; XCD x (x = b mod 8) owns slabs [x, x+1) * S (S = slabs / 8), and
// workgroup b takes slabs x*S + b/8, + a.nwg/8, ..., with the loads of the
// next two slabs in flight while a slab is summed and stored. The relay
// counts slabs. Measured back to back at 8 ranks x 64 Mi bf16, alternating
// on one machine: 0.385 ms with one slab in flight ahead against 0.400 ms for
// one workgroup per tile, and 0.381 ms with two; taking a tile's two slabs
// in a row before striding was 3 % slower than one workgroup per tile.
template <int DT, int RT>
__device__ void persistent_tiles(const ARArgs& a, uint32_t b) {
  constexpr uint64_t slab = 256ull * Elem<DT>::kPerVec;  // elements
  const uint32_t S = ((RT * a.tpc) >> 3) * kU;           // slabs per XCD
  const uint32_t spc = a.tpc * kU;                         // slabs per chunk
  const uint32_t x = b & 7u, step = a.nwg >> 3;
  uint32_t q = b >> 3;
  if (q >= S) return;
  uint32_t c = (x * S + q) / spc;
  uint32_t n = 0;  // slabs of chunk c finished by this workgroup
  uint64_t piece = 0;  // first element of the last slab stored
  v4u v0[RT], v1[RT], v2[RT];  // slabs q, q + step, q + 2 step
  load_slab<DT, RT>(a, (uint64_t)(x * S + q) * slab, v0);
  if (q + step < S) load_slab<DT, RT>(a, (uint64_t)(x * S + q + step) * slab, v1);
  for (;;) {
    const uint32_t q2 = q + step, q3 = q2 + step;
    if (q3 < S) load_slab<DT, RT>(a, (uint64_t)(x * S + q3) * slab, v2);
    piece = (uint64_t)(x * S + q) * slab;
    sum_store_slab<DT, RT>(a, piece, v0);
    ++n;
    if (q2 >= S) break;
    const uint32_t c2 = (x * S + q2) / spc;
    if (c2 != c) {  // next slab is in another chunk: close this one
      wg_stores_complete();
      if (threadIdx.x == 0) chunk_done(a, RT, c, x, n, kU, piece);
      c = c2;
      n = 0;
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      v0[r] = v1[r];
      v1[r] = v2[r];
    }
    q = q2;
  }
  wg_stores_complete();
  if (threadIdx.x == 0) chunk_done(a, RT, c, x, n, kU, piece);
}

// Rank-split form, used when the offsets are 16-byte aligned, R is 2, 4, 8
// or 16, there are at least 8192 tiles, and each chunk's pieces split evenly
// over the relay counters. The piece holding the end of the vector is summed
// element by element; pieces past it move nothing but still join the relay.
// Workgroup w takes piece w: max(512/R, 64) vectors of every rank (1 KiB per
// rank for R = 8 and 16), rank-major. Each wave loads two (four for R = 16)
// 64-vector runs of it (each within one rank, so the rank's window pointer is
// a scalar) into LDS; after a barrier every thread sums 32-bit words across
// the ranks in rank order; after another, each wave stores the same runs'
// positions of the sum to their ranks. So each thread issues two loads and
// two stores (four for R = 16), and the workgroup ends; pieces run in grid
// order, so at any time the chip reads and writes one narrow band of each
// rank's slice. Measured back to back at
// 8 ranks x 64 Mi bf16 in a stand-alone copy of the data path: 0.341 ms
// without the relay, 0.348 ms with it, against 0.389 ms for one tile per
// workgroup with eight loads and eight stores per thread. A relay of two
// levels ((chunk, XCD), then chunk) took 0.411 ms: 2048 arrivals on each
// first-level counter queue behind each other, so the first level is spread
// over kSplitFan counters per (chunk, XCD).
// Piece w's stores are done in every wave: three relay levels, (chunk, XCD,
// k) with k = (w / 8) mod kSplitFan, then (chunk, XCD), then chunk; the
// pieces of a chunk split evenly over them. The workgroup completing a chunk
// applies one SignalInc at every rank.
template <int RT>
__device__ inline void split_done(const ARArgs& a, uint32_t w, uint64_t start) {
  wg_stores_complete();
  if (threadIdx.x != 0) return;
  const uint32_t c = w / a.ppc, x = w & 7u, k = (w >> 3) & (kSplitFan - 1);
  const bool last =
      relay_arrive(a.relay + (9 * RT + (c * 8 + x) * kSplitFan + k) * a.rstride, a.ppc / (8 * kSplitFan), false) &&
      relay_arrive(a.relay + (RT + c * 8 + x) * a.rstride, kSplitFan, false) &&
      relay_arrive(a.relay + c * a.rstride, 8, false);
  if (last) {
    if (a.lit) litmus_record(a.lit_last + c, start);
    for (uint32_t d = 0; d < RT; ++d) atomic_add_u64(a.sig + (size_t)d * a.sig_stride, 1ull);
  }
}

template <int DT, int RT>
__device__ void split_piece(const ARArgs& a, uint32_t w) {
  using E = Elem<DT>;
  constexpr uint32_t V = RT <= 8 ? 512 / RT : 64;  // vectors per rank in a piece
  constexpr int kRuns = RT * V / 256;               // 64-vector runs per wave: 2, or 4 for R = 16
  static_assert(V % 64 == 0, "a 64-lane run must lie within one rank");
  constexpr uint64_t pe = (uint64_t)V * E::kPerVec;  // elements per piece
  __shared__ v4u part[RT * V];  // rank-major
  __shared__ v4u total[V];
  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint64_t start = (uint64_t)w * pe;
  if (start + pe > a.count) {
    // the piece holding the end of the vector (element by element, rank
    // order) or one past it (nothing to move); it still joins the relay
    const uint32_t nbytes = static_cast<uint32_t>(pe * E::kSize);
    for (uint64_t k = start + tid; k < a.count; k += 256) {
      const uint64_t sb = a.send_off + k * E::kSize;
      float acc = E::load1(a.send.p[0] + sb);
#pragma unroll
      for (int r = 1; r < RT; ++r) acc = acc + E::load1(a.send.p[r] + sb);
      const uint32_t off = static_cast<uint32_t>((k - start) * E::kSize);
#pragma unroll
      for (int d = 0; d < RT; ++d) E::store1(rsrc(a.recv.p[d] + a.recv_off + start * E::kSize, nbytes), off, acc);
    }
    split_done<RT>(a, w, start);
    return;
  }
  v4u x[kRuns];
  char* dst[kRuns];  // read before the barriers, so the stores need not wait for them
#pragma unroll
  for (int u = 0; u < kRuns; ++u) {
    const uint32_t q = (kRuns * wave + u) * 64;  // first rank-major vector of the run
    const char* src = a.send.p[q / V] + a.send_off + start * E::kSize;
    x[u] = load16_stream(reinterpret_cast<const v4u*>(src + (q % V + lane) * 16u));
    dst[u] = a.recv.p[q / V];
  }
#pragma unroll
  for (int u = 0; u < kRuns; ++u) part[(kRuns * wave + u) * 64 + lane] = x[u];
  __syncthreads();
  const uint32_t* p32 = reinterpret_cast<const uint32_t*>(part);
  uint32_t* t32 = reinterpret_cast<uint32_t*>(total);
  for (uint32_t j = tid; j < 4 * V; j += 256) {
    const uint32_t w0 = p32[j];
    if constexpr (DT == VR_DT_BF16) {
      float lo = bf16lo(w0), hi = bf16hi(w0);
#pragma unroll
      for (int r = 1; r < RT; ++r) {
        const uint32_t wr = p32[r * 4 * V + j];
        lo = lo + bf16lo(wr);
        hi = hi + bf16hi(wr);
      }
      t32[j] = bf16_rne(lo) | (bf16_rne(hi) << 16);
    } else {
      float acc = __uint_as_float(w0);
#pragma unroll
      for (int r = 1; r < RT; ++r) acc = acc + __uint_as_float(p32[r * 4 * V + j]);
      t32[j] = __float_as_uint(acc);
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kRuns; ++u) {
    const uint32_t q = (kRuns * wave + u) * 64;
    const __amdgpu_buffer_rsrc_t rd = rsrc(dst[u] + a.recv_off + start * E::kSize, V * 16u);
    store16_agent_stream(rd, (q % V + lane) * 16u, total[q % V + lane]);
  }
  split_done<RT>(a, w, start);
}

template <int DT, int RT, bool ALIGNED, int FORM>
__global__ __launch_bounds__(256) void k_allreduce(const ARArgs a) {
  const uint32_t R = RT ? RT : a.R;
  const uint32_t nwork = R * a.tpc;
  const uint32_t b = blockIdx.x;
  if (b >= a.nwg) {  // receiver d waits for one SignalInc per owner
    const uint32_t d = b - a.nwg;
    if (!a.lit) {
      if (threadIdx.x == 0)
        wait_reached(a.sig + (size_t)d * a.sig_stride, a.target.v[d], 64, a.timeout_ns, a.err, VR_ASYNC_TIMEOUT);
    } else if (receiver_wait(a.sig + (size_t)d * a.sig_stride, a.target.v[d], a.timeout_ns, a.err)) {
      ar_litmus<DT>(a, R, d);
    }
    return;
  }
  if constexpr (FORM == kLoop) {
    static_assert(RT != 0 && ALIGNED, "the looping form needs a compiled rank count and aligned tiles");
    persistent_tiles<DT, RT>(a, b);
    return;
  }
  if constexpr (FORM == kSplit) {
    static_assert(RT != 0 && RT <= 16 && ALIGNED, "the rank-split form needs R <= 16, compiled, and aligned tiles");
    split_piece<DT, RT>(a, b);
    return;
  }
  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs (b % 8);
  // give XCD x the contiguous tile range [x, x+1) * nwork/8 -- for R = 8
  // exactly owner x's chunk -- so each XCD streams one region and the owners'
  // relay counters are hit in parallel rather than one at a time.
  const uint32_t w = (nwork & 7u) == 0 ? (b & 7u) * (nwork >> 3) + (b >> 3) : b;
  const uint32_t c = w / a.tpc, j = w % a.tpc;
  constexpr uint64_t tile = 256ull * kU * Elem<DT>::kPerVec;
  const uint64_t cbeg = (uint64_t)c * a.csz;
  const uint64_t cend = std::min<uint64_t>(a.count, cbeg + a.csz);
  const uint64_t start = cbeg + (uint64_t)j * tile;
  const uint64_t end = std::min<uint64_t>(cend, start + tile);
  if (start < end) reduce_tile<DT, RT, ALIGNED>(a, start, end);
  wg_stores_complete();
  if (threadIdx.x == 0) chunk_done(a, R, c, b & 7u, 1, 1, start);
}

template <int DT, int RT, bool AL, int FORM>
void launch_t(const ARArgs& a, uint32_t grid, hipStream_t st) {
  hipLaunchKernelGGL((k_allreduce<DT, RT, AL, FORM>), dim3(grid), dim3(256), 0, st, a);
}

template <int DT, int RT>
void launch_r(const ARArgs& a, int form, uint32_t grid, hipStream_t st) {
  if (form == kSplit) launch_t<DT, RT, true, kSplit>(a, grid, st);
  else if (form == kLoop) launch_t<DT, RT, true, kLoop>(a, grid, st);
  else launch_t<DT, RT, true, kOneTile>(a, grid, st);
}

template <int DT>
void launch_dt(const ARArgs& a, bool aligned, int form, uint32_t grid, hipStream_t st) {
  if (!aligned) return launch_t<DT, 0, false, kOneTile>(a, grid, st);
  switch (a.R) {
    case 2: return launch_r<DT, 2>(a, form, grid, st);
    case 4: return launch_r<DT, 4>(a, form, grid, st);
    case 8: return launch_r<DT, 8>(a, form, grid, st);
    case 16: return launch_r<DT, 16>(a, form, grid, st);
    default: return launch_t<DT, 0, true, kOneTile>(a, grid, st);
  }
}

constexpr uint32_t kLoopWorkgroups = 4096;  // workgroups of the looping form

}  // namespace

vrResult_t launch_allreduce(vrComm* c, const vrWindow* send, size_t send_off, const vrWindow* recv, size_t recv_off,
                            size_t count, int dtype, uint32_t sig, const U64Tab& target, bool wait, hipStream_t st) {
  ARArgs a;
  const int R = c->nranks;
  bool aligned = ((send_off | recv_off) & 15) == 0;
  for (int r = 0; r < VR_MAX_RANKS; ++r) {
    a.send.p[r] = send->base[r];
    a.recv.p[r] = recv->base[r];
  }
  a.target = target;
  a.send_off = send_off;
  a.recv_off = recv_off;
  a.count = count;
  const uint64_t tile = 256ull * kU * (dtype == VR_DT_F32 ? 4 : 8);
  const uint64_t per = (count + R - 1) / R;
  a.csz = (per + tile - 1) / tile * tile;
  const uint64_t tpc = std::max<uint64_t>(1, a.csz / tile);
  if (tpc * R > 0x7FFFFFFFull) return VR_ERR_INVALID_ARGUMENT;
  a.tpc = static_cast<uint32_t>(tpc);
  a.sig = c->sig + sig;
  a.sig_stride = c->req.signal_count;
  // [R] per chunk, then [R][8] per (chunk, XCD), then (rank-split form)
  // [R][8][kSplitFan] per (chunk, XCD, k)
  a.relay = c->relay + kRelayColl;
  a.rstride = relay_stride((9 + 8 * kSplitFan) * R);
  a.err = c->err;
  a.timeout_ns = kDefaultTimeoutNs;
  a.lit = c->litmus;
  a.lit_last = c->lit_last;
  a.lit_seed = c->lit_seed++;
  a.R = R;
  a.wait = wait;
  // rank-split form: aligned offsets, R = 2, 4, 8 or 16, at least 8192
  // tiles, and each chunk's pieces (a tile is min(R, 8) pieces) a multiple
  // of the 8 * kSplitFan first-level relay counters (the count need not
  // fill them).
  // Looping form: every tile full, aligned, a rank count with a compiled
  // kernel (2, 4, 8, 16), the tiles splitting evenly over the XCDs, and at
  // least two tiles per looping workgroup. Smaller shapes run one tile per
  // workgroup: at 4 ranks x 1 Mi fp32 (512 tiles) that took 12.6 us against
  // 13.2 us for the rank-split form (flushed, alternating on one machine).
  const uint32_t nwork = a.tpc * R;
  const bool full = aligned && (R == 2 || R == 4 || R == 8 || R == 16) && count == (uint64_t)R * a.csz;
  int form = kOneTile;
  a.ppc = 0;
  const uint32_t ppt = std::min(R, 8);  // rank-split pieces per tile
  if (aligned && (R == 2 || R == 4 || R == 8 || R == 16) && (a.tpc * ppt) % (8 * kSplitFan) == 0 &&
      nwork >= 2 * kLoopWorkgroups && (uint64_t)a.tpc * ppt * R <= 0x7FFFFFFFull) {
    form = kSplit;
    a.ppc = a.tpc * ppt;  // pieces per chunk
    a.nwg = a.ppc * R;
  } else if (full && (nwork & 7u) == 0 && nwork >= 2 * kLoopWorkgroups) {
    form = kLoop;
    a.nwg = kLoopWorkgroups;
  } else {
    a.nwg = nwork;
  }
  const uint32_t grid = a.nwg + (wait ? R : 0);
  if (dtype == VR_DT_F32) launch_dt<VR_DT_F32>(a, aligned, form, grid, st);
  else launch_dt<VR_DT_BF16>(a, aligned, form, grid, st);
  return hipGetLastError() == hipSuccess ? VR_OK : VR_ERR_HIP;
}

}  // namespace vr
