// Communicator, windows, one-sided primitives and the C ABI entry points.
//
// GIN page (lpnh.cn/news/2681042): one-sided transfers (put/get), signals
// and counters, signal and counter methods. Symmetric page
// (zwxr.cn/news/250719): window registration flags, alignment and the
// deregister-before-free cleanup order.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <set>
#include <vector>

#include "vr_device.hpp"
#include "vr_internal.hpp"

using namespace vr;

namespace {

std::mutex g_mu;
std::set<vrComm*> g_comms;

// Scratch of vr_dispatch_noalloc: a file-scope device array, so each GPU the
// library runs on holds its own copy (allocated with the code object and kept
// until the process ends). In host code `scratch` names a host-side stand-in,
// not a device address: the device address of each GPU's copy is taken once
// per device with hipGetSymbolAddress (in vr_comm_create, with that device
// current) and only that address is ever handed to a kernel.
static __device__ __align__(256) char scratch[VR_DISPATCH_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 256;
char* g_noalloc_scratch[kMaxDevices];  // per device, under g_mu; null until looked up

// The current device's copy of `scratch` (looked up on the first call per
// device). Called with the device current; VR_ERR_HIP if the lookup fails.
vrResult_t noalloc_scratch_init(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return VR_ERR_HIP;
  std::lock_guard<std::mutex> g(g_mu);
  if (g_noalloc_scratch[dev]) return VR_OK;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
    (void)hipGetLastError();
    return VR_ERR_HIP;
  }
  g_noalloc_scratch[dev] = static_cast<char*>(p);
  return VR_OK;
}
char* noalloc_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> g(g_mu);
  return g_noalloc_scratch[dev];
}

// Bytes per workgroup of a put: one 16-byte load and store per thread.
// Measured on a 1 GiB copy back to back (stand-alone, one machine): 4 KiB
// tiles 0.325 ms, 8 KiB 0.345 ms, 16 KiB (four per thread) 0.365 ms, each
// with its relay; the relay then needs the first-level fan-out below (per
// XCD only, 4 KiB tiles took 0.597 ms: 32,768 arrivals per counter).
constexpr uint32_t kPutTile = 4096;
constexpr uint32_t kPutFan = 8;  // first-level relay counters per XCD

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool valid_req(int nranks, const vrCommRequirements* req) {
  if (nranks < 1 || nranks > VR_MAX_RANKS || !req) return false;
  if (req->signal_count < 1 || req->signal_count > 65536) return false;
  if (req->counter_count > 65536) return false;
  if (req->context_count < 1 || req->context_count > 1024) return false;
  if (req->barrier_count > 65536) return false;
  return true;
}

struct Layout {
  size_t sig, cnt, err, relay, bar, lit, ring, total;
};
Layout layout(int R, const vrCommRequirements& q) {
  Layout l;
  l.sig = 0;
  l.cnt = align_up(l.sig + sizeof(uint64_t) * R * q.signal_count, 256);
  l.err = align_up(l.cnt + sizeof(uint64_t) * R * std::max<uint32_t>(q.counter_count, 1), 256);
  l.relay = align_up(l.err + 256, 256);
  l.bar = align_up(l.relay + sizeof(uint32_t) * kRelaySlots, 256);
  l.lit = align_up(l.bar + sizeof(uint64_t) * std::max<uint32_t>(q.barrier_count, 1), 256);
  l.ring = align_up(l.lit + sizeof(uint64_t) * R * R, 256);
  l.total = align_up(l.ring + 2 * sizeof(uint64_t) * R * q.context_count, 256);
  return l;
}

bool live(vrComm* c) {
  std::lock_guard<std::mutex> g(g_mu);
  return c && g_comms.count(c);
}
// A call runs with the communicator's device current: the null stream, a
// device synchronize and a symbol lookup all resolve against the current
// device, and a launch there would address this communicator's memory from
// another GPU.
bool on_device(const vrComm* c) {
  int d = -1;
  return hipGetDevice(&d) == hipSuccess && d == c->device;
}
bool has_win(vrComm* c, vrWindow* w) { return w && c->windows.count(w); }
bool rank_ok(vrComm* c, int r) { return r >= 0 && r < c->nranks; }
bool span_ok(const vrWindow* w, size_t off, size_t n) { return off <= w->bytes && n <= w->bytes - off; }
bool overlap(const char* a, size_t an, const char* b, size_t bn) {
  if (!an || !bn) return false;
  return a < b + bn && b < a + an;
}
hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }
vrResult_t hip_ok(hipError_t e) { return e == hipSuccess ? VR_OK : VR_ERR_HIP; }

size_t sidx(const vrComm* c, int rank, uint32_t id) { return (size_t)rank * c->req.signal_count + id; }

// [p, p + bytes) lies in one device allocation on the communicator's device
// (nothing to check when bytes is 0). Kernels dereference these pointers, so
// a host or foreign pointer is refused here instead of faulting the GPU.
bool dev_span_ok(const vrComm* c, const void* p, size_t bytes) {
  if (!bytes) return true;
  if (!p) return false;
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (attr.type != hipMemoryTypeDevice || attr.device != c->device) return false;
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return static_cast<const char*>(p) >= static_cast<const char*>(base) &&
         bytes <= size - (size_t)(static_cast<const char*>(p) - static_cast<const char*>(base));
}

// Whether [off, off + n) of rank's slice (any rank when rank < 0) touches a
// word in use as a VA signal: such words are accessed by signal operations
// only (GIN page, VA signals).
bool va_touch(const vrWindow* w, int rank, size_t off, size_t n) {
  if (!n || w->va_words.empty()) return false;
  for (const auto& kv : w->va_words) {
    const uint64_t o = kv.first.second;
    if ((rank < 0 || kv.first.first == rank) && o < off + n && off < o + 8) return true;
  }
  return false;
}
// A VA signal word: 8-byte aligned, inside the window, which carries strict ordering.
vrResult_t check_va_word(vrComm* c, const vrWindow* w, size_t off) {
  if (!has_win(c, const_cast<vrWindow*>(w))) return VR_ERR_INVALID_ARGUMENT;
  if (off % 8 || !span_ok(w, off, 8)) return VR_ERR_INVALID_ARGUMENT;
  if (!(w->flags & VR_WIN_STRICT_ORDERING)) return VR_ERR_INVALID_USAGE;
  return VR_OK;
}
bool is_va(uint32_t kind) { return kind == VR_VA_SIGNAL_INC || kind == VR_VA_SIGNAL_ADD; }

// Checks that a signal action may be applied (Inc/Add not mixed since the
// last reset: GIN page, strong and weak signals).
vrResult_t check_signal_mode(const vrComm* c, int peer, uint32_t id, uint32_t kind) {
  const uint8_t m = c->sig_mode[sidx(c, peer, id)];
  const uint8_t want = kind == VR_SIGNAL_INC ? 1 : 2;
  return (m && m != want) ? VR_ERR_INVALID_USAGE : VR_OK;
}
void note_signal(vrComm* c, int peer, uint32_t id, uint32_t kind, uint64_t amount, bool known) {
  const size_t i = sidx(c, peer, id);
  c->sig_mode[i] = kind == VR_SIGNAL_INC ? 1 : 2;
  c->expect[i] += amount;
  if (!known) c->expect_known[i] = 0;
}

vrResult_t check_remote(vrComm* c, int peer, const vrRemoteAction& a) {
  if (a.reserved) return VR_ERR_INVALID_ARGUMENT;
  if (a.kind == VR_ACTION_NONE) return VR_OK;
  if (is_va(a.kind)) {
    vrResult_t r = check_va_word(c, a.window, a.offset);
    if (r != VR_OK) return r;
    const auto it = a.window->va_words.find({peer, a.offset});
    const uint8_t want = a.kind == VR_VA_SIGNAL_INC ? 1 : 2;
    return (it != a.window->va_words.end() && it->second && it->second != want) ? VR_ERR_INVALID_USAGE : VR_OK;
  }
  if (a.kind != VR_SIGNAL_INC && a.kind != VR_SIGNAL_ADD) return VR_ERR_INVALID_ARGUMENT;
  if (a.id >= c->req.signal_count) return VR_ERR_INVALID_ARGUMENT;
  return check_signal_mode(c, peer, a.id, a.kind);
}
// The word a remote action adds to, and how much.
uint64_t* remote_word(vrComm* c, int peer, const vrRemoteAction& a, uint64_t* add) {
  *add = (a.kind == VR_SIGNAL_INC || a.kind == VR_VA_SIGNAL_INC) ? 1 : a.value;
  if (is_va(a.kind)) return reinterpret_cast<uint64_t*>(a.window->base[peer] + a.offset);
  return c->sig + sidx(c, peer, a.id);
}
// Enters a VA signal word in the window's table before the operation that
// updates it is enqueued, so that the bookkeeping after a successful launch
// only assigns to an existing entry and cannot fail. The word counts as a
// signal from here on, as after a wait or a read of it.
vrResult_t va_reserve(vrWindow* w, int rank, uint64_t off) {
  try {
    w->va_words.emplace(std::make_pair(rank, off), 0);
  } catch (...) {
    return VR_ERR_OUT_OF_RESOURCES;
  }
  return VR_OK;
}
// Host bookkeeping once a remote action has been enqueued (its VA word, if
// any, entered by va_reserve).
void note_remote(vrComm* c, int peer, const vrRemoteAction& a, uint64_t add) {
  if (is_va(a.kind)) a.window->va_words[{peer, a.offset}] = a.kind == VR_VA_SIGNAL_INC ? 1 : 2;
  else note_signal(c, peer, a.id, a.kind, add, true);
}
vrResult_t check_local(vrComm* c, const vrLocalAction& a) {
  if (a.kind == VR_ACTION_NONE) return VR_OK;
  if (a.kind != VR_COUNTER_INC) return VR_ERR_INVALID_ARGUMENT;
  if (a.id >= c->req.counter_count) return VR_ERR_INVALID_ARGUMENT;
  return VR_OK;
}

// ---- kernels -------------------------------------------------------------------
struct PutArgs {
  char* dst;
  const char* src;
  uint64_t bytes;
  uint32_t parts;
  int dir;           // 0: disjoint ranges; +1 / -1: overlapping, copy forward / backward
  uint32_t* relay;
  uint64_t* sig;     // remote action target or null
  uint64_t add;
  uint64_t* cnt;     // local action target or null
};

// Overlapping copy by one workgroup, in the direction that never overwrites
// bytes not yet read: each round loads a chunk into registers, waits for the
// loads, meets at a barrier, then stores.
__device__ void memmove_wg(char* dst, const char* src, uint64_t n, int dir) {
  constexpr uint32_t kChunk = 256 * 16;
  const uint32_t t = threadIdx.x;
  const uint64_t nchunks = (n + kChunk - 1) / kChunk;
  for (uint64_t k = 0; k < nchunks; ++k) {
    const uint64_t c = dir > 0 ? k : nchunks - 1 - k;
    const uint64_t base = c * kChunk;
    const uint32_t len = static_cast<uint32_t>(std::min<uint64_t>(kChunk, n - base));
    uint8_t v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t i = t * 16 + j;
      v[j] = i < len ? static_cast<uint8_t>(src[base + i]) : 0;
    }
    wait_vmem();
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rd = rsrc(dst + base, len);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t i = t * 16 + j;
      if (i < len) store1_agent(rd, i, v[j]);
    }
    wait_vmem();
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_put(PutArgs a) {
  if (a.dir == 0) {
    const uint64_t off = (uint64_t)blockIdx.x * kPutTile;
    if (off < a.bytes) {
      const uint32_t n = static_cast<uint32_t>(std::min<uint64_t>(kPutTile, a.bytes - off));
      copy_any<1>(a.dst + off, a.src + off, n, threadIdx.x, 256);
    }
  } else {
    memmove_wg(a.dst, a.src, a.bytes, a.dir);
  }
  wg_stores_complete();
  if (threadIdx.x != 0) return;
  // three-level relay for many tiles: tiles b with b mod 8 = x (workgroup b
  // runs on XCD b mod 8) and (b / 8) mod kPutFan = k, then the XCD's k, then
  // the XCDs; each counter on its own 256-byte span. Counters: [0] total,
  // [1 + x] per XCD, [9 + x * kPutFan + k] first level.
  bool last;
  if (a.parts >= 16) {
    const uint32_t b = blockIdx.x, x = b & 7u, k = (b >> 3) % kPutFan;
    const uint32_t n1 = (a.parts - 1 - (8 * k + x)) / (8 * kPutFan) + 1;  // tiles with b mod 8F = 8k + x
    const uint32_t nk = std::min(kPutFan, (a.parts - x + 7) / 8);         // first-level counters of XCD x in use
    last = relay_arrive(a.relay + (9 + x * kPutFan + k) * kRelaySpread, n1, false) &&
           relay_arrive(a.relay + (1 + x) * kRelaySpread, nk, false) && relay_arrive(a.relay, 8, false);
  } else {
    last = relay_arrive(a.relay, a.parts, false);
  }
  if (last) {
    if (a.sig) atomic_add_u64(a.sig, a.add);
    if (a.cnt) atomic_add_u64(a.cnt, 1ull);
  }
}

__global__ void k_signal(uint64_t* sig, uint64_t add) {
  if (threadIdx.x == 0) atomic_add_u64(sig, add);
}

// After copy-engine puts (all complete in stream order): thread (s, d) applies
// the SignalInc of put (s, d) at d; then, in workgroup d + 1, receiver d waits.
__global__ void k_ce_complete(uint64_t* sig, uint32_t stride, int R, vr::U64Tab target, int wait,
                              uint64_t timeout_ns, uint32_t* err) {
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < R * R; i += blockDim.x) atomic_add_u64(sig + (size_t)(i % R) * stride, 1ull);
    return;
  }
  const int d = blockIdx.x - 1;
  if (wait && threadIdx.x == 0) wait_reached(sig + (size_t)d * stride, target.v[d], 64, timeout_ns, err, VR_ASYNC_TIMEOUT);
}

__global__ void k_wait(const uint64_t* word, uint64_t least, int bits, uint64_t timeout_ns, uint32_t* err) {
  if (threadIdx.x == 0) wait_reached(word, least, bits, timeout_ns, err, VR_ASYNC_TIMEOUT);
}

__global__ void k_store0(uint64_t* word) {
  if (threadIdx.x == 0) store8_agent(word, 0ull);
}

vrResult_t enqueue_copy(vrComm* c, char* dst, const char* src, size_t bytes, uint64_t* sig,
                        uint64_t add, uint64_t* cnt, hipStream_t st) {
  PutArgs a;
  a.dst = dst;
  a.src = src;
  a.bytes = bytes;
  a.dir = 0;
  if (overlap(dst, bytes, src, bytes) && dst != src) a.dir = dst < src ? 1 : -1;
  const uint64_t tiles = a.dir ? 1 : std::max<uint64_t>(1, (bytes + kPutTile - 1) / kPutTile);
  if (tiles > 0xFFFFFFFFull) return VR_ERR_INVALID_ARGUMENT;
  a.parts = static_cast<uint32_t>(tiles);
  a.relay = c->relay + kRelaySingle;
  a.sig = sig;
  a.add = add;
  a.cnt = cnt;
  hipLaunchKernelGGL(k_put, dim3(a.parts), dim3(256), 0, st, a);
  return hip_ok(hipGetLastError());
}

}  // namespace

// ---- internal helpers used by the collectives ---------------------------------------
namespace vr {
// Copy-engine puts: ops spread over the internal streams, forked from and
// joined back into st (default-priority streams).
struct CeCopy {
  char* dst;
  const char* src;
  size_t bytes;
};
// The internal streams and events, created on first use: all of them or
// none (a partial set would be indexed past its end by the next call).
static vrResult_t ce_setup(vrComm* c) {
  hipStream_t ss[VR_CE_STREAMS];
  hipEvent_t es[VR_CE_STREAMS + 1];
  int nss = 0, nes = 0;
  while (nss < VR_CE_STREAMS && hipStreamCreateWithFlags(&ss[nss], hipStreamNonBlocking) == hipSuccess) ++nss;
  while (nss == VR_CE_STREAMS && nes <= VR_CE_STREAMS && hipEventCreateWithFlags(&es[nes], hipEventDisableTiming) == hipSuccess)
    ++nes;
  const bool ok = nss == VR_CE_STREAMS && nes == VR_CE_STREAMS + 1;
  if (ok) {
    try {
      c->ce_streams.assign(ss, ss + nss);
      c->ce_events.assign(es, es + nes);
      return VR_OK;
    } catch (...) {
      c->ce_streams.clear();
      c->ce_events.clear();
    }
  }
  for (int i = 0; i < nss; ++i) (void)hipStreamDestroy(ss[i]);
  for (int i = 0; i < nes; ++i) (void)hipEventDestroy(es[i]);
  return ok ? VR_ERR_OUT_OF_RESOURCES : VR_ERR_HIP;
}

vrResult_t ce_puts(vrComm* c, const std::vector<CeCopy>& ops, hipStream_t st) {
  if (c->ce_streams.empty()) {
    const vrResult_t r = ce_setup(c);
    if (r != VR_OK) return r;
  }
  const int n = std::min<int>(VR_CE_STREAMS, std::max<int>(1, (int)ops.size()));
  if (hipEventRecord(c->ce_events[0], st) != hipSuccess) return VR_ERR_HIP;
  for (int i = 0; i < n; ++i)
    if (hipStreamWaitEvent(c->ce_streams[i], c->ce_events[0], 0) != hipSuccess) return VR_ERR_HIP;
  for (size_t k = 0; k < ops.size(); ++k)
    if (ops[k].bytes && hipMemcpyAsync(ops[k].dst, ops[k].src, ops[k].bytes, hipMemcpyDeviceToDeviceNoCU,
                                       c->ce_streams[k % n]) != hipSuccess)
      return VR_ERR_HIP;
  for (int i = 0; i < n; ++i) {
    if (hipEventRecord(c->ce_events[1 + i], c->ce_streams[i]) != hipSuccess) return VR_ERR_HIP;
    if (hipStreamWaitEvent(st, c->ce_events[1 + i], 0) != hipSuccess) return VR_ERR_HIP;
  }
  return VR_OK;
}
vrResult_t ce_complete(vrComm* c, uint32_t sig, const U64Tab& target, bool wait, hipStream_t st) {
  hipLaunchKernelGGL(k_ce_complete, dim3(1 + c->nranks), dim3(256), 0, st, c->sig + sig, c->req.signal_count,
                     c->nranks, target, wait ? 1 : 0, kDefaultTimeoutNs, c->err);
  return hip_ok(hipGetLastError());
}

vrDevComm device_view(const vrComm* c) {
  vrDevComm v;
  v.nranks = c->nranks;
  v.signal_count = c->req.signal_count;
  v.counter_count = c->req.counter_count;
  v.barrier_count = c->req.barrier_count;
  v.signals = c->sig;
  v.counters = c->cnt;
  v.barriers = c->bar;
  v.error = c->err;
  return v;
}
vrDevWindow device_view(const vrWindow* w) {
  vrDevWindow v;
  for (int r = 0; r < VR_MAX_RANKS; ++r) v.base[r] = w->base[r];
  v.bytes = w->bytes;
  return v;
}

vrResult_t ensure_scratch(vrComm* c, size_t bytes) {
  if (bytes <= c->scratch_bytes) return VR_OK;
  // the previous scratch may still be in use by enqueued work
  if (c->scratch) {
    if (hipDeviceSynchronize() != hipSuccess) return VR_ERR_HIP;
    if (hipFree(c->scratch) != hipSuccess) return VR_ERR_HIP;
    c->scratch = nullptr;
    c->scratch_bytes = 0;
  }
  void* p = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess) return VR_ERR_OUT_OF_RESOURCES;
  if (hipMemset(p, 0, bytes) != hipSuccess) {
    (void)hipFree(p);
    return VR_ERR_HIP;
  }
  c->scratch = static_cast<char*>(p);
  c->scratch_bytes = bytes;
  return VR_OK;
}
}  // namespace vr

// ---- C ABI -------------------------------------------------------------------------------
extern "C" {

const char* vr_error_string(vrResult_t r) {
  switch (r) {
    case VR_OK: return "VR_OK";
    case VR_ERR_INVALID_ARGUMENT: return "VR_ERR_INVALID_ARGUMENT";
    case VR_ERR_INVALID_USAGE: return "VR_ERR_INVALID_USAGE";
    case VR_ERR_OUT_OF_RESOURCES: return "VR_ERR_OUT_OF_RESOURCES";
    case VR_ERR_HIP: return "VR_ERR_HIP";
    case VR_ERR_TIMEOUT: return "VR_ERR_TIMEOUT";
    case VR_ERR_UNSUPPORTED_DEVICE: return "VR_ERR_UNSUPPORTED_DEVICE";
    case VR_ERR_INTERNAL: return "VR_ERR_INTERNAL";
    case VR_ERR_DEVICE_CHECK: return "VR_ERR_DEVICE_CHECK";
    default: return "VR_ERR_UNKNOWN";
  }
}

int vr_version(void) { return 100; }

size_t vr_comm_workspace_bytes(int nranks, const vrCommRequirements* req) {
  if (!valid_req(nranks, req)) return 0;
  return layout(nranks, *req).total;
}

vrResult_t vr_comm_create(int nranks, const vrCommRequirements* req, void* workspace,
                          size_t workspace_bytes, vrComm_t* out) {
  if (!out || !valid_req(nranks, req)) return VR_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  const Layout l = layout(nranks, *req);
  if (workspace && (workspace_bytes < l.total || (reinterpret_cast<uintptr_t>(workspace) & 255)))
    return VR_ERR_INVALID_ARGUMENT;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return VR_ERR_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return VR_ERR_HIP;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return VR_ERR_UNSUPPORTED_DEVICE;
  vrComm* c = new (std::nothrow) vrComm();
  if (!c) return VR_ERR_OUT_OF_RESOURCES;
  c->device = dev;
  c->nranks = nranks;
  c->req = *req;
  c->owns_ws = workspace == nullptr;
  c->ws_bytes = l.total;
  if (workspace) {
    c->ws = static_cast<char*>(workspace);
  } else {
    void* p = nullptr;
    if (hipMalloc(&p, l.total) != hipSuccess) {
      delete c;
      return VR_ERR_OUT_OF_RESOURCES;
    }
    c->ws = static_cast<char*>(p);
  }
  if (hipMemset(c->ws, 0, l.total) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
      noalloc_scratch_init(dev) != VR_OK) {
    if (c->owns_ws) (void)hipFree(c->ws);
    delete c;
    return VR_ERR_HIP;
  }
  c->sig = reinterpret_cast<uint64_t*>(c->ws + l.sig);
  c->cnt = reinterpret_cast<uint64_t*>(c->ws + l.cnt);
  c->err = reinterpret_cast<uint32_t*>(c->ws + l.err);
  c->relay = reinterpret_cast<uint32_t*>(c->ws + l.relay);
  c->bar = reinterpret_cast<uint64_t*>(c->ws + l.bar);
  c->lit_last = reinterpret_cast<uint64_t*>(c->ws + l.lit);
  c->litmus = nullptr;
  c->lit_seed = 0;
  c->trace = nullptr;
  c->trace_words = 0;
  c->ring_bases = reinterpret_cast<uint64_t*>(c->ws + l.ring);
  c->ring_gens = c->ring_bases + (size_t)nranks * req->context_count;
  c->ring_gen = 0;
  c->scratch = nullptr;
  c->scratch_bytes = 0;
  const size_t ns = (size_t)nranks * req->signal_count;
  try {  // host tables: a failed allocation is an error code, never an exception through the C ABI
    c->bar_expect.assign(req->barrier_count, 0);
    c->expect.assign(ns, 0);
    c->expect_known.assign(ns, 1);
    c->sig_mode.assign(ns, 0);
    std::lock_guard<std::mutex> g(g_mu);
    g_comms.insert(c);
  } catch (...) {
    if (c->owns_ws) (void)hipFree(c->ws);
    delete c;
    return VR_ERR_OUT_OF_RESOURCES;
  }
  *out = c;
  return VR_OK;
}

vrResult_t vr_comm_destroy(vrComm_t c) {
  if (!live(c)) return VR_ERR_INVALID_ARGUMENT;
  if (!c->windows.empty()) return VR_ERR_INVALID_USAGE;
  // any device may be current here: switch to the communicator's for the
  // synchronize and the frees, then give the caller's back
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(c->device) != hipSuccess) return VR_ERR_HIP;
  (void)hipDeviceSynchronize();
  if (c->owns_ws) (void)hipFree(c->ws);
  if (c->scratch) (void)hipFree(c->scratch);
  for (hipStream_t s : c->ce_streams) (void)hipStreamDestroy(s);
  for (hipEvent_t e : c->ce_events) (void)hipEventDestroy(e);
  {
    std::lock_guard<std::mutex> g(g_mu);
    g_comms.erase(c);
  }
  delete c;
  (void)hipSetDevice(prev);
  return VR_OK;
}

vrResult_t vr_comm_get_async_error(vrComm_t c, vrResult_t* out, uint32_t* bits) {
  if (!live(c) || !out) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  uint32_t b = 0;
  if (hipMemcpy(&b, c->err, sizeof(b), hipMemcpyDeviceToHost) != hipSuccess) return VR_ERR_HIP;
  if (b && hipMemset(c->err, 0, sizeof(uint32_t)) != hipSuccess) return VR_ERR_HIP;
  if (bits) *bits = b;
  if (b & VR_ASYNC_TIMEOUT) *out = VR_ERR_TIMEOUT;
  else if (b & VR_ASYNC_CAPACITY) *out = VR_ERR_OUT_OF_RESOURCES;
  else if (b) *out = VR_ERR_DEVICE_CHECK;
  else *out = VR_OK;
  return VR_OK;
}

vrResult_t vr_comm_set_litmus(vrComm_t c, uint64_t* litmus) {
  if (!live(c)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (litmus && !dev_span_ok(c, litmus, 2 * sizeof(uint64_t))) return VR_ERR_INVALID_ARGUMENT;
  c->litmus = litmus;
  return VR_OK;
}

vrResult_t vr_comm_set_trace(vrComm_t c, uint64_t* stamps, size_t words) {
  if (!live(c)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (stamps && (!words || !dev_span_ok(c, stamps, words * sizeof(uint64_t)))) return VR_ERR_INVALID_ARGUMENT;
  c->trace = stamps;
  c->trace_words = stamps ? words : 0;
  return VR_OK;
}

vrResult_t vr_comm_query(vrComm_t c, int* nranks, vrCommRequirements* req) {
  if (!live(c)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (nranks) *nranks = c->nranks;
  if (req) *req = c->req;
  return VR_OK;
}

vrResult_t vr_window_register(vrComm_t c, void* const* bases, size_t bytes, uint32_t flags,
                              vrWindow_t* out) {
  if (!live(c) || !bases || !out || bytes == 0) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (flags & ~(VR_WIN_COLL_SYMMETRIC | VR_WIN_STRICT_ORDERING)) return VR_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  const int R = c->nranks;
  for (int r = 0; r < R; ++r) {
    char* b = static_cast<char*>(bases[r]);
    if (!b || (reinterpret_cast<uintptr_t>(b) % VR_WIN_REQUIRED_ALIGNMENT)) return VR_ERR_INVALID_ARGUMENT;
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, b) != hipSuccess) return VR_ERR_INVALID_ARGUMENT;
    if (attr.type != hipMemoryTypeDevice || attr.device != c->device) return VR_ERR_INVALID_ARGUMENT;
    hipDeviceptr_t pbase = nullptr;
    size_t psize = 0;
    if (hipMemGetAddressRange(&pbase, &psize, b) != hipSuccess) return VR_ERR_INVALID_ARGUMENT;
    if (b + bytes > static_cast<char*>(pbase) + psize) return VR_ERR_INVALID_ARGUMENT;
    for (int q = 0; q < r; ++q)
      if (overlap(b, bytes, static_cast<char*>(bases[q]), bytes)) return VR_ERR_INVALID_ARGUMENT;
  }
  vrWindow* w = new (std::nothrow) vrWindow();
  if (!w) return VR_ERR_OUT_OF_RESOURCES;
  w->comm = c;
  w->bytes = bytes;
  w->flags = flags;
  w->nranks = R;
  for (int r = 0; r < VR_MAX_RANKS; ++r) w->base[r] = r < R ? static_cast<char*>(bases[r]) : nullptr;
  try {
    c->windows.insert(w);
  } catch (...) {
    delete w;
    return VR_ERR_OUT_OF_RESOURCES;
  }
  *out = w;
  return VR_OK;
}

vrResult_t vr_window_deregister(vrComm_t c, vrWindow_t w) {
  if (!live(c) || !has_win(c, w)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  (void)hipDeviceSynchronize();  // no enqueued work may still use the window
  c->windows.erase(w);
  delete w;
  return VR_OK;
}

vrResult_t vr_put(vrComm_t c, int ctx, int rank, int peer, vrWindow_t dst, size_t dst_off,
                  vrWindow_t src, size_t src_off, size_t bytes, vrRemoteAction remote,
                  vrLocalAction local, void* stream) {
  if (!live(c) || !rank_ok(c, rank) || !rank_ok(c, peer)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (ctx < 0 || (uint32_t)ctx >= c->req.context_count) return VR_ERR_INVALID_ARGUMENT;
  if (!has_win(c, dst) || !has_win(c, src)) return VR_ERR_INVALID_ARGUMENT;
  if (!span_ok(dst, dst_off, bytes) || !span_ok(src, src_off, bytes)) return VR_ERR_INVALID_ARGUMENT;
  vrResult_t r = check_remote(c, peer, remote);
  if (r != VR_OK) return r;
  if ((r = check_local(c, local)) != VR_OK) return r;
  if (va_touch(dst, peer, dst_off, bytes) || va_touch(src, rank, src_off, bytes)) return VR_ERR_INVALID_USAGE;
  if (is_va(remote.kind) && ((remote.window == dst && overlap(dst->base[peer] + dst_off, bytes,
                                                               dst->base[peer] + remote.offset, 8)) ||
                             (remote.window == src && overlap(src->base[rank] + src_off, bytes,
                                                               src->base[peer] + remote.offset, 8))))
    return VR_ERR_INVALID_USAGE;  // the put would move the signal word's own bytes
  if (is_va(remote.kind) && (r = va_reserve(remote.window, peer, remote.offset)) != VR_OK) return r;
  uint64_t* sig = nullptr;
  uint64_t add = 0;
  if (remote.kind != VR_ACTION_NONE) sig = remote_word(c, peer, remote, &add);
  uint64_t* cnt = local.kind == VR_COUNTER_INC ? c->cnt + (size_t)rank * c->req.counter_count + local.id : nullptr;
  r = enqueue_copy(c, dst->base[peer] + dst_off, src->base[rank] + src_off, bytes, sig, add, cnt, S(stream));
  if (r == VR_OK && sig) note_remote(c, peer, remote, add);
  return r;
}

vrResult_t vr_get(vrComm_t c, int ctx, int rank, int peer, vrWindow_t remote, size_t remote_off,
                  vrWindow_t localw, size_t local_off, size_t bytes, vrLocalAction local, void* stream) {
  if (!live(c) || !rank_ok(c, rank) || !rank_ok(c, peer)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (ctx < 0 || (uint32_t)ctx >= c->req.context_count) return VR_ERR_INVALID_ARGUMENT;
  if (!has_win(c, remote) || !has_win(c, localw)) return VR_ERR_INVALID_ARGUMENT;
  if (!span_ok(remote, remote_off, bytes) || !span_ok(localw, local_off, bytes)) return VR_ERR_INVALID_ARGUMENT;
  vrResult_t r = check_local(c, local);
  if (r != VR_OK) return r;
  if (va_touch(remote, peer, remote_off, bytes) || va_touch(localw, rank, local_off, bytes))
    return VR_ERR_INVALID_USAGE;
  uint64_t* cnt = local.kind == VR_COUNTER_INC ? c->cnt + (size_t)rank * c->req.counter_count + local.id : nullptr;
  return enqueue_copy(c, localw->base[rank] + local_off, remote->base[peer] + remote_off, bytes, nullptr, 0,
                      cnt, S(stream));
}

vrResult_t vr_signal(vrComm_t c, int ctx, int rank, int peer, vrRemoteAction remote, void* stream) {
  if (!live(c) || !rank_ok(c, rank) || !rank_ok(c, peer)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (ctx < 0 || (uint32_t)ctx >= c->req.context_count) return VR_ERR_INVALID_ARGUMENT;
  if (remote.kind == VR_ACTION_NONE) return VR_ERR_INVALID_ARGUMENT;
  vrResult_t r = check_remote(c, peer, remote);
  if (r != VR_OK) return r;
  if (is_va(remote.kind) && (r = va_reserve(remote.window, peer, remote.offset)) != VR_OK) return r;
  uint64_t add = 0;
  uint64_t* word = remote_word(c, peer, remote, &add);
  hipLaunchKernelGGL(k_signal, dim3(1), dim3(64), 0, S(stream), word, add);
  r = hip_ok(hipGetLastError());
  if (r == VR_OK) note_remote(c, peer, remote, add);
  return r;
}

static vrResult_t wait_word(vrComm* c, uint64_t* word, uint64_t least, int bits, uint64_t timeout_ns,
                            void* stream) {
  if (timeout_ns == 0) timeout_ns = kDefaultTimeoutNs;
  hipLaunchKernelGGL(k_wait, dim3(1), dim3(64), 0, S(stream), word, least, bits, timeout_ns, c->err);
  return hip_ok(hipGetLastError());
}

vrResult_t vr_signal_wait(vrComm_t c, int rank, uint32_t id, uint64_t least, int bits, uint64_t timeout_ns,
                          void* stream) {
  if (!live(c) || !rank_ok(c, rank) || id >= c->req.signal_count) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (bits < 1 || bits > VR_SIGNAL_BITS) return VR_ERR_INVALID_ARGUMENT;
  return wait_word(c, c->sig + sidx(c, rank, id), least, bits, timeout_ns, stream);
}

static vrResult_t va_prepare(vrComm* c, vrWindow* w, int rank, size_t off) {
  if (!live(c) || !rank_ok(c, rank)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  vrResult_t r = check_va_word(c, w, off);
  if (r != VR_OK) return r;
  try {
    w->va_words.emplace(std::make_pair(rank, (uint64_t)off), 0);  // a signal from now on
  } catch (...) {
    return VR_ERR_OUT_OF_RESOURCES;
  }
  return VR_OK;
}

vrResult_t vr_va_signal_wait(vrComm_t c, vrWindow_t w, int rank, size_t off, uint64_t least, int bits,
                             uint64_t timeout_ns, void* stream) {
  if (bits < 1 || bits > VR_SIGNAL_BITS) return VR_ERR_INVALID_ARGUMENT;
  vrResult_t r = va_prepare(c, w, rank, off);
  if (r != VR_OK) return r;
  return wait_word(c, reinterpret_cast<uint64_t*>(w->base[rank] + off), least, bits, timeout_ns, stream);
}

vrResult_t vr_counter_wait(vrComm_t c, int rank, uint32_t id, uint64_t least, int bits, uint64_t timeout_ns,
                           void* stream) {
  if (!live(c) || !rank_ok(c, rank) || id >= c->req.counter_count) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (bits < 1 || bits > VR_COUNTER_BITS) return VR_ERR_INVALID_ARGUMENT;
  return wait_word(c, c->cnt + (size_t)rank * c->req.counter_count + id, least, bits, timeout_ns, stream);
}

static vrResult_t read_word(const uint64_t* word, int bits, uint64_t* out) {
  uint64_t v = 0;
  if (hipMemcpy(&v, word, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return VR_ERR_HIP;
  *out = bits >= 64 ? v : (v & ((1ull << bits) - 1));
  return VR_OK;
}

vrResult_t vr_signal_read(vrComm_t c, int rank, uint32_t id, int bits, uint64_t* out) {
  if (!live(c) || !rank_ok(c, rank) || id >= c->req.signal_count || !out) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (bits < 1 || bits > VR_SIGNAL_BITS) return VR_ERR_INVALID_ARGUMENT;
  return read_word(c->sig + sidx(c, rank, id), bits, out);
}

vrResult_t vr_va_signal_read(vrComm_t c, vrWindow_t w, int rank, size_t off, int bits, uint64_t* out) {
  if (!out || bits < 1 || bits > VR_SIGNAL_BITS) return VR_ERR_INVALID_ARGUMENT;
  vrResult_t r = va_prepare(c, w, rank, off);
  if (r != VR_OK) return r;
  return read_word(reinterpret_cast<uint64_t*>(w->base[rank] + off), bits, out);
}

vrResult_t vr_va_signal_reset(vrComm_t c, vrWindow_t w, int rank, size_t off, void* stream) {
  vrResult_t r = va_prepare(c, w, rank, off);
  if (r != VR_OK) return r;
  hipLaunchKernelGGL(k_store0, dim3(1), dim3(64), 0, S(stream), reinterpret_cast<uint64_t*>(w->base[rank] + off));
  r = hip_ok(hipGetLastError());
  if (r == VR_OK) w->va_words[{rank, (uint64_t)off}] = 0;
  return r;
}

vrResult_t vr_comm_device_view(vrComm_t c, vrDevComm* out) {
  if (!live(c) || !out) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  *out = device_view(c);
  return VR_OK;
}

vrResult_t vr_window_device_view(vrComm_t c, vrWindow_t w, vrDevWindow* out) {
  if (!live(c) || !has_win(c, w) || !out) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  *out = device_view(w);
  return VR_OK;
}

vrResult_t vr_barrier_expected(vrComm_t c, uint32_t index, uint64_t* out) {
  if (!live(c) || index >= c->req.barrier_count || !out) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  *out = c->bar_expect[index];
  return VR_OK;
}

vrResult_t vr_barrier_advance(vrComm_t c, uint32_t index, uint64_t arrivals) {
  if (!live(c) || index >= c->req.barrier_count) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  c->bar_expect[index] += arrivals;
  return VR_OK;
}

vrResult_t vr_barrier(vrComm_t c, uint32_t index, uint32_t fence, uint64_t timeout_ns, void* stream) {
  if (!live(c) || index >= c->req.barrier_count) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (fence & ~(VR_FENCE_PUT | VR_FENCE_GET)) return VR_ERR_INVALID_ARGUMENT;
  const uint64_t target = c->bar_expect[index] + c->nranks;
  vrResult_t r = launch_barrier(c, index, target, fence, timeout_ns ? timeout_ns : kDefaultTimeoutNs, S(stream));
  if (r == VR_OK) c->bar_expect[index] = target;
  return r;
}

vrResult_t vr_counter_read(vrComm_t c, int rank, uint32_t id, int bits, uint64_t* out) {
  if (!live(c) || !rank_ok(c, rank) || id >= c->req.counter_count || !out) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (bits < 1 || bits > VR_COUNTER_BITS) return VR_ERR_INVALID_ARGUMENT;
  return read_word(c->cnt + (size_t)rank * c->req.counter_count + id, bits, out);
}

vrResult_t vr_signal_reset(vrComm_t c, int rank, uint32_t id, void* stream) {
  if (!live(c) || !rank_ok(c, rank) || id >= c->req.signal_count) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  hipLaunchKernelGGL(k_store0, dim3(1), dim3(64), 0, S(stream), c->sig + sidx(c, rank, id));
  vrResult_t r = hip_ok(hipGetLastError());
  if (r == VR_OK) {
    const size_t i = sidx(c, rank, id);
    c->expect[i] = 0;
    c->expect_known[i] = 1;
    c->sig_mode[i] = 0;
  }
  return r;
}

vrResult_t vr_counter_reset(vrComm_t c, int rank, uint32_t id, void* stream) {
  if (!live(c) || !rank_ok(c, rank) || id >= c->req.counter_count) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  hipLaunchKernelGGL(k_store0, dim3(1), dim3(64), 0, S(stream),
                     c->cnt + (size_t)rank * c->req.counter_count + id);
  return hip_ok(hipGetLastError());
}

vrResult_t vr_signal_expected(vrComm_t c, int rank, uint32_t id, uint64_t* out) {
  if (!live(c) || !rank_ok(c, rank) || id >= c->req.signal_count || !out) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  const size_t i = sidx(c, rank, id);
  if (!c->expect_known[i]) return VR_ERR_INVALID_USAGE;
  *out = c->expect[i];
  return VR_OK;
}

// ---- collectives: validation and bookkeeping; kernels live in their own files ---------------
static bool any_overlap(const vrWindow* a, size_t aoff, size_t an, const vrWindow* b, size_t boff, size_t bn,
                        int R) {
  for (int i = 0; i < R; ++i)
    for (int j = 0; j < R; ++j)
      if (overlap(a->base[i] + aoff, an, b->base[j] + boff, bn)) return true;
  return false;
}

// Targets for an Inc-type completion signal that rises by `amount` at every rank.
static vrResult_t inc_targets(vrComm* c, uint32_t sig, uint64_t amount, bool wait, U64Tab* t) {
  if (sig >= c->req.signal_count) return VR_ERR_INVALID_ARGUMENT;
  for (int d = 0; d < c->nranks; ++d) {
    if (check_signal_mode(c, d, sig, VR_SIGNAL_INC) != VR_OK) return VR_ERR_INVALID_USAGE;
    if (wait && !c->expect_known[sidx(c, d, sig)]) return VR_ERR_INVALID_USAGE;
  }
  for (int d = 0; d < VR_MAX_RANKS; ++d)
    t->v[d] = d < c->nranks ? c->expect[sidx(c, d, sig)] + amount : 0;
  return VR_OK;
}
static void commit_inc(vrComm* c, uint32_t sig, uint64_t amount) {
  for (int d = 0; d < c->nranks; ++d) note_signal(c, d, sig, VR_SIGNAL_INC, amount, true);
}

vrResult_t vr_allreduce(vrComm_t c, vrWindow_t send, size_t send_off, vrWindow_t recv, size_t recv_off,
                        size_t count, int dtype, int op, uint32_t sig, uint32_t flags, void* stream) {
  if (!live(c) || !has_win(c, send) || !has_win(c, recv)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if ((dtype != VR_DT_F32 && dtype != VR_DT_BF16) || op != VR_OP_SUM) return VR_ERR_INVALID_ARGUMENT;
  if (flags & ~VR_COLL_NO_WAIT) return VR_ERR_INVALID_ARGUMENT;
  const size_t es = dtype == VR_DT_F32 ? 4 : 2;
  if (count > (size_t(1) << 40) || (send_off % es) || (recv_off % es)) return VR_ERR_INVALID_ARGUMENT;
  const size_t n = count * es;
  if (!span_ok(send, send_off, n) || !span_ok(recv, recv_off, n)) return VR_ERR_INVALID_ARGUMENT;
  if (any_overlap(send, send_off, n, recv, recv_off, n, c->nranks)) return VR_ERR_INVALID_ARGUMENT;
  if (va_touch(send, -1, send_off, n) || va_touch(recv, -1, recv_off, n)) return VR_ERR_INVALID_USAGE;
  const bool wait = !(flags & VR_COLL_NO_WAIT);
  U64Tab t;
  vrResult_t r = inc_targets(c, sig, c->nranks, wait, &t);
  if (r != VR_OK) return r;
  r = launch_allreduce(c, send, send_off, recv, recv_off, count, dtype, sig, t, wait, S(stream));
  if (r == VR_OK) commit_inc(c, sig, c->nranks);
  return r;
}

vrResult_t vr_alltoall(vrComm_t c, vrWindow_t send, size_t send_off, vrWindow_t recv, size_t recv_off,
                       size_t block, uint32_t sig, uint32_t flags, void* stream) {
  if (!live(c) || !has_win(c, send) || !has_win(c, recv)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (flags & ~(VR_COLL_NO_WAIT | VR_COLL_COPY_ENGINE)) return VR_ERR_INVALID_ARGUMENT;
  const int R = c->nranks;
  if (block > (size_t(1) << 40)) return VR_ERR_INVALID_ARGUMENT;
  const size_t n = block * R;
  if (!span_ok(send, send_off, n) || !span_ok(recv, recv_off, n)) return VR_ERR_INVALID_ARGUMENT;
  if (any_overlap(send, send_off, n, recv, recv_off, n, R)) return VR_ERR_INVALID_ARGUMENT;
  if (va_touch(send, -1, send_off, n) || va_touch(recv, -1, recv_off, n)) return VR_ERR_INVALID_USAGE;
  const bool wait = !(flags & VR_COLL_NO_WAIT);
  U64Tab t;
  vrResult_t r = inc_targets(c, sig, R, wait, &t);
  if (r != VR_OK) return r;
  if (flags & VR_COLL_COPY_ENGINE) {
    std::vector<CeCopy> ops;
    try {
      ops.reserve((size_t)R * R);  // the pushes below then cannot throw
    } catch (...) {
      return VR_ERR_OUT_OF_RESOURCES;
    }
    for (int s = 0; s < R; ++s)  // destination-major, so consecutive copies target different ranks
      for (int d = 0; d < R; ++d)
        ops.push_back({recv->base[(d + s) % R] + recv_off + (size_t)s * block,
                       send->base[s] + send_off + (size_t)((d + s) % R) * block, block});
    r = ce_puts(c, ops, S(stream));
    if (r == VR_OK) r = ce_complete(c, sig, t, wait, S(stream));
  } else {
    r = launch_alltoall(c, send, send_off, recv, recv_off, block, sig, t, wait, S(stream));
  }
  if (r == VR_OK) commit_inc(c, sig, R);
  return r;
}

vrResult_t vr_alltoall_sessions(vrComm_t c, vrWindow_t send, size_t send_off, vrWindow_t recv, size_t recv_off,
                                size_t block, uint32_t sig, uint32_t index, uint32_t flags, void* stream) {
  if (!live(c) || !has_win(c, send) || !has_win(c, recv)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (flags || index >= c->req.barrier_count) return VR_ERR_INVALID_ARGUMENT;
  const int R = c->nranks;
  if (block > (size_t(1) << 40)) return VR_ERR_INVALID_ARGUMENT;
  const size_t n = block * R;
  if (!span_ok(send, send_off, n) || !span_ok(recv, recv_off, n)) return VR_ERR_INVALID_ARGUMENT;
  if (any_overlap(send, send_off, n, recv, recv_off, n, R)) return VR_ERR_INVALID_ARGUMENT;
  if (va_touch(send, -1, send_off, n) || va_touch(recv, -1, recv_off, n)) return VR_ERR_INVALID_USAGE;
  U64Tab t;
  vrResult_t r = inc_targets(c, sig, R, true, &t);
  if (r != VR_OK) return r;
  const uint64_t base = c->bar_expect[index];
  r = launch_alltoall_sessions(c, device_view(send), send_off, device_view(recv), recv_off, block, sig, t, index,
                               base, S(stream));
  if (r == VR_OK) {
    commit_inc(c, sig, R);
    c->bar_expect[index] = base + 2ull * R;
  }
  return r;
}

vrResult_t vr_signal_pingpong(vrComm_t c, vrWindow_t w, size_t off, size_t bytes, uint32_t iters, uint32_t sig,
                              uint32_t flags, void* stream) {
  if (!live(c) || !has_win(c, w)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if ((flags & ~(VR_PINGPONG_SAME_XCD | VR_PINGPONG_WAVES)) ||
      (flags & (VR_PINGPONG_SAME_XCD | VR_PINGPONG_WAVES)) == (VR_PINGPONG_SAME_XCD | VR_PINGPONG_WAVES))
    return VR_ERR_INVALID_ARGUMENT;
  if (c->nranks < 2 || iters == 0 || bytes > (size_t(1) << 20)) return VR_ERR_INVALID_ARGUMENT;
  if (!span_ok(w, off, 2 * bytes)) return VR_ERR_INVALID_ARGUMENT;
  if (va_touch(w, 0, off, 2 * bytes) || va_touch(w, 1, off, 2 * bytes)) return VR_ERR_INVALID_USAGE;
  if (sig >= c->req.signal_count) return VR_ERR_INVALID_ARGUMENT;
  uint64_t base[2];
  for (int r = 0; r < 2; ++r) {
    if (check_signal_mode(c, r, sig, VR_SIGNAL_INC) != VR_OK) return VR_ERR_INVALID_USAGE;
    if (!c->expect_known[sidx(c, r, sig)]) return VR_ERR_INVALID_USAGE;
    base[r] = c->expect[sidx(c, r, sig)];
  }
  vrResult_t r = launch_pingpong(c, w, off, bytes, iters, sig, base, (flags & VR_PINGPONG_SAME_XCD) != 0,
                                 (flags & VR_PINGPONG_WAVES) != 0, S(stream));
  if (r == VR_OK)
    for (int q = 0; q < 2; ++q) note_signal(c, q, sig, VR_SIGNAL_INC, iters, true);
  return r;
}

vrResult_t vr_allgather(vrComm_t c, vrWindow_t send, size_t send_off, vrWindow_t recv, size_t recv_off,
                        size_t bytes, uint32_t sig, uint32_t flags, void* stream) {
  if (!live(c) || !has_win(c, send) || !has_win(c, recv)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (flags & ~(VR_COLL_NO_WAIT | VR_COLL_COPY_ENGINE)) return VR_ERR_INVALID_ARGUMENT;
  const int R = c->nranks;
  if (bytes > (size_t(1) << 40)) return VR_ERR_INVALID_ARGUMENT;
  if (!span_ok(send, send_off, bytes) || !span_ok(recv, recv_off, bytes * R)) return VR_ERR_INVALID_ARGUMENT;
  if (any_overlap(send, send_off, bytes, recv, recv_off, bytes * R, R)) return VR_ERR_INVALID_ARGUMENT;
  if (va_touch(send, -1, send_off, bytes) || va_touch(recv, -1, recv_off, bytes * R))
    return VR_ERR_INVALID_USAGE;
  const bool wait = !(flags & VR_COLL_NO_WAIT);
  U64Tab t;
  vrResult_t r = inc_targets(c, sig, R, wait, &t);
  if (r != VR_OK) return r;
  if (flags & VR_COLL_COPY_ENGINE) {
    std::vector<CeCopy> ops;
    try {
      ops.reserve((size_t)R * R);  // the pushes below then cannot throw
    } catch (...) {
      return VR_ERR_OUT_OF_RESOURCES;
    }
    for (int s = 0; s < R; ++s)
      for (int d = 0; d < R; ++d)
        ops.push_back({recv->base[(d + s) % R] + recv_off + (size_t)s * bytes, send->base[s] + send_off, bytes});
    r = ce_puts(c, ops, S(stream));
    if (r == VR_OK) r = ce_complete(c, sig, t, wait, S(stream));
  } else {
    r = launch_allgather(c, send, send_off, recv, recv_off, bytes, sig, t, wait, S(stream));
  }
  if (r == VR_OK) commit_inc(c, sig, R);
  return r;
}

static vrResult_t dispatch_common(vrComm_t c, vrWindow_t x, size_t x_off, size_t row_bytes, const int32_t* topk,
                                  int T, int K, int E, vrWindow_t recv, size_t recv_off, size_t cap,
                                  int32_t* counts_out, int32_t* src_out, int32_t* experts_out, int32_t* send_pos,
                                  bool dedup, uint32_t sig_counts, uint32_t sig_rows, uint32_t flags, void* stream,
                                  bool noalloc = false) {
  if (!live(c) || !has_win(c, x) || !has_win(c, recv)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (flags & ~VR_COLL_NO_WAIT) return VR_ERR_INVALID_ARGUMENT;
  const int R = c->nranks;
  if ((!topk && T > 0) || !counts_out || (!src_out && cap > 0)) return VR_ERR_INVALID_ARGUMENT;
  if (dedup && !experts_out && cap > 0) return VR_ERR_INVALID_ARGUMENT;
  if (T < 0 || T >= 65536 || K < 1 || K > 64 || E < R || E % R || E > 1024)
    return VR_ERR_INVALID_ARGUMENT;
  if (row_bytes == 0 || row_bytes > (size_t(1) << 30) || cap > (size_t(1) << 31)) return VR_ERR_INVALID_ARGUMENT;
  if (!span_ok(x, x_off, row_bytes * T) || !span_ok(recv, recv_off, row_bytes * cap)) return VR_ERR_INVALID_ARGUMENT;
  if (any_overlap(x, x_off, row_bytes * T, recv, recv_off, row_bytes * cap, R)) return VR_ERR_INVALID_ARGUMENT;
  if (va_touch(x, -1, x_off, row_bytes * T) || va_touch(recv, -1, recv_off, row_bytes * cap))
    return VR_ERR_INVALID_USAGE;
  if (sig_counts >= c->req.signal_count || sig_rows >= c->req.signal_count || sig_counts == sig_rows)
    return VR_ERR_INVALID_ARGUMENT;
  const size_t RT = (size_t)R * T, n4 = sizeof(int32_t);
  if (!dev_span_ok(c, topk, RT * K * n4) || !dev_span_ok(c, counts_out, (size_t)E * n4) ||
      !dev_span_ok(c, src_out, (size_t)R * cap * n4) ||
      (send_pos && !dev_span_ok(c, send_pos, RT * (dedup ? (size_t)R : (size_t)K) * n4)) ||
      (dedup && !dev_span_ok(c, experts_out, (size_t)R * cap * K * n4)))
    return VR_ERR_INVALID_ARGUMENT;
  const bool wait = !(flags & VR_COLL_NO_WAIT);
  U64Tab tc;
  vrResult_t r = inc_targets(c, sig_counts, R, true, &tc);
  if (r != VR_OK) return r;
  for (int d = 0; d < R; ++d)
    if (check_signal_mode(c, d, sig_rows, VR_SIGNAL_ADD) != VR_OK) return VR_ERR_INVALID_USAGE;
  const size_t need = dispatch_scratch_bytes(R, T, dedup ? R : E, dedup ? E : 0);
  char* scr = nullptr;
  if (noalloc) {
    // the GPU's fixed scratch array; nothing is allocated
    if (need > VR_DISPATCH_NOALLOC_SCRATCH_BYTES) return VR_ERR_INVALID_ARGUMENT;
    scr = noalloc_scratch(c->device);
    if (!scr) return VR_ERR_HIP;
  } else {
    r = ensure_scratch(c, need);
    if (r != VR_OK) return r;
    scr = c->scratch;
  }
  r = launch_dispatch(c, x, x_off, row_bytes, topk, T, K, E, recv, recv_off, cap, counts_out, src_out, send_pos,
                      experts_out, dedup, sig_counts, sig_rows, tc, wait, scr, S(stream));
  if (r == VR_OK) {
    commit_inc(c, sig_counts, R);
    for (int d = 0; d < R; ++d) note_signal(c, d, sig_rows, VR_SIGNAL_ADD, 0, false);
  }
  return r;
}

vrResult_t vr_dispatch(vrComm_t c, vrWindow_t x, size_t x_off, size_t row_bytes, const int32_t* topk,
                       int T, int K, int E, vrWindow_t recv, size_t recv_off, size_t cap, int32_t* counts_out,
                       int32_t* src_out, int32_t* send_pos, uint32_t sig_counts, uint32_t sig_rows, uint32_t flags,
                       void* stream) {
  return dispatch_common(c, x, x_off, row_bytes, topk, T, K, E, recv, recv_off, cap, counts_out, src_out, nullptr,
                         send_pos, false, sig_counts, sig_rows, flags, stream);
}

vrResult_t vr_dispatch_noalloc(vrComm_t c, vrWindow_t x, size_t x_off, size_t row_bytes, const int32_t* topk,
                               int T, int K, int E, vrWindow_t recv, size_t recv_off, size_t cap,
                               int32_t* counts_out, int32_t* src_out, int32_t* send_pos, uint32_t sig_counts,
                               uint32_t sig_rows, uint32_t flags, void* stream) {
  return dispatch_common(c, x, x_off, row_bytes, topk, T, K, E, recv, recv_off, cap, counts_out, src_out, nullptr,
                         send_pos, false, sig_counts, sig_rows, flags, stream, true);
}

vrResult_t vr_dispatch_dedup(vrComm_t c, vrWindow_t x, size_t x_off, size_t row_bytes, const int32_t* topk,
                             int T, int K, int E, vrWindow_t recv, size_t recv_off, size_t cap,
                             int32_t* counts_out, int32_t* src_out, int32_t* experts_out, int32_t* send_pos,
                             uint32_t sig_counts, uint32_t sig_rows, uint32_t flags, void* stream) {
  return dispatch_common(c, x, x_off, row_bytes, topk, T, K, E, recv, recv_off, cap, counts_out, src_out,
                         experts_out, send_pos, true, sig_counts, sig_rows, flags, stream);
}

static vrResult_t combine_common(vrComm_t c, vrWindow_t y, size_t y_off, size_t cap, size_t row_bytes, int dtype,
                                 const int32_t* topk, const float* weights, const int32_t* send_pos, int T, int K,
                                 int E, bool dedup, vrWindow_t out, size_t out_off, uint32_t sig, uint32_t flags,
                                 void* stream) {
  if (!live(c) || !has_win(c, y) || !has_win(c, out)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (flags & ~VR_COLL_NO_WAIT) return VR_ERR_INVALID_ARGUMENT;
  const int R = c->nranks;
  if (dtype != VR_DT_F32 && dtype != VR_DT_BF16) return VR_ERR_INVALID_ARGUMENT;
  const size_t es = dtype == VR_DT_F32 ? 4 : 2;
  if (T < 0 || T >= 65536 || K < 1 || K > 64 || E < R || E % R || E > 1024) return VR_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!send_pos || (!dedup && (!topk || !weights)))) return VR_ERR_INVALID_ARGUMENT;
  if (row_bytes == 0 || row_bytes > (size_t(1) << 30) || row_bytes % es || y_off % es || out_off % es)
    return VR_ERR_INVALID_ARGUMENT;
  if (cap > (size_t(1) << 31)) return VR_ERR_INVALID_ARGUMENT;
  if (!span_ok(y, y_off, row_bytes * cap) || !span_ok(out, out_off, row_bytes * T)) return VR_ERR_INVALID_ARGUMENT;
  if (any_overlap(y, y_off, row_bytes * cap, out, out_off, row_bytes * T, R)) return VR_ERR_INVALID_ARGUMENT;
  if (va_touch(y, -1, y_off, row_bytes * cap) || va_touch(out, -1, out_off, row_bytes * T))
    return VR_ERR_INVALID_USAGE;
  const size_t RT = (size_t)R * T;
  if (!dev_span_ok(c, send_pos, RT * (dedup ? (size_t)R : (size_t)K) * sizeof(int32_t)) ||
      (!dedup && (!dev_span_ok(c, topk, RT * K * sizeof(int32_t)) || !dev_span_ok(c, weights, RT * K * sizeof(float)))))
    return VR_ERR_INVALID_ARGUMENT;
  const bool wait = !(flags & VR_COLL_NO_WAIT);
  U64Tab t;
  vrResult_t r = inc_targets(c, sig, R, wait, &t);
  if (r != VR_OK) return r;
  r = launch_combine(c, y, y_off, cap, row_bytes, dtype, topk, weights, send_pos, T, K, E, dedup, out, out_off, sig,
                     t, wait, S(stream));
  if (r == VR_OK) commit_inc(c, sig, R);
  return r;
}

vrResult_t vr_combine(vrComm_t c, vrWindow_t y, size_t y_off, size_t cap, size_t row_bytes, int dtype,
                      const int32_t* topk, const float* weights, const int32_t* send_pos, int T, int K, int E,
                      vrWindow_t out, size_t out_off, uint32_t sig, uint32_t flags, void* stream) {
  return combine_common(c, y, y_off, cap, row_bytes, dtype, topk, weights, send_pos, T, K, E, false, out, out_off,
                        sig, flags, stream);
}

vrResult_t vr_combine_dedup(vrComm_t c, vrWindow_t y, size_t y_off, size_t cap, size_t row_bytes, int dtype,
                            const int32_t* send_pos, int T, vrWindow_t out, size_t out_off, uint32_t sig,
                            uint32_t flags, void* stream) {
  if (!live(c)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  const int R = c->nranks;  // a row per destination rank: K = E = R entries per token
  return combine_common(c, y, y_off, cap, row_bytes, dtype, nullptr, nullptr, send_pos, T, R, R, true, out, out_off,
                        sig, flags, stream);
}

vrResult_t vr_ring_exchange(vrComm_t c, vrWindow_t send, vrWindow_t recv, size_t put_bytes, size_t puts_per_rank,
                            int contexts, uint32_t sig_base, uint32_t cnt_base, vrWindow_t sig_window,
                            size_t sig_window_off, uint64_t* litmus, uint32_t flags, void* stream) {
  if (!live(c) || !has_win(c, send) || !has_win(c, recv)) return VR_ERR_INVALID_ARGUMENT;
  if (!on_device(c)) return VR_ERR_INVALID_USAGE;
  if (flags & ~(VR_COLL_NO_WAIT | VR_RING_WEAK)) return VR_ERR_INVALID_ARGUMENT;
  if (litmus && !dev_span_ok(c, litmus, 2 * sizeof(uint64_t))) return VR_ERR_INVALID_ARGUMENT;
  const int R = c->nranks;
  if (contexts < 1 || (uint32_t)contexts > c->req.context_count) return VR_ERR_INVALID_ARGUMENT;
  if (put_bytes == 0 || put_bytes % 16 || put_bytes > 65536) return VR_ERR_INVALID_ARGUMENT;
  if (puts_per_rank == 0 || puts_per_rank % contexts || puts_per_rank > (size_t(1) << 32))
    return VR_ERR_INVALID_ARGUMENT;
  if ((uint64_t)cnt_base + contexts > c->req.counter_count) return VR_ERR_INVALID_ARGUMENT;
  const bool va = sig_window != nullptr;
  if (!va && (uint64_t)sig_base + contexts > c->req.signal_count) return VR_ERR_INVALID_ARGUMENT;
  const size_t n = put_bytes * puts_per_rank;
  if (!span_ok(send, 0, n) || !span_ok(recv, 0, n)) return VR_ERR_INVALID_ARGUMENT;
  if (any_overlap(send, 0, n, recv, 0, n, R)) return VR_ERR_INVALID_ARGUMENT;
  if (va_touch(send, -1, 0, n) || va_touch(recv, -1, 0, n)) return VR_ERR_INVALID_USAGE;
  const uint64_t per_ctx = puts_per_rank / contexts;
  uint64_t* ctx0[VR_MAX_RANKS];
  if (va) {
    // one VA signal word per context, consecutive, in every rank's slice
    vrResult_t r = check_va_word(c, sig_window, sig_window_off);
    if (r != VR_OK) return r;
    if (!span_ok(sig_window, sig_window_off, (size_t)8 * contexts)) return VR_ERR_INVALID_ARGUMENT;
    if ((sig_window == send && any_overlap(send, 0, n, sig_window, sig_window_off, (size_t)8 * contexts, R)) ||
        (sig_window == recv && any_overlap(recv, 0, n, sig_window, sig_window_off, (size_t)8 * contexts, R)))
      return VR_ERR_INVALID_USAGE;  // the messages would move the signal words' own bytes
    for (int d = 0; d < R; ++d) {
      for (int k = 0; k < contexts; ++k) {
        const auto it = sig_window->va_words.find({d, sig_window_off + 8ull * k});
        if (it != sig_window->va_words.end() && it->second == 2) return VR_ERR_INVALID_USAGE;
      }
      ctx0[d] = reinterpret_cast<uint64_t*>(sig_window->base[d] + sig_window_off);
    }
    for (int d = 0; d < R; ++d)
      for (int k = 0; k < contexts; ++k)
        if (vrResult_t e = va_reserve(sig_window, d, sig_window_off + 8ull * k)) return e;
  } else {
    for (int d = 0; d < R; ++d) {
      for (int k = 0; k < contexts; ++k)
        if (check_signal_mode(c, d, sig_base + k, VR_SIGNAL_INC) != VR_OK) return VR_ERR_INVALID_USAGE;
      ctx0[d] = c->sig + sidx(c, d, sig_base);
    }
  }
  const bool wait = !(flags & VR_COLL_NO_WAIT);
  vrResult_t r = launch_ring(c, send, recv, put_bytes, puts_per_rank, contexts, ctx0, cnt_base, wait,
                             (flags & VR_RING_WEAK) != 0, litmus, S(stream));
  if (r == VR_OK)
    for (int d = 0; d < R; ++d)
      for (int k = 0; k < contexts; ++k) {
        if (va) sig_window->va_words[{d, sig_window_off + 8ull * k}] = 1;
        else note_signal(c, d, sig_base + k, VR_SIGNAL_INC, per_ctx, true);
      }
  return r;
}

}  // extern "C"
