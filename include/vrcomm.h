/*
 * vrcomm.h -- one-sided window put/get with integer signals and counters,
 * and the collectives built on them, for R virtual ranks that share one
 * AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by page and section (the pages are not reproduced here):
 *   GIN page         NCCL GIN device API walkthrough, lpnh.cn/news/2681042
 *   Symmetric page   NCCL symmetric-memory examples, zwxr.cn/news/250719
 *   GDA survey       "GPUDirect Async" survey, 10100.com/article/158785524
 *
 * Model. A communicator (vrComm_t) holds R virtual ranks on the current HIP
 * device. Each rank owns a slice of every registered window: R device
 * pointers, one per rank, all of the same size ("symmetric": one offset names
 * the same slot on every rank). Every rank can address every other rank's
 * slices directly (on one GPU all memory is load/store accessible), so a put
 * or get is a copy performed by GPU workgroups, and a signal is an atomic add
 * at agent scope on a 64-bit word owned by the receiving rank.
 *
 * Conventions (every function):
 *   - Returns a vrResult_t; nothing throws across this interface.
 *   - Argument errors are reported synchronously, before anything is
 *     enqueued, and leave the communicator unchanged.
 *   - Errors found by device code (a wait that timed out, a dispatch that
 *     overflowed its receive capacity, an expert id out of range, a litmus
 *     violation) set bits in the communicator's device error word; read them
 *     with vr_comm_get_async_error after synchronizing the stream.
 *   - Memory: windows, inputs and outputs are owned by the caller; the
 *     library owns only its signal/counter words and small scratch buffers.
 *     The dispatch scratch (count rows, block prefixes: about
 *     R*(T/64)*E*4 bytes) is grown on the first vr_dispatch or
 *     vr_dispatch_dedup that needs more than any call before it on the
 *     communicator: that call synchronizes the device, frees the old buffer
 *     and allocates (hipMalloc) before enqueuing. Later calls of that size or
 *     smaller allocate nothing, so a caller that must not allocate (graph
 *     capture, a serving loop) makes one call of its largest shape first, or
 *     uses vr_dispatch_noalloc. Every other operation allocates nothing.
 *   - Device pointers are plain device addresses on the communicator's device.
 *     Array arguments (routing ids, weights, positions, counts, tags, the
 *     litmus words) must lie, for their whole stated size, inside one device
 *     allocation on that device; a host pointer, a buffer on another device or
 *     a span that runs past the end of its allocation is
 *     VR_ERR_INVALID_ARGUMENT. (A buffer carved from a larger allocation, as
 *     torch's caching allocator does, is only checked against that
 *     allocation.)
 *     A stream is a hipStream_t passed as void* (NULL = the null stream).
 *   - A communicator is not thread-safe, and the operations issued on one
 *     communicator must execute in issue order: use one stream per
 *     communicator, or order the streams yourself. Operations that share a
 *     signal id must be stream-ordered.
 *   - HIP graphs: an operation whose kernel waits in-kernel takes the
 *     signal's target from the library's expected value when it is enqueued,
 *     so a captured call keeps that target on every replay, and from the
 *     second replay on its waits would find it already reached. Capture a
 *     vr_signal_reset of the signal at every rank (a kernel, not a memset)
 *     before the operation, so that every replay starts from 0 and waits for
 *     exactly its own signals; or capture with VR_COLL_NO_WAIT.
 *   - Device: a communicator lives on the device current at vr_comm_create.
 *     Every later call but vr_comm_destroy must be made with that device
 *     current, else it returns VR_ERR_INVALID_USAGE and does nothing;
 *     vr_comm_destroy selects the device itself and restores the caller's.
 */
#ifndef VRCOMM_H
#define VRCOMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- result codes ---------------------------------------------------------- */
typedef int vrResult_t;
#define VR_OK                      0
#define VR_ERR_INVALID_ARGUMENT    1  /* a value is out of range, misaligned or NULL */
#define VR_ERR_INVALID_USAGE       2  /* legal values, but the call breaks a usage rule */
#define VR_ERR_OUT_OF_RESOURCES    3  /* allocation failed, or a dispatch overflowed (async) */
#define VR_ERR_HIP                 4  /* a HIP runtime call failed */
#define VR_ERR_TIMEOUT             5  /* a device-side wait gave up (async) */
#define VR_ERR_UNSUPPORTED_DEVICE  6  /* the current device is not gfx950 */
#define VR_ERR_INTERNAL            7
#define VR_ERR_DEVICE_CHECK        8  /* a device-side check failed (async): bad expert id, litmus */

/* Human-readable name of a result code. Never NULL. */
const char* vr_error_string(vrResult_t r);

/* Library version as major*10000 + minor*100 + patch. */
int vr_version(void);

/* ---- limits and flags --------------------------------------------------------- */
#define VR_MAX_RANKS               64
#define VR_WIN_DEFAULT             0x00u
#define VR_WIN_COLL_SYMMETRIC      0x01u  /* Symmetric page, window registration flags */
#define VR_WIN_STRICT_ORDERING     0x02u
#define VR_WIN_REQUIRED_ALIGNMENT  4096u  /* Symmetric page: required window alignment */
#define VR_SIGNAL_BITS             64
#define VR_COUNTER_BITS            56     /* GIN page, counter methods: at most 56 bits */

/* ---- handles and requirement records ------------------------------------------- */
typedef struct vrComm* vrComm_t;
typedef struct vrWindow* vrWindow_t;

/* Resources a communicator provides to each rank (GIN page, host-side setup of
 * the AlltoAll example: signal and barrier counts requested up front).
 * signal_count   signals per rank (ids 0..signal_count-1), 1..65536
 * counter_count  counters per rank, 0..65536
 * context_count  ordering contexts per rank, 1..1024 (GIN page, ncclGin:
 *                several contexts spread traffic; a context orders the puts
 *                of the one issuer that owns it)
 * barrier_count  barrier-session slots shared by the ranks, 0..65536 (GIN
 *                page, ncclGinBarrierSession: one slot per cooperating group
 *                that syncs). */
typedef struct {
  uint32_t signal_count;
  uint32_t counter_count;
  uint32_t context_count;
  uint32_t barrier_count;
} vrCommRequirements;

/* Fence levels of a barrier-session sync (GIN page, sync and fence levels):
 * bit flags, combined with |. */
#define VR_FENCE_NONE  0x0u  /* pure synchronization */
#define VR_FENCE_PUT   0x1u  /* puts other members issued before the sync, aimed at the caller, are visible */
#define VR_FENCE_GET   0x2u  /* gets the caller issued before the sync have landed */

/* Device views for kernels written against include/vrcomm_device.hpp: plain
 * structs passed by value. Pointers are device addresses owned by the
 * communicator or the window and valid until it is destroyed / deregistered. */
typedef struct {
  int nranks;
  uint32_t signal_count, counter_count, barrier_count;
  uint64_t* signals;   /* [nranks][signal_count] */
  uint64_t* counters;  /* [nranks][counter_count] */
  uint64_t* barriers;  /* [barrier_count] */
  uint32_t* error;     /* VR_ASYNC_* bits */
} vrDevComm;
typedef struct {
  char* base[VR_MAX_RANKS];  /* rank r's slice (NULL past nranks) */
  uint64_t bytes;
} vrDevWindow;

/* Remote action, applied at the peer after the put's payload has landed
 * (GIN page, one-sided transfers and signals and counters).
 *   kind  VR_ACTION_NONE, VR_SIGNAL_INC (add 1) or VR_SIGNAL_ADD (add value)
 *         on signal `id`; or VR_VA_SIGNAL_INC / VR_VA_SIGNAL_ADD on the VA
 *         signal at (window, offset) (GIN page, VA signals)
 *   id    signal id at the peer (id signals)
 *   strong nonzero: the signal also covers every earlier put of the same
 *         context to the same peer (GIN page, strong and weak signals). This
 *         library always publishes a signal after all earlier stores of the
 *         issuing context, so weak signals get the strong guarantee too.
 *   window, offset  VA signals: the signal is the little-endian uint64 at
 *         byte `offset` (a multiple of 8) of the peer's slice of `window`,
 *         which must be registered with VR_WIN_STRICT_ORDERING
 *         (VR_ERR_INVALID_USAGE otherwise). Once a word has served as a VA
 *         signal (action, wait, read or reset), puts, gets and collectives
 *         whose data ranges touch it are refused with VR_ERR_INVALID_USAGE:
 *         the word is accessed by signal operations only. NULL / 0 for id
 *         signals.
 * A signal must not receive both SignalInc and SignalAdd without a reset in
 * between (GIN page, strong and weak signals); the library rejects such a
 * call with VR_ERR_INVALID_USAGE. */
#define VR_ACTION_NONE     0u
#define VR_SIGNAL_INC      1u
#define VR_SIGNAL_ADD      2u
#define VR_COUNTER_INC     3u
#define VR_VA_SIGNAL_INC   4u
#define VR_VA_SIGNAL_ADD   5u
typedef struct {
  uint32_t kind;
  uint32_t id;
  uint64_t value;
  uint32_t strong;
  uint32_t reserved;  /* must be 0 */
  vrWindow_t window;  /* VA signals only */
  uint64_t offset;    /* VA signals only */
} vrRemoteAction;

/* Local action, applied at the issuing rank once the source bytes have been
 * read (GIN page, counter methods): kind VR_ACTION_NONE or VR_COUNTER_INC. */
typedef struct {
  uint32_t kind;
  uint32_t id;
} vrLocalAction;

/* ---- communicator ---------------------------------------------------------------- */
/* Device bytes a communicator needs for its signal and counter words, error
 * word and relay counters; 0 on invalid arguments. */
size_t vr_comm_workspace_bytes(int nranks, const vrCommRequirements* req);

/* Create a communicator of nranks (1..VR_MAX_RANKS) virtual ranks on the
 * current HIP device. workspace: caller-owned device memory of at least
 * vr_comm_workspace_bytes() bytes, 256-byte aligned, or NULL to let the
 * library allocate it. The words are zeroed (synchronously) before return.
 * Errors: VR_ERR_INVALID_ARGUMENT, VR_ERR_UNSUPPORTED_DEVICE (not gfx950; the
 * analog of a device communicator that cannot be created, GIN page, host-side
 * setup), VR_ERR_HIP, VR_ERR_OUT_OF_RESOURCES. */
vrResult_t vr_comm_create(int nranks, const vrCommRequirements* req, void* workspace,
                          size_t workspace_bytes, vrComm_t* out);

/* Destroy a communicator. VR_ERR_INVALID_USAGE while windows are still
 * registered (Symmetric page, example 1 step 7: deregister windows, then free
 * memory, then destroy the communicator). Synchronizes the device. */
vrResult_t vr_comm_destroy(vrComm_t comm);

/* Read and clear the device error word. Synchronize the streams that ran the
 * communicator's work first. *out is VR_OK, or the code of the first set bit
 * in the order TIMEOUT, OUT_OF_RESOURCES, DEVICE_CHECK. *bits (may be NULL)
 * receives the raw bit set. */
#define VR_ASYNC_TIMEOUT       0x1u
#define VR_ASYNC_CAPACITY      0x2u
#define VR_ASYNC_BAD_EXPERT    0x4u
#define VR_ASYNC_LITMUS        0x8u
vrResult_t vr_comm_get_async_error(vrComm_t comm, vrResult_t* out, uint32_t* bits);

/* Strong-signal litmus for the collectives (GIN page, strong and weak
 * signals: a signal seen at the peer means every earlier put of the context to
 * that peer is visible there). litmus: device uint64[2] or NULL (off, the
 * default). While it is set, the receivers of later vr_allreduce,
 * vr_alltoall, vr_allgather (compute-unit paths), vr_dispatch,
 * vr_dispatch_noalloc and vr_dispatch_dedup calls on the communicator check,
 * inside the kernel, right after their wait on the completion signal has ended
 * and they have acquired, that what the signal announced is visible: first,
 * whole, the piece (tile, slab or row) that the workgroup completing each
 * relay stored last, which it records before applying the signal; then one
 * seeded sample in every tile (every received row for the dispatch), each
 * against the senders' windows (for the AllReduce, the rank-order sum
 * recomputed from the send windows; for the dispatch, the token row named by
 * the row's source tag). litmus[0] counts the checks and litmus[1] the
 * mismatches; a mismatch also sets VR_ASYNC_LITMUS. The checks lengthen the
 * receivers' part of the kernel; calls with VR_COLL_NO_WAIT have no receivers
 * and check nothing. */
vrResult_t vr_comm_set_litmus(vrComm_t comm, uint64_t* litmus);

/* Phase timeline of the dispatch (a measuring aid: where the time of the
 * count exchange, the offsets and the row copies goes). stamps: device
 * uint64[words] or NULL (off, the default). While it is set, every workgroup
 * of a vr_dispatch, vr_dispatch_noalloc or vr_dispatch_dedup kernel writes the
 * device real-time clock (ns) at its phase boundaries into
 * stamps[w * 8 + phase], w its index in the grid -- the count workgroups
 * (R * ceil(T / 256), source-interleaved), then the put workgroups
 * (R * 4 * ceil(T / 256)), then the R receivers; words past `words` are not
 * written, and phases a workgroup does not reach keep their old value.
 * Count workgroup: 0 start, 1 histograms stored, 2 count row published (the
 * source's last block only). Put workgroup: 0 start, 1 entries ranked and
 * token-row loads issued, 2 count signal seen, 3 count rows loaded and
 * offsets computed, 4 source tags stored, 5 row stores issued, 6 row stores
 * complete, 7 row signals applied (the source's last block only). Receiver:
 * 0 start, 1 count signal seen, 2 row signal seen. */
vrResult_t vr_comm_set_trace(vrComm_t comm, uint64_t* stamps, size_t words);

/* Rank count and requirements of a communicator. */
vrResult_t vr_comm_query(vrComm_t comm, int* nranks, vrCommRequirements* req);

/* ---- windows ------------------------------------------------------------------------ */
/* Register a symmetric window: bases[r] is rank r's slice (device memory on
 * the communicator's device, VR_WIN_REQUIRED_ALIGNMENT-aligned, bytes long);
 * the R slices must not overlap. flags: VR_WIN_* bits. The memory stays owned
 * by the caller and must outlive the registration (Symmetric page, window
 * registration and cleanup order). Slices that start on 2 MiB boundaries run
 * the bandwidth-bound collectives fastest (slices offset by 4 KiB from them
 * measured up to 10 % slower). */
vrResult_t vr_window_register(vrComm_t comm, void* const* bases, size_t bytes, uint32_t flags,
                              vrWindow_t* out);

/* Deregister a window; must precede freeing its memory. Synchronizes the device. */
vrResult_t vr_window_deregister(vrComm_t comm, vrWindow_t win);

/* ---- one-sided primitives (each enqueues one kernel on the stream) --------------------- */
/* put: copy bytes from src (rank's slice, at src_off) to dst (peer's slice, at
 * dst_off), then apply the remote action at the peer and the local action at
 * the rank (GIN page, one-sided transfers: put). peer may equal rank
 * (loopback); when the source and destination bytes overlap in memory the
 * copy behaves like memmove (one workgroup copies in the safe direction).
 * bytes may be 0 (actions only). ctx < context_count. Offsets and sizes are
 * checked against the window size (VR_ERR_INVALID_ARGUMENT). */
vrResult_t vr_put(vrComm_t comm, int ctx, int rank, int peer, vrWindow_t dst, size_t dst_off,
                  vrWindow_t src, size_t src_off, size_t bytes, vrRemoteAction remote,
                  vrLocalAction local, void* stream);

/* get: copy bytes from remote (peer's slice, at remote_off) into local (rank's
 * slice, at local_off); the local action runs once the bytes have landed
 * (GIN page, one-sided transfers: get; completion management: flush). */
vrResult_t vr_get(vrComm_t comm, int ctx, int rank, int peer, vrWindow_t remote, size_t remote_off,
                  vrWindow_t local, size_t local_off, size_t bytes, vrLocalAction local_action,
                  void* stream);

/* signal: a remote action with no payload (GIN page, signal methods). */
vrResult_t vr_signal(vrComm_t comm, int ctx, int rank, int peer, vrRemoteAction remote, void* stream);

/* Wait on the stream until the low `bits` bits of rank's signal id reach
 * `least` in rolling (wrap-around) order: value - least, taken modulo
 * 2^bits, is below 2^(bits-1) (GIN page, signals and counters: rolling
 * comparison; signal methods: waitSignal). timeout_ns: give up after this
 * long and set VR_ASYNC_TIMEOUT (0 = 5 s). bits in 1..64. */
vrResult_t vr_signal_wait(vrComm_t comm, int rank, uint32_t id, uint64_t least, int bits,
                          uint64_t timeout_ns, void* stream);

/* VA signals (GIN page, VA signals): wait on, read or reset the uint64 word
 * at byte `offset` (a multiple of 8) of rank's slice of `win`, a window
 * registered with VR_WIN_STRICT_ORDERING (VR_ERR_INVALID_USAGE otherwise).
 * Semantics as vr_signal_wait / vr_signal_read / vr_signal_reset; the word
 * counts as a signal from then on (see vrRemoteAction). */
vrResult_t vr_va_signal_wait(vrComm_t comm, vrWindow_t win, int rank, size_t offset, uint64_t least,
                             int bits, uint64_t timeout_ns, void* stream);
vrResult_t vr_va_signal_read(vrComm_t comm, vrWindow_t win, int rank, size_t offset, int bits,
                             uint64_t* out);
vrResult_t vr_va_signal_reset(vrComm_t comm, vrWindow_t win, int rank, size_t offset, void* stream);

/* ---- barrier sessions and device views ---------------------------------------------- */
/* Fill the device views of a communicator and of one of its windows. */
vrResult_t vr_comm_device_view(vrComm_t comm, vrDevComm* out);
vrResult_t vr_window_device_view(vrComm_t comm, vrWindow_t win, vrDevWindow* out);

/* The value barrier slot `index` will hold once every operation enqueued so
 * far has run (every sync of a session adds its member count). A kernel that
 * syncs k times on the slot with m members targets base + m, ..., base + k*m;
 * vr_barrier_advance records those arrivals on the host. */
vrResult_t vr_barrier_expected(vrComm_t comm, uint32_t index, uint64_t* out);
vrResult_t vr_barrier_advance(vrComm_t comm, uint32_t index, uint64_t arrivals);

/* One sync of the R ranks on barrier slot `index` (GIN page,
 * ncclGinBarrierSession::sync), enqueued on the stream: one workgroup per
 * rank arrives, with the drains `fence` asks for, and waits for the others.
 * timeout_ns as vr_signal_wait. */
vrResult_t vr_barrier(vrComm_t comm, uint32_t index, uint32_t fence, uint64_t timeout_ns, void* stream);

/* Read the low `bits` bits of a signal now (synchronous device read; the
 * caller synchronizes the stream that modified it). */
vrResult_t vr_signal_read(vrComm_t comm, int rank, uint32_t id, int bits, uint64_t* out);

/* Reset a signal to 0 on the stream. Must not race with updates of the same
 * signal (GIN page, signal methods: resetSignal). Also clears its Inc/Add mode. */
vrResult_t vr_signal_reset(vrComm_t comm, int rank, uint32_t id, void* stream);

/* The value a signal will hold once every operation enqueued so far has run,
 * as tracked by the host (the library's counterpart of the pages' per-signal
 * shadow value, GIN page, signal methods). VR_ERR_INVALID_USAGE when an
 * enqueued operation added a device-computed amount (vr_dispatch's row
 * signal) and no reset followed. */
vrResult_t vr_signal_expected(vrComm_t comm, int rank, uint32_t id, uint64_t* out);

/* Counters: as the signal calls, with at most 56 bits (GIN page, counter methods). */
vrResult_t vr_counter_wait(vrComm_t comm, int rank, uint32_t id, uint64_t least, int bits,
                           uint64_t timeout_ns, void* stream);
vrResult_t vr_counter_read(vrComm_t comm, int rank, uint32_t id, int bits, uint64_t* out);
vrResult_t vr_counter_reset(vrComm_t comm, int rank, uint32_t id, void* stream);

/* ---- collectives (all R ranks in one call, stream-ordered) ------------------------------ */
#define VR_DT_F32   0
#define VR_DT_BF16  1
#define VR_OP_SUM   0
/* flags */
#define VR_COLL_NO_WAIT      0x1u  /* skip the in-kernel receiver waits (signals are still applied) */
/* vr_alltoall and vr_allgather: move the bytes with the copy engines (SDMA)
 * instead of compute units (Symmetric page, AllGather with the copy engine),
 * one copy per (s, d) spread over VR_CE_STREAMS internal streams that fork
 * from and join back into the caller's stream; then one kernel applies the
 * SignalIncs (each rank's signal rises by R) and, unless VR_COLL_NO_WAIT,
 * the receivers' waits. Offsets and sizes need no alignment. */
#define VR_COLL_COPY_ENGINE  0x4u
#define VR_CE_STREAMS        8
/* vr_ring_exchange only: weak SignalIncs (see there) */
#define VR_RING_WEAK         0x8u
/* vr_signal_pingpong only: rank 1's workgroup on rank 0's XCD */
#define VR_PINGPONG_SAME_XCD 0x10u
/* vr_signal_pingpong only: ranks 0 and 1 are the two waves of one workgroup */
#define VR_PINGPONG_WAVES    0x20u

/* Sum-AllReduce over `count` elements at send_off of every rank's send slice;
 * every rank's recv slice receives the sum at recv_off.
 * Result, per element: ((x_0 + x_1) + x_2) + ... + x_{R-1}, each addition an
 * IEEE binary32 addition rounded to nearest even (fixed rank order; the pages
 * fix no order). VR_DT_BF16: bf16 inputs widened exactly, fp32 accumulation,
 * bf16 output rounded to nearest even; any NaN becomes 0x7FC0.
 * Method: reduce-scatter, each owner pulling its chunk from every rank (get),
 * then all-gather, the owner putting the reduced chunk to every rank, with one
 * SignalInc on `sig` per (owner, receiver): every rank's signal rises by R.
 * Unless VR_COLL_NO_WAIT, each receiver waits in-kernel for its signal.
 * Symmetric page, AllReduce example; GIN page, put/get and signals.
 * Offsets must be multiples of the element size; send and recv ranges must
 * not overlap (VR_ERR_INVALID_ARGUMENT). */
vrResult_t vr_allreduce(vrComm_t comm, vrWindow_t send, size_t send_off, vrWindow_t recv,
                        size_t recv_off, size_t count, int dtype, int op, uint32_t sig,
                        uint32_t flags, void* stream);

/* Equal-block AlltoAll: block d of rank s's send slice (at send_off +
 * d*block_bytes) lands in rank d's recv slice at recv_off + s*block_bytes,
 * as one put per (s, d) with a SignalInc on `sig` at d: every rank's signal
 * rises by R, its own loopback block included (GIN page, pure-GIN AlltoAll
 * kernel). */
vrResult_t vr_alltoall(vrComm_t comm, vrWindow_t send, size_t send_off, vrWindow_t recv,
                       size_t recv_off, size_t block_bytes, uint32_t sig, uint32_t flags,
                       void* stream);

/* The pure-GIN AlltoAll kernel's structure (GIN page, the AlltoAll example),
 * written with include/vrcomm_device.hpp: every rank enters through a
 * barrier-session sync on slot `barrier_index` (VR_FENCE_NONE), puts its
 * blocks with a weak SignalInc on `sig` at each destination, waits until its
 * own signal has risen by R, and leaves through a second sync. Same result
 * and signal totals as vr_alltoall; the slot advances by 2R. */
vrResult_t vr_alltoall_sessions(vrComm_t comm, vrWindow_t send, size_t send_off, vrWindow_t recv,
                                size_t recv_off, size_t block_bytes, uint32_t sig, uint32_t barrier_index,
                                uint32_t flags, void* stream);

/* AllGather: rank s's bytes_per_rank bytes at send_off land in every rank's
 * recv slice at recv_off + s*bytes_per_rank, one put + SignalInc per (s, d)
 * (Symmetric page, AllGather example: segment k holds rank k's data). */
vrResult_t vr_allgather(vrComm_t comm, vrWindow_t send, size_t send_off, vrWindow_t recv,
                        size_t recv_off, size_t bytes_per_rank, uint32_t sig, uint32_t flags,
                        void* stream);

/* MoE token dispatch (GDA survey, opening section: tokens of a few hundred
 * bytes routed among dozens of experts).
 *   x, x_off        rank s's T token rows of row_bytes bytes each (window)
 *   topk_idx        device int32 [R][T][K]: expert ids in [0, num_experts),
 *                   or -1 for "not routed"; K in 1..64; may be NULL when T == 0
 *   num_experts     multiple of R, at most 1024; rank d owns experts
 *                   [d*E/R, (d+1)*E/R)
 *   recv, recv_off  rank d's receive rows (window), capacity recv_capacity_rows
 *   recv_expert_counts  device int32 [R][E/R]: rows received per local expert
 *   recv_src        device int32 [R][recv_capacity_rows]: (s << 16) | t per row
 *   send_pos        device int32 [R][T][K] or NULL: the receive row of every
 *                   routing entry at rank expert/(E/R), -1 for entries that are
 *                   not routed or whose row fell past the capacity (the
 *                   metadata vr_combine uses to find the rows again)
 * Layout of rank d's rows: by expert, then source rank, then token (a stable
 * sort of the routing entries on (expert, source, token)). A token whose
 * top-k names one expert more than once sends one row per entry, in k order
 * (reading; the pages do not say), and the counts and the row signal count
 * entries.
 * Method: (1) each rank counts its tokens per expert and puts its count row
 * to every rank with a SignalInc on sig_counts (each rises by R); (2) every
 * rank computes its offsets from the full count matrix; (3) each rank puts
 * every expert's rows, then one strong SignalAdd(rows sent to d) on
 * sig_rows at each d (GDA survey, section 4: a batch of puts closed by one
 * signal). Unless VR_COLL_NO_WAIT, each receiver waits in-kernel until
 * sig_rows has grown by the rows aimed at it. Rows past the capacity are
 * dropped and set VR_ASYNC_CAPACITY; out-of-range ids set VR_ASYNC_BAD_EXPERT.
 * T < 65536; row_bytes > 0; sig_counts != sig_rows. */
vrResult_t vr_dispatch(vrComm_t comm, vrWindow_t x, size_t x_off, size_t row_bytes,
                       const int32_t* topk_idx, int T, int K, int num_experts, vrWindow_t recv,
                       size_t recv_off, size_t recv_capacity_rows, int32_t* recv_expert_counts,
                       int32_t* recv_src, int32_t* send_pos, uint32_t sig_counts, uint32_t sig_rows,
                       uint32_t flags, void* stream);

/* vr_dispatch without any allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Arguments, results, signals and device checks are those of
 * vr_dispatch. Its scratch (count rows, block prefixes) is not the
 * communicator's growable buffer but a fixed array of
 * VR_DISPATCH_NOALLOC_SCRATCH_BYTES in the library's code object, one copy per
 * GPU, held until the process ends; the call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine). Every call on one GPU shares that
 * GPU's array, whatever its communicator: calls whose executions overlap on
 * one GPU (other streams, other communicators) race on it and must be
 * stream-ordered; each call writes every scratch word it reads, so nothing
 * needs clearing between calls. Limit: with NB = max(1, ceil(T / 256)), the
 * scratch R*NB*E*16 + R*NB*E*4 + R*R*E*4 + R*8 + R*4 bytes (each term rounded
 * up to a multiple of 256) must not exceed VR_DISPATCH_NOALLOC_SCRATCH_BYTES
 * (R = 8, E = 256: up to 25,600 tokens per rank); larger shapes return
 * VR_ERR_INVALID_ARGUMENT before anything is enqueued. In a replayed graph,
 * capture a vr_signal_reset of sig_counts and of sig_rows at every rank
 * before it: the count target then holds on every replay, and each
 * receiver's row target is taken on the device, so every replay may route
 * differently. */
#define VR_DISPATCH_NOALLOC_SCRATCH_BYTES (4u << 20)
vrResult_t vr_dispatch_noalloc(vrComm_t comm, vrWindow_t x, size_t x_off, size_t row_bytes,
                               const int32_t* topk_idx, int T, int K, int num_experts, vrWindow_t recv,
                               size_t recv_off, size_t recv_capacity_rows, int32_t* recv_expert_counts,
                               int32_t* recv_src, int32_t* send_pos, uint32_t sig_counts, uint32_t sig_rows,
                               uint32_t flags, void* stream);

/* MoE dispatch in the per-rank (dedup) layout (reading: the GDA survey's
 * dispatch, sending each token once to every rank that owns at least one of
 * its experts instead of once per expert). Rank d's rows are ordered by
 * source rank, then token; row i carries recv_src[d][i] = (s << 16) | t and
 * recv_experts[d][i][k] (device int32 [R][cap][K]) = the local expert index
 * of the token's entry k when that expert lives on d, else -1.
 * recv_expert_counts[d][j] counts the routing entries naming local expert j
 * (as vr_dispatch). send_pos (device int32 [R][T][R] or NULL): the row of
 * token (s, t) at each rank d, -1 where it is not sent (or fell past the
 * capacity). Count exchange, signals (sig_counts rises by R, sig_rows by the
 * rows aimed at each rank), checks and limits as vr_dispatch. */
vrResult_t vr_dispatch_dedup(vrComm_t comm, vrWindow_t x, size_t x_off, size_t row_bytes,
                             const int32_t* topk_idx, int T, int K, int num_experts, vrWindow_t recv,
                             size_t recv_off, size_t recv_capacity_rows, int32_t* recv_expert_counts,
                             int32_t* recv_src, int32_t* recv_experts, int32_t* send_pos, uint32_t sig_counts,
                             uint32_t sig_rows, uint32_t flags, void* stream);

/* Combine in the per-rank layout: every rank d holds one row per token it
 * received (its experts' outputs for that token, already mixed there), at
 * the row vr_dispatch_dedup placed it (send_pos, [R][T][R]). For each source s
 * and token t: acc = +0.0, then for d = 0..R-1 with send_pos[s][t][d] != -1,
 * acc = acc + y[d][send_pos[s][t][d]] (binary32 additions in rank order);
 * bf16 rows widened exactly, the result rounded to bf16 (RNE). Gets,
 * completion signal (each rank's `sig` rises by R), waits and checks as
 * vr_combine. */
vrResult_t vr_combine_dedup(vrComm_t comm, vrWindow_t y, size_t y_off, size_t y_capacity_rows,
                            size_t row_bytes, int dtype, const int32_t* send_pos, int T, vrWindow_t out,
                            size_t out_off, uint32_t sig, uint32_t flags, void* stream);

/* MoE combine, the inverse of vr_dispatch (reading: the GDA survey's opening
 * section describes the dispatch; its other half brings every expert output
 * back to the token's rank and mixes the K of them with the router weights).
 *   y, y_off        rank d's expert-output rows (window), y_capacity_rows of
 *                   row_bytes each, in the dispatch's receive layout: the row
 *                   for routing entry (s, t, k) is at send_pos[s][t][k]
 *   dtype           VR_DT_BF16 (rows of bf16) or VR_DT_F32
 *   topk_idx        device int32 [R][T][K], the routing given to vr_dispatch
 *   weights         device float [R][T][K], router weights
 *   send_pos        device int32 [R][T][K], as vr_dispatch wrote it
 *   out, out_off    rank s's T combined rows (window), row_bytes each
 * For each source s and token t: acc = +0.0, then for k = 0..K-1 in order,
 * for entries with a row (expert id and position not -1),
 * acc = acc + weights[s][t][k] * y[d][send_pos[s][t][k]] with d = expert / (E/R),
 * every product and sum rounded to binary32 (no fused multiply-add); bf16
 * rows are widened exactly and the result rounded to bf16 (RNE, NaN ->
 * 0x7FC0). Each row is read once with a get (GIN page, one-sided transfers);
 * once source s has read all its rows it applies a SignalInc on `sig` at
 * every rank d, so each rank's signal rises by R, and unless VR_COLL_NO_WAIT
 * each rank waits in-kernel for that (its rows may then be overwritten).
 * Device checks: an expert id outside [-1, E) sets VR_ASYNC_BAD_EXPERT, a
 * position outside [-1, y_capacity_rows) sets VR_ASYNC_CAPACITY; either entry
 * is skipped. row_bytes and both offsets must be multiples of the element
 * size; T < 65536, K in 1..64, num_experts a multiple of R up to 1024; the y
 * and out ranges must not overlap (VR_ERR_INVALID_ARGUMENT). */
vrResult_t vr_combine(vrComm_t comm, vrWindow_t y, size_t y_off, size_t y_capacity_rows,
                      size_t row_bytes, int dtype, const int32_t* topk_idx, const float* weights,
                      const int32_t* send_pos, int T, int K, int num_experts, vrWindow_t out,
                      size_t out_off, uint32_t sig, uint32_t flags, void* stream);

/* Ring exchange (GDA survey, section 4, the ring-exchange example): rank r
 * puts puts_per_rank messages of put_bytes each to rank (r+1) mod R, message
 * k from send offset k*put_bytes to recv offset k*put_bytes. Messages are
 * split into `contexts` contiguous ranges, each issued in order by one
 * workgroup; every message carries a strong SignalInc on signal
 * sig_base + ctx at the receiver (or, when sig_window is not NULL, on the
 * VA signal at sig_window_off + 8*ctx of the receiver's slice of
 * sig_window, a VR_WIN_STRICT_ORDERING window; sig_base is then unused) and
 * a CounterInc on counter cnt_base + ctx at the sender. Receivers wait in-kernel until each context signal has
 * grown by puts_per_rank / contexts. litmus (device uint64[2] or NULL): when
 * given, the waiting wavefronts repeatedly read a context signal v and check
 * that messages v-1 and an earlier one are visible, counting checks in
 * litmus[0] and violations in litmus[1] (and VR_ASYNC_LITMUS).
 * flags: VR_COLL_NO_WAIT, and VR_RING_WEAK: the SignalIncs are weak (GIN
 * page, strong and weak signals: each is ordered after its own put only),
 * so the library publishes per wavefront instead of per workgroup; a
 * reader that sees v may then find one of the first v messages missing.
 * litmus[1] counts such observations, which the weak rule allows; only a
 * missing message once the signal reads the context's full count sets
 * VR_ASYNC_LITMUS.
 * puts_per_rank must be a multiple of contexts; put_bytes a multiple of 16. */
vrResult_t vr_ring_exchange(vrComm_t comm, vrWindow_t send, vrWindow_t recv, size_t put_bytes,
                            size_t puts_per_rank, int contexts, uint32_t sig_base,
                            uint32_t cnt_base, vrWindow_t sig_window, size_t sig_window_off,
                            uint64_t* litmus, uint32_t flags, void* stream);

/* Signal ping-pong (GIN page, one-sided transfers: put with a SignalInc, and
 * the signal methods: wait; GDA survey, opening section: for messages of a few
 * hundred bytes the control path sets the time): ranks 0 and 1 make `iters`
 * round trips inside one kernel, written with the device API of
 * vrcomm_device.hpp. Round i: rank 0 puts bytes [off, off+bytes) of its slice
 * of `win` to the same range of rank 1's slice with a SignalInc on `sig` at
 * rank 1; rank 1 waits for that, then puts [off, off+bytes) of its slice to
 * [off+bytes, off+2*bytes) of rank 0's slice with a SignalInc on `sig` at
 * rank 0, which waits for it. Each of the two signals rises by iters; other
 * ranks are untouched. flags: VR_PINGPONG_SAME_XCD runs rank 1 on rank 0's
 * XCD (otherwise on the next one); VR_PINGPONG_WAVES makes the two ranks the
 * two waves of one workgroup, each with the wave-level put and publish of
 * vrcomm_device.hpp (not with VR_PINGPONG_SAME_XCD). Needs nranks >= 2, iters >= 1,
 * bytes <= 1 MiB (0 allowed: signals only), [off, off+2*bytes) inside the
 * window and clear of VA signal words, and both signals' values known to the
 * host (VR_ERR_INVALID_USAGE otherwise). A wait that times out sets
 * VR_ASYNC_TIMEOUT and ends the exchange. */
vrResult_t vr_signal_pingpong(vrComm_t comm, vrWindow_t win, size_t off, size_t bytes, uint32_t iters,
                              uint32_t sig, uint32_t flags, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* VRCOMM_H */
