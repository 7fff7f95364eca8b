/*
 * rc.h - tensor collectives over R logical ranks whose buffers all live in the
 * HBM of one GPU (gfx950).  C ABI; plain pointers and sizes only.
 *
 * The operations are the public tensor collective API of the ruCCL README
 * (ja), user guide section 2 "Tensor collective API" (register, all_reduce,
 * reduce, broadcast, finish_collective, reset_collective), with the call
 * contract of section 3 and the CollectiveError cases of section 4, plus
 * reduce_scatter_tensor and all_gather_into_tensor from the monarch
 * `Struct Communicator` page.  Every collective takes a stream, as the
 * Communicator methods do, and returns a status code.
 *
 * Two ways to call.  The whole-call entry points take all R ranks' arguments
 * at once (one rc_buf per logical rank), so the contract that every rank
 * issues matching collectives in the same order (ruCCL README section 3;
 * Communicator's Send/Sync safety note) holds by construction and mismatches
 * between ranks are detected inside one call.  The per-rank entry points
 * (rc_rank_*, below) take one rank's side per call, from that rank's own
 * thread, and match the ranks' calls by issue order.  Gradient syncs keyed by
 * parameter ID (ruCCL README section 6) come in both forms.
 *
 * Numerics.  Each collective reduces along the ring: for element counts N over
 * R ranks, the segment length is S = ceil(N/R) and segment c = [c*S,
 * min((c+1)*S, N)) is folded left in rank order (c+1), (c+2), ..., c (mod R),
 * the order a ring reduce-scatter leaves at segment c's owner (ruCCL README,
 * "CUDA tensor example": a ring AllReduce over logical ranks on one GPU).
 * float32 adds are IEEE round-to-nearest-even with subnormals kept; Mean is
 * one correctly rounded float32 division of the finished fold by R; int32 Sum
 * wraps; float32 Max returns the quiet NaN 0x7FC00000 if any operand is NaN
 * and otherwise the larger value, +0 above -0.  The result therefore does not
 * depend on the algorithm, tile size or grid, and every rank's output is
 * bit-identical.
 *
 * Errors.  Every argument is checked before anything is enqueued.  On an
 * error no buffer is touched, nothing is launched, the session stays as it
 * was, and rc_last_error() describes the failure.  Checks run in this order:
 *   NOT_REGISTERED; INVALID_ARGUMENT for malformed fields (enum values, ndim,
 *   negative dims, NULL or misaligned pointers that the op requires);
 *   DTYPE_MISMATCH; SHAPE_MISMATCH; OP_MISMATCH; INVALID_ARGUMENT for an op the
 *   dtype lacks (int32 Mean); ROOT_MISMATCH and INVALID_ARGUMENT for a root
 *   out of range; BROADCAST_SENDERS; INVALID_ARGUMENT for overlapping buffers.
 *
 * Graphs.  Single collectives (all_reduce, reduce, broadcast, reduce_scatter,
 * all_gather, send/recv) and the copy batches of all_to_all_single and the
 * list-form all_gather (up to 12 and 16 ranks) enqueue nothing but kernels,
 * so they can be captured into a HIP graph and replayed, and so can
 * rc_all_reduce_many_static.  Batched all-reduces (rc_all_reduce_many,
 * rc_all_reduce_params) with tensors under 64 MiB of traffic, and copy
 * batches beyond those sizes, upload descriptor tables from reused host
 * staging; on a capturing stream they return RC_ERR_INVALID_ARGUMENT before
 * enqueuing anything.  Per-rank calls join several streams and are not meant
 * for capture.
 *
 * Threads.  The library keeps one process-wide session behind a mutex; calls
 * from several threads are serialised.  A per-rank call blocks its thread,
 * without holding the mutex, until its peers' matching calls arrive.  The
 * caller orders whole-call collectives on its streams (the Communicator page
 * leaves issue order to the user).
 */
#ifndef RANKRED_RC_H
#define RANKRED_RC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RC_ABI_VERSION 3
#define RC_MAX_RANKS 16
#define RC_MAX_DIMS 8

/* Element types: the backend's float and int types are f32 and i32 (RUDA
 * "Training and state saving", "Configure training backend"). */
enum { RC_F32 = 0, RC_I32 = 1 };

/* Reduction operators: Sum and Mean (ruCCL README, "CUDA tensor example" and
 * section 6, ReduceOperation::Mean); Max (the ReduceOp of the Communicator's
 * all_reduce).  Mean is float32 only. */
enum { RC_SUM = 0, RC_MEAN = 1, RC_MAX = 2 };

/* Algorithm for all_reduce: DIRECT reads all R inputs once per element and
 * writes all R outputs; RING runs a reduce-scatter kernel, then an all-gather
 * kernel.  Both give the same bits.  AUTO picks DIRECT. */
enum { RC_ALGO_AUTO = 0, RC_ALGO_DIRECT = 1, RC_ALGO_RING = 2 };

/* Store cache hint for outputs (and load hint for inputs). */
enum { RC_CACHE_AUTO = 0, RC_CACHE_STREAMING = 1, RC_CACHE_NORMAL = 2 };

/* Status codes.  Codes 1-6 are the CollectiveError cases of the ruCCL README,
 * section 4 "Errors and lifecycle" (duplicate or missing registration, shape
 * mismatch, inconsistent reduction op or root, invalid broadcast sender
 * count); 7-9 are this library's plumbing; 10 is the parameter-ID agreement
 * that section 6 "Collective training" requires of a gradient sync. */
typedef enum {
    RC_OK = 0,
    RC_ERR_NOT_REGISTERED = 1,
    RC_ERR_DUPLICATE_REGISTRATION = 2,
    RC_ERR_SHAPE_MISMATCH = 3,
    RC_ERR_OP_MISMATCH = 4,
    RC_ERR_ROOT_MISMATCH = 5,
    RC_ERR_BROADCAST_SENDERS = 6,
    RC_ERR_DTYPE_MISMATCH = 7,
    RC_ERR_INVALID_ARGUMENT = 8,
    RC_ERR_DEVICE = 9,
    RC_ERR_PARAM_MISMATCH = 10  /* gradient maps with different parameter IDs */
} rc_status;

/* One logical rank's side of a collective (cf. the TensorCell argument of the
 * Communicator methods).  Buffers are dense, contiguous, in device memory of
 * the registered GPU, and aligned to the element size.  The element count is
 * the product of dims[0..ndim) (ndim 0 means a scalar, count 1); a count of 0
 * is a no-op that returns RC_OK once the fields check out.  Buffers of zero
 * elements may be NULL, except that broadcast still finds its sender as the
 * one non-NULL send.
 *   send  input, read only (never written unless recv == send);
 *   recv  output;
 *   dtype RC_F32 or RC_I32, equal on all ranks;
 *   op    RC_SUM / RC_MEAN / RC_MAX, equal on all ranks (reducing ops only;
 *         ignored by broadcast and all_gather);
 *   root  reduce: the receiving rank, equal on all ranks.  broadcast: -1 on
 *         all ranks, or the sender's index on all ranks.  Ignored otherwise.
 *   dims  shape, equal on all ranks; reduce_scatter: the input's shape (count
 *         divisible by R; recv holds count/R elements); all_gather: the
 *         shard's shape (recv holds R*count elements). */
typedef struct rc_buf {
    const void* send;
    void* recv;
    int32_t dtype;
    int32_t op;
    int32_t root;
    int32_t ndim;
    int64_t dims[RC_MAX_DIMS];
} rc_buf;

/* Session configuration (cf. CollectiveConfig::default() and
 * with_num_devices, ruCCL README section 3; the "strategy" set through the
 * config maps to algo).  Zero-initialise, set struct_size = sizeof(rc_config),
 * then set what you need; 0 selects the default of every field but device.
 *   device         GPU index, or -1 for the device current at rc_register
 *                  (cfg == NULL also means the current device)
 *   algo           RC_ALGO_*
 *   validate_only  nonzero: check arguments and return, never touch the GPU
 *                  (rc_register then makes no HIP call at all)
 *   tile_elems     elements per workgroup tile; 0: default; else a multiple
 *                  of 256 in [256, 65536]
 *   max_workgroups 0: one workgroup per tile (batched all-reduce: a
 *                  persistent grid sized from the CU count); > 0: a
 *                  persistent grid of at most this many workgroups
 *   cache_hint     RC_CACHE_*
 *   waves_per_cu   cap on workgroups (one wave each) resident per compute
 *                  unit, in [1, 32]; 0: the library's choice per collective.
 *                  With 0, launches that move 256 MiB or more are tuned
 *                  online: the first launches of each launch shape and size
 *                  class try three caps (five timed launches each, HIP
 *                  events read once complete, never waited on; none while
 *                  the stream is being captured) and later ones use the cap
 *                  with the lowest median time, the default cap unless
 *                  another beats it by 3%.  The cap changes timing only,
 *                  never the results.  With
 *                  RC_TUNE_LOG=1 in the environment each choice is printed
 *                  on stderr.
 *   reserved       must be 0 */
typedef struct rc_config {
    uint32_t struct_size;
    int32_t device;
    int32_t algo;
    int32_t validate_only;
    int64_t tile_elems;
    int32_t max_workgroups;
    int32_t cache_hint;
    int32_t waves_per_cu;
    int32_t reserved;
} rc_config;

/* register<B> (ruCCL README, section 2; section 3 for the config): open the
 * process-wide session for num_ranks logical ranks (1..RC_MAX_RANKS) on one
 * GPU.  cfg may be NULL for defaults; cfg->struct_size must equal
 * sizeof(rc_config).  Fails with RC_ERR_DUPLICATE_REGISTRATION while a session
 * is open, RC_ERR_INVALID_ARGUMENT for bad values, RC_ERR_DEVICE if the GPU is
 * not a gfx950 or cannot be queried.  Allocates nothing on the device. */
int rc_register(int num_ranks, const rc_config* cfg);

/* all_reduce<B> (ruCCL README section 2: the reduced result is returned to
 * every participant; Communicator.all_reduce).  bufs[r] for r < num_ranks;
 * every send and recv non-NULL; recv == send (in place) is allowed.  Every
 * rank's recv receives the same bits.  Enqueued on `stream` (a hipStream_t;
 * NULL is the null stream); returns once enqueued. */
int rc_all_reduce(const rc_buf* bufs, void* stream);

/* reduce<B> (ruCCL README section 2: reduce to the given root; non-root
 * participants receive nothing; Communicator.reduce).  Every send non-NULL;
 * the root's recv non-NULL (may equal its send); other ranks' recv may be
 * NULL and is never written.  The root receives the bits all_reduce gives. */
int rc_reduce(const rc_buf* bufs, void* stream);

/* broadcast<B> (ruCCL README section 2: the sender passes Some(tensor), the
 * receivers pass None; section 3: exactly one sender; Communicator.broadcast).
 * The sender is the one rank with send != NULL; all other sends must be NULL,
 * else RC_ERR_BROADCAST_SENDERS.  Every receiver's recv must be non-NULL and
 * receives the sender's bytes; the sender's recv, if non-NULL and not equal to
 * its send, receives them too. */
int rc_broadcast(const rc_buf* bufs, void* stream);

/* reduce_scatter_tensor (Communicator page: reduce, then scatter the result).
 * Each send holds count = R*M elements (dims describe it); rank r's recv
 * receives the M elements [r*M, (r+1)*M) of the reduction.  In place is
 * allowed as recv_r == send_r + r*M elements. */
int rc_reduce_scatter(const rc_buf* bufs, void* stream);

/* all_gather_into_tensor (Communicator page: gather every rank's tensor into
 * one output).  Each send is a shard of count = M elements; every recv holds
 * R*M elements and receives shard_0, ..., shard_{R-1} in rank order, bit for
 * bit.  In place is allowed as send_r == recv_r + r*M elements. */
int rc_all_gather(const rc_buf* bufs, void* stream);

/* all_gather, list form (Communicator.all_gather: one output tensor per
 * source rank).  bufs[r].send is rank r's shard of count M elements (dims
 * describe it); bufs[r].recv is not used.  recvs[r * num_ranks + k] is rank
 * r's output for rank k's shard (M elements), receiving it bit for bit.  The
 * output a rank keeps for its own shard may be the shard itself
 * (recvs[r * num_ranks + r] == bufs[r].send); any other overlap is
 * RC_ERR_INVALID_ARGUMENT.  recvs is read during the call only. */
int rc_all_gather_list(const rc_buf* bufs, void* const* recvs, void* stream);

/* all_to_all_single (Communicator page: split the input, scatter the splits
 * to all ranks, concatenate what is received).  Each send holds count = R*M
 * elements and each recv the same count; rank d's recv receives, at [s*M,
 * (s+1)*M), the elements [d*M, (d+1)*M) of rank s's send, bit for bit.  A
 * count not divisible by R is RC_ERR_SHAPE_MISMATCH; no in-place layout
 * exists (recv overlapping any send is RC_ERR_INVALID_ARGUMENT). */
int rc_all_to_all_single(const rc_buf* bufs, void* stream);

/* Communicator.send on rank src together with Communicator.recv on rank dst,
 * as one call: bufs[0] is the sender's side (send used), bufs[1] the
 * receiver's (recv used); dtype and shape must agree (RC_ERR_DTYPE_MISMATCH,
 * RC_ERR_SHAPE_MISMATCH); src and dst are different ranks in [0, num_ranks).
 * recv == send moves nothing. */
int rc_send_recv(int src, int dst, const rc_buf* bufs, void* stream);

/* Communicator.barrier.  With every rank's work issued on the one stream of
 * the whole-call entry points, it is already in order: this checks the
 * session and enqueues nothing.  The per-rank form below joins the ranks'
 * streams. */
int rc_barrier(void* stream);

/* Whole-gradient all-reduce (ruCCL README section 6, "Collective training":
 * grads.all_reduce_with(communicator, ReduceOperation::Mean) reduces every
 * gradient of a parameter set, with IDs, shapes, dtype and call order
 * matching across ranks).  bufs is [num_tensors][num_ranks], row-major: tensor
 * t's rank r is bufs[t * num_ranks + r].  Every tensor obeys the all_reduce
 * rules and is reduced with its own segments, so the bits equal num_tensors
 * separate rc_all_reduce calls.  Tensors are batched into few launches; the
 * session keeps a descriptor arena for this (allocated on first use, freed by
 * rc_finish / rc_reset). */
int rc_all_reduce_many(int num_tensors, const rc_buf* bufs, void* stream);

/* rc_all_reduce_many for callers that cannot allocate device memory: code
 * being captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, checks, launches and bits as
 * rc_all_reduce_many, but nothing is allocated and only kernels are enqueued:
 * the descriptor tables of the tensors that share the batched launch (those
 * moving under 64 MiB) are written by a small kernel into a static device
 * buffer of 1 MiB that the library holds on each GPU it runs on until the
 * process ends, instead of the session's arena; tensors that get launches of
 * their own use the occupancy tuner's choice so far without timing anything.
 * A call whose tables need more than 1 MiB (about 11,900 ring segments at 4
 * ranks, 3,700 at 16) returns RC_ERR_INVALID_ARGUMENT before enqueuing
 * anything.  Every call on a GPU shares that GPU's buffer and leaves its
 * tables there: calls that overlap on one GPU (from several threads, or on
 * streams that run concurrently) race and give wrong results; calls ordered
 * on one stream do not. */
int rc_all_reduce_many_static(int num_tensors, const rc_buf* bufs, void* stream);

/* One rank's entry of a gradient sync keyed by parameter ID.
 *   id   the parameter ID;
 *   acc  NULL, or that rank's gradients accumulated over earlier microbatches
 *        (the GradientsAccumulator of RUDA "Training and state saving":
 *        accumulate adds without averaging, grads() hands the sum over).
 *        Same shape and dtype as buf.send, read only.  The parameter is then
 *        reduced over acc + send, one add per element (float32 round to
 *        nearest even, int32 wrap) before the fold: the bits of adding the
 *        last microbatch with a separate accumulate and then syncing, in one
 *        pass over memory.  recv may equal acc (the accumulator's storage
 *        receives the result) as it may equal send.  Sum and Mean only.
 *   buf  the parameter's rc_buf with the all_reduce meaning (send: the
 *        rank's gradient, recv: its output, op: normally RC_MEAN). */
typedef struct rc_param {
    uint64_t id;
    const void* acc;
    rc_buf buf;
} rc_param;

/* Whole-gradient all-reduce keyed by parameter ID (ruCCL README section 6,
 * "Collective training": each rank's gradients form a map from parameter ID
 * to gradient, reduced with ReduceOperation::Mean; IDs, shapes and dtype
 * must agree on every rank).  Rank r lists num_params[r] entries
 * params[r][0 .. num_params[r]), in any order.  Entries are paired across
 * ranks by ID and each parameter is reduced on its own, so its bits equal
 * rc_all_reduce of its R buffers (of acc + send where acc is given); the
 * batch runs as rc_all_reduce_many does.  The arrays are read during the
 * call only.
 * Errors, in this order, nothing enqueued: a negative count, a NULL array
 * with a positive count, or an ID listed twice by one rank:
 * RC_ERR_INVALID_ARGUMENT; the ranks' ID sets differ (including their
 * sizes): RC_ERR_PARAM_MISMATCH; then each parameter, in ascending ID order,
 * gets the rc_all_reduce checks, and dtype and op must be the same for the
 * whole batch (as in rc_all_reduce_many); an acc given on some ranks only,
 * misaligned, overlapping an output other than its own rank's recv, or with
 * RC_MAX: RC_ERR_INVALID_ARGUMENT. */
int rc_all_reduce_params(const int* num_params, const rc_param* const* params, void* stream);

/* finish_collective<B> (ruCCL README sections 2 and 4: the normal end of the
 * peer's collective session).  Waits for all work on the session's GPU,
 * frees the session's scratch and closes the session.
 * RC_ERR_NOT_REGISTERED if no session is open. */
int rc_finish(void);

/* reset_collective<B> (ruCCL README sections 2 and 4): discard the
 * registration and any state of calls in progress, from any state.  It does
 * not complete, revoke or checkpoint work already enqueued; it waits only for
 * the kernels that read the session's scratch before freeing it.  Always
 * returns RC_OK. */
int rc_reset(void);

/* ------------------------------------------------------------------------
 * Per-rank front end.  Each logical rank registers itself and issues its own
 * side of every collective, typically from a thread of its own: register<B>
 * registers one peer (ruCCL README section 2), participants agree on the rank
 * count and call matching collectives in the same order (section 3), and on
 * the monarch Communicator page each rank builds and drives its own
 * communicator on its own thread or in its own process.
 *
 * The k-th collective call of every rank forms one collective.  Each call
 * blocks until all num_ranks ranks have made their k-th call; the last to
 * arrive checks the R descriptors against each other (the same checks and
 * codes as the whole-call API; a different collective kind on two ranks is
 * RC_ERR_OP_MISMATCH) and enqueues the kernels.  Every rank then returns the
 * same status.  Ordering: the kernels run after the work each rank had
 * enqueued on its own stream before its call, and each rank's stream waits
 * for the kernels before any work it enqueues after the call returns.  The
 * join is made when the last rank arrives, so work that another thread puts
 * on a waiting rank's stream in the meantime also precedes the kernels.
 * Ranks that pass the same stream as the launching rank cost no events.
 * A rank issues its calls one at a time: a call for a rank that already has
 * one in progress (on another thread) is RC_ERR_INVALID_ARGUMENT and joins
 * no collective.  A rank that never makes its call leaves the others
 * waiting; rc_reset releases them with RC_ERR_NOT_REGISTERED.  The
 * whole-call entry points
 * above reject a session opened here with RC_ERR_INVALID_ARGUMENT, and the
 * per-rank entry points report RC_ERR_NOT_REGISTERED for a rank that has not
 * registered in a per-rank session. */

/* register<B> for one peer.  The first call opens the session with
 * num_ranks and cfg; later calls must give the same num_ranks (else
 * RC_ERR_INVALID_ARGUMENT).  A rank registering twice, or any call while a
 * whole-call session is open, is RC_ERR_DUPLICATE_REGISTRATION.  rank in
 * [0, num_ranks). */
int rc_rank_register(int rank, int num_ranks, const rc_config* cfg);

/* Rank `rank`'s side of all_reduce / reduce / broadcast / reduce_scatter /
 * all_gather: buf is that rank's rc_buf with the meaning given above for the
 * whole-call entry point of the same name, stream is that rank's stream. */
int rc_rank_all_reduce(int rank, const rc_buf* buf, void* stream);
int rc_rank_reduce(int rank, const rc_buf* buf, void* stream);
int rc_rank_broadcast(int rank, const rc_buf* buf, void* stream);
int rc_rank_reduce_scatter(int rank, const rc_buf* buf, void* stream);
int rc_rank_all_gather(int rank, const rc_buf* buf, void* stream);

/* Rank `rank`'s side of rc_all_gather_list: buf describes its shard and
 * recvs[k], k < num_ranks, are its outputs for rank k's shard. */
int rc_rank_all_gather_list(int rank, const rc_buf* buf, void* const* recvs, void* stream);

/* Rank `rank`'s side of rc_all_to_all_single. */
int rc_rank_all_to_all_single(int rank, const rc_buf* buf, void* stream);

/* Communicator.send and recv on logical ranks.  Unlike the collectives, a
 * send from rank a to rank b is matched only with recvs on b from a: the k-th
 * such send meets the k-th such recv, whatever the other ranks call.  Each
 * call blocks until its peer's call arrives (a send and a recv that wait on
 * each other in opposite orders never complete, as with unbuffered
 * point-to-point).  buf.send is the sender's tensor, buf.recv the receiver's;
 * checks as rc_send_recv, reported to both sides.  A peer out of range or
 * equal to the rank: RC_ERR_INVALID_ARGUMENT, nothing matched. */
int rc_rank_send(int rank, const rc_buf* buf, int dst, void* stream);
int rc_rank_recv(int rank, const rc_buf* buf, int src, void* stream);

/* Communicator.barrier: the k-th barrier of every rank forms one barrier.
 * Work each rank enqueues after it is ordered after the work every rank had
 * enqueued before it; nothing else is launched. */
int rc_rank_barrier(int rank, void* stream);

/* Rank `rank`'s side of rc_all_reduce_params: its own num_params entries,
 * in any order.  The gradient sync as the pages call it, once per rank with
 * that rank's parameter map.  The array is read before the call returns. */
int rc_rank_all_reduce_params(int rank, int num_params, const rc_param* params, void* stream);

/* Communicator.split_all / split_from: a collective on rank's communicator
 * that makes a new communicator of some of its members.  Each rank that is
 * to be a member passes the same list of num_members distinct ranks of the
 * current communicator, in the new communicator's rank order (all ranks, in
 * order, is split_all); a rank that passes num_members = 0 stays out and
 * needs not know the list (the page's empty-ranks case).  *new_rank receives
 * the member's endpoint in the new communicator, or -1 for a rank left out.
 *
 * Endpoints.  The rank argument of every rc_rank_* call is an endpoint: a
 * registered rank's index in [0, num_ranks) addresses the world, and the
 * endpoints rc_rank_split returns address the new communicators (each is
 * comm_id * RC_MAX_RANKS + the member's rank in it).  Every collective,
 * gradient sync, send/recv and barrier works on any communicator, with ranks,
 * roots and peers counted within it.  A rank calls from one thread at a time
 * whichever endpoint it uses.
 * Errors: lists that differ between ranks, a listed rank that passed no
 * list, members out of range or listed twice, or new_rank NULL:
 * RC_ERR_INVALID_ARGUMENT for every rank. */
int rc_rank_split(int rank, int num_members, const int* members, int* new_rank);

/* finish_collective<B> for one peer: the rank leaves the session.  When the
 * last registered rank has finished, the session waits for the GPU, frees its
 * scratch and closes.  On a split-off communicator's endpoint it leaves that
 * communicator, which is dropped once all its members have left.  A world
 * rank that finishes leaves every communicator it belongs to.  Calls of other
 * members that wait for a rank that has left could never complete: they
 * return RC_ERR_NOT_REGISTERED at once, and so do later calls on a
 * communicator with a member that has left (send and recv only when the peer
 * has left).
 * RC_ERR_NOT_REGISTERED for a rank not registered; RC_ERR_INVALID_ARGUMENT
 * while the rank still has a call in progress on another thread. */
int rc_rank_finish(int rank);

/* Text for the last failure on the calling thread (valid until that thread's
 * next rc_* call); "" after success. */
const char* rc_last_error(void);

/* Name of a status code ("RC_OK", "RC_ERR_SHAPE_MISMATCH", ...). */
const char* rc_status_name(int status);

/* RC_ABI_VERSION of the loaded library. */
int rc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RANKRED_RC_H */
