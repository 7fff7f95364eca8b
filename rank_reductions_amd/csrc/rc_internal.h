// Internal structures shared by the host-only layers (session, validation,
// planning) and the HIP layer (kernels, launch).  Plain C++, no HIP types:
// the host-only files compile with an ordinary C++ compiler.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "rc.h"
#include "tiling.h"

namespace rc {

static_assert(kMaxRanks == RC_MAX_RANKS, "tiling.h and rc.h disagree on the rank limit");

// The first five are reductions or fan-outs over ring segments; the rest are
// the Communicator page's other methods: copies between ranks and a barrier.
enum class Coll { AllReduce, Reduce, Broadcast, ReduceScatter, AllGather, AllToAll, AllGatherList, SendRecv, Barrier };

// How a job's inputs are formed.
enum InMode : int32_t {
    kInFold = 0,  // fold R inputs: in[(c+1+k) % R] + c*in_stride, k = 0..R-1
    kInCopy = 1,  // copy one input: in[c] + c*in_stride
};

// Argument block of one launch that covers up to kMaxRanks jobs (segments).
// Job c spans elements [c*seg, min((c+1)*seg, n)) of the collective's index
// space.  Passed by value as the kernel argument.
struct JobArgs {
    const void* in[kMaxRanks];
    void* out[kMaxRanks];
    int64_t n;
    int64_t seg;
    int64_t in_stride;
    int64_t out_stride;
    int32_t tile_elems;     // elements per tile, a multiple of kBlock*kVec*unroll
    int32_t jobs;
    int32_t nranks;
    int32_t in_mode;
    int32_t out_mode;
    uint32_t out_mask;
    int32_t mean;           // divide the finished fold by nranks
    int32_t nontemporal;
    int32_t grid_2d;                     // one-shot 2-D grid (x: tile of job, y: job)
    // 2-D grid whose every tile is one whole round: each job has phase 0 and
    // exactly gridDim.x tiles of tile_elems = kBlock*kVec*unroll elements.
    // Such launches run the whole-tile kernels, which skip the head, lead,
    // tail and tile-count logic.
    int32_t full_tiles;
    int32_t total_tiles;                 // tile_prefix[jobs], below 2^31
    int32_t tile_prefix[kMaxRanks + 1];  // tiles before job j; past the last job: total_tiles
    uint8_t phase[kMaxRanks];            // job phase (phase_code of its reference stream)
    // fold jobs with accumulators: operand k of a job is acc[r] + in[r] for
    // its rank r, added before the fold (kernels instantiated for it only)
    const void* acc[kMaxRanks];
};

struct DeviceInfo {
    int device = 0;
    int cu_count = 0;
    int64_t l2_bytes = 0;
    int64_t lds_per_cu = 0;         // bytes of LDS per compute unit
    int64_t max_lds_per_block = 0;  // largest dynamic LDS one workgroup may take
    std::string arch;
};

struct Config {
    int device = -1;
    int algo = RC_ALGO_AUTO;
    bool validate_only = false;
    int64_t tile_elems = 0;
    int max_workgroups = 0;
    int cache_hint = RC_CACHE_AUTO;
    int waves_per_cu = 0;
    // folds moving this many bytes or more split off their aligned interior
    // (split_fold); not in rc_config: kSplitMinBytes, lowered by the CPU
    // replay of the planner to reach the split at small sizes
    int64_t split_min_bytes = -1;
};

// Result of validating one collective call.
struct Checked {
    Coll coll = Coll::AllReduce;
    int nranks = 0;
    int dtype = RC_F32;
    int op = RC_SUM;
    int root = -1;            // reduce root, or broadcast sender
    int64_t count = 0;        // element count described by dims
    const void* send[kMaxRanks] = {};
    void* recv[kMaxRanks] = {};
    // all_reduce over acc[r] + send[r] (a gradient sync's accumulators)
    bool has_acc = false;
    const void* acc[kMaxRanks] = {};
    // all_gather, list form: rank r's output for rank k's shard at [r*R + k]
    std::vector<void*> recv_list;
};

struct Error {
    int code = RC_OK;
    std::string msg;
};

// ---------------------------------------------------------------- validate.cpp
Error validate(Coll coll, int nranks, const rc_buf* bufs, Checked* out, void* const* recv_list = nullptr);
// send on rank src and recv on rank dst as one copy: bufs[0] is the sender's
// side, bufs[1] the receiver's.  The result is a SendRecv with send[0] and
// recv[0] set and root = src.
Error validate_send_recv(int nranks, int src, int dst, const rc_buf* bufs, Checked* out);
const char* coll_name(Coll c);
// Tensor t of a batched all-reduce; messages name the tensor index, or
// ids[t] when ids is given (a gradient sync's parameter IDs).  accs, when
// given, holds tensor t's accumulators at [t*R + r] (NULL: none).
Error validate_batch(int nranks, int num_tensors, const rc_buf* bufs,
                     std::vector<Checked>* out, const uint64_t* ids = nullptr,
                     const void* const* accs = nullptr);
// Pairs the ranks' gradient entries by parameter ID: rank r has counts[r]
// entries params[r][i].  On success bufs[t*R + r] and accs[t*R + r] are rank
// r's buffer and accumulator of the t-th smallest ID, order[t].
Error match_params(int nranks, const int* counts, const rc_param* const* params,
                   std::vector<rc_buf>* bufs, std::vector<const void*>* accs, std::vector<uint64_t>* order);
int64_t element_size(int dtype);

// ---------------------------------------------------------------- plan.cpp
// Unroll (16-byte vectors per lane per round) of a fold of `nin` inputs: about
// eight vector loads in flight per lane.  Shared by the planner and kernels.
constexpr int unroll_for(int nin) { return nin >= 8 ? 1 : (nin >= 4 ? 2 : (nin >= 2 ? 4 : 8)); }
// Unroll of the copy kernel (one input, up to 16 outputs per element).
constexpr int kCopyUnroll = 2;
// Elements per tile for a kernel of the given unroll under the session's config.
int tile_elems_for(int unroll, const Config& cfg);
// The stream a job's tiles align to: of the job's streams (its nin inputs,
// then its nout outputs, each at the job's first element), the one whose
// 256-byte alignment class carries the most weight, an output counting twice
// an input (a store sharing a line with a neighbouring tile costs more than a
// load); ties go to the class met first.  Returns its index in ins ++ outs.
int job_reference(const uintptr_t* ins, int nin, const uintptr_t* outs, int nout);
// Phase (phase_code) of a job whose reference stream starts at `ref`.
uint8_t phase_of(uintptr_t ref);
// job_reference and phase_of together.
uint8_t job_phase(const uintptr_t* ins, int nin, const uintptr_t* outs, int nout);

struct LaunchPlan {
    JobArgs args;
    int nin = 1;             // inputs folded per element (1 = copy)
    bool acc = false;        // each folded input is an accumulator plus a send
    int nout = 1;            // outputs written per element
    int unroll = 1;          // vectors per lane per round of the kernel
    int dtype = RC_F32;
    int op = RC_SUM;
    int64_t total_tiles = 0;
    int64_t grid = 0;        // workgroups launched along x
    int grid_y = 1;          // along y: the jobs, for one-shot launches
    int lds_bytes = 0;       // dynamic LDS per workgroup: caps workgroups per CU
    int waves = 0;           // workgroups (waves) per CU that lds_bytes allows; 0: no cap
    // a whole-tile fold without accumulators, or a whole-tile copy, some of
    // whose written outputs start a job off a 64-byte write burst, and no
    // output overlaps an input: it runs fold_table_shift_kernel or
    // copy_full_shift_kernel (tiling.h)
    bool shift_out = false;
    // A fold whose jobs are not whole tiles, split (split_fold): the FoldTable
    // kernels' edge form, whose first `edges` workgroups of each job do the
    // job's head, lead and what follows its interior on the general path,
    // and the next `interior` the whole tiles of its aligned interior, job c's
    // starting job_off[c] elements in.  grid = edges + interior.
    bool split = false;
    int edges = 0;
    int64_t interior = 0;
    int64_t job_off[kMaxRanks] = {};
};

// Builds the launches of one validated call: one for most collectives, two
// for the ring all-reduce.  Empty when there is nothing to do.
std::vector<LaunchPlan> plan(const Checked& ck, const Config& cfg, const DeviceInfo& dev);
// Whether a whole-tile fold or copy of these jobs (element size es) runs the
// shifted kernel (LaunchPlan::shift_out); job_off: where the launch starts
// in each job (LaunchPlan::job_off).
bool shifted_outputs_pay(const JobArgs& a, int64_t es, const int64_t* job_off);
// Turns a fold launch whose jobs are not whole tiles into a split one
// (LaunchPlan::split); false: it stays on the general kernel.
bool split_fold(LaunchPlan* lp, const Config& cfg, const DeviceInfo& dev, int64_t es);

// Batched all-reduce: job and pointer tables for tensors [t0, t1).
struct BatchPlan {
    std::vector<BatchJob> jobs;
    // [job][2R] or, with accumulators, [job][3R]: fold operands in order,
    // their accumulators in the same order, then the outputs
    std::vector<const void*> ptrs;
    bool acc = false;
    // a batch of copies instead of folds: ptrs is [job][1 + nout], the
    // source then nout destinations, all at the job's first element
    bool copy = false;
    int nout = 0;
    std::vector<int32_t> group_job;  // job holding tile g << kGroupShift, per group g
    int64_t total_tiles = 0;
    int tile_elems = 0;
    int nranks = 0;
    int dtype = RC_F32;
    int op = RC_SUM;
    int nontemporal = 1;
    int64_t grid = 0;
    int grid_y = 1;     // copies of equal-length jobs: y = job, x = tile of the job
    int grid_2d = 0;
    int lds_bytes = 0;
    int waves = 0;  // workgroups (waves) per CU that lds_bytes allows; 0: no cap
    // a copy batch small enough to pass its table in the kernel arguments
    // (no descriptor upload before the launch)
    bool by_value = false;
    // by value, and every job whole one-round tiles on a 256-byte boundary
    // (phase 0, len = grid * tile_elems): the whole-tile copy kernel
    bool full_tiles = false;
    // whole tiles, some destination starts its job off a 64-byte write
    // burst, and no destination overlaps a source: the shifted copy kernel
    // (tiling.h)
    bool shift_out = false;
};
// Whether a whole-tile copy batch runs the shifted kernel
// (BatchPlan::shift_out; element size es).
bool shifted_copies_pay(const BatchPlan& bp, int64_t es);
// Capacity of the by-value copy table: all_to_all_single up to 12 ranks
// (R*R jobs of 2 pointers) and every list-form all_gather (R jobs of 1+R).
constexpr int kMaxCopyArgJobs = 256;
constexpr int kMaxCopyArgPtrs = 288;
BatchPlan plan_batch(const std::vector<Checked>& tensors, const Config& cfg, const DeviceInfo& dev);
// The copy jobs of all_to_all_single and of the list form of all_gather.
BatchPlan plan_copies(const Checked& ck, const Config& cfg, const DeviceInfo& dev);
// Whether a validated call runs as a batch of copies (plan_copies) rather
// than through plan().
inline bool runs_as_copies(Coll c) { return c == Coll::AllToAll || c == Coll::AllGatherList; }

// A batched all-reduce splits into tensors large enough to run as launches of
// their own (their kernel time dwarfs a launch boundary, and they avoid the
// batched kernel's per-tile job lookup) and the rest, batched into one launch.
constexpr int64_t kOwnLaunchBytes = int64_t(64) << 20;  // HBM bytes moved per tensor
void split_batch(const std::vector<Checked>& tensors, std::vector<Checked>* own,
                 std::vector<Checked>* batched);

// Workgroups resident per CU that keep HBM busiest for a kernel streaming
// `nin` inputs and `nout` outputs per element with `unroll` vectors per lane:
// the rule aims at `kib` KiB of traffic in flight per CU, a store counting
// `store_weight` of a load.
struct InFlightRule {
    double kib;
    double store_weight;
};
constexpr InFlightRule kFoldRule{110.0, 0.65};     // general fold and copy kernels
constexpr InFlightRule kCopyBatchRule{60.0, 0.5};  // batched copies; whole-tile copies
constexpr InFlightRule kFullFoldRule{85.0, 0.52};  // whole-tile folds
// Whole-tile folds with accumulators (fold_table_acc_kernel) run at most this
// many waves per CU.  Sweeps of W = 4..10, in place and not, two runs each:
// 2 and 4 ranks (8 KiB of loads per wave either way) peak at 6 (4 x 64 MiB
// 122.3-123.1 us against 126.7-128.0 at the rule's 8, 128-130 at 4 and 5),
// 8 ranks at 4-5, where the rule already lands.
constexpr int kAccTableMaxWaves = 6;
int auto_waves_per_cu(int nin, int nout, int unroll, const InFlightRule& rule = kFoldRule);
// Grid and LDS reservation of a launch of `total_tiles` tiles.
void shape_launch(int64_t total_tiles, int nin, int nout, int unroll, const Config& cfg,
                  const DeviceInfo& dev, int64_t* grid, int* lds_bytes,
                  const InFlightRule& rule = kFoldRule);

// LDS reservation per one-wave workgroup that lets `waves` of them share a CU.
int lds_for_waves(const DeviceInfo& dev, int waves);

// Occupancy tuner.  The fastest waves per CU for a launch shape differs
// between otherwise identical boxes (5 on some, 7 on others for the 8-rank
// all-reduce: 161 against 167 us and the reverse), and the wave count changes
// timing only, never results.  So the first launches of each large shape try
// the rule's W and the two values below it, kTuneSamples timed launches each
// (HIP events read once they have completed, never waited on), and every
// later launch of that shape uses the candidate with the lowest median time
// per byte.  A candidate other than the rule's W must beat the rule's median
// by kTuneMargin: launch times of one shape spread by up to +-10%, a lucky
// sample once sent a 4-rank all-reduce to a wave count that ran 30% slower
// in steady state, and a switch 1.6% ahead in calibration ran 9% slower,
// while the largest gain seen from a right switch is 3.6%.  Used when
// waves_per_cu is left to the library, for launches that move at least
// kTuneMinBytes.
constexpr int kTuneCands = 3;
constexpr int kTuneSamples = 5;
constexpr double kTuneMargin = 0.03;
constexpr int64_t kTuneMinBytes = int64_t(256) << 20;
// Fold launches that move this much or more split off their aligned
// interior onto the whole-tile kernels (split_fold).  Ragged 4- and 8-rank
// all-reduces of 64 and 128 MiB ran 1-8% faster split, same box; at 32 MiB,
// latency-bound (about 10 us a call), the two forms were within noise.
constexpr int64_t kSplitMinBytes = int64_t(64) << 20;
struct TunePending {
    int ticket;     // device timer
    int cand;       // candidate index
    int64_t bytes;  // bytes the timed launch moves
};
struct TuneEntry {
    int ncand = 0;
    int cand[kTuneCands] = {};
    int issued[kTuneCands] = {};
    int got[kTuneCands] = {};
    float us[kTuneCands][kTuneSamples] = {};  // time per GiB of each timed launch
    float median_us[kTuneCands] = {};         // set once every candidate has kTuneSamples times
    std::vector<TunePending> pending;  // timed launches not read yet
    int chosen = 0;  // 0 until every candidate has kTuneSamples times
};
// Waves per CU for the next launch of a shape whose rule gives rule_waves;
// *cand >= 0 asks the caller to time this launch and report it to tune_record.
int tune_pick(TuneEntry& t, int rule_waves, int* cand);
void tune_record(TuneEntry& t, int cand, float us);

// ---------------------------------------------------------------- kernels_*.hip
// Kernel argument blocks of the table-driven launches, passed by value.

// A launch over a job table in device memory: tile t belongs to job
// find_job(jobs, group_job, ngroups, njobs, t).
struct BatchArgs {
    const BatchJob* jobs;
    const int32_t* group_job;
    const void* const* ptrs;  // [job][2R], or [job][3R] with accumulators: operands, accumulators, outputs
    int64_t total_tiles;
    int64_t ngroups;
    int32_t njobs;
    int32_t tile_elems;
    int32_t mean;
    int32_t grid_2d;  // copies: y = job, x = tile of the job
};

// A copy batch whose table travels in the kernel arguments: job j =
// blockIdx.y copies ptrs[j*(1+NR)] to the next NR pointers; every job has
// len elements.
struct CopyArgs {
    const void* ptrs[kMaxCopyArgPtrs];
    int64_t len;
    int32_t tile_elems;
    int32_t pad;
    uint8_t phase[kMaxCopyArgJobs];
};

// Argument block of a whole-tile fold (the all-reduce, reduce and
// reduce_scatter of whole, aligned tiles: every large workload's launch; a
// gradient sync's fold with accumulators of up to kAccSlot ranks).  Job c's
// fold operands are listed in ring order and already offset to its first
// element, so a workgroup fetches its R input pointers, the output bases and
// its job's output mask in one round of scalar loads, with no index or
// stride arithmetic before its HBM loads; the JobArgs form measured 3%
// slower on the 8-rank all-reduce.  With accumulators, operand k's
// accumulator sits in slot kAccSlot + k of the job's row.
constexpr int kAccSlot = kMaxRanks / 2;
struct FoldTable {
    const void* in[kMaxRanks][kMaxRanks];  // [job][k]: operand k at the first element the launch folds
    void* out[kMaxRanks];                  // output bases; job c's outputs start c*out_stride elements in
    int64_t out_off[kMaxRanks];            // ... and the launch writes from out_off[c] elements further
    int64_t out_stride;
    uint32_t mask[kMaxRanks];              // outputs job c writes
    int32_t mean;                          // divide the finished fold by the rank count
    int32_t pad;
    // A split fold (LaunchPlan::split): workgroups x < edges of job c do the
    // job's tiles outside its interior on the general path (job c has len[c]
    // elements and phase[c]; its tile skipped_tile(x, 1, interior)); the next
    // `interior` do the whole tiles of its interior.  Unused otherwise.
    int64_t len[kMaxRanks];
    uint8_t phase[kMaxRanks];
    int32_t edges;
    int32_t interior;
};

// The FoldTable of a whole-tile fold (full_tiles or split, kInFold; with
// accumulators only for nin <= kAccSlot and full_tiles): job c's operands in
// ring order from the element its launch starts at (job_off[c] for a split),
// its output mask and, for a split, its length, phase and edge tiles.
FoldTable fold_table_of(const LaunchPlan& p);

// A piece of a descriptor table written into device memory by a kernel (the
// allocation-free batched all-reduce's way of placing its tables).
constexpr int kTableChunkWords = 896;
struct TableChunk {
    uint32_t* dst;
    uint32_t nwords;
    uint32_t pad;
    uint32_t words[kTableChunkWords];
};

using FoldFn = void (*)(JobArgs);
using FoldTableFn = void (*)(FoldTable);
using BatchFn = void (*)(BatchArgs);
using CopyArgsFn = void (*)(CopyArgs);
using TableFn = void (*)(TableChunk);

// The kernel instantiation for a launch; nullptr if none exists.  Fold
// kernels (kernels_fold.hip, built once per dtype and cache hint):
// op RC_SUM / RC_MEAN / RC_MAX, acc (accumulators: Sum and Mean only), full
// (whole-tile kernel), u1 (the whole-tile fold of 4-7 ranks with one vector
// per lane), nin = ranks folded.
FoldFn fold_fn_f32_nt(int op, bool acc, bool full, bool u1, int nin);
FoldFn fold_fn_f32_cached(int op, bool acc, bool full, bool u1, int nin);
FoldFn fold_fn_i32_nt(int op, bool acc, bool full, bool u1, int nin);
FoldFn fold_fn_i32_cached(int op, bool acc, bool full, bool u1, int nin);
// Whole-tile folds without accumulators, over a FoldTable (same files);
// shift: the kernel for launches with outputs off a 64-byte write burst
// (LaunchPlan::shift_out); edges: the form of split folds (LaunchPlan::split,
// unroll kUnroll only).
FoldTableFn fold_table_fn_f32_nt(int op, bool u1, bool shift, bool edges, int nin);
FoldTableFn fold_table_fn_f32_cached(int op, bool u1, bool shift, bool edges, int nin);
FoldTableFn fold_table_fn_i32_nt(int op, bool u1, bool shift, bool edges, int nin);
FoldTableFn fold_table_fn_i32_cached(int op, bool u1, bool shift, bool edges, int nin);
// Whole-tile folds with accumulators of nin <= kAccSlot ranks, over a
// FoldTable (same files; Sum and Mean, unroll unroll_for(2 * nin)).
FoldTableFn fold_table_acc_fn_f32_nt(int op, int nin);
FoldTableFn fold_table_acc_fn_f32_cached(int op, int nin);
FoldTableFn fold_table_acc_fn_i32_nt(int op, int nin);
FoldTableFn fold_table_acc_fn_i32_cached(int op, int nin);
// Batched folds (kernels_batch.hip, once per cache hint).
BatchFn batch_fn_nt(int dtype, int op, bool acc, int nin);
BatchFn batch_fn_cached(int dtype, int op, bool acc, int nin);
// Copies to nr outputs (kernels_copy.hip): single copies, copy batches over
// a device table, copy batches by value, and the table writer; shift (with
// full only): the whole-tile kernel that writes outputs off a 64-byte burst
// over burst-aligned ranges.
FoldFn copy_fn(bool nt, bool full, bool shift, int nr);
BatchFn copy_batch_fn(bool nt, int nr);
CopyArgsFn copy_args_fn(bool nt, bool full, bool shift, int nr);
TableFn table_write_fn();

// ---------------------------------------------------------------- device.hip
// All return RC_OK or RC_ERR_DEVICE with a message.
Error device_open(const Config& cfg, DeviceInfo* info);
Error device_launch(const LaunchPlan& p, void* stream);
Error device_launch_batch(const BatchPlan& p, void* stream);
// The same batch with its tables in the library's static device scratch
// (kStaticScratchBytes per GPU, reserved when the library loads) instead of
// the session's arena: no allocation, no host staging, nothing but kernel
// launches (a table writer, then the batch).  RC_ERR_INVALID_ARGUMENT when
// the tables exceed the scratch.  Calls that overlap on one GPU race on it.
constexpr size_t kStaticScratchBytes = size_t(1) << 20;
size_t batch_table_bytes(const BatchPlan& p);
Error device_launch_batch_static(const BatchPlan& p, void* stream);
Error device_finish();   // wait for the GPU, free scratch
void device_reset();     // wait for kernels reading scratch, free scratch
// Events that order the per-rank front end's streams around a launch.
Error device_event_create(void** ev);
void device_event_destroy(void* ev);
Error device_event_record(void* ev, void* stream);
Error device_stream_wait(void* stream, void* ev);
// Whether work enqueued on `stream` is being captured into a graph.
Error device_stream_capturing(void* stream, bool* capturing);
// Launch timers for the occupancy tuner: a start and a stop event around
// kernels on `stream`.  timer_read never blocks: *done stays false while
// either event is pending; once both completed it gives the time between
// them and releases the ticket.  device_finish / device_reset free them all.
Error device_timer_start(void* stream, int* ticket);
Error device_timer_stop(int ticket, void* stream);
Error device_timer_read(int ticket, bool* done, float* us);

}  // namespace rc
