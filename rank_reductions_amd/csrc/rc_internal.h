// Internal structures shared by the host-only layers (session, validation,
// planning) and the HIP layer (kernels, launch).  Plain C++, no HIP types:
// the host-only files compile with an ordinary C++ compiler.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "rc.h"

namespace rc {

constexpr int kMaxRanks = RC_MAX_RANKS;
constexpr int kBlock = 256;          // threads per workgroup (4 wave64s)
constexpr int kVec = 4;              // elements per 16-byte vector
constexpr uint8_t kScalarOnly = 0xFF;  // job phase: pointers not co-aligned

enum class Coll { AllReduce, Reduce, Broadcast, ReduceScatter, AllGather };

// How a job's inputs are formed.
enum InMode : int32_t {
    kInFold = 0,  // fold R inputs: in[(c+1+k) % R] + c*in_stride, k = 0..R-1
    kInCopy = 1,  // copy one input: in[c] + c*in_stride
};

// Which ranks' outputs a job writes (each at out[r] + c*out_stride).
enum OutMode : int32_t {
    kOutMask = 0,       // the ranks in out_mask
    kOutOwner = 1,      // only rank c
    kOutMaskButOwner = 2,  // the ranks in out_mask except rank c
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
    int64_t tile_prefix[kMaxRanks + 1];  // tiles before job j
    uint8_t phase[kMaxRanks];            // leading scalar elements, or kScalarOnly
};

// One segment of one tensor in a batched all-reduce (device descriptor).
struct BatchJob {
    int64_t tile_begin;  // first tile of this job in the launch's tile space
    int64_t start;       // element offset of the segment in its tensor
    int64_t len;         // elements in the segment (> 0)
    int32_t tensor;      // index into the pointer table
    int32_t c;           // segment index (sets the fold rotation)
    int32_t phase;       // leading scalar elements, or kScalarOnly
    int32_t pad;
};

struct DeviceInfo {
    int device = 0;
    int cu_count = 0;
    int64_t l2_bytes = 0;
    std::string arch;
};

struct Config {
    int device = -1;
    int algo = RC_ALGO_AUTO;
    bool validate_only = false;
    int64_t tile_elems = 0;
    int max_workgroups = 0;
    int cache_hint = RC_CACHE_AUTO;
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
};

struct Error {
    int code = RC_OK;
    std::string msg;
};

// ---------------------------------------------------------------- validate.cpp
Error validate(Coll coll, int nranks, const rc_buf* bufs, Checked* out);
// Tensor t of a batched all-reduce; messages name the tensor index.
Error validate_batch(int nranks, int num_tensors, const rc_buf* bufs,
                     std::vector<Checked>* out);
int64_t element_size(int dtype);

// ---------------------------------------------------------------- plan.cpp
// Unroll (16-byte vectors per lane per round) for a job's input count: about
// 16 vector loads in flight per lane.  Shared by the planner and the kernels.
constexpr int unroll_for(int nin) { return nin >= 16 ? 1 : (nin >= 8 ? 2 : 4); }
// Elements per tile for a job's input count under the session's config.
int tile_elems_for(int nin, const Config& cfg);
// Job phase: number of scalar elements before every pointer is 16-byte
// aligned, or kScalarOnly when the pointers disagree modulo 16 bytes.
uint8_t job_phase(const uintptr_t* addrs, int naddrs, int64_t elem_size, int64_t len);
// Tiles for one job of `len` elements.
int64_t job_tiles(int64_t len, uint8_t phase, int64_t tile_elems);

struct LaunchPlan {
    JobArgs args;
    int nin = 1;             // inputs folded per element (1 = copy)
    int dtype = RC_F32;
    int op = RC_SUM;
    int64_t total_tiles = 0;
};

// Builds the launches of one validated call: one for most collectives, two
// for the ring all-reduce.  Empty when there is nothing to do.
std::vector<LaunchPlan> plan(const Checked& ck, const Config& cfg);

// Batched all-reduce: job and pointer tables for tensors [t0, t1).
struct BatchPlan {
    std::vector<BatchJob> jobs;
    std::vector<const void*> ptrs;  // [tensor][2R]: R inputs, then R outputs
    int64_t total_tiles = 0;
    int tile_elems = 0;
    int nranks = 0;
    int dtype = RC_F32;
    int op = RC_SUM;
    int nontemporal = 1;
};
BatchPlan plan_batch(const std::vector<Checked>& tensors, const Config& cfg);

int grid_for(int64_t total_tiles, const Config& cfg, const DeviceInfo& dev);

// ---------------------------------------------------------------- device.hip
// All return RC_OK or RC_ERR_DEVICE with a message.
Error device_open(const Config& cfg, DeviceInfo* info);
Error device_launch(const LaunchPlan& p, int grid, void* stream);
Error device_launch_batch(const BatchPlan& p, int grid, void* stream);
Error device_finish();   // wait for the GPU, free scratch
void device_reset();     // wait for kernels reading scratch, free scratch

}  // namespace rc
