// HIP side of the session: device query, launches on the caller's stream, the
// descriptor arena of the batched all-reduce, and the static scratch of its
// allocation-free variant.
//
// The arena holds the job and pointer tables of batched launches (the
// gradient all-reduces, and copy batches too large for kernel arguments).
// Tables are written into pinned host staging and copied to device memory
// with one asynchronous copy on the caller's stream, ahead of the kernel.  Two
// arenas alternate; before one is rewritten the host waits on the event
// recorded after the last kernel that read it.  Copy batches that fit travel
// in the kernel arguments instead and need no upload.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "rc_internal.h"

namespace rc {

// Device scratch of the allocation-free batched all-reduce: its job, group
// and pointer tables are written here by kernels.  Each GPU holds its own
// copy, at an address looked up once per device (resolve_scratch) and kept in
// g_scratch_ptr; in host code the name is only a handle and is never passed
// to a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};

// ---------------------------------------------------------------- launches

hipError_t launch_jobs(const LaunchPlan& p, hipStream_t stream) {
    const bool nt = p.args.nontemporal != 0;
    const bool full = p.args.full_tiles != 0;
    if (full && p.args.in_mode == kInFold && p.acc && p.nin <= kAccSlot) {
        FoldTableFn tf;
        if (p.dtype == RC_F32)
            tf = nt ? fold_table_acc_fn_f32_nt(p.op, p.nin) : fold_table_acc_fn_f32_cached(p.op, p.nin);
        else
            tf = nt ? fold_table_acc_fn_i32_nt(p.op, p.nin) : fold_table_acc_fn_i32_cached(p.op, p.nin);
        if (!tf || p.split || p.shift_out || p.unroll != unroll_for(2 * p.nin)) return hipErrorInvalidValue;
        hipLaunchKernelGGL(tf, dim3(p.grid, p.grid_y), dim3(kBlock), p.lds_bytes, stream, fold_table_of(p));
        return hipGetLastError();
    }
    if ((full || p.split) && p.args.in_mode == kInFold && !p.acc) {
        const bool u1 = p.nin >= 4 && p.nin < 8 && p.unroll == 1;
        const bool sh = p.shift_out;
        const bool ed = p.split;
        FoldTableFn tf;
        if (p.dtype == RC_F32)
            tf = nt ? fold_table_fn_f32_nt(p.op, u1, sh, ed, p.nin) : fold_table_fn_f32_cached(p.op, u1, sh, ed, p.nin);
        else
            tf = nt ? fold_table_fn_i32_nt(p.op, u1, sh, ed, p.nin) : fold_table_fn_i32_cached(p.op, u1, sh, ed, p.nin);
        if (!tf || p.unroll != (u1 ? 1 : unroll_for(p.nin))) return hipErrorInvalidValue;
        // the shifted kernel stages a round in the LDS that caps occupancy
        const int lds = sh ? std::max(p.lds_bytes, shift_lds_bytes(p.unroll)) : p.lds_bytes;
        hipLaunchKernelGGL(tf, dim3(p.grid, p.grid_y), dim3(kBlock), lds, stream, fold_table_of(p));
        return hipGetLastError();
    }
    FoldFn fn;
    if (p.args.in_mode == kInCopy) {
        fn = copy_fn(nt, full, p.shift_out, p.args.nranks);
    } else {
        // the one-vector whole-tile all-reduce of 4-7 ranks (see plan)
        const bool mid = !p.acc && p.nin >= 4 && p.nin < 8;
        const bool u1 = full && mid && p.unroll == 1;
        if (mid && !full && p.unroll != 2) return hipErrorInvalidValue;  // no general kernel with one vector
        if (p.dtype == RC_F32) fn = nt ? fold_fn_f32_nt(p.op, p.acc, full, u1, p.nin)
                                       : fold_fn_f32_cached(p.op, p.acc, full, u1, p.nin);
        else fn = nt ? fold_fn_i32_nt(p.op, p.acc, full, u1, p.nin) : fold_fn_i32_cached(p.op, p.acc, full, u1, p.nin);
    }
    if (!fn) return hipErrorInvalidValue;
    // the shifted copy stages a round in the LDS that caps occupancy
    const int lds = p.shift_out ? std::max(p.lds_bytes, shift_lds_bytes(p.unroll)) : p.lds_bytes;
    hipLaunchKernelGGL(fn, dim3(p.grid, p.grid_y), dim3(kBlock), lds, stream, p.args);
    return hipGetLastError();
}

hipError_t launch_batch(const BatchJob* jobs, const int32_t* group_job, const void* const* ptrs,
                        const BatchPlan& p, hipStream_t stream) {
    const bool nt = p.nontemporal != 0;
    BatchFn fn;
    if (p.copy) fn = copy_batch_fn(nt, p.nout);
    else fn = nt ? batch_fn_nt(p.dtype, p.op, p.acc, p.nranks) : batch_fn_cached(p.dtype, p.op, p.acc, p.nranks);
    if (!fn) return hipErrorInvalidValue;
    BatchArgs a;
    a.jobs = jobs;
    a.group_job = group_job;
    a.ptrs = ptrs;
    a.total_tiles = p.total_tiles;
    a.ngroups = (int64_t)p.group_job.size();
    a.njobs = (int32_t)p.jobs.size();
    a.tile_elems = p.tile_elems;
    a.mean = p.op == RC_MEAN ? 1 : 0;
    a.grid_2d = p.grid_2d;
    hipLaunchKernelGGL(fn, dim3(p.grid, p.grid_y), dim3(kBlock), p.lds_bytes, stream, a);
    return hipGetLastError();
}

hipError_t launch_copy_args(const BatchPlan& p, hipStream_t stream) {
    if (!p.by_value || p.jobs.size() > (size_t)kMaxCopyArgJobs || p.ptrs.size() > (size_t)kMaxCopyArgPtrs)
        return hipErrorInvalidValue;
    CopyArgsFn fn = copy_args_fn(p.nontemporal != 0, p.full_tiles, p.shift_out, p.nout);
    if (!fn) return hipErrorInvalidValue;
    CopyArgs a{};
    for (size_t i = 0; i < p.ptrs.size(); ++i) a.ptrs[i] = p.ptrs[i];
    a.len = p.jobs[0].len;
    a.tile_elems = p.tile_elems;
    for (size_t j = 0; j < p.jobs.size(); ++j) {
        if (p.jobs[j].len != a.len) return hipErrorInvalidValue;  // equal lengths only
        a.phase[j] = (uint8_t)p.jobs[j].phase;
    }
    const int lds = p.shift_out ? std::max(p.lds_bytes, shift_lds_bytes(kCopyUnroll)) : p.lds_bytes;
    hipLaunchKernelGGL(fn, dim3(p.grid, p.grid_y), dim3(kBlock), lds, stream, a);
    return hipGetLastError();
}

struct Arena {
    void* host = nullptr;    // pinned staging
    void* dev = nullptr;     // device copy read by the kernel
    size_t cap = 0;
    hipEvent_t done = nullptr;
    bool pending = false;    // `done` recorded after the last kernel reading it
};

// A launch timer of the occupancy tuner: start and stop events, reused.
struct Timer {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
    bool used = false;
};

struct DeviceState {
    int device = -1;
    Arena arena[2];
    int next = 0;
    std::vector<Timer> timers;
} g;

void free_timers() {
    for (Timer& t : g.timers) {
        if (t.start) (void)hipEventDestroy(t.start);
        if (t.stop) (void)hipEventDestroy(t.stop);
    }
    g.timers.clear();
}

Error hip_fail(const char* what, hipError_t e) {
    return Error{RC_ERR_DEVICE, std::string(what) + ": " + hipGetErrorName(e) + " (" +
                                    hipGetErrorString(e) + ")"};
}

// Makes the session's device current for the scope of a call.
struct DeviceGuard {
    int prev = -1;
    hipError_t err = hipSuccess;
    DeviceGuard() {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != g.device) err = hipSetDevice(g.device);
        else prev = -1;
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

Error wait_arena(Arena& a) {
    if (a.pending) {
        hipError_t e = hipEventSynchronize(a.done);
        if (e != hipSuccess) return hip_fail("hipEventSynchronize", e);
        a.pending = false;
    }
    return {};
}

void free_arena(Arena& a) {
    if (a.pending) (void)hipEventSynchronize(a.done);
    if (a.host) (void)hipHostFree(a.host);
    if (a.dev) (void)hipFree(a.dev);
    if (a.done) (void)hipEventDestroy(a.done);
    a = Arena{};
}

Error ensure_arena(Arena& a, size_t bytes) {
    if (a.cap >= bytes) return {};
    free_arena(a);
    size_t cap = 64 << 10;
    while (cap < bytes) cap *= 2;
    hipError_t e = hipHostMalloc(&a.host, cap, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail("hipHostMalloc", e);
    e = hipMalloc(&a.dev, cap);
    if (e != hipSuccess) {
        free_arena(a);
        return hip_fail("hipMalloc", e);
    }
    e = hipEventCreateWithFlags(&a.done, hipEventDisableTiming);
    if (e != hipSuccess) {
        free_arena(a);
        return hip_fail("hipEventCreateWithFlags", e);
    }
    a.cap = cap;
    return {};
}

// Where a batch's tables sit in its descriptor block: [jobs][group index]
// [pointer table], each 256-byte aligned.
struct TableLayout {
    size_t group_off;
    size_t ptr_off;
    size_t bytes;
};

TableLayout table_layout(const BatchPlan& p) {
    auto align = [](size_t v) { return (v + 255) & ~size_t(255); };
    TableLayout t;
    t.group_off = align(p.jobs.size() * sizeof(BatchJob));
    t.ptr_off = align(t.group_off + p.group_job.size() * sizeof(int32_t));
    t.bytes = t.ptr_off + p.ptrs.size() * sizeof(void*);
    return t;
}

// Bytes [off, off + n) of a batch's descriptor block into dst (the gaps
// between the tables are zero).
void read_tables(const BatchPlan& p, const TableLayout& t, size_t off, size_t n, char* dst) {
    std::memset(dst, 0, n);
    const struct {
        const void* src;
        size_t at, len;
    } parts[3] = {{p.jobs.data(), 0, p.jobs.size() * sizeof(BatchJob)},
                  {p.group_job.data(), t.group_off, p.group_job.size() * sizeof(int32_t)},
                  {p.ptrs.data(), t.ptr_off, p.ptrs.size() * sizeof(void*)}};
    for (const auto& q : parts) {
        const size_t lo = std::max(off, q.at), hi = std::min(off + n, q.at + q.len);
        if (lo < hi) std::memcpy(dst + (lo - off), static_cast<const char*>(q.src) + (lo - q.at), hi - lo);
    }
}

void write_tables(const BatchPlan& p, const TableLayout& t, char* dst) { read_tables(p, t, 0, t.bytes, dst); }

// Looks up the address of GPU dev's copy of `scratch` once per device, with
// that device current (rc_register's set-up of each session calls it).
Error resolve_scratch(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return Error{RC_ERR_DEVICE, "device index beyond the scratch table"};
    if (g_scratch_ptr[dev]) return {};
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e == hipSuccess && prev != dev) e = hipSetDevice(dev);
    if (e != hipSuccess) return hip_fail("hipSetDevice", e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev >= 0 && prev != dev) (void)hipSetDevice(prev);
    if (e != hipSuccess) return hip_fail("hipGetSymbolAddress(scratch)", e);
    if (!p) return Error{RC_ERR_DEVICE, "hipGetSymbolAddress(scratch) gave NULL"};
    g_scratch_ptr[dev] = p;
    return {};
}

}  // namespace

size_t batch_table_bytes(const BatchPlan& p) { return table_layout(p).bytes; }

Error device_launch_batch_static(const BatchPlan& p, void* stream) {
    if (p.jobs.empty()) return {};
    if (p.by_value) return Error{RC_ERR_INVALID_ARGUMENT, "device_launch_batch_static: by-value batch"};
    const TableLayout t = table_layout(p);
    if (t.bytes > kStaticScratchBytes)
        return Error{RC_ERR_INVALID_ARGUMENT,
                     "the batched tensors' descriptor tables need " + std::to_string(t.bytes) +
                         " bytes, more than the " + std::to_string(kStaticScratchBytes) +
                         " bytes of static scratch: use rc_all_reduce_many, or fewer small tensors per call"};
    DeviceGuard guard;
    if (guard.err != hipSuccess) return hip_fail("hipSetDevice", guard.err);
    if (g.device < 0 || g.device >= kMaxDevices || !g_scratch_ptr[g.device])
        return Error{RC_ERR_DEVICE, "static scratch not resolved for this device"};
    char* base = static_cast<char*>(g_scratch_ptr[g.device]);
    // the tables as 32-bit words (their size is a multiple of 8 bytes), in
    // pieces small enough for kernel arguments
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t words = t.bytes / 4;
    TableChunk c;
    c.pad = 0;
    for (size_t w0 = 0; w0 < words; w0 += kTableChunkWords) {
        const size_t n = words - w0 < (size_t)kTableChunkWords ? words - w0 : (size_t)kTableChunkWords;
        c.dst = reinterpret_cast<uint32_t*>(base) + w0;
        c.nwords = (uint32_t)n;
        read_tables(p, t, w0 * 4, n * 4, reinterpret_cast<char*>(c.words));
        hipLaunchKernelGGL(table_write_fn(), dim3(1), dim3(kBlock), 0, s, c);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail("table writer launch", e);
    }
    const hipError_t e = launch_batch(reinterpret_cast<const BatchJob*>(base),
                                      reinterpret_cast<const int32_t*>(base + t.group_off),
                                      reinterpret_cast<const void* const*>(base + t.ptr_off), p, s);
    if (e != hipSuccess) return hip_fail("kernel launch", e);
    return {};
}

Error device_open(const Config& cfg, DeviceInfo* info) {
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess) return hip_fail("hipGetDeviceCount", e);
    if (count <= 0) return Error{RC_ERR_DEVICE, "no GPU visible"};
    int dev = cfg.device;
    if (dev < 0) {
        e = hipGetDevice(&dev);
        if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    }
    if (dev >= count) return Error{RC_ERR_INVALID_ARGUMENT, "device index out of range"};
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail("hipGetDeviceProperties", e);
    const std::string arch = prop.gcnArchName;
    if (arch.compare(0, 6, "gfx950") != 0)
        return Error{RC_ERR_DEVICE, "GPU " + std::to_string(dev) + " is " + arch +
                                        "; this library is built for gfx950 only"};
    info->device = dev;
    info->cu_count = prop.multiProcessorCount;
    info->l2_bytes = prop.l2CacheSize;
    info->lds_per_cu = (int64_t)prop.maxSharedMemoryPerMultiProcessor;
    info->max_lds_per_block = (int64_t)prop.sharedMemPerBlock;
    info->arch = arch;
    Error err = resolve_scratch(dev);
    if (err.code) return err;
    g.device = dev;
    g.next = 0;
    return {};
}

Error device_launch(const LaunchPlan& p, void* stream) {
    DeviceGuard guard;
    if (guard.err != hipSuccess) return hip_fail("hipSetDevice", guard.err);
    hipError_t e = launch_jobs(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("kernel launch", e);
    return {};
}

Error device_launch_batch(const BatchPlan& p, void* stream) {
    if (p.jobs.empty()) return {};
    DeviceGuard guard;
    if (guard.err != hipSuccess) return hip_fail("hipSetDevice", guard.err);
    if (p.by_value) {
        const hipError_t e = launch_copy_args(p, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail("kernel launch", e);
        return {};
    }
    Arena& a = g.arena[g.next];
    Error err = wait_arena(a);
    if (err.code) return err;
    const TableLayout t = table_layout(p);
    err = ensure_arena(a, t.bytes);
    if (err.code) return err;
    write_tables(p, t, static_cast<char*>(a.host));
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(a.dev, a.host, t.bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail("hipMemcpyAsync", e);
    const char* dev = static_cast<const char*>(a.dev);
    e = launch_batch(reinterpret_cast<const BatchJob*>(dev), reinterpret_cast<const int32_t*>(dev + t.group_off),
                     reinterpret_cast<const void* const*>(dev + t.ptr_off), p, s);
    if (e != hipSuccess) return hip_fail("kernel launch", e);
    e = hipEventRecord(a.done, s);
    if (e != hipSuccess) return hip_fail("hipEventRecord", e);
    a.pending = true;
    g.next ^= 1;
    return {};
}

Error device_finish() {
    DeviceGuard guard;
    if (guard.err != hipSuccess) return hip_fail("hipSetDevice", guard.err);
    hipError_t e = hipDeviceSynchronize();
    for (Arena& a : g.arena) free_arena(a);
    free_timers();
    g.device = -1;
    if (e != hipSuccess) return hip_fail("hipDeviceSynchronize", e);
    return {};
}

void device_reset() {
    if (g.device < 0) return;
    DeviceGuard guard;
    for (Arena& a : g.arena) free_arena(a);
    free_timers();  // destroying a pending event is allowed: the runtime defers it
    g.device = -1;
}

Error device_event_create(void** ev) {
    DeviceGuard guard;
    if (guard.err != hipSuccess) return hip_fail("hipSetDevice", guard.err);
    hipEvent_t e = nullptr;
    hipError_t st = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (st != hipSuccess) return hip_fail("hipEventCreateWithFlags", st);
    *ev = e;
    return {};
}

void device_event_destroy(void* ev) {
    if (ev) (void)hipEventDestroy(static_cast<hipEvent_t>(ev));
}

Error device_event_record(void* ev, void* stream) {
    hipError_t st = hipEventRecord(static_cast<hipEvent_t>(ev), static_cast<hipStream_t>(stream));
    if (st != hipSuccess) return hip_fail("hipEventRecord", st);
    return {};
}

Error device_stream_wait(void* stream, void* ev) {
    hipError_t st = hipStreamWaitEvent(static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(ev), 0);
    if (st != hipSuccess) return hip_fail("hipStreamWaitEvent", st);
    return {};
}

Error device_stream_capturing(void* stream, bool* capturing) {
    hipStreamCaptureStatus status = hipStreamCaptureStatusNone;
    hipError_t st = hipStreamIsCapturing(static_cast<hipStream_t>(stream), &status);
    if (st != hipSuccess) return hip_fail("hipStreamIsCapturing", st);
    *capturing = status != hipStreamCaptureStatusNone;
    return {};
}

}  // namespace rc

namespace rc {

Error device_timer_start(void* stream, int* ticket) {
    DeviceGuard guard;
    if (guard.err != hipSuccess) return hip_fail("hipSetDevice", guard.err);
    size_t i = 0;
    while (i < g.timers.size() && g.timers[i].used) ++i;
    if (i == g.timers.size()) {
        // Timing only: nothing reads the timed launch's data on the strength
        // of these events, so they skip the system-scope fence (its cache
        // writeback and invalidation would otherwise slow the launch being
        // timed; calibration then read ~2% above the steady state).
        Timer t;
        hipError_t e = hipEventCreateWithFlags(&t.start, hipEventDisableSystemFence);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&t.stop, hipEventDisableSystemFence);
        if (e != hipSuccess) {
            if (t.start) (void)hipEventDestroy(t.start);
            return hip_fail("hipEventCreateWithFlags", e);
        }
        g.timers.push_back(t);
    }
    const hipError_t e = hipEventRecord(g.timers[i].start, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("hipEventRecord", e);
    g.timers[i].used = true;
    *ticket = (int)i;
    return {};
}

Error device_timer_stop(int ticket, void* stream) {
    if (ticket < 0 || ticket >= (int)g.timers.size() || !g.timers[ticket].used)
        return Error{RC_ERR_DEVICE, "device_timer_stop: unknown ticket"};
    const hipError_t e = hipEventRecord(g.timers[ticket].stop, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("hipEventRecord", e);
    return {};
}

Error device_timer_read(int ticket, bool* done, float* us) {
    *done = false;
    if (ticket < 0 || ticket >= (int)g.timers.size() || !g.timers[ticket].used)
        return Error{RC_ERR_DEVICE, "device_timer_read: unknown ticket"};
    Timer& t = g.timers[ticket];
    hipError_t e = hipEventQuery(t.stop);
    if (e == hipErrorNotReady) return {};
    if (e != hipSuccess) return hip_fail("hipEventQuery", e);
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, t.start, t.stop);
    if (e != hipSuccess) return hip_fail("hipEventElapsedTime", e);
    t.used = false;
    *done = true;
    *us = ms * 1000.0f;
    return {};
}

}  // namespace rc
