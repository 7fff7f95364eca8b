// HIP side of the session: device query, launches on the caller's stream, and
// the descriptor arena of the batched all-reduce.
//
// The arena holds the job and pointer tables of batched launches (the
// gradient all-reduces, and copy batches too large for kernel arguments).
// Tables are written into pinned host staging and copied to device memory
// with one asynchronous copy on the caller's stream, ahead of the kernel.  Two
// arenas alternate; before one is rewritten the host waits on the event
// recorded after the last kernel that read it.  Copy batches that fit travel
// in the kernel arguments instead and need no upload.
#include <hip/hip_runtime.h>

#include <cstring>
#include <string>
#include <vector>

#include "rc_internal.h"

namespace rc {

hipError_t launch_jobs(const LaunchPlan& p, hipStream_t stream);
hipError_t launch_copy_args(const BatchPlan& p, hipStream_t stream);
hipError_t launch_batch(const BatchJob* jobs, const int32_t* group_job, const void* const* ptrs,
                        const BatchPlan& p, hipStream_t stream);

namespace {

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

}  // namespace

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
    // arena layout: [jobs][group index][pointer table], each 256-byte aligned
    auto align = [](size_t v) { return (v + 255) & ~size_t(255); };
    const size_t job_bytes = p.jobs.size() * sizeof(BatchJob);
    const size_t group_off = align(job_bytes);
    const size_t group_bytes = p.group_job.size() * sizeof(int32_t);
    const size_t ptr_off = align(group_off + group_bytes);
    const size_t bytes = ptr_off + p.ptrs.size() * sizeof(void*);
    err = ensure_arena(a, bytes);
    if (err.code) return err;
    char* host = static_cast<char*>(a.host);
    std::memcpy(host, p.jobs.data(), job_bytes);
    std::memcpy(host + group_off, p.group_job.data(), group_bytes);
    std::memcpy(host + ptr_off, p.ptrs.data(), p.ptrs.size() * sizeof(void*));
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(a.dev, a.host, bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail("hipMemcpyAsync", e);
    const char* dev = static_cast<const char*>(a.dev);
    const BatchJob* jobs = reinterpret_cast<const BatchJob*>(dev);
    const int32_t* group_job = reinterpret_cast<const int32_t*>(dev + group_off);
    const void* const* ptrs = reinterpret_cast<const void* const*>(dev + ptr_off);
    e = launch_batch(jobs, group_job, ptrs, p, s);
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
        Timer t;
        hipError_t e = hipEventCreate(&t.start);
        if (e == hipSuccess) e = hipEventCreate(&t.stop);
        if (e != hipSuccess) {
            if (t.start) (void)hipEventDestroy(t.start);
            return hip_fail("hipEventCreate", e);
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
