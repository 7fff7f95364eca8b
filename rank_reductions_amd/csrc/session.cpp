// The C ABI and the session state machine.
//
// Lifecycle (ruCCL README (ja), section 2 "Tensor collective API" and section
// 4 "Errors and lifecycle"): register opens the session, finish_collective is
// the normal end, reset_collective discards the registration and in-flight
// state without completing, checkpointing or recovering anything.  Duplicate
// and missing registration are CollectiveError cases.  Host-only C++: the GPU
// is reached only through the device_* functions.
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "rc_internal.h"

namespace rc {
namespace {

struct Session {
    bool registered = false;
    int nranks = 0;
    Config cfg;
    DeviceInfo dev;
};

std::mutex g_mu;
Session g_s;
thread_local std::string t_err;

int report(const Error& e) {
    t_err = e.code ? e.msg : std::string();
    return e.code;
}

int ok() {
    t_err.clear();
    return RC_OK;
}

Error read_config(const rc_config* in, Config* cfg) {
    *cfg = Config{};
    if (!in) return {};
    if (in->struct_size != sizeof(rc_config))
        return Error{RC_ERR_INVALID_ARGUMENT,
                     "rc_register: cfg->struct_size must be sizeof(rc_config) = " +
                         std::to_string(sizeof(rc_config))};
    if (in->algo < RC_ALGO_AUTO || in->algo > RC_ALGO_RING)
        return Error{RC_ERR_INVALID_ARGUMENT, "rc_register: unknown algo"};
    if (in->cache_hint < RC_CACHE_AUTO || in->cache_hint > RC_CACHE_NORMAL)
        return Error{RC_ERR_INVALID_ARGUMENT, "rc_register: unknown cache_hint"};
    if (in->tile_elems < 0 || in->tile_elems > 65536 || in->tile_elems % 256 != 0)
        return Error{RC_ERR_INVALID_ARGUMENT,
                     "rc_register: tile_elems must be 0 or a multiple of 256 up to 65536"};
    if (in->max_workgroups < 0)
        return Error{RC_ERR_INVALID_ARGUMENT, "rc_register: max_workgroups is negative"};
    if (in->waves_per_cu < 0 || in->waves_per_cu > 32)
        return Error{RC_ERR_INVALID_ARGUMENT, "rc_register: waves_per_cu must be in [0, 32]"};
    if (in->device < -1) return Error{RC_ERR_INVALID_ARGUMENT, "rc_register: device < -1"};
    if (in->reserved != 0) return Error{RC_ERR_INVALID_ARGUMENT, "rc_register: reserved must be 0"};
    cfg->device = in->device;
    cfg->algo = in->algo;
    cfg->validate_only = in->validate_only != 0;
    cfg->tile_elems = in->tile_elems;
    cfg->max_workgroups = in->max_workgroups;
    cfg->cache_hint = in->cache_hint;
    cfg->waves_per_cu = in->waves_per_cu;
    return {};
}

int collective(Coll coll, const rc_buf* bufs, void* stream) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_s.registered)
        return report(Error{RC_ERR_NOT_REGISTERED, "no session: call rc_register first"});
    Checked ck;
    Error e = validate(coll, g_s.nranks, bufs, &ck);
    if (e.code) return report(e);
    if (g_s.cfg.validate_only) return ok();
    for (const LaunchPlan& p : plan(ck, g_s.cfg, g_s.dev)) {
        e = device_launch(p, stream);
        if (e.code) return report(e);
    }
    return ok();
}

}  // namespace
}  // namespace rc

using namespace rc;

extern "C" {

int rc_register(int num_ranks, const rc_config* cfg) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_s.registered)
        return report(Error{RC_ERR_DUPLICATE_REGISTRATION, "rc_register: a session is already open"});
    if (num_ranks < 1 || num_ranks > RC_MAX_RANKS)
        return report(Error{RC_ERR_INVALID_ARGUMENT, "rc_register: num_ranks must be in [1, 16]"});
    Config c;
    Error e = read_config(cfg, &c);
    if (e.code) return report(e);
    DeviceInfo dev;
    if (!c.validate_only) {
        e = device_open(c, &dev);
        if (e.code) return report(e);
    }
    g_s.registered = true;
    g_s.nranks = num_ranks;
    g_s.cfg = c;
    g_s.dev = dev;
    return ok();
}

int rc_all_reduce(const rc_buf* bufs, void* stream) { return collective(Coll::AllReduce, bufs, stream); }
int rc_reduce(const rc_buf* bufs, void* stream) { return collective(Coll::Reduce, bufs, stream); }
int rc_broadcast(const rc_buf* bufs, void* stream) { return collective(Coll::Broadcast, bufs, stream); }
int rc_reduce_scatter(const rc_buf* bufs, void* stream) {
    return collective(Coll::ReduceScatter, bufs, stream);
}
int rc_all_gather(const rc_buf* bufs, void* stream) { return collective(Coll::AllGather, bufs, stream); }

int rc_all_reduce_many(int num_tensors, const rc_buf* bufs, void* stream) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_s.registered)
        return report(Error{RC_ERR_NOT_REGISTERED, "no session: call rc_register first"});
    std::vector<Checked> cks;
    Error e = validate_batch(g_s.nranks, num_tensors, bufs, &cks);
    if (e.code) return report(e);
    if (g_s.cfg.validate_only) return ok();
    std::vector<Checked> own, batched;
    split_batch(cks, &own, &batched);
    for (const Checked& ck : own) {
        for (const LaunchPlan& p : plan(ck, g_s.cfg, g_s.dev)) {
            e = device_launch(p, stream);
            if (e.code) return report(e);
        }
    }
    const BatchPlan bp = plan_batch(batched, g_s.cfg, g_s.dev);
    if (bp.total_tiles == 0) return ok();
    e = device_launch_batch(bp, stream);
    return report(e);
}

int rc_finish(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_s.registered)
        return report(Error{RC_ERR_NOT_REGISTERED, "rc_finish: no session is open"});
    Error e;
    if (!g_s.cfg.validate_only) e = device_finish();
    g_s = Session{};
    return report(e);
}

int rc_reset(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_s.registered && !g_s.cfg.validate_only) device_reset();
    g_s = Session{};
    return ok();
}

const char* rc_last_error(void) { return t_err.c_str(); }

const char* rc_status_name(int status) {
    switch (status) {
        case RC_OK: return "RC_OK";
        case RC_ERR_NOT_REGISTERED: return "RC_ERR_NOT_REGISTERED";
        case RC_ERR_DUPLICATE_REGISTRATION: return "RC_ERR_DUPLICATE_REGISTRATION";
        case RC_ERR_SHAPE_MISMATCH: return "RC_ERR_SHAPE_MISMATCH";
        case RC_ERR_OP_MISMATCH: return "RC_ERR_OP_MISMATCH";
        case RC_ERR_ROOT_MISMATCH: return "RC_ERR_ROOT_MISMATCH";
        case RC_ERR_BROADCAST_SENDERS: return "RC_ERR_BROADCAST_SENDERS";
        case RC_ERR_DTYPE_MISMATCH: return "RC_ERR_DTYPE_MISMATCH";
        case RC_ERR_INVALID_ARGUMENT: return "RC_ERR_INVALID_ARGUMENT";
        case RC_ERR_DEVICE: return "RC_ERR_DEVICE";
        default: return "RC_UNKNOWN_STATUS";
    }
}

int rc_abi_version(void) { return RC_ABI_VERSION; }

}  // extern "C"
