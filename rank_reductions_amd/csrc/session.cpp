// The C ABI and the session state machine.
//
// Lifecycle (ruCCL README (ja), section 2 "Tensor collective API" and section
// 4 "Errors and lifecycle"): register opens the session, finish_collective is
// the normal end, reset_collective discards the registration and in-flight
// state without completing, checkpointing or recovering anything.  Duplicate
// and missing registration are CollectiveError cases.
//
// Two front ends share one process-wide session.  The whole-call entry points
// take all R ranks' arguments at once.  The per-rank entry points take one
// rank's side per call (section 3: every participant calls matching
// collectives in the same order; the monarch Communicator page: one thread or
// process per rank); the k-th calls of all ranks are matched into one
// collective, checked, and launched by the last rank to arrive.  Host-only
// C++: the GPU is reached only through the device_* functions.
#include <algorithm>
#include <condition_variable>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "rc_internal.h"

namespace rc {
namespace {

enum class Mode { None, Whole, PerRank };

// What a per-rank call is: one of the collectives (its Coll kind), a gradient
// sync, or a communicator split.
enum Form : uint8_t { kCollective = 0, kParams = 1, kSplit = 2 };

// One collective of the per-rank front end, filled in as ranks arrive.
struct Slot {
    std::vector<Coll> kinds;
    std::vector<rc_buf> bufs;
    std::vector<uint8_t> have_buf;
    std::vector<void*> streams;
    std::vector<uint8_t> form;  // per rank: kCollective, kParams or kSplit
    // gradient sync (all_reduce_params): each rank's entries
    std::vector<int> pcount;
    std::vector<std::vector<rc_param>> params;
    // all_gather, list form: each rank's R outputs
    std::vector<std::vector<void*>> recvs;
    // split: each rank's member list (has_list 0: the rank gave none) and,
    // once matched, its endpoint in the new communicator or -1
    std::vector<uint8_t> has_list;
    std::vector<std::vector<int>> members;
    std::vector<int> result;
    uint32_t arrived = 0;
    int left = 0;
    bool done = false;
    bool abandoned = false;  // a member finished before arriving: the ranks that came get an error
    int status = RC_OK;
    std::string msg;
};

// The per-rank session's events, used only by the launching rank under the
// session lock and reused by every collective (each wait is enqueued right
// after the record it reads, before the event can be recorded again).
struct RankEvents {
    std::vector<void*> arrive;  // one per distinct stream other than the launch stream
    void* done = nullptr;
    ~RankEvents() {
        for (void* ev : arrive) device_event_destroy(ev);
        device_event_destroy(done);
    }
};

// One send/recv pair of the per-rank front end: side 0 is the sender's, side 1
// the receiver's.
struct PairSlot {
    rc_buf bufs[2] = {};
    bool have[2] = {false, false};
    bool null_buf = false;
    void* streams[2] = {nullptr, nullptr};
    bool done = false;
    bool abandoned = false;
    int left = 0;
    int status = RC_OK;
    std::string msg;
};

// A communicator of the per-rank front end: the registered world (id 0), or
// one split off another (the Communicator page's split_all and split_from).
// A member is addressed by its endpoint, id * RC_MAX_RANKS + its rank in the
// communicator, so the world's endpoints are its rank indices.
struct Comm {
    std::vector<int> world;     // world rank of each member, in communicator rank order
    uint32_t fin_mask = 0;      // members that have finished
    std::vector<uint64_t> seq;  // calls issued per member
    std::map<uint64_t, std::shared_ptr<Slot>> slots;
    // point-to-point: the k-th send from src to dst meets the k-th recv on dst from src
    std::map<std::pair<int, int>, uint64_t> sends_posted, recvs_posted;
    std::map<std::tuple<int, int, uint64_t>, std::shared_ptr<PairSlot>> pairs;
    int size() const { return (int)world.size(); }
};

// Launch shape for the occupancy tuner: kernel family (fold, copy, copy
// batch), whole tiles (2: whole tiles with outputs shifted onto 64-byte
// bursts), inputs, accumulators, outputs, unroll and size class.
using TuneKey = std::tuple<int, int, int, int, int, int, int>;

struct Session {
    Mode mode = Mode::None;
    int nranks = 0;
    Config cfg;
    DeviceInfo dev;
    // per-rank front end
    uint32_t reg_mask = 0;   // world ranks registered
    uint32_t fin_mask = 0;   // world ranks finished
    uint32_t busy_mask = 0;  // world ranks with a call in progress
    std::map<int, Comm> comms;
    int next_comm = 1;
    std::shared_ptr<RankEvents> events;
    // occupancy tuner, per launch shape (tune_key)
    std::map<TuneKey, TuneEntry> tune;
};

// The power of two of the bytes a launch moves (the tuner's size class).
int size_class(int64_t moved) { return 63 - __builtin_clzll((unsigned long long)std::max<int64_t>(moved, 1)); }

std::mutex g_mu;
std::condition_variable g_cv;
Session g_s;
uint64_t g_generation = 0;  // bumped when the session is reset or closed
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

// Opens the session (caller holds g_mu and has checked that none is open).
Error open_session(Mode mode, int num_ranks, const rc_config* cfg) {
    if (num_ranks < 1 || num_ranks > RC_MAX_RANKS)
        return Error{RC_ERR_INVALID_ARGUMENT, "register: num_ranks must be in [1, 16]"};
    Config c;
    Error e = read_config(cfg, &c);
    if (e.code) return e;
    DeviceInfo dev;
    if (!c.validate_only) {
        e = device_open(c, &dev);
        if (e.code) return e;
    }
    auto events = std::make_shared<RankEvents>();
    if (mode == Mode::PerRank && !c.validate_only) {
        events->arrive.assign(num_ranks, nullptr);
        for (int r = 0; r < num_ranks && !e.code; ++r) e = device_event_create(&events->arrive[r]);
        if (!e.code) e = device_event_create(&events->done);
        if (e.code) return e;
    }
    g_s = Session{};
    g_s.mode = mode;
    g_s.nranks = num_ranks;
    g_s.cfg = c;
    g_s.dev = dev;
    if (mode == Mode::PerRank) {
        Comm& world = g_s.comms[0];
        for (int r = 0; r < num_ranks; ++r) world.world.push_back(r);
        world.seq.assign(num_ranks, 0);
    }
    g_s.events = std::move(events);
    return {};
}

// Drops the session; waiting per-rank calls wake up and see the new generation.
void close_session() {
    g_s = Session{};
    ++g_generation;
    g_cv.notify_all();
}

// With RC_TUNE_LOG=1 in the environment, each choice of the occupancy tuner
// is reported on stderr: the launch shape, the rule's wave count, and each
// candidate's median time per GiB moved.
void log_tune_choice(const TuneKey& key, int rule_waves, const TuneEntry& t) {
    static const bool on = [] {
        const char* v = std::getenv("RC_TUNE_LOG");
        return v && std::strcmp(v, "0") != 0 && *v;
    }();
    if (!on) return;
    static const char* const kinds[] = {"fold", "copy", "copy batch"};
    const int kind = std::get<0>(key);
    std::string line = std::string("rankred tune: ") + (kind >= 0 && kind < 3 ? kinds[kind] : "?") + " whole-tile " +
                       std::to_string(std::get<1>(key)) + " in " + std::to_string(std::get<2>(key)) + " acc " +
                       std::to_string(std::get<3>(key)) + " out " + std::to_string(std::get<4>(key)) + " unroll " +
                       std::to_string(std::get<5>(key)) + " 2^" + std::to_string(std::get<6>(key)) +
                       " B: rule W=" + std::to_string(rule_waves) + ", chose W=" + std::to_string(t.chosen) + " (";
    for (int i = 0; i < t.ncand; ++i) {
        char buf[64];
        std::snprintf(buf, sizeof buf, "%sW=%d %.1f us/GiB", i ? ", " : "", t.cand[i], (double)t.median_us[i]);
        line += buf;
    }
    std::fprintf(stderr, "%s)\n", line.c_str());
}

// Runs `run(lds_bytes)`, one launch whose rule allows rule_waves waves per
// CU, under the occupancy tuner when it applies: the entry `key` picks the
// wave count, and a launch chosen for timing is bracketed by a timer.
// run(-1) keeps the plan's own reservation.  `capturing` caches whether
// `stream` is being captured (-1: not asked yet).  With `timed` false the
// launch makes no event or capture query at all: it takes the tuner's
// choice for the shape if there is one, else the rule's wave count.
template <class Run>
Error launch_tuned(const TuneKey& key, int rule_waves, int64_t moved, void* stream, int* capturing, bool timed,
                   Run run) {
    if (g_s.cfg.waves_per_cu > 0 || g_s.cfg.max_workgroups > 0 || rule_waves <= 0 || moved < kTuneMinBytes)
        return run(-1);
    if (!timed) {
        const auto it = g_s.tune.find(key);
        const int w = it != g_s.tune.end() ? it->second.chosen : 0;
        return run(w > 0 && w != rule_waves ? lds_for_waves(g_s.dev, w) : -1);
    }
    if (*capturing < 0) {
        bool c = false;
        Error e = device_stream_capturing(stream, &c);
        if (e.code) return e;
        *capturing = c ? 1 : 0;
    }
    TuneEntry& t = g_s.tune[key];
    // read the timed launches that have completed, without waiting; a
    // capturing call makes no event calls at all
    for (size_t i = 0; !*capturing && i < t.pending.size();) {
        bool done = false;
        float us = 0.0f;
        Error e = device_timer_read(t.pending[i].ticket, &done, &us);
        if (e.code) return e;
        if (done) {  // launches of one size class differ by up to 2x: compare time per GiB
            const bool open = !t.chosen;
            tune_record(t, t.pending[i].cand, (float)(us * (double)(int64_t(1) << 30) / (double)t.pending[i].bytes));
            if (open && t.chosen) log_tune_choice(key, rule_waves, t);
            t.pending.erase(t.pending.begin() + (std::ptrdiff_t)i);
        } else {
            ++i;
        }
    }
    int cand = -1;
    const int waves = tune_pick(t, rule_waves, &cand);
    if (*capturing && cand >= 0) {  // a captured launch is replayed later: not timed here
        --t.issued[cand];
        cand = -1;
    }
    const int lds = waves == rule_waves ? -1 : lds_for_waves(g_s.dev, waves);
    if (cand < 0) return run(lds);
    int ticket = -1;
    Error e = device_timer_start(stream, &ticket);
    if (!e.code) e = run(lds);
    if (!e.code) e = device_timer_stop(ticket, stream);
    if (e.code) return e;
    t.pending.push_back(TunePending{ticket, cand, moved});
    return {};
}

// Enqueues one validated collective.  With `timed` false nothing but kernel
// launches is enqueued (see launch_tuned).
Error launch(const Checked& ck, void* stream, bool timed = true) {
    const int64_t es = element_size(ck.dtype);
    int capturing = -1;  // asked once, when a launch could be tuned
    if (runs_as_copies(ck.coll)) {
        BatchPlan bp = plan_copies(ck, g_s.cfg, g_s.dev);
        if (!bp.total_tiles) return {};
        if (!bp.by_value) {  // tables through the arena: not capturable (see launch_batch)
            bool c = false;
            Error e = device_stream_capturing(stream, &c);
            if (e.code) return e;
            if (c)
                return Error{RC_ERR_INVALID_ARGUMENT, std::string(coll_name(ck.coll)) +
                                                          " with this many ranks cannot be captured into a graph"};
            return device_launch_batch(bp, stream);
        }
        int64_t elems = 0;  // every job reads len elements and writes them nout times
        for (const BatchJob& jb : bp.jobs) elems += jb.len;
        const int64_t moved = (1 + bp.nout) * elems * es;
        const TuneKey key{2, (bp.full_tiles ? 1 : 0) + (bp.shift_out ? 1 : 0), 1, 0, bp.nout, kCopyUnroll,
                          size_class(moved)};
        return launch_tuned(key, bp.waves, moved, stream, &capturing, timed, [&](int lds) {
            if (lds >= 0) bp.lds_bytes = lds;
            return device_launch_batch(bp, stream);
        });
    }
    for (LaunchPlan& p : plan(ck, g_s.cfg, g_s.dev)) {
        int64_t elems = 0;  // the launch's jobs: every element read from nin inputs, written nout times
        for (int c = 0; c < p.args.jobs; ++c)
            elems += std::max<int64_t>(0, std::min(p.args.seg, p.args.n - (int64_t)c * p.args.seg));
        const int64_t moved = (int64_t)(p.nin * (p.acc ? 2 : 1) + p.nout) * elems * es;
        if (!p.args.grid_2d) {
            Error e = device_launch(p, stream);
            if (e.code) return e;
            continue;
        }
        // a split fold runs the whole-tile kernels: tuned with them
        const TuneKey key{(int)p.args.in_mode, (p.args.full_tiles || p.split ? 1 : 0) + (p.shift_out ? 1 : 0), p.nin,
                          p.acc ? 1 : 0, p.nout, p.unroll, size_class(moved)};
        Error e = launch_tuned(key, p.waves, moved, stream, &capturing, timed, [&](int lds) {
            if (lds >= 0) p.lds_bytes = lds;
            return device_launch(p, stream);
        });
        if (e.code) return e;
    }
    return {};
}

// Registration checks of the whole-call entry points.
Error whole_call_session() {
    if (g_s.mode == Mode::None) return Error{RC_ERR_NOT_REGISTERED, "no session: call rc_register first"};
    if (g_s.mode == Mode::PerRank)
        return Error{RC_ERR_INVALID_ARGUMENT, "the session was opened per rank: use the rc_rank_* entry points"};
    return {};
}

int collective(Coll coll, const rc_buf* bufs, void* stream, void* const* recv_list = nullptr) {
    std::lock_guard<std::mutex> lock(g_mu);
    Error reg = whole_call_session();
    if (reg.code) return report(reg);
    Checked ck;
    Error e = validate(coll, g_s.nranks, bufs, &ck, recv_list);
    if (e.code) return report(e);
    if (g_s.cfg.validate_only) return ok();
    return report(launch(ck, stream));
}

// A validated batch of all-reduces: tensors large enough get launches of
// their own, the rest share one batched launch (one for tensors with
// accumulators and one for tensors without, when both occur).  With
// `use_static` the batched launches take their tables from the library's
// static scratch, and nothing but kernels is enqueued.
Error launch_batch(const std::vector<Checked>& cks, void* stream, bool use_static = false) {
    std::vector<Checked> own, batched;
    split_batch(cks, &own, &batched);
    if (use_static) {
        // every check before anything is enqueued
        BatchPlan parts[2];
        for (const bool acc : {false, true}) {
            std::vector<Checked> part;
            for (const Checked& ck : batched)
                if (ck.has_acc == acc) part.push_back(ck);
            parts[acc] = plan_batch(part, g_s.cfg, g_s.dev);
            const size_t need = batch_table_bytes(parts[acc]);
            if (parts[acc].total_tiles && need > kStaticScratchBytes)
                return Error{RC_ERR_INVALID_ARGUMENT,
                             "all_reduce_many_static: the tables of the " + std::to_string(part.size()) +
                                 " tensors under 64 MiB of traffic need " + std::to_string(need) +
                                 " bytes, more than the " + std::to_string(kStaticScratchBytes) +
                                 " bytes of static scratch"};
        }
        for (const Checked& ck : own) {
            Error e = launch(ck, stream, false);
            if (e.code) return e;
        }
        for (const BatchPlan& bp : parts) {
            if (bp.total_tiles == 0) continue;
            Error e = device_launch_batch_static(bp, stream);
            if (e.code) return e;
        }
        return {};
    }
    if (!batched.empty()) {
        // the batched launch uploads its tables from host staging that later
        // calls reuse, so a graph replay would read stale tables: refuse
        // capture before anything is enqueued
        bool capturing = false;
        Error e = device_stream_capturing(stream, &capturing);
        if (e.code) return e;
        if (capturing)
            return Error{RC_ERR_INVALID_ARGUMENT,
                         "the batched all-reduce cannot be captured into a graph (its descriptor tables are "
                         "uploaded from reused host staging); tensors of 64 MiB and more can be"};
    }
    for (const Checked& ck : own) {
        Error e = launch(ck, stream);
        if (e.code) return e;
    }
    for (const bool acc : {false, true}) {
        std::vector<Checked> part;
        for (const Checked& ck : batched)
            if (ck.has_acc == acc) part.push_back(ck);
        const BatchPlan bp = plan_batch(part, g_s.cfg, g_s.dev);
        if (bp.total_tiles == 0) continue;
        Error e = device_launch_batch(bp, stream);
        if (e.code) return e;
    }
    return {};
}

// Runs `enqueue` (the kernels of one matched collective) on `stream`, the
// last rank's, ordered against every rank's stream.  Every other rank is
// blocked inside its call and has enqueued nothing since making it, so an
// event recorded on its stream now marks that rank's call point; after the
// kernels, the same streams wait on `done` before anything the ranks enqueue
// once they return.  Each distinct stream is joined once, and a stream shared
// with the launching rank needs no event at all.
template <class Enqueue>
Error launch_joined(const std::vector<void*>& streams, void* stream, Enqueue enqueue) {
    RankEvents& ev = *g_s.events;
    std::vector<void*> others;
    for (void* s : streams)
        if (s != stream && std::find(others.begin(), others.end(), s) == others.end()) others.push_back(s);
    Error e;
    for (size_t i = 0; i < others.size() && !e.code; ++i) {
        e = device_event_record(ev.arrive[i], others[i]);
        if (!e.code) e = device_stream_wait(stream, ev.arrive[i]);
    }
    if (!e.code) e = enqueue();
    if (!e.code && !others.empty()) e = device_event_record(ev.done, stream);
    for (size_t i = 0; i < others.size() && !e.code; ++i) e = device_stream_wait(others[i], ev.done);
    return e;
}

const char* kind_name(const Slot& s, int r) {
    if (s.form[r] == kParams) return "all_reduce_params";
    if (s.form[r] == kSplit) return "split";
    return coll_name(s.kinds[r]);
}

// Pairs a gradient sync's entries by parameter ID and validates the batch.
Error check_params(int R, const std::vector<int>& counts, const std::vector<const rc_param*>& params,
                   std::vector<Checked>* cks) {
    std::vector<rc_buf> bufs;
    std::vector<const void*> accs;
    std::vector<uint64_t> order;
    Error e = match_params(R, counts.data(), params.data(), &bufs, &accs, &order);
    if (e.code) return e;
    return validate_batch(R, (int)order.size(), bufs.data(), cks, order.data(), accs.data());
}

// Communicator.split_all / split_from: the members named by the ranks that
// pass a list form a new communicator in that order; ranks that pass none are
// left out (the page's empty-list case) and get -1.  Every rank that passes a
// list must pass the same one, and every listed rank must pass it.
Error complete_split(Slot& s, const Comm& parent) {
    const int R = parent.size();
    int first = -1;
    for (int r = 0; r < R; ++r)
        if (s.has_list[r]) {
            if (first < 0) first = r;
            else if (s.members[r] != s.members[first])
                return Error{RC_ERR_INVALID_ARGUMENT, "split: ranks " + std::to_string(first) + " and " +
                                                          std::to_string(r) + " pass different member lists"};
        }
    s.result.assign(R, -1);
    if (first < 0) return {};  // nobody named a member: no communicator
    const std::vector<int>& list = s.members[first];
    std::vector<uint8_t> seen(R, 0);
    for (int m : list) {
        if (m < 0 || m >= R) return Error{RC_ERR_INVALID_ARGUMENT, "split: member " + std::to_string(m) + " outside the communicator"};
        if (seen[m]++) return Error{RC_ERR_INVALID_ARGUMENT, "split: member " + std::to_string(m) + " listed twice"};
        if (!s.has_list[m])
            return Error{RC_ERR_INVALID_ARGUMENT, "split: rank " + std::to_string(m) + " is listed but passed no list"};
    }
    if (g_s.next_comm >= (1 << 26)) return Error{RC_ERR_INVALID_ARGUMENT, "split: too many communicators"};
    const int id = g_s.next_comm++;
    Comm& c = g_s.comms[id];
    for (size_t i = 0; i < list.size(); ++i) {
        c.world.push_back(parent.world[list[i]]);
        s.result[list[i]] = id * RC_MAX_RANKS + (int)i;
    }
    c.seq.assign(list.size(), 0);
    return {};
}

// The last rank of a slot: check the R sides against each other and launch.
void complete_slot(Slot& s, const Comm& cm, void* stream) {
    if (s.status != RC_OK) return;  // an argument error recorded at arrival
    const int R = cm.size();
    for (int r = 1; r < R; ++r) {
        if (s.kinds[r] != s.kinds[0] || s.form[r] != s.form[0]) {
            s.status = RC_ERR_OP_MISMATCH;
            s.msg = std::string("rank ") + std::to_string(r) + " called " + kind_name(s, r) +
                    " where rank 0 called " + kind_name(s, 0);
            return;
        }
    }
    Error e;
    if (s.form[0] == kSplit) {
        e = complete_split(s, cm);
    } else if (s.kinds[0] == Coll::Barrier && s.form[0] == kCollective) {
        // Communicator.barrier: no data, only the stream join
        if (!g_s.cfg.validate_only) e = launch_joined(s.streams, stream, [] { return Error{}; });
    } else if (s.form[0] == kParams) {
        std::vector<const rc_param*> params(R);
        for (int r = 0; r < R; ++r) params[r] = s.params[r].data();
        std::vector<Checked> cks;
        e = check_params(R, s.pcount, params, &cks);
        if (!e.code && !g_s.cfg.validate_only)
            e = launch_joined(s.streams, stream, [&] { return launch_batch(cks, stream); });
    } else {
        for (int r = 0; r < R; ++r) {
            if (!s.have_buf[r]) {
                s.status = RC_ERR_INVALID_ARGUMENT;
                s.msg = "rank " + std::to_string(r) + " passed a NULL rc_buf";
                return;
            }
        }
        std::vector<void*> recv_list;
        if (s.kinds[0] == Coll::AllGatherList)
            for (int r = 0; r < R; ++r) recv_list.insert(recv_list.end(), s.recvs[r].begin(), s.recvs[r].end());
        Checked ck;
        e = validate(s.kinds[0], R, s.bufs.data(), &ck, recv_list.empty() ? nullptr : recv_list.data());
        if (!e.code && !g_s.cfg.validate_only)
            e = launch_joined(s.streams, stream, [&] { return launch(ck, stream); });
    }
    if (e.code) s.result.assign(R, -1);
    s.status = e.code;
    s.msg = e.msg;
}

// One rank's side of a per-rank call.
struct RankArgs {
    Coll coll = Coll::AllReduce;
    Form form = kCollective;
    const rc_buf* buf = nullptr;
    int count = 0;                     // all_reduce_params entries, or split members
    const rc_param* entries = nullptr;
    const int* members = nullptr;
    bool missing_out = false;          // split without a place for its result
    void* const* recvs = nullptr;      // all_gather list form: R outputs
};

// Resolves an endpoint of the per-rank front end (the caller holds g_mu).
Error resolve(int ep, int* id, int* local, int* world) {
    if (g_s.mode != Mode::PerRank)
        return Error{RC_ERR_NOT_REGISTERED, "no per-rank session: call rc_rank_register first"};
    if (ep < 0) return Error{RC_ERR_INVALID_ARGUMENT, "rank outside [0, num_ranks)"};
    *id = ep / RC_MAX_RANKS;
    *local = ep % RC_MAX_RANKS;
    auto it = g_s.comms.find(*id);
    if (it == g_s.comms.end() || *local >= it->second.size()) {
        if (*id == 0) return Error{RC_ERR_INVALID_ARGUMENT, "rank outside [0, num_ranks)"};
        return Error{RC_ERR_NOT_REGISTERED, "endpoint " + std::to_string(ep) + " names no communicator"};
    }
    *world = it->second.world[*local];
    if (!((g_s.reg_mask >> *world) & 1u) || ((g_s.fin_mask >> *world) & 1u) ||
        ((it->second.fin_mask >> *local) & 1u))
        return Error{RC_ERR_NOT_REGISTERED, "rank " + std::to_string(ep) + " is not registered"};
    return {};
}

// Whether member `local` of `cm` has left: it finished its endpoint in a
// split-off communicator, or its world rank, which ends all its endpoints.
bool member_left(const Comm& cm, int local) {
    return ((cm.fin_mask >> local) & 1u) || ((g_s.fin_mask >> cm.world[local]) & 1u);
}

Error check_members(const Comm& cm) {
    for (int i = 0; i < cm.size(); ++i)
        if (member_left(cm, i))
            return Error{RC_ERR_NOT_REGISTERED, "rank " + std::to_string(i) +
                                                    " of this communicator has finished: the call cannot complete"};
    return {};
}

// Member `local` of `cm` is leaving: the calls of other members that wait for
// it could never complete, so they end now with RC_ERR_NOT_REGISTERED (later
// calls are refused by check_members).  The caller holds g_mu and notifies.
void abandon_waits(Comm& cm, int local) {
    const std::string why = "rank " + std::to_string(local) + " of the communicator finished before joining this ";
    for (auto& kv : cm.slots) {
        Slot& s = *kv.second;
        if (s.done || ((s.arrived >> local) & 1u)) continue;
        s.status = RC_ERR_NOT_REGISTERED;
        s.msg = why + "call";
        s.abandoned = true;
        s.done = true;
    }
    for (auto& kv : cm.pairs) {
        PairSlot& p = *kv.second;
        const int src = std::get<0>(kv.first), dst = std::get<1>(kv.first);
        if (p.done || !((src == local && !p.have[0]) || (dst == local && !p.have[1]))) continue;
        p.status = RC_ERR_NOT_REGISTERED;
        p.msg = why + (src == local ? "send" : "recv");
        p.abandoned = true;
        p.done = true;
    }
}

Error claim(int world) {
    const uint32_t bit = 1u << world;
    if (g_s.busy_mask & bit)
        return Error{RC_ERR_INVALID_ARGUMENT,
                     "rank " + std::to_string(world) + " already has a call in progress on another thread"};
    g_s.busy_mask |= bit;
    return {};
}

int rank_collective(const RankArgs& a, int ep, void* stream, int* split_result = nullptr) {
    std::unique_lock<std::mutex> lock(g_mu);
    int id = 0, rank = 0, world = 0;
    Error e0 = resolve(ep, &id, &rank, &world);
    if (!e0.code) e0 = check_members(g_s.comms[id]);
    if (!e0.code) e0 = claim(world);
    if (e0.code) return report(e0);
    Comm& cm = g_s.comms[id];
    const int R = cm.size();
    const uint64_t gen = g_generation;
    const uint64_t k = cm.seq[rank]++;
    std::shared_ptr<Slot>& sp = cm.slots[k];
    if (!sp) {
        sp = std::make_shared<Slot>();
        sp->kinds.assign(R, Coll::AllReduce);
        sp->bufs.assign(R, rc_buf{});
        sp->have_buf.assign(R, 0);
        sp->streams.assign(R, nullptr);
        sp->form.assign(R, kCollective);
        sp->pcount.assign(R, 0);
        sp->params.assign(R, {});
        sp->recvs.assign(R, {});
        sp->has_list.assign(R, 0);
        sp->members.assign(R, {});
    }
    std::shared_ptr<Slot> s = sp;
    s->kinds[rank] = a.coll;
    s->form[rank] = a.form;
    auto arg_error = [&](const std::string& msg) {
        if (s->status == RC_OK) {
            s->status = RC_ERR_INVALID_ARGUMENT;
            s->msg = "rank " + std::to_string(rank) + ": " + msg;
        }
    };
    if (a.form == kParams) {
        // copied now: the caller's arrays need only live through the call
        if (a.count < 0 || (a.count > 0 && !a.entries)) {
            arg_error("all_reduce_params needs num_params >= 0 and a non-NULL params array");
        } else {
            s->pcount[rank] = a.count;
            s->params[rank].assign(a.entries, a.entries + a.count);
        }
    } else if (a.form == kSplit) {
        if (a.missing_out) {
            arg_error("split needs somewhere to return the new rank");
        } else if (a.count < 0 || (a.count > 0 && !a.members)) {
            arg_error("split needs num_members >= 0 and a non-NULL members array");
        } else if (a.count > 0) {
            s->has_list[rank] = 1;
            s->members[rank].assign(a.members, a.members + a.count);
        }
    } else if (a.buf) {
        s->bufs[rank] = *a.buf;
        s->have_buf[rank] = 1;
    } else if (a.coll == Coll::Barrier) {
        s->have_buf[rank] = 1;  // nothing to describe
    }
    if (a.form == kCollective && a.coll == Coll::AllGatherList) {
        if (a.recvs) s->recvs[rank].assign(a.recvs, a.recvs + R);
        else arg_error("all_gather_list needs its recvs array");
    }
    s->streams[rank] = stream;
    s->arrived |= 1u << rank;
    if (s->arrived == (uint32_t)((1ull << R) - 1)) {
        complete_slot(*s, cm, stream);
        s->done = true;
        g_cv.notify_all();
    } else {
        g_cv.wait(lock, [&] { return s->done || g_generation != gen; });
        if (g_generation != gen)
            return report(Error{RC_ERR_NOT_REGISTERED, "the session was reset or closed while rank " +
                                                           std::to_string(ep) + " waited"});
    }
    g_s.busy_mask &= ~(1u << world);
    const Error e{s->status, s->msg};
    if (split_result) *split_result = s->result.empty() ? -1 : s->result[rank];
    // the communicator outlives every call in progress on it (a member cannot
    // finish while it is inside a call), so cm is still valid here; nobody
    // joins an abandoned slot after it ended
    if (++s->left == (s->abandoned ? __builtin_popcount(s->arrived) : R)) cm.slots.erase(k);
    return report(e);
}

// Communicator.send / recv on logical ranks: pairs are matched per ordered
// (src, dst) of one communicator in issue order, independently of the other
// ranks' calls.  The first side to arrive waits for its peer; the second
// validates both sides and copies on its stream, joined with the peer's.
int rank_p2p(bool is_send, int ep, int peer, const rc_buf* buf, void* stream) {
    std::unique_lock<std::mutex> lock(g_mu);
    int id = 0, rank = 0, world = 0;
    Error e0 = resolve(ep, &id, &rank, &world);
    if (e0.code) return report(e0);
    Comm& cm = g_s.comms[id];
    const int R = cm.size();
    if (peer < 0 || peer >= R || peer == rank)
        return report(Error{RC_ERR_INVALID_ARGUMENT, std::string(is_send ? "send: dst " : "recv: src ") +
                                                         std::to_string(peer) + " is not another rank"});
    if (member_left(cm, peer))
        return report(Error{RC_ERR_NOT_REGISTERED, std::string(is_send ? "send: dst " : "recv: src ") +
                                                       std::to_string(peer) + " has finished"});
    e0 = claim(world);
    if (e0.code) return report(e0);
    const uint64_t gen = g_generation;
    const int src = is_send ? rank : peer, dst = is_send ? peer : rank;
    const int side = is_send ? 0 : 1;
    const uint64_t k = (is_send ? cm.sends_posted : cm.recvs_posted)[{src, dst}]++;
    const auto key = std::make_tuple(src, dst, k);
    std::shared_ptr<PairSlot>& sp = cm.pairs[key];
    if (!sp) sp = std::make_shared<PairSlot>();
    std::shared_ptr<PairSlot> s = sp;
    s->have[side] = true;
    if (buf) s->bufs[side] = *buf;
    else s->null_buf = true;
    s->streams[side] = stream;
    if (s->have[0] && s->have[1]) {
        Error e;
        if (s->null_buf) e = Error{RC_ERR_INVALID_ARGUMENT, "send_recv: a side passed a NULL rc_buf"};
        Checked ck;
        if (!e.code) e = validate_send_recv(R, src, dst, s->bufs, &ck);
        if (!e.code && !g_s.cfg.validate_only) {
            const std::vector<void*> streams = {s->streams[0], s->streams[1]};
            e = launch_joined(streams, stream, [&] { return launch(ck, stream); });
        }
        s->status = e.code;
        s->msg = e.msg;
        s->done = true;
        g_cv.notify_all();
    } else {
        g_cv.wait(lock, [&] { return s->done || g_generation != gen; });
        if (g_generation != gen)
            return report(Error{RC_ERR_NOT_REGISTERED, "the session was reset or closed while rank " +
                                                           std::to_string(ep) + " waited"});
    }
    g_s.busy_mask &= ~(1u << world);
    const Error e{s->status, s->msg};
    if (++s->left == (s->abandoned ? (int)s->have[0] + (int)s->have[1] : 2)) cm.pairs.erase(key);
    return report(e);
}

}  // namespace
}  // namespace rc

using namespace rc;

extern "C" {

int rc_register(int num_ranks, const rc_config* cfg) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_s.mode != Mode::None)
        return report(Error{RC_ERR_DUPLICATE_REGISTRATION, "rc_register: a session is already open"});
    return report(open_session(Mode::Whole, num_ranks, cfg));
}

int rc_all_reduce(const rc_buf* bufs, void* stream) { return collective(Coll::AllReduce, bufs, stream); }
int rc_reduce(const rc_buf* bufs, void* stream) { return collective(Coll::Reduce, bufs, stream); }
int rc_broadcast(const rc_buf* bufs, void* stream) { return collective(Coll::Broadcast, bufs, stream); }
int rc_reduce_scatter(const rc_buf* bufs, void* stream) {
    return collective(Coll::ReduceScatter, bufs, stream);
}
int rc_all_gather(const rc_buf* bufs, void* stream) { return collective(Coll::AllGather, bufs, stream); }
int rc_all_gather_list(const rc_buf* bufs, void* const* recvs, void* stream) {
    return collective(Coll::AllGatherList, bufs, stream, recvs);
}
int rc_all_to_all_single(const rc_buf* bufs, void* stream) { return collective(Coll::AllToAll, bufs, stream); }

int rc_send_recv(int src, int dst, const rc_buf* bufs, void* stream) {
    std::lock_guard<std::mutex> lock(g_mu);
    Error e = whole_call_session();
    if (e.code) return report(e);
    Checked ck;
    e = validate_send_recv(g_s.nranks, src, dst, bufs, &ck);
    if (e.code) return report(e);
    if (g_s.cfg.validate_only) return ok();
    return report(launch(ck, stream));
}

int rc_barrier(void* stream) {
    (void)stream;  // every rank's work is on the one stream of the calls, already in order
    std::lock_guard<std::mutex> lock(g_mu);
    return report(whole_call_session());
}

int rc_all_reduce_many(int num_tensors, const rc_buf* bufs, void* stream) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_s.mode == Mode::None)
        return report(Error{RC_ERR_NOT_REGISTERED, "no session: call rc_register first"});
    if (g_s.mode == Mode::PerRank)
        return report(Error{RC_ERR_INVALID_ARGUMENT, "the session was opened per rank"});
    std::vector<Checked> cks;
    Error e = validate_batch(g_s.nranks, num_tensors, bufs, &cks);
    if (e.code) return report(e);
    if (g_s.cfg.validate_only) return ok();
    return report(launch_batch(cks, stream));
}

int rc_all_reduce_many_static(int num_tensors, const rc_buf* bufs, void* stream) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_s.mode == Mode::None)
        return report(Error{RC_ERR_NOT_REGISTERED, "no session: call rc_register first"});
    if (g_s.mode == Mode::PerRank)
        return report(Error{RC_ERR_INVALID_ARGUMENT, "the session was opened per rank"});
    std::vector<Checked> cks;
    Error e = validate_batch(g_s.nranks, num_tensors, bufs, &cks);
    if (e.code) return report(e);
    if (g_s.cfg.validate_only) return ok();
    return report(launch_batch(cks, stream, true));
}

int rc_all_reduce_params(const int* num_params, const rc_param* const* params, void* stream) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_s.mode == Mode::None)
        return report(Error{RC_ERR_NOT_REGISTERED, "no session: call rc_register first"});
    if (g_s.mode == Mode::PerRank)
        return report(Error{RC_ERR_INVALID_ARGUMENT, "the session was opened per rank"});
    const int R = g_s.nranks;
    if (!num_params || !params)
        return report(Error{RC_ERR_INVALID_ARGUMENT, "all_reduce_params: NULL num_params or params"});
    std::vector<int> counts(num_params, num_params + R);
    std::vector<Checked> cks;
    Error e = check_params(R, counts, std::vector<const rc_param*>(params, params + R), &cks);
    if (e.code) return report(e);
    if (g_s.cfg.validate_only) return ok();
    return report(launch_batch(cks, stream));
}

int rc_finish(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_s.mode == Mode::None)
        return report(Error{RC_ERR_NOT_REGISTERED, "rc_finish: no session is open"});
    if (g_s.mode == Mode::PerRank)
        return report(Error{RC_ERR_INVALID_ARGUMENT, "rc_finish: the session was opened per rank; "
                                                     "every rank calls rc_rank_finish"});
    Error e;
    if (!g_s.cfg.validate_only) e = device_finish();
    close_session();
    return report(e);
}

int rc_reset(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_s.mode != Mode::None && !g_s.cfg.validate_only) device_reset();
    close_session();
    return ok();
}

int rc_rank_register(int rank, int num_ranks, const rc_config* cfg) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_s.mode == Mode::Whole)
        return report(Error{RC_ERR_DUPLICATE_REGISTRATION, "rc_rank_register: a whole-call session is open"});
    if (g_s.mode == Mode::None) {
        Error e = open_session(Mode::PerRank, num_ranks, cfg);
        if (e.code) return report(e);
    } else if (num_ranks != g_s.nranks) {
        return report(Error{RC_ERR_INVALID_ARGUMENT, "rc_rank_register: num_ranks " + std::to_string(num_ranks) +
                                                         " differs from the session's " +
                                                         std::to_string(g_s.nranks)});
    }
    if (rank < 0 || rank >= g_s.nranks)
        return report(Error{RC_ERR_INVALID_ARGUMENT, "rc_rank_register: rank outside [0, num_ranks)"});
    if ((g_s.reg_mask >> rank) & 1u)
        return report(Error{RC_ERR_DUPLICATE_REGISTRATION,
                            "rc_rank_register: rank " + std::to_string(rank) + " is already registered"});
    g_s.reg_mask |= 1u << rank;
    return ok();
}

static int rank_call(Coll coll, int rank, const rc_buf* buf, void* stream) {
    RankArgs a;
    a.coll = coll;
    a.buf = buf;
    return rank_collective(a, rank, stream);
}

int rc_rank_all_reduce(int rank, const rc_buf* buf, void* stream) {
    return rank_call(Coll::AllReduce, rank, buf, stream);
}
int rc_rank_reduce(int rank, const rc_buf* buf, void* stream) { return rank_call(Coll::Reduce, rank, buf, stream); }
int rc_rank_broadcast(int rank, const rc_buf* buf, void* stream) {
    return rank_call(Coll::Broadcast, rank, buf, stream);
}
int rc_rank_reduce_scatter(int rank, const rc_buf* buf, void* stream) {
    return rank_call(Coll::ReduceScatter, rank, buf, stream);
}
int rc_rank_all_gather(int rank, const rc_buf* buf, void* stream) {
    return rank_call(Coll::AllGather, rank, buf, stream);
}
int rc_rank_all_gather_list(int rank, const rc_buf* buf, void* const* recvs, void* stream) {
    RankArgs a;
    a.coll = Coll::AllGatherList;
    a.buf = buf;
    a.recvs = recvs;
    return rank_collective(a, rank, stream);
}
int rc_rank_all_to_all_single(int rank, const rc_buf* buf, void* stream) {
    return rank_call(Coll::AllToAll, rank, buf, stream);
}
int rc_rank_send(int rank, const rc_buf* buf, int dst, void* stream) { return rank_p2p(true, rank, dst, buf, stream); }
int rc_rank_recv(int rank, const rc_buf* buf, int src, void* stream) { return rank_p2p(false, rank, src, buf, stream); }
int rc_rank_barrier(int rank, void* stream) {
    RankArgs a;
    a.coll = Coll::Barrier;
    return rank_collective(a, rank, stream);
}
int rc_rank_all_reduce_params(int rank, int num_params, const rc_param* params, void* stream) {
    RankArgs a;
    a.form = kParams;
    a.count = num_params;
    a.entries = params;
    return rank_collective(a, rank, stream);
}

int rc_rank_split(int rank, int num_members, const int* members, int* new_rank) {
    RankArgs a;
    a.form = kSplit;
    a.count = num_members;
    a.members = members;
    a.missing_out = new_rank == nullptr;
    int result = -1;
    const int rc = rank_collective(a, rank, nullptr, &result);
    if (new_rank) *new_rank = rc == RC_OK ? result : -1;
    return rc;
}

int rc_rank_finish(int rank) {
    std::lock_guard<std::mutex> lock(g_mu);
    int id = 0, local = 0, world = 0;
    if (resolve(rank, &id, &local, &world).code)
        return report(Error{RC_ERR_NOT_REGISTERED, "rc_rank_finish: rank is not registered"});
    if ((g_s.busy_mask >> world) & 1u)  // a call of this rank is still waiting on another thread
        return report(Error{RC_ERR_INVALID_ARGUMENT, "rc_rank_finish: the rank has a call in progress"});
    if (id != 0) {
        // a split-off communicator goes away when all its members have finished
        Comm& c = g_s.comms[id];
        c.fin_mask |= 1u << local;
        abandon_waits(c, local);
        g_cv.notify_all();
        if (c.fin_mask == (uint32_t)((1ull << c.size()) - 1)) g_s.comms.erase(id);
        return ok();
    }
    g_s.fin_mask |= 1u << world;
    // the world rank leaves every communicator it belongs to
    for (auto& kv : g_s.comms) {
        Comm& c = kv.second;
        const auto it = std::find(c.world.begin(), c.world.end(), world);
        if (it != c.world.end()) abandon_waits(c, (int)(it - c.world.begin()));
    }
    g_cv.notify_all();
    if (g_s.fin_mask != g_s.reg_mask) return ok();
    Error e;
    if (!g_s.cfg.validate_only) e = device_finish();
    close_session();
    return report(e);
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
        case RC_ERR_PARAM_MISMATCH: return "RC_ERR_PARAM_MISMATCH";
        default: return "RC_UNKNOWN_STATUS";
    }
}

int rc_abi_version(void) { return RC_ABI_VERSION; }

}  // extern "C"
