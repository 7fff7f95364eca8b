// Host-only stress of the C ABI in validate-only sessions (no GPU): many
// threads issue valid and invalid collectives while others register, finish
// and reset.  Built with AddressSanitizer or ThreadSanitizer by the tests; the
// program checks that every call returns a documented status and that a
// valid call in an open session succeeds.  Links session.cpp, validate.cpp,
// plan.cpp and stub device functions (validate-only sessions never reach them).
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

#include "rc.h"
#include "rc_internal.h"

namespace rc {
// validate-only sessions never call into the device layer
Error device_open(const Config&, DeviceInfo*) { return Error{RC_ERR_DEVICE, "no device in this test"}; }
Error device_launch(const LaunchPlan&, void*) { return Error{RC_ERR_DEVICE, "no device in this test"}; }
Error device_launch_batch(const BatchPlan&, void*) { return Error{RC_ERR_DEVICE, "no device in this test"}; }
size_t batch_table_bytes(const BatchPlan&) { return 0; }
Error device_launch_batch_static(const BatchPlan&, void*) { return Error{RC_ERR_DEVICE, "no device in this test"}; }
Error device_finish() { return {}; }
void device_reset() {}
Error device_event_create(void**) { return Error{RC_ERR_DEVICE, "no device in this test"}; }
void device_event_destroy(void*) {}
Error device_event_record(void*, void*) { return Error{RC_ERR_DEVICE, "no device in this test"}; }
Error device_stream_wait(void*, void*) { return Error{RC_ERR_DEVICE, "no device in this test"}; }
Error device_timer_start(void*, int*) { return Error{RC_ERR_DEVICE, "no device in this test"}; }
Error device_timer_stop(int, void*) { return Error{RC_ERR_DEVICE, "no device in this test"}; }
Error device_timer_read(int, bool* done, float*) {
    *done = false;
    return Error{RC_ERR_DEVICE, "no device in this test"};
}
Error device_stream_capturing(void*, bool* c) {
    *c = false;
    return Error{RC_ERR_DEVICE, "no device in this test"};
}
}  // namespace rc

namespace {

std::atomic<int> g_bad{0};

rc_buf buf(uintptr_t s, uintptr_t r, int64_t n, int dtype = RC_F32, int op = RC_SUM, int root = 0) {
    rc_buf b;
    std::memset(&b, 0, sizeof b);
    b.send = reinterpret_cast<const void*>(s);
    b.recv = reinterpret_cast<void*>(r);
    b.dtype = dtype;
    b.op = op;
    b.root = root;
    b.ndim = 1;
    b.dims[0] = n;
    return b;
}

void worker(int id, int iters, int R) {
    std::mt19937 rng(id);
    std::vector<rc_buf> bufs(R);
    for (int i = 0; i < iters; ++i) {
        const int64_t n = 1 + rng() % 100000;
        const uintptr_t base = 0x100000000ull + (uintptr_t)id * 0x10000000ull;
        for (int r = 0; r < R; ++r) bufs[r] = buf(base + r * 0x800000ull, base + 0x8000000ull + r * 0x800000ull, n);
        const int kind = rng() % 6;
        if (kind == 5) bufs[rng() % R].dims[0] += 1;  // shape mismatch
        int rc = 0;
        switch (kind) {
            case 0: rc = rc_all_reduce(bufs.data(), nullptr); break;
            case 1: rc = rc_reduce(bufs.data(), nullptr); break;
            case 2:
                for (int r = 1; r < R; ++r) bufs[r].send = nullptr;
                rc = rc_broadcast(bufs.data(), nullptr);
                break;
            case 3: rc = rc_all_gather(bufs.data(), nullptr); break;
            case 4: rc = rc_all_reduce_many(1, bufs.data(), nullptr); break;
            default: rc = rc_all_reduce(bufs.data(), nullptr); break;
        }
        const char* err = rc_last_error();
        if (rc < 0 || rc > RC_ERR_PARAM_MISMATCH) ++g_bad;
        if (rc == RC_OK && err[0] != '\0') ++g_bad;
        if (rc != RC_OK && err[0] == '\0') ++g_bad;
        if (kind == 5 && rc == RC_OK) ++g_bad;  // a mismatch must never pass
    }
}

void lifecycle(int iters, int R) {
    rc_config cfg;
    std::memset(&cfg, 0, sizeof cfg);
    cfg.struct_size = sizeof cfg;
    cfg.device = -1;
    cfg.validate_only = 1;
    for (int i = 0; i < iters; ++i) {
        const int rc = rc_register(R, &cfg);
        if (rc != RC_OK && rc != RC_ERR_DUPLICATE_REGISTRATION) ++g_bad;
        if (i % 3 == 0) {
            const int f = rc_finish();
            if (f != RC_OK && f != RC_ERR_NOT_REGISTERED) ++g_bad;
        } else if (i % 3 == 1) {
            if (rc_reset() != RC_OK) ++g_bad;
        }
    }
}

// Random field values (pointers are never dereferenced in validate-only
// sessions): every call must return a documented status without crashing.
void fuzz(int iters, int R) {
    std::mt19937_64 rng(99);
    std::vector<rc_buf> bufs(R * 3);
    for (int i = 0; i < iters; ++i) {
        for (rc_buf& b : bufs) {
            b.send = (rng() % 4) ? reinterpret_cast<const void*>(rng() & 0xFFFFFFFFFFFull) : nullptr;
            b.recv = (rng() % 4) ? reinterpret_cast<void*>(rng() & 0xFFFFFFFFFFFull) : nullptr;
            b.dtype = (int32_t)(rng() % 4) - 1;
            b.op = (int32_t)(rng() % 5) - 1;
            b.root = (int32_t)(rng() % (R + 3)) - 2;
            b.ndim = (int32_t)(rng() % 11) - 1;
            for (int d = 0; d < RC_MAX_DIMS; ++d)
                b.dims[d] = (rng() % 8 == 0) ? (int64_t)(rng() >> 1) * ((rng() % 2) ? 1 : -1) : (int64_t)(rng() % 70);
        }
        std::vector<void*> recvs(R * R);
        for (void*& p : recvs) p = (rng() % 8) ? reinterpret_cast<void*>(rng() & 0xFFFFFFFFFFFull) : nullptr;
        int rc;
        switch (rng() % 9) {
            case 0: rc = rc_all_reduce(bufs.data(), nullptr); break;
            case 1: rc = rc_reduce(bufs.data(), nullptr); break;
            case 2: rc = rc_broadcast(bufs.data(), nullptr); break;
            case 3: rc = rc_reduce_scatter(bufs.data(), nullptr); break;
            case 4: rc = rc_all_gather(bufs.data(), nullptr); break;
            case 5: rc = rc_all_to_all_single(bufs.data(), nullptr); break;
            case 6: rc = rc_all_gather_list(bufs.data(), (rng() % 5) ? recvs.data() : nullptr, nullptr); break;
            case 7: rc = rc_send_recv((int)(rng() % (R + 2)) - 1, (int)(rng() % (R + 2)) - 1, bufs.data(), nullptr); break;
            default: rc = rc_all_reduce_many(3, bufs.data(), nullptr); break;
        }
        if (rc < 0 || rc > RC_ERR_PARAM_MISMATCH) ++g_bad;
    }
}

// Per-rank front end: one thread per rank, calls matched by issue order; every
// 7th collective has a shape mismatch on rank 0, which every rank must see.
void rank_thread(int rank, int R, int iters) {
    for (int i = 0; i < iters; ++i) {
        int64_t n = 1 + (i * 7919) % 5000;
        if (i % 7 == 3 && rank == 0) n += 1;
        const uintptr_t base = 0x200000000ull + (uintptr_t)rank * 0x1000000ull;
        rc_buf b = buf(base, base + 0x800000ull, n);
        int rc;
        switch (i % 3) {
            case 0: rc = rc_rank_all_reduce(rank, &b, nullptr); break;
            case 1: rc = rc_rank_reduce(rank, &b, nullptr); break;
            default: rc = rc_rank_all_gather(rank, &b, nullptr); break;
        }
        const int want = i % 7 == 3 ? RC_ERR_SHAPE_MISMATCH : RC_OK;
        if (rc != want) ++g_bad;
    }
    if (rc_rank_finish(rank) != RC_OK) ++g_bad;
}

void rank_session(int R, int iters) {
    rc_config cfg;
    std::memset(&cfg, 0, sizeof cfg);
    cfg.struct_size = sizeof cfg;
    cfg.device = -1;
    cfg.validate_only = 1;
    for (int r = 0; r < R; ++r)
        if (rc_rank_register(r, R, &cfg) != RC_OK) ++g_bad;
    std::vector<std::thread> ts;
    for (int r = 0; r < R; ++r) ts.emplace_back(rank_thread, r, R, iters);
    for (auto& t : ts) t.join();
}

// Communicator splits under threads: the six ranks split into two groups of
// three over and over, run collectives, a send/recv ring and a barrier inside
// their group, and leave it.
void group_thread(int rank, int rounds) {
    const int evens[3] = {0, 2, 4}, odds[3] = {5, 3, 1};
    const int parity = rank % 2;
    const uintptr_t base = 0x400000000ull + (uintptr_t)rank * 0x1000000ull;
    for (int it = 0; it < rounds; ++it) {
        int ep_even = -2, ep_odd = -2;
        if (rc_rank_split(rank, parity ? 0 : 3, evens, &ep_even) != RC_OK) ++g_bad;
        if (rc_rank_split(rank, parity ? 3 : 0, odds, &ep_odd) != RC_OK) ++g_bad;
        const int ep = parity ? ep_odd : ep_even;
        if (ep < RC_MAX_RANKS || (parity ? ep_even : ep_odd) != -1) {
            ++g_bad;
            return;
        }
        const int local = ep % RC_MAX_RANKS, size = 3;
        for (int j = 0; j < 12; ++j) {
            rc_buf b = buf(base, base + 0x800000ull, 1 + (j * 131) % 3000);
            if (rc_rank_all_reduce(ep, &b, nullptr) != RC_OK) ++g_bad;
        }
        rc_buf s = buf(base, 0, 64), d = buf(0, base + 0x800000ull, 64);
        const int nxt = (local + 1) % size, prv = (local + size - 1) % size;
        int a, c;
        if (local % 2 == 0) {
            a = rc_rank_send(ep, &s, nxt, nullptr);
            c = rc_rank_recv(ep, &d, prv, nullptr);
        } else {
            c = rc_rank_recv(ep, &d, prv, nullptr);
            a = rc_rank_send(ep, &s, nxt, nullptr);
        }
        if (a != RC_OK || c != RC_OK) ++g_bad;
        if (rc_rank_barrier(ep, nullptr) != RC_OK) ++g_bad;
        if (rc_rank_finish(ep) != RC_OK) ++g_bad;
    }
    if (rc_rank_finish(rank) != RC_OK) ++g_bad;
}

void group_session(int rounds) {
    rc_config cfg;
    std::memset(&cfg, 0, sizeof cfg);
    cfg.struct_size = sizeof cfg;
    cfg.device = -1;
    cfg.validate_only = 1;
    for (int r = 0; r < 6; ++r)
        if (rc_rank_register(r, 6, &cfg) != RC_OK) ++g_bad;
    std::vector<std::thread> ts;
    for (int r = 0; r < 6; ++r) ts.emplace_back(group_thread, r, rounds);
    for (auto& t : ts) t.join();
}

// A rank leaving early: in each round one rank finishes after `stop` calls
// while the others keep calling.  Their next call must end with
// RC_ERR_NOT_REGISTERED, released from its wait or refused at once, and the
// session must close once they have finished too.
void leave_thread(int rank, int R, int round) {
    const int leaver = round % R, stop = round % 5;
    const uintptr_t base = 0x600000000ull + (uintptr_t)rank * 0x1000000ull;
    for (int i = 0; !(rank == leaver && i == stop); ++i) {
        rc_buf b = buf(base, base + 0x800000ull, 1 + (i * 37) % 2000);
        const int rc = (i % 2) ? rc_rank_all_reduce(rank, &b, nullptr) : rc_rank_barrier(rank, nullptr);
        if (i < stop) {
            if (rc != RC_OK) ++g_bad;
            continue;
        }
        if (rc != RC_ERR_NOT_REGISTERED) ++g_bad;
        break;
    }
    if (rc_rank_finish(rank) != RC_OK) ++g_bad;
}

void leave_session(int R, int rounds) {
    rc_config cfg;
    std::memset(&cfg, 0, sizeof cfg);
    cfg.struct_size = sizeof cfg;
    cfg.device = -1;
    cfg.validate_only = 1;
    for (int round = 0; round < rounds; ++round) {
        for (int r = 0; r < R; ++r)
            if (rc_rank_register(r, R, &cfg) != RC_OK) ++g_bad;  // a new session each round
        std::vector<std::thread> ts;
        for (int r = 0; r < R; ++r) ts.emplace_back(leave_thread, r, R, round);
        for (auto& t : ts) t.join();
    }
}

}  // namespace

int main() {
    rank_session(6, 3000);
    group_session(200);
    leave_session(6, 300);
    const int R = 8;
    rc_config cfg;
    std::memset(&cfg, 0, sizeof cfg);
    cfg.struct_size = sizeof cfg;
    cfg.device = -1;
    cfg.validate_only = 1;
    if (rc_register(R, &cfg) != RC_OK) return 2;
    // with the session held open, every valid call must succeed
    {
        std::vector<rc_buf> bufs(R);
        for (int r = 0; r < R; ++r) bufs[r] = buf(0x10000 * (r + 1), 0x1000000 + 0x10000 * r, 1000);
        if (rc_all_reduce(bufs.data(), nullptr) != RC_OK) return 3;
    }
    fuzz(20000, R);
    std::vector<std::thread> ts;
    for (int t = 0; t < 6; ++t) ts.emplace_back(worker, t, 3000, R);
    ts.emplace_back(lifecycle, 2000, R);
    for (auto& t : ts) t.join();
    rc_reset();
    std::printf("abi stress: %d bad results\n", g_bad.load());
    return g_bad.load() ? 1 : 0;
}
