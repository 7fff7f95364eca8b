// Argument checks for every collective, producing the CollectiveError cases of
// the ruCCL README (ja), section 4 "Errors and lifecycle": shape mismatch,
// inconsistent reduction op or root, invalid broadcast sender count.  The
// call contract they enforce is section 3 "Registration and call contract":
// ranks call matching collectives with the same shape, op and root, and each
// broadcast has exactly one sender.  Host-only C++; nothing here touches HIP.
#include <algorithm>
#include <cstdio>
#include <string>
#include <vector>

#include "rc_internal.h"

namespace rc {
namespace {

// Largest element count accepted per buffer (2^44 elements = 64 TiB of f32).
constexpr int64_t kMaxCount = int64_t(1) << 44;

std::string fmt(const char* f, long long a = 0, long long b = 0, long long c = 0) {
    char buf[256];
    std::snprintf(buf, sizeof buf, f, a, b, c);
    return buf;
}

Error fail(int code, std::string msg) { return Error{code, std::move(msg)}; }

bool reduces(Coll c) {
    return c == Coll::AllReduce || c == Coll::Reduce || c == Coll::ReduceScatter;
}

Error count_of(const rc_buf& b, int r, int64_t* count) {
    if (b.ndim < 0 || b.ndim > RC_MAX_DIMS)
        return fail(RC_ERR_INVALID_ARGUMENT, fmt("rank %lld: ndim %lld outside [0, 8]", r, b.ndim));
    int64_t n = 1;
    for (int d = 0; d < b.ndim; ++d) {
        if (b.dims[d] < 0)
            return fail(RC_ERR_INVALID_ARGUMENT, fmt("rank %lld: dims[%lld] is negative", r, d));
        if (b.dims[d] == 0) n = 0;
        else if (n != 0) {
            if (b.dims[d] > kMaxCount || n > kMaxCount / b.dims[d])
                return fail(RC_ERR_INVALID_ARGUMENT, fmt("rank %lld: element count too large", r));
            n *= b.dims[d];
        }
    }
    *count = n;
    return {};
}

// A byte range [lo, hi) of device memory that one call reads or writes.
// Reads may overlap reads.  A read may overlap a write only as the exact
// in-place layout the collective allows: same `tag`, and read.lo - write.lo
// equal to the read's `delta`.
struct Range {
    uintptr_t lo, hi;
    int tag;        // -1: never in place
    int64_t delta;  // allowed read.lo - write.lo
    int owner;      // rank (for messages)
    int tensor;
};

Error check_overlaps(std::vector<Range>& writes, const std::vector<Range>& reads) {
    std::sort(writes.begin(), writes.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
    for (size_t i = 1; i < writes.size(); ++i) {
        if (writes[i].lo < writes[i - 1].hi)
            return fail(RC_ERR_INVALID_ARGUMENT,
                        fmt("output of rank %lld (tensor %lld) overlaps another output",
                            writes[i].owner, writes[i].tensor));
    }
    for (const Range& rd : reads) {
        // first write that ends after rd.lo
        auto it = std::upper_bound(writes.begin(), writes.end(), rd.lo,
                                   [](uintptr_t v, const Range& w) { return v < w.hi; });
        for (; it != writes.end() && it->lo < rd.hi; ++it) {
            const bool in_place = rd.tag >= 0 && it->tag == rd.tag &&
                                  (int64_t)(rd.lo - it->lo) == rd.delta;
            if (!in_place)
                return fail(RC_ERR_INVALID_ARGUMENT,
                            fmt("input of rank %lld (tensor %lld) overlaps an output "
                                "other than its allowed in-place position",
                                rd.owner, rd.tensor));
        }
    }
    return {};
}

bool misaligned(const void* p, int64_t esize) {
    return (reinterpret_cast<uintptr_t>(p) % (uintptr_t)esize) != 0;
}

// Collect the ranges of a validated call into reads/writes.
void ranges_of(const Checked& ck, int tensor, std::vector<Range>* writes, std::vector<Range>* reads) {
    const int R = ck.nranks;
    const int64_t b = element_size(ck.dtype);
    const int64_t n = ck.count;
    auto at = [](const void* p) { return reinterpret_cast<uintptr_t>(p); };
    const int tag0 = tensor * kMaxRanks;
    switch (ck.coll) {
        case Coll::AllReduce:
            for (int r = 0; r < R; ++r) {
                writes->push_back({at(ck.recv[r]), at(ck.recv[r]) + n * b, tag0 + r, 0, r, tensor});
                reads->push_back({at(ck.send[r]), at(ck.send[r]) + n * b, tag0 + r, 0, r, tensor});
                // an accumulator may be its own rank's output, like send
                if (ck.has_acc)
                    reads->push_back({at(ck.acc[r]), at(ck.acc[r]) + n * b, tag0 + r, 0, r, tensor});
            }
            break;
        case Coll::Reduce:
            for (int r = 0; r < R; ++r)
                reads->push_back({at(ck.send[r]), at(ck.send[r]) + n * b, tag0 + r, 0, r, tensor});
            writes->push_back({at(ck.recv[ck.root]), at(ck.recv[ck.root]) + n * b, tag0 + ck.root, 0,
                               ck.root, tensor});
            break;
        case Coll::Broadcast: {
            const int s = ck.root;
            reads->push_back({at(ck.send[s]), at(ck.send[s]) + n * b, -1, 0, s, tensor});
            for (int r = 0; r < R; ++r) {
                if (!ck.recv[r] || (r == s && ck.recv[r] == ck.send[s])) continue;
                writes->push_back({at(ck.recv[r]), at(ck.recv[r]) + n * b, -1, 0, r, tensor});
            }
            break;
        }
        case Coll::ReduceScatter: {
            const int64_t m = n / R;
            for (int r = 0; r < R; ++r) {
                reads->push_back({at(ck.send[r]), at(ck.send[r]) + n * b, tag0 + r, -(int64_t)r * m * b, r,
                                  tensor});
                writes->push_back({at(ck.recv[r]), at(ck.recv[r]) + m * b, tag0 + r, 0, r, tensor});
            }
            break;
        }
        case Coll::AllGather:
            for (int r = 0; r < R; ++r) {
                reads->push_back({at(ck.send[r]), at(ck.send[r]) + n * b, tag0 + r, (int64_t)r * n * b, r,
                                  tensor});
                writes->push_back({at(ck.recv[r]), at(ck.recv[r]) + R * n * b, tag0 + r, 0, r, tensor});
            }
            break;
        case Coll::AllToAll:  // no in-place layout: chunks move between ranks
            for (int r = 0; r < R; ++r) {
                reads->push_back({at(ck.send[r]), at(ck.send[r]) + n * b, -1, 0, r, tensor});
                writes->push_back({at(ck.recv[r]), at(ck.recv[r]) + n * b, -1, 0, r, tensor});
            }
            break;
        case Coll::AllGatherList:
            // rank k's output for its own shard may be the shard itself
            for (int k = 0; k < R; ++k) {
                reads->push_back({at(ck.send[k]), at(ck.send[k]) + n * b, tag0 + k, 0, k, tensor});
                for (int r = 0; r < R; ++r) {
                    const uintptr_t o = at(ck.recv_list[(size_t)r * R + k]);
                    writes->push_back({o, o + n * b, r == k ? tag0 + k : -1, 0, r, tensor});
                }
            }
            break;
        case Coll::SendRecv:
            reads->push_back({at(ck.send[0]), at(ck.send[0]) + n * b, tag0, 0, ck.root, tensor});
            writes->push_back({at(ck.recv[0]), at(ck.recv[0]) + n * b, tag0, 0, ck.root, tensor});
            break;
        case Coll::Barrier:
            break;
    }
}

// Every check except the overlap check.
Error validate_fields(Coll coll, int R, const rc_buf* bufs, Checked* ck) {
    if (!bufs) return fail(RC_ERR_INVALID_ARGUMENT, "bufs is NULL");
    ck->coll = coll;
    ck->nranks = R;
    // 1. malformed fields and required pointers
    int64_t count[kMaxRanks];
    for (int r = 0; r < R; ++r) {
        const rc_buf& b = bufs[r];
        if (b.dtype != RC_F32 && b.dtype != RC_I32)
            return fail(RC_ERR_INVALID_ARGUMENT, fmt("rank %lld: unknown dtype %lld", r, b.dtype));
        if (reduces(coll) && b.op != RC_SUM && b.op != RC_MEAN && b.op != RC_MAX)
            return fail(RC_ERR_INVALID_ARGUMENT, fmt("rank %lld: unknown op %lld", r, b.op));
        Error e = count_of(b, r, &count[r]);
        if (e.code) return e;
        const int64_t es = element_size(b.dtype);
        const bool need_send = coll != Coll::Broadcast;
        const bool need_recv = coll == Coll::AllReduce || coll == Coll::ReduceScatter ||
                               coll == Coll::AllGather || coll == Coll::AllToAll;
        // zero-element buffers may be NULL (nothing is read or written)
        if (need_send && !b.send && count[r] > 0)
            return fail(RC_ERR_INVALID_ARGUMENT, fmt("rank %lld: send is NULL", r));
        if (need_recv && !b.recv && count[r] > 0)
            return fail(RC_ERR_INVALID_ARGUMENT, fmt("rank %lld: recv is NULL", r));
        if ((b.send && misaligned(b.send, es)) || (b.recv && misaligned(b.recv, es)))
            return fail(RC_ERR_INVALID_ARGUMENT,
                        fmt("rank %lld: buffer not aligned to the %lld-byte element", r, es));
    }
    // 2. dtype, shape, op agree across ranks
    for (int r = 1; r < R; ++r)
        if (bufs[r].dtype != bufs[0].dtype)
            return fail(RC_ERR_DTYPE_MISMATCH, fmt("rank %lld dtype %lld differs from rank 0's %lld", r,
                                                   bufs[r].dtype, bufs[0].dtype));
    for (int r = 1; r < R; ++r) {
        bool same = bufs[r].ndim == bufs[0].ndim;
        for (int d = 0; same && d < bufs[0].ndim; ++d) same = bufs[r].dims[d] == bufs[0].dims[d];
        if (!same) return fail(RC_ERR_SHAPE_MISMATCH, fmt("rank %lld shape differs from rank 0's", r));
    }
    if ((coll == Coll::ReduceScatter || coll == Coll::AllToAll) && count[0] % R != 0)
        return fail(RC_ERR_SHAPE_MISMATCH,
                    fmt("input of %lld elements does not split over %lld ranks", count[0], R));
    if (reduces(coll)) {
        for (int r = 1; r < R; ++r)
            if (bufs[r].op != bufs[0].op)
                return fail(RC_ERR_OP_MISMATCH,
                            fmt("rank %lld op %lld differs from rank 0's %lld", r, bufs[r].op, bufs[0].op));
        if (bufs[0].op == RC_MEAN && bufs[0].dtype != RC_F32)
            return fail(RC_ERR_INVALID_ARGUMENT, "Mean is defined for float32 only");
    }
    ck->dtype = bufs[0].dtype;
    ck->op = reduces(coll) ? bufs[0].op : RC_SUM;
    ck->count = count[0];
    // 3. root
    if (coll == Coll::Reduce || coll == Coll::Broadcast) {
        for (int r = 1; r < R; ++r)
            if (bufs[r].root != bufs[0].root)
                return fail(RC_ERR_ROOT_MISMATCH,
                            fmt("rank %lld root %lld differs from rank 0's %lld", r, bufs[r].root,
                                bufs[0].root));
        const int root = bufs[0].root;
        if (coll == Coll::Reduce) {
            if (root < 0 || root >= R)
                return fail(RC_ERR_INVALID_ARGUMENT, fmt("root %lld outside [0, %lld)", root, R));
            if (!bufs[root].recv && count[0] > 0)
                return fail(RC_ERR_INVALID_ARGUMENT, fmt("root rank %lld: recv is NULL", root));
            ck->root = root;
        } else {
            if (root < -1 || root >= R)
                return fail(RC_ERR_INVALID_ARGUMENT, fmt("broadcast root %lld outside [-1, %lld)", root, R));
            int senders = 0, sender = -1;
            for (int r = 0; r < R; ++r)
                if (bufs[r].send) ++senders, sender = r;
            if (senders != 1)
                return fail(RC_ERR_BROADCAST_SENDERS,
                            fmt("broadcast needs exactly one sender (non-NULL send), got %lld", senders));
            if (root >= 0 && root != sender)
                return fail(RC_ERR_ROOT_MISMATCH,
                            fmt("broadcast root %lld is not the sender %lld", root, sender));
            for (int r = 0; r < R; ++r)
                if (r != sender && !bufs[r].recv && count[0] > 0)
                    return fail(RC_ERR_INVALID_ARGUMENT, fmt("receiver %lld: recv is NULL", r));
            ck->root = sender;
        }
    }
    for (int r = 0; r < R; ++r) {
        ck->send[r] = bufs[r].send;
        ck->recv[r] = bufs[r].recv;
    }
    if (coll == Coll::Reduce)
        for (int r = 0; r < R; ++r)
            if (r != ck->root) ck->recv[r] = nullptr;  // never written
    return {};
}

}  // namespace

int64_t element_size(int /*dtype*/) { return 4; }

const char* coll_name(Coll c) {
    switch (c) {
        case Coll::AllReduce: return "all_reduce";
        case Coll::Reduce: return "reduce";
        case Coll::Broadcast: return "broadcast";
        case Coll::ReduceScatter: return "reduce_scatter";
        case Coll::AllGather: return "all_gather";
        case Coll::AllToAll: return "all_to_all_single";
        case Coll::AllGatherList: return "all_gather_list";
        case Coll::SendRecv: return "send_recv";
        case Coll::Barrier: return "barrier";
    }
    return "?";
}

Error validate(Coll coll, int R, const rc_buf* bufs, Checked* ck, void* const* recv_list) {
    Error e = validate_fields(coll, R, bufs, ck);
    if (!e.code && coll == Coll::AllGatherList) {
        // the list form's outputs: R per rank, each a shard's size
        if (!recv_list) {
            e = fail(RC_ERR_INVALID_ARGUMENT, "recvs is NULL");
        } else {
            ck->recv_list.assign(recv_list, recv_list + (size_t)R * R);
            for (int i = 0; i < R * R && !e.code; ++i) {
                void* o = ck->recv_list[i];
                if (!o && ck->count > 0)
                    e = fail(RC_ERR_INVALID_ARGUMENT,
                             fmt("rank %lld: output for rank %lld's shard is NULL", i / R, i % R));
                else if (o && misaligned(o, element_size(ck->dtype)))
                    e = fail(RC_ERR_INVALID_ARGUMENT,
                             fmt("rank %lld: output for rank %lld's shard is misaligned", i / R, i % R));
            }
        }
    }
    if (e.code) {
        std::string prefix = std::string(coll_name(coll)) + ": ";
        e.msg = prefix + e.msg;
        return e;
    }
    if (ck->count == 0) return {};
    std::vector<Range> writes, reads;
    ranges_of(*ck, 0, &writes, &reads);
    e = check_overlaps(writes, reads);
    if (e.code) e.msg = std::string(coll_name(coll)) + ": " + e.msg;
    return e;
}

// Communicator.send on rank src and recv on rank dst.  The two sides must
// describe the same dtype and shape; the sender's send and the receiver's
// recv are required (when non-empty), and they may be the same buffer (then
// nothing moves) but must not overlap otherwise.
Error validate_send_recv(int R, int src, int dst, const rc_buf* bufs, Checked* ck) {
    if (!bufs) return fail(RC_ERR_INVALID_ARGUMENT, "send_recv: bufs is NULL");
    if (src < 0 || src >= R || dst < 0 || dst >= R)
        return fail(RC_ERR_INVALID_ARGUMENT, fmt("send_recv: src %lld or dst %lld outside [0, %lld)", src, dst, R));
    if (src == dst) return fail(RC_ERR_INVALID_ARGUMENT, "send_recv: a rank cannot send to itself");
    int64_t count[2];
    for (int i = 0; i < 2; ++i) {
        const rc_buf& b = bufs[i];
        const int rank = i ? dst : src;
        if (b.dtype != RC_F32 && b.dtype != RC_I32)
            return fail(RC_ERR_INVALID_ARGUMENT, fmt("send_recv: rank %lld: unknown dtype %lld", rank, b.dtype));
        Error e = count_of(b, rank, &count[i]);
        if (e.code) return e;
        const void* p = i ? static_cast<const void*>(b.recv) : b.send;
        if (!p && count[i] > 0)
            return fail(RC_ERR_INVALID_ARGUMENT,
                        fmt(i ? "send_recv: receiver %lld: recv is NULL" : "send_recv: sender %lld: send is NULL", rank));
        if (p && misaligned(p, element_size(b.dtype)))
            return fail(RC_ERR_INVALID_ARGUMENT, fmt("send_recv: rank %lld: buffer not aligned", rank));
    }
    if (bufs[1].dtype != bufs[0].dtype)
        return fail(RC_ERR_DTYPE_MISMATCH, fmt("send_recv: receiver %lld dtype differs from sender %lld's", dst, src));
    bool same = bufs[1].ndim == bufs[0].ndim;
    for (int d = 0; same && d < bufs[0].ndim; ++d) same = bufs[1].dims[d] == bufs[0].dims[d];
    if (!same) return fail(RC_ERR_SHAPE_MISMATCH, fmt("send_recv: receiver %lld shape differs from sender %lld's", dst, src));
    ck->coll = Coll::SendRecv;
    ck->nranks = 2;
    ck->dtype = bufs[0].dtype;
    ck->op = RC_SUM;
    ck->root = src;
    ck->count = count[0];
    ck->send[0] = bufs[0].send;
    ck->recv[0] = bufs[1].recv;
    if (ck->count == 0) return {};
    std::vector<Range> writes, reads;
    ranges_of(*ck, 0, &writes, &reads);
    Error e = check_overlaps(writes, reads);
    if (e.code) e.msg = "send_recv: " + e.msg;
    return e;
}

Error validate_batch(int R, int num_tensors, const rc_buf* bufs, std::vector<Checked>* out,
                     const uint64_t* ids, const void* const* accs) {
    const char* who = ids ? "all_reduce_params" : "all_reduce_many";
    auto name = [&](int t) {
        return ids ? "parameter " + std::to_string(ids[t]) : "tensor " + std::to_string(t);
    };
    if (num_tensors < 0) return fail(RC_ERR_INVALID_ARGUMENT, std::string(who) + ": num_tensors is negative");
    if (num_tensors > 0 && !bufs) return fail(RC_ERR_INVALID_ARGUMENT, std::string(who) + ": bufs is NULL");
    out->assign(num_tensors, Checked{});
    for (int t = 0; t < num_tensors; ++t) {
        Error e = validate_fields(Coll::AllReduce, R, bufs + (int64_t)t * R, &(*out)[t]);
        if (e.code) {
            e.msg = std::string(who) + ": " + name(t) + ": " + e.msg;
            return e;
        }
    }
    // ops and dtypes must agree across the whole batch: one launch family
    for (int t = 1; t < num_tensors; ++t) {
        if ((*out)[t].dtype != (*out)[0].dtype)
            return fail(RC_ERR_DTYPE_MISMATCH,
                        std::string(who) + ": " + name(t) + " dtype differs from " + name(0) + "'s");
        if ((*out)[t].op != (*out)[0].op)
            return fail(RC_ERR_OP_MISMATCH, std::string(who) + ": " + name(t) + " op differs from " + name(0) + "'s");
    }
    // accumulators (RUDA "Training and state saving": accumulate adds without
    // averaging), on every rank or on none, for Sum and Mean
    for (int t = 0; accs && t < num_tensors; ++t) {
        Checked& ck = (*out)[t];
        if (ck.count == 0) continue;
        int given = 0;
        for (int r = 0; r < R; ++r) given += accs[(int64_t)t * R + r] != nullptr;
        if (given == 0) continue;
        if (given != R)
            return fail(RC_ERR_INVALID_ARGUMENT, std::string(who) + ": " + name(t) +
                                                     ": acc is given on some ranks only");
        if (ck.op == RC_MAX)
            return fail(RC_ERR_INVALID_ARGUMENT, std::string(who) + ": " + name(t) +
                                                     ": accumulated gradients reduce with Sum or Mean");
        for (int r = 0; r < R; ++r) {
            ck.acc[r] = accs[(int64_t)t * R + r];
            if (misaligned(ck.acc[r], element_size(ck.dtype)))
                return fail(RC_ERR_INVALID_ARGUMENT, std::string(who) + ": " + name(t) + ": rank " +
                                                         std::to_string(r) + ": acc is misaligned");
        }
        ck.has_acc = true;
    }
    std::vector<Range> writes, reads;
    for (int t = 0; t < num_tensors; ++t)
        if ((*out)[t].count) ranges_of((*out)[t], t, &writes, &reads);
    Error e = check_overlaps(writes, reads);
    if (e.code) e.msg = std::string(who) + ": " + e.msg;
    return e;
}

// Gradient sync keyed by parameter ID (ruCCL README section 6, "Collective
// training": IDs, shapes and dtype agree on every rank).  Each rank's entries
// are sorted by ID; a repeated ID within a rank is an argument error, and ID
// lists that differ between ranks are a parameter mismatch named by the first
// ID that one side lacks.
Error match_params(int R, const int* counts, const rc_param* const* params, std::vector<rc_buf>* bufs,
                   std::vector<const void*>* accs, std::vector<uint64_t>* order) {
    std::vector<std::vector<int>> perm(R);
    auto id_of = [&](int r, int i) { return params[r][perm[r][i]].id; };
    for (int r = 0; r < R; ++r) {
        if (counts[r] < 0)
            return fail(RC_ERR_INVALID_ARGUMENT, fmt("all_reduce_params: rank %lld: num_params is negative", r));
        if (counts[r] > 0 && !params[r])
            return fail(RC_ERR_INVALID_ARGUMENT, fmt("all_reduce_params: rank %lld: params is NULL", r));
        perm[r].resize(counts[r]);
        for (int i = 0; i < counts[r]; ++i) perm[r][i] = i;
        const rc_param* pr = params[r];
        std::sort(perm[r].begin(), perm[r].end(), [pr](int a, int b) { return pr[a].id < pr[b].id; });
        for (int i = 1; i < counts[r]; ++i)
            if (id_of(r, i) == id_of(r, i - 1))
                return fail(RC_ERR_INVALID_ARGUMENT, "all_reduce_params: rank " + std::to_string(r) +
                                                         " lists parameter " + std::to_string(id_of(r, i)) +
                                                         " twice");
    }
    for (int r = 1; r < R; ++r) {
        // walk both sorted lists to the first ID present on one side only
        int i = 0, j = 0;
        while (i < counts[0] || j < counts[r]) {
            const bool has0 = i < counts[0], hasr = j < counts[r];
            const uint64_t a = has0 ? id_of(0, i) : 0, b = hasr ? id_of(r, j) : 0;
            if (has0 && hasr && a == b) {
                ++i, ++j;
                continue;
            }
            const bool missing_on_r = has0 && (!hasr || a < b);
            const uint64_t pid = missing_on_r ? a : b;
            return fail(RC_ERR_PARAM_MISMATCH,
                        "all_reduce_params: parameter " + std::to_string(pid) +
                            (missing_on_r ? " is on rank 0 but not on rank " + std::to_string(r)
                                          : " is on rank " + std::to_string(r) + " but not on rank 0"));
        }
    }
    const int P = R ? counts[0] : 0;
    order->resize(P);
    bufs->assign((size_t)P * R, rc_buf{});
    accs->assign((size_t)P * R, nullptr);
    for (int t = 0; t < P; ++t) {
        (*order)[t] = id_of(0, t);
        for (int r = 0; r < R; ++r) {
            const rc_param& e = params[r][perm[r][t]];
            (*bufs)[(size_t)t * R + r] = e.buf;
            (*accs)[(size_t)t * R + r] = e.acc;
        }
    }
    return {};
}

}  // namespace rc
