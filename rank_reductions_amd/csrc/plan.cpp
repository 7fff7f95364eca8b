// Chunk scheduler: turns a validated collective into launch plans - ring
// segments (jobs), their alignment phase, tiles per job, the grid and the
// occupancy cap.
//
// Segmentation follows the ring of the ruCCL README (ja), "CUDA tensor
// example": S = ceil(N/R) elements per segment, segment c owned by rank c and
// folded in rank order (c+1), ..., c.  reduce_scatter_tensor and
// all_gather_into_tensor (monarch Communicator page) use shards of M = N/R
// elements, which are exactly those segments.  Host-only C++.
//
// Launch shape.  Every workgroup is one wave and takes one tile.  One-shot
// launches use a 2-D grid (x: tile of the job, y: job), dispatched in order, so
// the tiles in flight form one compact window of each rank's buffers.  How
// many waves a CU holds at once is capped through an LDS reservation: on
// MI355X, HBM efficiency for these many-stream patterns peaks at about 110 KiB
// of load traffic per CU in flight, counting a store as 0.65 of a load; more
// waves open more DRAM rows at once and lose bandwidth, fewer leave it idle.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "rc_internal.h"

namespace rc {

namespace {

constexpr int64_t kMaxTileElems = 65536;

uintptr_t addr(const void* p, int64_t elem_off, int64_t esize) {
    return reinterpret_cast<uintptr_t>(p) + (uintptr_t)(elem_off * esize);
}

// A job's streams at its first element: the inputs it reads, then the
// outputs it writes.
struct JobAddrs {
    std::vector<uintptr_t> ins, outs;
};

// Fill per-job phase and tile counts of a single-launch plan.  Tile indices
// are 32-bit in the kernels: tiles grow until the total stays below 2^31.
void finish_jobs(LaunchPlan* p, const std::vector<JobAddrs>& job_addrs) {
    JobArgs& a = p->args;
    for (int c = 0; c < a.jobs; ++c) {
        const JobAddrs& ad = job_addrs[c];
        a.phase[c] = job_len(a.n, a.seg, c) ? job_phase(ad.ins.data(), (int)ad.ins.size(), ad.outs.data(),
                                                         (int)ad.outs.size())
                                            : 0;
    }
    int64_t prefix[kMaxRanks + 1];
    for (;;) {
        prefix[0] = 0;
        for (int c = 0; c < a.jobs; ++c) prefix[c + 1] = prefix[c] + tiles_of(job_len(a.n, a.seg, c), a.phase[c], a.tile_elems);
        if (prefix[a.jobs] < (int64_t(1) << 31)) break;
        a.tile_elems *= 2;
    }
    for (int c = 0; c <= kMaxRanks; ++c) a.tile_prefix[c] = (int32_t)prefix[std::min(c, a.jobs)];
    for (int c = a.jobs; c < kMaxRanks; ++c) a.phase[c] = 0;
    a.total_tiles = (int32_t)prefix[a.jobs];
    p->total_tiles = prefix[a.jobs];
}

int nontemporal_of(const Config& cfg) {
    return cfg.cache_hint == RC_CACHE_NORMAL ? 0 : 1;
}

// Group index of a batch: the job holding the first tile of every group of
// 2^kGroupShift tiles.
void build_groups(BatchPlan* bp) {
    const int64_t groups = (bp->total_tiles + (int64_t(1) << kGroupShift) - 1) >> kGroupShift;
    bp->group_job.resize(groups);
    size_t j = 0;
    for (int64_t g = 0; g < groups; ++g) {
        const int64_t t = g << kGroupShift;
        while (j + 1 < bp->jobs.size() && bp->jobs[j + 1].tile_begin <= t) ++j;
        bp->group_job[g] = (int32_t)j;
    }
}

}  // namespace

int tile_elems_for(int unroll, const Config& cfg) {
    const int64_t step = (int64_t)kBlock * kVec * unroll;
    int64_t te = cfg.tile_elems > 0 ? cfg.tile_elems : step;
    te = ((te + step - 1) / step) * step;
    te = std::min<int64_t>(std::max<int64_t>(te, step), std::max<int64_t>(step, kMaxTileElems));
    return (int)te;
}

int job_reference(const uintptr_t* ins, int nin, const uintptr_t* outs, int nout) {
    // weight of each stream's 256-byte class, counted over all streams
    const int n = nin + nout;
    int best = 0, best_w = -1;
    for (int i = 0; i < n; ++i) {
        const uintptr_t cls = (i < nin ? ins[i] : outs[i - nin]) % kTileAlignBytes;
        bool seen = false;
        for (int j = 0; j < i && !seen; ++j) seen = (j < nin ? ins[j] : outs[j - nin]) % kTileAlignBytes == cls;
        if (seen) continue;
        int w = 0;
        for (int j = i; j < n; ++j)
            if ((j < nin ? ins[j] : outs[j - nin]) % kTileAlignBytes == cls) w += j < nin ? 1 : 2;
        if (w > best_w) {
            best = i;
            best_w = w;
        }
    }
    return best;
}

uint8_t phase_of(uintptr_t ref) {
    // elements are 4 bytes and 4-byte aligned (validation checks it)
    const int head = (int)(((16 - ref % 16) % 16) / 4);
    const uintptr_t first_vec = ref + (uintptr_t)(head * 4);
    const int lead = (int)(((kTileAlignBytes - first_vec % kTileAlignBytes) % kTileAlignBytes) / 16);
    return phase_code(head, lead);
}

uint8_t job_phase(const uintptr_t* ins, int nin, const uintptr_t* outs, int nout) {
    if (nin + nout == 0) return 0;
    const int r = job_reference(ins, nin, outs, nout);
    return phase_of(r < nin ? ins[r] : outs[r - nin]);
}

int auto_waves_per_cu(int nin, int nout, int unroll, const InFlightRule& rule) {
    // each wave moves (nin + nout) * unroll KiB per round (64 lanes x 16 B);
    // stores are posted and hold the wave only part of the time
    const double kib_per_wave = ((double)nin + rule.store_weight * nout) * unroll;
    const long w = std::lround(rule.kib / std::max(kib_per_wave, 1.0));
    return (int)std::min<long>(32, std::max<long>(2, w));
}

int lds_for_waves(const DeviceInfo& dev, int waves) {
    // One workgroup is one wave; reserving lds_per_cu / waves bytes of LDS per
    // workgroup lets at most `waves` of them sit on a CU at a time.
    int64_t lds = 0;
    if (dev.lds_per_cu > 0 && waves > 0 && waves < 32) {
        lds = (dev.lds_per_cu / waves) / 512 * 512;
        lds = std::min(lds, dev.max_lds_per_block);
    }
    return (int)std::max<int64_t>(lds, 0);
}

int tune_pick(TuneEntry& t, int rule_waves, int* cand) {
    *cand = -1;
    if (t.ncand == 0)
        for (int w = rule_waves; w >= std::max(2, rule_waves - (kTuneCands - 1)); --w) t.cand[t.ncand++] = w;
    if (t.chosen) return t.chosen;
    // candidates in turn, the one with the fewest timed launches first
    int pick = -1;
    for (int i = 0; i < t.ncand; ++i)
        if (t.issued[i] < kTuneSamples && (pick < 0 || t.issued[i] < t.issued[pick])) pick = i;
    if (pick < 0) return t.cand[0];  // every sample issued, some not read yet
    ++t.issued[pick];
    *cand = pick;
    return t.cand[pick];
}

void tune_record(TuneEntry& t, int cand, float us) {
    if (cand < 0 || cand >= t.ncand || t.chosen || t.got[cand] >= kTuneSamples) return;
    t.us[cand][t.got[cand]++] = us;
    for (int i = 0; i < t.ncand; ++i)
        if (t.got[i] < kTuneSamples) return;
    for (int i = 0; i < t.ncand; ++i) {
        float v[kTuneSamples];
        std::copy(t.us[i], t.us[i] + kTuneSamples, v);
        std::sort(v, v + kTuneSamples);
        t.median_us[i] = v[kTuneSamples / 2];
    }
    int best = 0;  // candidate 0 is the rule's W
    for (int i = 1; i < t.ncand; ++i)
        if (t.median_us[i] < t.median_us[best]) best = i;
    if (best != 0 && t.median_us[best] > (1.0 - kTuneMargin) * t.median_us[0]) best = 0;
    t.chosen = t.cand[best];
}

void shape_launch(int64_t total_tiles, int nin, int nout, int unroll, const Config& cfg,
                  const DeviceInfo& dev, int64_t* grid, int* lds_bytes, const InFlightRule& rule) {
    const int waves = cfg.waves_per_cu > 0 ? cfg.waves_per_cu : auto_waves_per_cu(nin, nout, unroll, rule);
    *lds_bytes = lds_for_waves(dev, waves);
    int64_t g = total_tiles;
    if (cfg.max_workgroups > 0) g = std::min<int64_t>(g, cfg.max_workgroups);
    *grid = std::max<int64_t>(1, std::min<int64_t>(g, 0x7FFFFFFF));
}

namespace {

// A byte range [lo, hi).
struct Span {
    uintptr_t lo, hi;
};

// Whether shifting pays and is safe (tiling.h): some destination starts its
// job off a 64-byte write burst, and no destination overlaps a source.  The
// shifted kernels write up to kBurstElems - 1 elements ahead of each tile,
// which the previous tile reads when an output aliases an input (a call in
// place).
bool shift_pays(bool off_burst, const std::vector<Span>& srcs, const std::vector<Span>& dsts) {
    if (!off_burst) return false;
    for (const Span& d : dsts)
        for (const Span& r : srcs)
            if (d.lo < r.hi && r.lo < d.hi) return false;
    return true;
}

}  // namespace

bool shifted_outputs_pay(const JobArgs& a, int64_t es, const int64_t* job_off) {
    bool off = false;
    std::vector<Span> srcs, dsts;
    auto at = [](const void* p, int64_t bytes) { return reinterpret_cast<uintptr_t>(p) + (uintptr_t)bytes; };
    for (int c = 0; c < a.jobs; ++c) {
        const int64_t len = job_len(a.n, a.seg, c);
        if (len == 0) continue;
        // a fold reads every rank's input at the job's place, a copy its own
        if (a.in_mode == kInFold) {
            for (int r = 0; r < a.nranks; ++r)
                srcs.push_back({at(a.in[r], c * a.in_stride * es), at(a.in[r], (c * a.in_stride + len) * es)});
        } else {
            srcs.push_back({at(a.in[c], c * a.in_stride * es), at(a.in[c], (c * a.in_stride + len) * es)});
        }
        const uint32_t mask = out_mask_of(a.out_mode, a.out_mask, c);
        for (int o = 0; o < a.nranks; ++o) {
            if (!((mask >> o) & 1u)) continue;
            const uintptr_t lo = at(a.out[o], c * a.out_stride * es);
            dsts.push_back({lo, lo + (uintptr_t)(len * es)});
            // where the launch starts writing the job (its interior, if split)
            if (burst_offset(lo + (uintptr_t)((job_off ? job_off[c] : 0) * es))) off = true;
        }
    }
    return shift_pays(off, srcs, dsts);
}

// The same for a copy batch: ptrs[j * (1 + nout)] is job j's source, the
// next nout its destinations, each at the job's first element.
bool shifted_copies_pay(const BatchPlan& bp, int64_t es) {
    bool off = false;
    std::vector<Span> srcs, dsts;
    const size_t per = 1 + (size_t)bp.nout;
    for (size_t j = 0; j < bp.jobs.size(); ++j) {
        const uintptr_t bytes = (uintptr_t)(bp.jobs[j].len * es);
        for (size_t i = 0; i < per; ++i) {
            const uintptr_t lo = reinterpret_cast<uintptr_t>(bp.ptrs[j * per + i]);
            (i == 0 ? srcs : dsts).push_back({lo, lo + bytes});
            if (i > 0 && burst_offset(lo)) off = true;
        }
    }
    return shift_pays(off, srcs, dsts);
}

// A fold launch whose jobs are not whole tiles (segment lengths or buffers
// off the 256-byte grid) runs its round inside the general kernel, 2-3%
// slower than the whole-tile kernels, plus the lead tiles.  When it moves
// kSplitMinBytes or more and every job has whole tiles after its first, it
// runs on the edge form of the FoldTable kernels instead (LaunchPlan::split):
// per job, `edges` workgroups for the tiles outside the interior (tile 0,
// with the scalars and the lead, and those past the interior) and
// `interior` workgroups for the first whole tiles after tile 0 (the fewest
// any job has), from element job_interior_start.  Each element is still
// folded once, in the same order.
bool split_fold(LaunchPlan* lp, const Config& cfg, const DeviceInfo& dev, int64_t es) {
    const JobArgs& a = lp->args;
    if (!a.grid_2d || a.full_tiles || a.in_mode != kInFold || lp->acc || cfg.max_workgroups > 0 ||
        a.tile_elems != kBlock * kVec * lp->unroll || lp->unroll != unroll_for(lp->nin) || a.jobs < 1)
        return false;
    int64_t elems = 0, interior = INT64_MAX;
    int64_t widest = 0;
    int64_t off[kMaxRanks] = {};
    for (int c = 0; c < a.jobs; ++c) {
        const int64_t len = job_len(a.n, a.seg, c);
        const JobSplit s = job_split(len, a.phase[c], a.tile_elems);
        interior = std::min(interior, job_interior_tiles(s));
        off[c] = job_interior_start(s);
        elems += len;
        widest = std::max<int64_t>(widest, a.tile_prefix[c + 1] - a.tile_prefix[c]);
    }
    const int64_t min_bytes = cfg.split_min_bytes >= 0 ? cfg.split_min_bytes : kSplitMinBytes;
    if (interior < 1 || (int64_t)(lp->nin + lp->nout) * elems * es < min_bytes) return false;
    lp->split = true;
    lp->interior = interior;
    lp->edges = (int)(widest - interior);
    for (int c = 0; c < a.jobs; ++c) lp->job_off[c] = off[c];
    // the interior carries the launch: the whole-tile occupancy rule
    int64_t grid = 0;
    shape_launch(a.jobs * interior, lp->nin, lp->nout, lp->unroll, cfg, dev, &grid, &lp->lds_bytes, kFullFoldRule);
    lp->waves = cfg.waves_per_cu > 0 ? cfg.waves_per_cu : auto_waves_per_cu(lp->nin, lp->nout, lp->unroll, kFullFoldRule);
    lp->grid = lp->edges + interior;
    lp->shift_out = shifted_outputs_pay(lp->args, es, lp->job_off);
    return true;
}

FoldTable fold_table_of(const LaunchPlan& p) {
    const JobArgs& a = p.args;
    FoldTable t{};
    for (int c = 0; c < a.jobs; ++c) {
        // the interior of a split fold starts job_off[c] elements into the job
        const int64_t off = (int64_t)c * a.in_stride + p.job_off[c];
        for (int k = 0; k < p.nin; ++k) {
            const int r = fold_rank(c, k, p.nin);
            t.in[c][k] = static_cast<const uint32_t*>(a.in[r]) + off;
            // accumulators only where they fit beside the operands (the
            // table kernels' case); past kAccSlot ranks the table is unused
            if (p.acc && p.nin <= kAccSlot) t.in[c][kAccSlot + k] = static_cast<const uint32_t*>(a.acc[r]) + off;
        }
        t.mask[c] = out_mask_of(a.out_mode, a.out_mask, c);
        t.out_off[c] = p.job_off[c];
        t.len[c] = job_len(a.n, a.seg, c);
        t.phase[c] = a.phase[c];
    }
    t.edges = p.split ? p.edges : 0;
    t.interior = (int32_t)(p.split ? p.interior : p.grid);
    for (int r = 0; r < a.nranks; ++r) t.out[r] = a.out[r];
    t.out_stride = a.out_stride;
    t.mean = a.mean;
    return t;
}

std::vector<LaunchPlan> plan(const Checked& ck, const Config& cfg, const DeviceInfo& dev) {
    std::vector<LaunchPlan> out;
    if (ck.count == 0) return out;
    const int R = ck.nranks;
    const int64_t es = element_size(ck.dtype);
    const uint32_t all = (1u << R) - 1u;

    LaunchPlan p{};
    JobArgs& a = p.args;
    a = JobArgs{};
    a.nranks = R;
    a.nontemporal = nontemporal_of(cfg);
    p.dtype = ck.dtype;
    p.op = ck.op;

    std::vector<JobAddrs> ad;
    auto fold_setup = [&](int64_t n, int64_t seg, int64_t in_stride, int64_t out_stride) {
        p.nin = R;
        p.acc = ck.has_acc;
        p.unroll = unroll_for(ck.has_acc ? 2 * R : R);
        a.in_mode = kInFold;
        a.n = n;
        a.seg = seg;
        a.in_stride = in_stride;
        a.out_stride = out_stride;
        a.jobs = R;
        a.mean = ck.op == RC_MEAN;
        a.tile_elems = tile_elems_for(p.unroll, cfg);
        for (int r = 0; r < R; ++r) {
            a.in[r] = ck.send[r];
            a.out[r] = ck.recv[r];
            a.acc[r] = ck.has_acc ? ck.acc[r] : nullptr;
        }
    };
    auto copy_setup = [&](LaunchPlan& q) {
        q.nin = 1;
        q.unroll = kCopyUnroll;
        q.args.in_mode = kInCopy;
        q.args.tile_elems = tile_elems_for(kCopyUnroll, cfg);
    };
    auto fold_addrs = [&](uint32_t mask_for_owner_only, bool owner_only) {
        ad.assign(R, {});
        for (int c = 0; c < R; ++c) {
            for (int r = 0; r < R; ++r) ad[c].ins.push_back(addr(a.in[r], (int64_t)c * a.in_stride, es));
            if (p.acc)
                for (int r = 0; r < R; ++r) ad[c].ins.push_back(addr(a.acc[r], (int64_t)c * a.in_stride, es));
            for (int r = 0; r < R; ++r) {
                const bool writes = owner_only ? (r == c) : ((mask_for_owner_only >> r) & 1u);
                if (writes) ad[c].outs.push_back(addr(a.out[r], (int64_t)c * a.out_stride, es));
            }
        }
    };

    switch (ck.coll) {
        case Coll::AllReduce:
        case Coll::Reduce: {
            const int64_t S = (ck.count + R - 1) / R;
            const bool ring = ck.coll == Coll::AllReduce && cfg.algo == RC_ALGO_RING;
            fold_setup(ck.count, S, S, S);
            if (!ring) {
                a.out_mode = kOutMask;
                a.out_mask = ck.coll == Coll::Reduce ? (1u << ck.root) : all;
                fold_addrs(a.out_mask, false);
                finish_jobs(&p, ad);
                out.push_back(p);
                break;
            }
            // ring phase 1: the fold of segment c lands in rank c's output
            a.out_mode = kOutOwner;
            a.out_mask = all;
            fold_addrs(0, true);
            finish_jobs(&p, ad);
            out.push_back(p);
            if (R == 1) break;
            // ring phase 2: rank c's finished segment is copied to every other rank
            LaunchPlan q{};
            JobArgs& b = q.args;
            b = JobArgs{};
            copy_setup(q);
            q.dtype = ck.dtype;
            q.op = ck.op;
            b.nranks = R;
            b.nontemporal = a.nontemporal;
            b.out_mode = kOutMaskButOwner;
            b.out_mask = all;
            b.n = ck.count;
            b.seg = S;
            b.in_stride = S;
            b.out_stride = S;
            b.jobs = R;
            for (int r = 0; r < R; ++r) {
                b.in[r] = ck.recv[r];
                b.out[r] = ck.recv[r];
            }
            ad.assign(R, {});
            for (int c = 0; c < R; ++c) {
                ad[c].ins.push_back(addr(ck.recv[c], (int64_t)c * S, es));
                for (int r = 0; r < R; ++r)
                    if (r != c) ad[c].outs.push_back(addr(ck.recv[r], (int64_t)c * S, es));
            }
            finish_jobs(&q, ad);
            out.push_back(q);
            break;
        }
        case Coll::ReduceScatter: {
            const int64_t M = ck.count / R;
            fold_setup(ck.count, M, M, 0);
            a.out_mode = kOutOwner;
            a.out_mask = all;
            fold_addrs(0, true);
            finish_jobs(&p, ad);
            out.push_back(p);
            break;
        }
        case Coll::Broadcast: {
            const int s = ck.root;
            copy_setup(p);
            a.out_mode = kOutMask;
            a.n = ck.count;
            a.seg = ck.count;
            a.in_stride = 0;
            a.out_stride = 0;
            a.jobs = 1;
            a.in[0] = ck.send[s];
            uint32_t mask = 0;
            for (int r = 0; r < R; ++r) {
                a.out[r] = ck.recv[r];
                if (ck.recv[r] && !(r == s && ck.recv[r] == ck.send[s])) mask |= 1u << r;
            }
            a.out_mask = mask;
            if (!mask) break;
            ad.assign(1, {});
            ad[0].ins.push_back(addr(a.in[0], 0, es));
            for (int r = 0; r < R; ++r)
                if ((mask >> r) & 1u) ad[0].outs.push_back(addr(a.out[r], 0, es));
            finish_jobs(&p, ad);
            out.push_back(p);
            break;
        }
        case Coll::SendRecv: {
            // one job: the sender's buffer to the receiver's (nothing when they coincide)
            copy_setup(p);
            a.nranks = 1;
            a.out_mode = kOutMask;
            a.n = ck.count;
            a.seg = ck.count;
            a.in_stride = 0;
            a.out_stride = 0;
            a.jobs = 1;
            a.in[0] = ck.send[0];
            a.out[0] = ck.recv[0];
            a.out_mask = ck.send[0] != ck.recv[0] ? 1u : 0u;
            if (!a.out_mask) break;
            ad.assign(1, {});
            ad[0].ins.push_back(addr(a.in[0], 0, es));
            ad[0].outs.push_back(addr(a.out[0], 0, es));
            finish_jobs(&p, ad);
            out.push_back(p);
            break;
        }
        case Coll::AllToAll:
        case Coll::AllGatherList:  // batches of copies: plan_copies
        case Coll::Barrier:        // no kernel
            break;
        case Coll::AllGather: {
            const int64_t M = ck.count;
            copy_setup(p);
            a.out_mode = kOutMask;
            a.out_mask = all;
            a.n = M * R;
            a.seg = M;
            a.in_stride = 0;
            a.out_stride = M;
            a.jobs = R;
            for (int r = 0; r < R; ++r) {
                a.in[r] = ck.send[r];
                a.out[r] = ck.recv[r];
            }
            // in place: rank c's shard already sits at its place in rank c's output
            ad.assign(R, {});
            for (int c = 0; c < R; ++c) {
                ad[c].ins.push_back(addr(a.in[c], 0, es));
                for (int r = 0; r < R; ++r) ad[c].outs.push_back(addr(a.out[r], (int64_t)c * M, es));
            }
            finish_jobs(&p, ad);
            out.push_back(p);
            break;
        }
    }
    for (LaunchPlan& lp : out) {
        const JobArgs& ja = lp.args;
        const int in_mask = __builtin_popcount(ja.out_mask);
        lp.nout = ja.out_mode == kOutOwner ? 1 : in_mask - (ja.out_mode == kOutMaskButOwner ? 1 : 0);
        const int loads = lp.acc ? 2 * lp.nin : lp.nin;
        if (cfg.max_workgroups > 0) {
            shape_launch(lp.total_tiles, loads, lp.nout, lp.unroll, cfg, dev, &lp.grid, &lp.lds_bytes);
            lp.waves = cfg.waves_per_cu > 0 ? cfg.waves_per_cu : auto_waves_per_cu(loads, lp.nout, lp.unroll);
            continue;
        }
        // one-shot: x = tiles of the longest job, y = jobs
        int64_t widest = 0;
        for (int c = 0; c < ja.jobs; ++c) widest = std::max<int64_t>(widest, ja.tile_prefix[c + 1] - ja.tile_prefix[c]);
        bool full = widest > 0 && ja.tile_elems == (int64_t)kBlock * kVec * lp.unroll;
        for (int c = 0; c < ja.jobs && full; ++c) {
            const int64_t len = job_len(ja.n, ja.seg, c);
            full = ja.phase[c] == 0 && ja.tile_prefix[c + 1] - ja.tile_prefix[c] == widest &&
                   len == widest * (int64_t)ja.tile_elems;
        }
        // whole-tile kernels carry their own occupancy rules (fitted per shape)
        const InFlightRule& rule = !full ? kFoldRule : (ja.in_mode == kInCopy ? kCopyBatchRule : kFullFoldRule);
        shape_launch(lp.total_tiles, loads, lp.nout, lp.unroll, cfg, dev, &lp.grid, &lp.lds_bytes, rule);
        lp.waves = cfg.waves_per_cu > 0 ? cfg.waves_per_cu : auto_waves_per_cu(loads, lp.nout, lp.unroll, rule);
        if (full && lp.acc && lp.nin <= kAccSlot && cfg.waves_per_cu <= 0 && lp.waves > kAccTableMaxWaves) {
            lp.waves = kAccTableMaxWaves;
            lp.lds_bytes = lds_for_waves(dev, lp.waves);
        }
        // A whole-tile all-reduce of 4-7 ranks runs one vector per lane:
        // 4 x 64 MiB 82.1-82.2 us at W=7 against 83.3-83.6 at the best W with
        // two (three boxes); 5, 6 and 7 ranks of 2^21 elements per segment
        // 64.2 / 93.0 / 126.6 us against 66.8 / 96.7 / 131.9.  Whole tiles of
        // two vectors are whole tiles of one, and the two-vector rule's wave
        // count (7, 6, 5, 4) is where one vector peaks.  A reduce to one
        // output stays at two (26.5 against 27.8 us for 4 ranks).
        if (full && ja.in_mode == kInFold && !lp.acc && lp.nin >= 4 && lp.nin < 8 && lp.nout == lp.nin &&
            lp.unroll == 2 && cfg.tile_elems <= 0) {
            lp.unroll = 1;
            lp.args.tile_elems /= 2;
            for (int c = 0; c <= kMaxRanks; ++c) lp.args.tile_prefix[c] *= 2;
            lp.args.total_tiles *= 2;
            lp.total_tiles *= 2;
            widest *= 2;
        }
        lp.args.grid_2d = 1;
        lp.args.full_tiles = full ? 1 : 0;
        lp.grid = std::max<int64_t>(1, widest);
        lp.grid_y = ja.jobs;
        if (full && !lp.acc) lp.shift_out = shifted_outputs_pay(lp.args, es, lp.job_off);
    }
    // folds whose jobs are not whole tiles: their aligned interiors on the
    // FoldTable kernels, the edges in the same launch
    for (LaunchPlan& lp : out) split_fold(&lp, cfg, dev, es);
    return out;
}

void split_batch(const std::vector<Checked>& tensors, std::vector<Checked>* own,
                 std::vector<Checked>* batched) {
    own->clear();
    batched->clear();
    for (const Checked& ck : tensors) {
        if (ck.count == 0) continue;
        const int64_t moved = (ck.has_acc ? 3 : 2) * (int64_t)ck.nranks * ck.count * element_size(ck.dtype);
        (moved >= kOwnLaunchBytes ? own : batched)->push_back(ck);
    }
}

BatchPlan plan_batch(const std::vector<Checked>& tensors, const Config& cfg, const DeviceInfo& dev) {
    BatchPlan bp;
    if (tensors.empty()) return bp;
    const int R = tensors[0].nranks;
    bp.acc = tensors[0].has_acc;  // the caller batches tensors with and without accumulators apart
    const int loads = bp.acc ? 2 * R : R;
    const int unroll = unroll_for(loads);
    bp.nranks = R;
    bp.dtype = tensors[0].dtype;
    bp.op = tensors[0].op;
    bp.tile_elems = tile_elems_for(unroll, cfg);
    bp.nontemporal = nontemporal_of(cfg);
    const int64_t es = element_size(bp.dtype);
    int64_t tiles = 0;
    std::vector<uintptr_t> ins, outs;
    ins.reserve(2 * R);
    outs.reserve(R);
    for (const Checked& ck : tensors) {
        if (ck.count == 0) continue;
        const int64_t S = (ck.count + R - 1) / R;
        for (int c = 0; c < R; ++c) {
            const int64_t start = (int64_t)c * S;
            const int64_t len = std::min(S, ck.count - start);
            if (len <= 0) continue;
            ins.clear();
            outs.clear();
            for (int k = 0; k < R; ++k) ins.push_back(addr(ck.send[fold_rank(c, k, R)], start, es));
            if (bp.acc)
                for (int k = 0; k < R; ++k) ins.push_back(addr(ck.acc[fold_rank(c, k, R)], start, es));
            for (int r = 0; r < R; ++r) outs.push_back(addr(ck.recv[r], start, es));
            BatchJob j{};
            j.tile_begin = tiles;
            j.len = len;
            j.phase = job_phase(ins.data(), (int)ins.size(), outs.data(), (int)outs.size());
            tiles += tiles_of(len, (uint8_t)j.phase, bp.tile_elems);
            bp.jobs.push_back(j);
            for (uintptr_t a : ins) bp.ptrs.push_back(reinterpret_cast<const void*>(a));
            for (uintptr_t a : outs) bp.ptrs.push_back(reinterpret_cast<const void*>(a));
        }
    }
    bp.total_tiles = tiles;
    build_groups(&bp);
    shape_launch(tiles, loads, R, unroll, cfg, dev, &bp.grid, &bp.lds_bytes);
    return bp;
}

// all_to_all_single (Communicator page: split, scatter, concatenate): job
// (d, s) copies chunk d of rank s's input to chunk s of rank d's output.  The
// list form of all_gather: job k copies rank k's shard to every rank's output
// for shard k.
BatchPlan plan_copies(const Checked& ck, const Config& cfg, const DeviceInfo& dev) {
    BatchPlan bp;
    if (ck.count == 0) return bp;
    const int R = ck.nranks;
    const int64_t es = element_size(ck.dtype);
    bp.copy = true;
    bp.nranks = R;
    bp.dtype = ck.dtype;
    bp.op = RC_SUM;
    bp.nontemporal = nontemporal_of(cfg);
    bp.tile_elems = tile_elems_for(kCopyUnroll, cfg);
    std::vector<uintptr_t> ad;  // the source, then the destinations
    int64_t tiles = 0;
    auto add_job = [&](int64_t len) {
        BatchJob j{};
        j.tile_begin = tiles;
        j.len = len;
        j.phase = job_phase(ad.data(), 1, ad.data() + 1, (int)ad.size() - 1);
        tiles += tiles_of(len, (uint8_t)j.phase, bp.tile_elems);
        bp.jobs.push_back(j);
        for (uintptr_t a : ad) bp.ptrs.push_back(reinterpret_cast<const void*>(a));
    };
    if (ck.coll == Coll::AllToAll) {
        const int64_t m = ck.count / R;
        bp.nout = 1;
        for (int d = 0; d < R; ++d)
            for (int s = 0; s < R; ++s) {
                ad.assign({addr(ck.send[s], (int64_t)d * m, es), addr(ck.recv[d], (int64_t)s * m, es)});
                add_job(m);
            }
    } else {
        bp.nout = R;
        for (int k = 0; k < R; ++k) {
            ad.assign(1, addr(ck.send[k], 0, es));
            for (int r = 0; r < R; ++r) ad.push_back(addr(ck.recv_list[(size_t)r * R + k], 0, es));
            add_job(ck.count);
        }
    }
    bp.total_tiles = tiles;
    build_groups(&bp);
    // measured: the batched copies peak at less traffic in flight than the
    // single-collective kernels (all_to_all and the list all_gather alike)
    shape_launch(tiles, 1, bp.nout, kCopyUnroll, cfg, dev, &bp.grid, &bp.lds_bytes, kCopyBatchRule);
    bp.waves = cfg.waves_per_cu > 0 ? cfg.waves_per_cu : auto_waves_per_cu(1, bp.nout, kCopyUnroll, kCopyBatchRule);
    if (cfg.max_workgroups <= 0 && !bp.jobs.empty()) {
        // every job has the same length: a one-shot 2-D grid needs no job lookup
        int64_t widest = 0;
        for (size_t j = 0; j < bp.jobs.size(); ++j) {
            const int64_t next = j + 1 < bp.jobs.size() ? bp.jobs[j + 1].tile_begin : tiles;
            widest = std::max(widest, next - bp.jobs[j].tile_begin);
        }
        bp.grid_2d = 1;
        bp.grid = std::max<int64_t>(1, widest);
        bp.grid_y = (int)bp.jobs.size();
        bp.by_value = bp.jobs.size() <= (size_t)kMaxCopyArgJobs && bp.ptrs.size() <= (size_t)kMaxCopyArgPtrs;
        bool full = bp.by_value && bp.tile_elems == kBlock * kVec * kCopyUnroll;
        for (const BatchJob& jb : bp.jobs)
            full = full && jb.phase == 0 && jb.len == bp.grid * (int64_t)bp.tile_elems;
        bp.full_tiles = full;
        bp.shift_out = full && shifted_copies_pay(bp, es);
    }
    return bp;
}

}  // namespace rc
