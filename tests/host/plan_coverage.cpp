// Replays, on the CPU, the index arithmetic the kernels apply to a launch plan
// (job lookup, scalar head, 16-byte vector body in rounds, scalar tail, the
// element-by-element path and the batched group lookup) and checks that every
// element of every job is produced exactly once and that every address read
// or written lies inside the buffer it belongs to.  Links the host-only
// planner and validator; no GPU involved.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "rc_internal.h"

using namespace rc;

namespace {

struct Buffer {
    uintptr_t lo, hi;
};

std::vector<Buffer> g_bufs;
int g_fail = 0;

void fail(const std::string& what) {
    if (g_fail < 20) std::fprintf(stderr, "FAIL: %s\n", what.c_str());
    ++g_fail;
}

// buffers are allocated at increasing addresses, so g_bufs is sorted by lo
bool inside(uintptr_t a, int64_t bytes) {
    auto it = std::upper_bound(g_bufs.begin(), g_bufs.end(), a,
                               [](uintptr_t v, const Buffer& b) { return v < b.lo; });
    if (it == g_bufs.begin()) return false;
    --it;
    return a >= it->lo && a + (uintptr_t)bytes <= it->hi;
}

// Enumerate the elements tile lt of a job touches, in the kernels' loop
// structure (job_tile: rounds of U vectors per lane over the tile's vectors,
// then the job's scalars on tile 0), with the index arithmetic of tiling.h.
template <class F>
void tile_elements(int64_t len, int phase, int64_t lt, int64_t te, int unroll, F&& visit) {
    const JobSplit s = job_split(len, (uint8_t)phase, te);
    int64_t v0, v1;
    tile_vectors(s, lt, &v0, &v1);
    const int64_t step = (int64_t)kBlock * unroll;
    for (int64_t vb = v0; vb < v1; vb += step)
        for (int u = 0; u < unroll; ++u)
            for (int tid = 0; tid < kBlock; ++tid) {
                const int64_t v = vb + (int64_t)u * kBlock + tid;
                if (v < v1) visit(s.head + v * kVec, 16);
            }
    if (lt == 0)
        for (int tid = 0; tid < kBlock; ++tid)
            if (tid < scalars_of(s, len)) visit(scalar_elem(s, tid), 4);
}

// fold_table_shift_kernel's writes of one output whose job starts m elements
// past a 64-byte burst boundary (tiling.h): tile lt of ntiles whole tiles of
// T elements, shifted onto the output's bursts.
template <class F>
void shifted_tile_writes(int64_t lt, int64_t ntiles, int64_t T, int m, F&& visit) {
    const bool first = lt == 0, last = lt == ntiles - 1;
    const int64_t e0 = lt * T;
    for (int64_t w = 0; w < T; w += kVec) {
        const int lo = shifted_first(first, w, m);
        if (lo == 0) visit(e0 + w - m, 16);
        else
            for (int i = lo; i < kVec; ++i) visit(e0 + w - m + i, 4);
    }
    for (int lane = 0; lane < kBlock; ++lane)
        if (shifted_tail(last, m, lane)) visit(e0 + T - m + lane, 4);
}

// Elements of one output of one job written per (job-relative) element.
struct WriteCount {
    std::vector<uint8_t> hits;
    bool bad = false;
};

// Checks one write of `bytes` at job element e of an output whose job starts
// at address base: inside the buffer and 4-byte aligned (16-byte writes off
// the 16-byte grid rely on the unaligned access mode); counts the elements.
void count_write(WriteCount& wc, uintptr_t base, int64_t e, int bytes, int64_t len, const std::string& what) {
    const uintptr_t ad = base + (uintptr_t)(e * 4);
    if (!inside(ad, bytes)) {
        if (!wc.bad) fail(what + ": write outside its buffer");
        wc.bad = true;
    }
    if (ad % 4) {
        if (!wc.bad) fail(what + ": write off the element grid");
        wc.bad = true;
    }
    for (int i = 0; i < bytes / 4; ++i) {
        if (e + i < 0 || e + i >= len) {
            if (!wc.bad) fail(what + ": write outside its job");
            wc.bad = true;
        } else {
            wc.hits[(size_t)(e + i)] += 1;
        }
    }
}

void expect_once(const WriteCount& wc, const std::string& what) {
    for (size_t i = 0; i < wc.hits.size(); ++i)
        if (wc.hits[i] != 1) {
            fail(what + ": element " + std::to_string(i) + " written " + std::to_string(wc.hits[i]) + " times");
            return;
        }
}

// The phase must put the job's tiles on the grid of a stream of the heaviest
// 256-byte alignment class (outputs weigh 2, inputs 1): some stream of such a
// class reaches a 16-byte boundary after `head` elements and a 256-byte one
// `lead` vectors later.  Brute force over the classes, independent of the
// planner's own choice.
bool phase_fits_heaviest(const std::vector<uintptr_t>& ins, const std::vector<uintptr_t>& outs, uint8_t phase) {
    std::vector<std::pair<uintptr_t, int>> w;  // class, weight
    auto add = [&](uintptr_t a, int wt) {
        for (auto& c : w)
            if (c.first == a % kTileAlignBytes) {
                c.second += wt;
                return;
            }
        w.push_back({a % kTileAlignBytes, wt});
    };
    for (uintptr_t a : ins) add(a, 1);
    for (uintptr_t a : outs) add(a, 2);
    int best = 0;
    for (auto& c : w) best = std::max(best, c.second);
    for (auto& c : w) {
        if (c.second != best) continue;
        const uintptr_t v = c.first + (uintptr_t)phase_head(phase) * 4;
        if (v % 16 == 0 && (v + (uintptr_t)phase_lead(phase) * 16) % kTileAlignBytes == 0) return true;
    }
    return w.empty();
}

int g_table_plans = 0;      // plans whose launch carries a FoldTable
int g_acc_table_plans = 0;  // ... with accumulators

void check_plan(const LaunchPlan& p, const std::string& name) {
    const JobArgs& a = p.args;
    if (a.tile_elems % (kBlock * kVec * p.unroll)) fail(name + ": tile not a multiple of a round");
    if (p.grid < 1 || p.grid > 0x7FFFFFFF) fail(name + ": grid out of range");
    std::vector<std::vector<uint8_t>> seen(a.jobs);
    std::vector<std::vector<WriteCount>> writes(a.jobs, std::vector<WriteCount>(a.nranks));
    for (int c = 0; c < a.jobs; ++c) {
        seen[c].assign((size_t)job_len(a.n, a.seg, c), 0);
        for (auto& wc : writes[c]) wc.hits.assign((size_t)job_len(a.n, a.seg, c), 0);
    }
    if (p.split) {
        // the interior: whole tiles from job_off[c], inside the job, starting on
        // a 256-byte boundary of a stream of the job's heaviest class, after
        // the general kernel's tile 0; edges: the job's other general tiles
        if (a.full_tiles || a.in_mode != kInFold || p.acc || !a.grid_2d) fail(name + ": split off a plain fold");
        if (p.grid != p.edges + p.interior || p.interior < 1) fail(name + ": split grid is not edges + interior");
        int64_t widest = 0;
        for (int c = 0; c < a.jobs; ++c) widest = std::max<int64_t>(widest, a.tile_prefix[c + 1] - a.tile_prefix[c]);
        if (p.edges != widest - p.interior) fail(name + ": split edges do not reach the widest job");
        for (int c = 0; c < a.jobs; ++c) {
            const int64_t len = job_len(a.n, a.seg, c);
            const JobSplit sp = job_split(len, a.phase[c], a.tile_elems);
            if (p.job_off[c] != job_interior_start(sp) || p.job_off[c] + p.interior * a.tile_elems > len ||
                p.interior > job_interior_tiles(sp))
                fail(name + ": split interior past its job");
            std::vector<uintptr_t> ins, outs;
            for (int k = 0; k < p.nin; ++k)
                ins.push_back((uintptr_t)a.in[(c + 1 + k) % p.nin] + (uintptr_t)(c * a.in_stride * 4));
            for (int o = 0; o < a.nranks; ++o)
                if ((out_mask_of(a.out_mode, a.out_mask, c) >> o) & 1u)
                    outs.push_back((uintptr_t)a.out[o] + (uintptr_t)(c * a.out_stride * 4));
            // the phase that makes the interior start element a 256-byte
            // boundary of the heaviest class: (job_off * 4) mod 256 = 0 there
            bool aligned = false;
            for (uintptr_t x : ins) aligned |= (x + (uintptr_t)(p.job_off[c] * 4)) % kTileAlignBytes == 0;
            for (uintptr_t x : outs) aligned |= (x + (uintptr_t)(p.job_off[c] * 4)) % kTileAlignBytes == 0;
            if (!aligned) fail(name + ": split interior of job " + std::to_string(c) + " on no stream's boundary");
        }
    }
    const int64_t total = a.total_tiles;
    if (total != a.tile_prefix[a.jobs] || total != p.total_tiles) fail(name + ": tile totals disagree");
    if (p.shift_out) {
        // the shifted kernel only for whole-tile folds, and never where an
        // output's bytes overlap an input's (its writes ahead of a tile would
        // race the previous tile's reads)
        if (!(a.full_tiles || p.split) || p.acc) fail(name + ": shifted kernel off a whole-tile launch");
        for (int c = 0; c < a.jobs; ++c) {
            const int64_t len = job_len(a.n, a.seg, c);
            for (int o = 0; o < a.nranks; ++o) {
                if (!((out_mask_of(a.out_mode, a.out_mask, c) >> o) & 1u)) continue;
                const uintptr_t olo = (uintptr_t)a.out[o] + (uintptr_t)(c * a.out_stride * 4);
                for (int d = 0; d < a.jobs; ++d)
                    for (int r = 0; r < a.nranks; ++r) {
                        if (a.in_mode != kInFold && r != d) continue;  // a copy job reads its own source
                        const uintptr_t ilo = (uintptr_t)a.in[r] + (uintptr_t)(d * a.in_stride * 4);
                        if (olo < ilo + (uintptr_t)(job_len(a.n, a.seg, d) * 4) && ilo < olo + (uintptr_t)(len * 4))
                            fail(name + ": shifted kernel with an output over an input");
                    }
            }
        }
    }
    for (int c = a.jobs; c <= kMaxRanks; ++c)
        if (a.tile_prefix[c] != total) fail(name + ": prefix past the last job is not the total");
    // the FoldTable of a whole-tile or split fold (built by the launch layer's
    // own host code): every job's operands, and accumulators, at the ranks of
    // the ring order from the element the launch starts at; its mask, length,
    // phase and edge tiles.  The replay below takes its addresses from the
    // JobArgs, so the two must agree.
    if (a.in_mode == kInFold && a.grid_2d && (a.full_tiles || p.split) && (!p.acc || p.nin <= kAccSlot)) {
        const FoldTable t = fold_table_of(p);
        for (int c = 0; c < a.jobs; ++c) {
            const uintptr_t off = (uintptr_t)((c * a.in_stride + p.job_off[c]) * 4);
            for (int k = 0; k < p.nin; ++k) {
                if ((uintptr_t)t.in[c][k] != (uintptr_t)a.in[(c + 1 + k) % p.nin] + off)
                    fail(name + ": table operand " + std::to_string(k) + " of job " + std::to_string(c));
                if (p.acc && (uintptr_t)t.in[c][kAccSlot + k] != (uintptr_t)a.acc[(c + 1 + k) % p.nin] + off)
                    fail(name + ": table accumulator " + std::to_string(k) + " of job " + std::to_string(c));
            }
            if (t.mask[c] != out_mask_of(a.out_mode, a.out_mask, c) || t.out_off[c] != p.job_off[c] ||
                t.len[c] != job_len(a.n, a.seg, c) || t.phase[c] != a.phase[c])
                fail(name + ": table row of job " + std::to_string(c));
        }
        for (int r = 0; r < a.nranks; ++r)
            if (t.out[r] != a.out[r]) fail(name + ": table output base");
        if (t.out_stride != a.out_stride || t.mean != a.mean || t.edges != (p.split ? p.edges : 0) ||
            t.interior != (p.split ? p.interior : p.grid))
            fail(name + ": table launch fields");
        ++g_table_plans;
        if (p.acc) ++g_acc_table_plans;
    }
    // the tiles the launch visits: (job, tile, whole) with whole tiles from
    // job_off[c] (the whole-tile kernels, a split fold's interior) or the
    // general kernel's tile of the job
    struct Visit {
        int c;
        int64_t lt;
        bool whole;
    };
    std::vector<Visit> visits;
    const int64_t nwhole = p.split ? p.interior : p.grid;  // whole tiles per job
    if (a.grid_2d) {
        if (p.grid_y != a.jobs) fail(name + ": 2-D grid height is not the job count");
        for (int c = 0; c < p.grid_y; ++c)
            for (int64_t bx = 0; bx < p.grid; ++bx) {
                if (p.split && bx < p.edges) {  // an edge tile, on the general path
                    const int64_t lt = skipped_tile((int)bx, 1, (int)p.interior);
                    if (lt < a.tile_prefix[c + 1] - a.tile_prefix[c]) visits.push_back({c, lt, false});
                    continue;
                }
                if (!a.full_tiles && !p.split) {
                    if (bx < a.tile_prefix[c + 1] - a.tile_prefix[c]) visits.push_back({c, bx, false});
                    continue;
                }
                // a whole tile; the shifted kernel's workgroup takes tile xcd_group_tile
                const int64_t x = p.split ? bx - p.edges : bx;
                const int64_t lt = p.shift_out ? xcd_group_tile(x, nwhole) : x;
                if (lt < 0 || lt >= nwhole) fail(name + ": grouped tile out of range");
                visits.push_back({c, lt, true});
            }
        if (a.full_tiles) {
            // the kernels then take every tile as whole: check that it is
            for (int c = 0; c < a.jobs; ++c) {
                const int64_t len = std::max<int64_t>(0, std::min(a.seg, a.n - (int64_t)c * a.seg));
                if (a.tile_elems != kBlock * kVec * p.unroll || a.phase[c] != 0 ||
                    a.tile_prefix[c + 1] - a.tile_prefix[c] != p.grid ||
                    len != p.grid * (int64_t)a.tile_elems)
                    fail(name + ": full_tiles set on a job that is not whole tiles");
            }
        }
    } else {
        if (p.grid_y != 1) fail(name + ": 1-D launch with a 2-D grid");
        for (int64_t b = 0; b < p.grid; ++b)
            for (int64_t t = b; t < total; t += p.grid) {
                // the kernels' lookup (tiling.h)
                const int c = job_of(a.tile_prefix, (int)t);
                if (c >= a.jobs || t < a.tile_prefix[c] || t >= a.tile_prefix[c + 1]) {
                    fail(name + ": job index past the last job");
                    return;
                }
                visits.push_back({c, t - a.tile_prefix[c], false});
            }
    }
    for (const Visit& vis : visits) {
        const int c = vis.c;
        const int64_t lt = vis.lt;
        const int64_t start = (int64_t)c * a.seg;
        const int64_t len = std::min(a.seg, a.n - start);
        const uint32_t mask = out_mask_of(a.out_mode, a.out_mask, c);
        const int64_t joff = p.job_off[c];  // where a split interior starts in the job
        auto visit_tile = [&](auto&& visit) {
            if (vis.whole) {
                // the whole-tile kernels: one round of whole 16-byte vectors
                // from joff + lt*tile_elems
                for (int64_t e = joff + lt * a.tile_elems; e < joff + (lt + 1) * a.tile_elems; e += kVec) visit(e, 16);
            } else {
                tile_elements(len, a.phase[c], lt, a.tile_elems, p.unroll, visit);
            }
        };
        visit_tile([&](int64_t e, int bytes) {
            const int n = bytes / 4;
            for (int i = 0; i < n; ++i) {
                if (e + i < 0 || e + i >= len) fail(name + ": element outside its job");
                else seen[c][e + i] += 1;
            }
            // every access 4-byte aligned (vectors off the reference's grid
            // rely on the unaligned access mode for the rest)
            if (a.in_mode == kInFold) {
                for (int k = 0; k < p.nin; ++k) {
                    const uintptr_t base = (uintptr_t)a.in[(c + 1 + k) % p.nin] + (uintptr_t)(c * a.in_stride * 4);
                    const uintptr_t ad = base + (uintptr_t)(e * 4);
                    if (!inside(ad, bytes)) fail(name + ": input read outside its buffer");
                    if (ad % 4) fail(name + ": input read off the element grid");
                    if (p.acc) {
                        const uintptr_t aa = (uintptr_t)a.acc[(c + 1 + k) % p.nin] +
                                             (uintptr_t)(c * a.in_stride * 4) + (uintptr_t)(e * 4);
                        if (!inside(aa, bytes)) fail(name + ": accumulator read outside its buffer");
                        if (aa % 4) fail(name + ": accumulator read off the element grid");
                    }
                }
            } else {
                const uintptr_t ad = (uintptr_t)a.in[c] + (uintptr_t)(c * a.in_stride * 4) + (uintptr_t)(e * 4);
                if (!inside(ad, bytes)) fail(name + ": copy read outside its buffer");
                if (ad % 4) fail(name + ": copy read off the element grid");
            }
        });
        // the shifted kernel's reads ahead of the tile: pre_vectors vectors
        // of every operand, inside the job and the operand's buffer
        if (p.shift_out && vis.whole) {
            int mmax = 0;
            for (int o = 0; o < a.nranks; ++o)
                if ((mask >> o) & 1u)
                    mmax = std::max(mmax, burst_offset((uintptr_t)a.out[o] + (uintptr_t)((c * a.out_stride + joff) * 4)));
            const int npre = pre_vectors(mmax, lt == 0);
            for (int lane = 0; lane < npre; ++lane) {
                const int64_t e = joff + lt * a.tile_elems - (int64_t)(npre - lane) * kVec;
                if (e < 0 || e + kVec > len) fail(name + ": read ahead of a tile outside its job");
                for (int k = 0; k < p.nin; ++k) {
                    const void* src = a.in_mode == kInFold ? a.in[(c + 1 + k) % p.nin] : a.in[c];
                    const uintptr_t ad = (uintptr_t)src + (uintptr_t)(c * a.in_stride * 4) + (uintptr_t)(e * 4);
                    if (!inside(ad, 16)) fail(name + ": read ahead of a tile outside its buffer");
                }
            }
        }
        // writes, output by output, as the kernel makes them
        for (int o = 0; o < a.nranks; ++o) {
            if (!((mask >> o) & 1u)) continue;
            const uintptr_t base = (uintptr_t)a.out[o] + (uintptr_t)(c * a.out_stride * 4);
            WriteCount& wc = writes[c][o];
            const int m = p.shift_out && vis.whole ? burst_offset(base + (uintptr_t)(joff * 4)) : 0;
            if (m) {
                shifted_tile_writes(lt, nwhole, a.tile_elems, m, [&](int64_t e, int bytes) {
                    count_write(wc, base, joff + e, bytes, len, name);
                });
                // burst-aligned: every 16-byte write starts on a 16-byte boundary
                shifted_tile_writes(lt, nwhole, a.tile_elems, m, [&](int64_t e, int bytes) {
                    if (bytes == 16 && (base + (uintptr_t)((joff + e) * 4)) % 16)
                        fail(name + ": shifted vector write off grid");
                });
            } else {
                visit_tile([&](int64_t e, int bytes) { count_write(wc, base, e, bytes, len, name); });
            }
        }
    }
    for (int c = 0; c < a.jobs; ++c)
        for (int o = 0; o < a.nranks; ++o)
            if ((out_mask_of(a.out_mode, a.out_mask, c) >> o) & 1u)
                expect_once(writes[c][o], name + ": job " + std::to_string(c) + " output " + std::to_string(o));
    // each job's phase follows a stream of its heaviest alignment class
    for (int c = 0; c < a.jobs; ++c) {
        if (job_len(a.n, a.seg, c) == 0) continue;
        uint32_t mask = out_mask_of(a.out_mode, a.out_mask, c);
        std::vector<uintptr_t> ins, outs;
        if (a.in_mode == kInFold) {
            for (int k = 0; k < p.nin; ++k)
                ins.push_back((uintptr_t)a.in[(c + 1 + k) % p.nin] + (uintptr_t)(c * a.in_stride * 4));
            if (p.acc)
                for (int k = 0; k < p.nin; ++k)
                    ins.push_back((uintptr_t)a.acc[(c + 1 + k) % p.nin] + (uintptr_t)(c * a.in_stride * 4));
        } else {
            ins.push_back((uintptr_t)a.in[c] + (uintptr_t)(c * a.in_stride * 4));
        }
        for (int o = 0; o < a.nranks; ++o)
            if ((mask >> o) & 1u) outs.push_back((uintptr_t)a.out[o] + (uintptr_t)(c * a.out_stride * 4));
        if (!phase_fits_heaviest(ins, outs, a.phase[c]))
            fail(name + ": job " + std::to_string(c) + " is not tiled on its heaviest alignment class");
    }
    for (int c = 0; c < a.jobs; ++c) {
        const int64_t len = std::max<int64_t>(0, std::min(a.seg, a.n - (int64_t)c * a.seg));
        for (int64_t e = 0; e < len; ++e) {
            if (seen[c][e] != 1) {
                fail(name + ": job " + std::to_string(c) + " element " + std::to_string(e) + " produced " +
                     std::to_string(seen[c][e]) + " times");
                return;
            }
        }
    }
}

uintptr_t g_next = 0x100000;

uintptr_t alloc(int64_t bytes, int misalign_elems) {
    const uintptr_t a = (g_next + 255) / 256 * 256 + (uintptr_t)misalign_elems * 4;
    g_next = a + (uintptr_t)bytes + 4096;
    g_bufs.push_back({a, a + (uintptr_t)bytes});
    return a;
}

rc_buf make(const void* s, void* r, int64_t n, int op = RC_SUM, int root = 0) {
    rc_buf b{};
    b.send = s;
    b.recv = r;
    b.dtype = RC_F32;
    b.op = op;
    b.root = root;
    b.ndim = 1;
    b.dims[0] = n;
    return b;
}

}  // namespace

int main(int argc, char** argv) {
    const int iters = argc > 1 ? std::atoi(argv[1]) : 300;
    std::mt19937_64 rng(12345);
    DeviceInfo dev;
    dev.cu_count = 256;
    dev.lds_per_cu = 160 * 1024;
    dev.max_lds_per_block = 64 * 1024;
    int plans = 0;
    int full_plans = 0;  // plans whose kernels take the whole-tile path
    int split_plans = 0;  // folds split into a whole-tile interior and edges
    // job_phase: the head reaches a 16-byte boundary and the lead a 256-byte
    // one of a stream of the heaviest alignment class
    for (int i = 0; i < 20000; ++i) {
        const int nin = 1 + (int)(rng() % 6), nout = (int)(rng() % 6);
        std::vector<uintptr_t> ins, outs;
        const uintptr_t base = 0x10000 + (uintptr_t)(rng() % 8192) * 4;
        for (int k = 0; k < nin + nout; ++k) {
            // a few classes only, so that ties and majorities both occur
            const uintptr_t a = base + 4096 * (uintptr_t)(1 + rng() % 5) + 4 * (uintptr_t)(rng() % 3);
            (k < nin ? ins : outs).push_back(a);
        }
        const uint8_t ph = job_phase(ins.data(), nin, outs.data(), nout);
        if (!phase_fits_heaviest(ins, outs, ph)) fail("job_phase: not on the heaviest class");
        const int ref = job_reference(ins.data(), nin, outs.data(), nout);
        if (ref < 0 || ref >= nin + nout || phase_of(ref < nin ? ins[ref] : outs[ref - nin]) != ph)
            fail("job_reference and job_phase disagree");
    }
    for (int it = 0; it < iters; ++it) {
        g_bufs.clear();
        const int R = 1 + (int)(rng() % 16);
        const int sizes[] = {0, 1, 2, 3, 5, 7, 64, 255, 256, 257, 1000, 4099, 20000, 65537};
        int64_t n = sizes[rng() % 14];
        if (rng() % 3 == 0) n = (int64_t)(rng() % 50000);
        if (rng() % 4 == 0) n = (int64_t)R * 4096 * (int64_t)(1 + rng() % 3);  // whole tiles per segment
        Config cfg;
        cfg.algo = rng() % 2 ? RC_ALGO_RING : RC_ALGO_DIRECT;
        const int64_t tiles[] = {0, 0, 256, 1024, 4096};
        cfg.tile_elems = tiles[rng() % 5];
        cfg.max_workgroups = rng() % 3 == 0 ? (int)(1 + rng() % 50) : 0;
        cfg.waves_per_cu = (int)(rng() % 9);
        if (rng() % 2) cfg.split_min_bytes = 0;  // split folds whatever their size
        const int mis_mode = (int)(rng() % 3);  // 0 aligned, 1 common offset, 2 mixed offsets
        auto mis = [&](int r) { return mis_mode == 0 ? 0 : (mis_mode == 1 ? 1 + (int)(it % 3) : (r * 3 + it) % 4); };
        const int coll = (int)(rng() % 5);
        std::vector<rc_buf> bufs(R);
        if (coll == 3) n = (n / R) * R;  // reduce_scatter needs R | n
        for (int r = 0; r < R; ++r) {
            const int64_t out_n = coll == 3 ? n / R : (coll == 4 ? n * R : n);
            void* s = (void*)alloc(std::max<int64_t>(n, 1) * 4, mis_mode == 3 ? 0 : mis(r));
            void* o = (void*)alloc(std::max<int64_t>(out_n, 1) * 4, mis(r + 1));
            bufs[r] = make(s, o, n, RC_SUM, coll == 2 ? -1 : (int)(it % R));
        }
        Coll kind = Coll::AllReduce;
        if (coll == 1) kind = Coll::Reduce;
        if (coll == 2) {
            kind = Coll::Broadcast;
            for (int r = 0; r < R; ++r)
                if (r != (int)(it % R)) bufs[r].send = nullptr;
        }
        if (coll == 3) kind = Coll::ReduceScatter;
        if (coll == 4) kind = Coll::AllGather;
        Checked ck;
        Error e = validate(kind, R, bufs.data(), &ck);
        if (e.code) {
            fail("validation rejected a valid call: " + e.msg);
            continue;
        }
        if (kind == Coll::AllReduce && rng() % 2) {  // a gradient sync's accumulators
            ck.has_acc = true;
            for (int r = 0; r < R; ++r) ck.acc[r] = (const void*)alloc(std::max<int64_t>(n, 1) * 4, mis(r + 2));
        }
        for (const LaunchPlan& p : plan(ck, cfg, dev)) {
            check_plan(p, "coll " + std::to_string(coll) + " R=" + std::to_string(R) + " n=" + std::to_string(n) +
                              " mis=" + std::to_string(mis_mode) + (ck.has_acc ? " acc" : ""));
            ++plans;
            if (p.args.full_tiles) ++full_plans;
            if (p.split) ++split_plans;
        }
    }
    {
        // whole-tile all-reduces of 4-7 ranks run one vector per lane: their
        // plans replay like any other, with tiles of 256 elements
        for (int R = 4; R < 8; ++R) {
        g_bufs.clear();
        const int64_t n = (int64_t)R * 4096 * 3;
        std::vector<rc_buf> bufs(R);
        for (int r = 0; r < R; ++r) bufs[r] = make((void*)alloc(n * 4, 0), (void*)alloc(n * 4, 0), n);
        Checked ck;
        if (validate(Coll::AllReduce, R, bufs.data(), &ck).code) fail("all-reduce rejected");
        Config cfg;
        for (const LaunchPlan& p : plan(ck, cfg, dev)) {
            check_plan(p, "whole-tile all-reduce of " + std::to_string(R) + " ranks");
            ++plans;
            if (!p.args.full_tiles || p.unroll != 1 || p.args.tile_elems != kBlock * kVec)
                fail("whole-tile all-reduce of 4-7 ranks does not run one vector per lane");
        }
        }
    }
    {
        // whole-tile gradient syncs with accumulators, in place into them and
        // not, direct and ring: up to kAccSlot ranks on the table kernel
        for (int R = 1; R <= 10; ++R)
            for (int variant = 0; variant < 4; ++variant) {
                g_bufs.clear();
                const int64_t n = (int64_t)R * 4096 * 2;
                const bool in_place = variant & 1;
                std::vector<rc_buf> bufs(R);
                std::vector<const void*> accs(R);
                for (int r = 0; r < R; ++r) {
                    accs[r] = (const void*)alloc(n * 4, 0);
                    void* o = in_place ? (void*)accs[r] : (void*)alloc(n * 4, 0);
                    bufs[r] = make((void*)alloc(n * 4, 0), o, n);
                }
                Checked ck;
                if (validate(Coll::AllReduce, R, bufs.data(), &ck).code) fail("all-reduce rejected");
                ck.has_acc = true;
                for (int r = 0; r < R; ++r) ck.acc[r] = accs[r];
                Config cfg;
                cfg.algo = variant & 2 ? RC_ALGO_RING : RC_ALGO_DIRECT;
                const int before = g_acc_table_plans;
                for (const LaunchPlan& p : plan(ck, cfg, dev)) {
                    check_plan(p, "whole-tile sync with accumulators, R=" + std::to_string(R) +
                                      (in_place ? " in place" : "") + (variant & 2 ? " ring" : ""));
                    ++plans;
                    if (p.acc && !p.args.full_tiles) fail("whole-tile sync with accumulators off the whole-tile path");
                }
                if ((g_acc_table_plans > before) != (R <= kAccSlot))
                    fail("sync with accumulators of " + std::to_string(R) + " ranks: table kernel " +
                         (R <= kAccSlot ? "not taken" : "taken"));
            }
    }
    // whole-tile folds with outputs off a 64-byte burst (offsets 0..15
    // elements): the shifted kernel, except in place
    int shifted_plans = 0;
    for (int it = 0; it < iters; ++it) {
        g_bufs.clear();
        const int R = 1 + (int)(rng() % 16);
        // up to 128 tiles per job: several whole groups of tiles per XCD and a
        // partial one; sometimes a ragged length (split: the interior shifted)
        int64_t n = (int64_t)R * 4096 * (int64_t)(1 + rng() % 8);
        if (rng() % 3 == 0) n += (int64_t)R * (1 + (int64_t)(rng() % 40));
        // all_reduce, reduce, reduce_scatter, broadcast, all_gather (of shards of n / R)
        const int coll = (int)(rng() % 5);
        const bool in_place = (coll == 0 || coll == 3) && rng() % 4 == 0;
        const int op = coll >= 3 ? RC_SUM : (rng() % 2 ? RC_SUM : RC_MEAN);
        const int root = (int)(it % R);
        const int64_t in_n = coll == 4 ? n / R : n;
        std::vector<rc_buf> bufs(R);
        for (int r = 0; r < R; ++r) {
            const int64_t out_n = coll == 2 ? n / R : n;
            void* sb = (void*)alloc(in_n * 4, rng() % 2 ? 0 : (int)(rng() % 16));
            void* ob = in_place ? sb : (void*)alloc(out_n * 4, (int)(rng() % 16));
            bufs[r] = make(coll == 3 && r != root ? nullptr : sb, ob, in_n, op, coll == 1 || coll == 3 ? root : 0);
        }
        Checked ck;
        const Coll kinds[] = {Coll::AllReduce, Coll::Reduce, Coll::ReduceScatter, Coll::Broadcast, Coll::AllGather};
        const Coll kind = kinds[coll];
        const Error ve = validate(kind, R, bufs.data(), &ck);
        if (ve.code) {
            fail("whole-tile fold with outputs off a burst rejected: " + ve.msg);
            continue;
        }
        Config cfg;
        cfg.algo = rng() % 4 == 0 ? RC_ALGO_RING : RC_ALGO_DIRECT;
        cfg.split_min_bytes = 0;
        for (const LaunchPlan& p : plan(ck, cfg, dev)) {
            if (p.split) ++split_plans;
            check_plan(p, "outputs off a burst: coll " + std::to_string(coll) + " R=" + std::to_string(R) +
                              (in_place ? " in place" : ""));
            ++plans;
            if (p.shift_out) ++shifted_plans;
            // in place an all-reduce's fold writes over its inputs (the ring's
            // all-gather phase reads only the owner's segment and writes the
            // other ranks', and a broadcast sender's own buffer is not
            // written: those may shift)
            if (in_place && p.args.in_mode == kInFold && p.shift_out)
                fail("shifted fold chosen for an all-reduce in place");
        }
    }
    // batched plans: job lookup through the group index, and coverage
    int batches = 0;
    for (int it = 0; it < iters / 3; ++it) {
        g_bufs.clear();
        const int R = 1 + (int)(rng() % 8);
        const int T = 1 + (int)(rng() % 40);
        const bool with_acc = rng() % 2;  // every tensor with accumulators, or none
        std::vector<rc_buf> rows;
        std::vector<const void*> accs;
        for (int t = 0; t < T; ++t) {
            int64_t n = (int64_t)(rng() % 4) == 0 ? (int64_t)(rng() % 300000) : (int64_t)(rng() % 700);
            const int mis_mode = (int)(rng() % 3);
            for (int r = 0; r < R; ++r) {
                const int m = mis_mode == 0 ? 0 : (mis_mode == 1 ? 2 : (r + t) % 4);
                void* s = (void*)alloc(std::max<int64_t>(n, 1) * 4, m);
                void* o = (void*)alloc(std::max<int64_t>(n, 1) * 4, m);
                rows.push_back(make(s, o, n, RC_MEAN));
                accs.push_back(with_acc ? (const void*)alloc(std::max<int64_t>(n, 1) * 4, mis_mode == 2 ? (r + t + 1) % 4 : m)
                                        : nullptr);
            }
        }
        std::vector<Checked> cks;
        Error e = validate_batch(R, T, rows.data(), &cks, nullptr, accs.data());
        if (e.code) {
            fail("batch validation rejected a valid call: " + e.msg);
            continue;
        }
        Config cfg;
        cfg.waves_per_cu = (int)(rng() % 9);
        std::vector<Checked> nonempty;
        for (const Checked& ck : cks)
            if (ck.count) nonempty.push_back(ck);
        const BatchPlan bp = plan_batch(nonempty, cfg, dev);
        if (!nonempty.empty() && bp.acc != with_acc) fail("batched plan lost the accumulators");
        const int unroll = unroll_for(with_acc ? 2 * R : R);
        const int ptrs_per_job = (with_acc ? 3 : 2) * R;
        if (bp.ptrs.size() != bp.jobs.size() * (size_t)ptrs_per_job) fail("batched pointer table has the wrong size");
        std::vector<std::vector<uint8_t>> seen(bp.jobs.size());
        std::vector<std::vector<WriteCount>> bwrites(bp.jobs.size(), std::vector<WriteCount>(R));
        for (size_t j = 0; j < bp.jobs.size(); ++j) {
            seen[j].assign((size_t)bp.jobs[j].len, 0);
            for (auto& wc : bwrites[j]) wc.hits.assign((size_t)bp.jobs[j].len, 0);
        }
        const int64_t ngroups = (int64_t)bp.group_job.size();
        for (size_t j = 0; j < bp.jobs.size(); ++j) {
            const auto* tp = &bp.ptrs[j * ptrs_per_job];
            const int nins = (with_acc ? 2 : 1) * R;
            std::vector<uintptr_t> ins, outs;
            for (int k = 0; k < ptrs_per_job; ++k) (k < nins ? ins : outs).push_back((uintptr_t)tp[k]);
            if (!phase_fits_heaviest(ins, outs, (uint8_t)bp.jobs[j].phase))
                fail("batched job not tiled on its heaviest alignment class");
        }
        for (int64_t t = 0; t < bp.total_tiles; ++t) {
            const int64_t g = t >> kGroupShift;
            if (g >= ngroups) {
                fail("group index out of range");
                break;
            }
            const int lo = find_job(bp.jobs.data(), bp.group_job.data(), ngroups, (int)bp.jobs.size(), t);
            const BatchJob& jb = bp.jobs[lo];
            const int64_t next = lo + 1 < (int)bp.jobs.size() ? bp.jobs[lo + 1].tile_begin : bp.total_tiles;
            if (!(jb.tile_begin <= t && t < next)) fail("group lookup found the wrong job");
            const int nreads = (with_acc ? 2 : 1) * R;
            tile_elements(jb.len, jb.phase, t - jb.tile_begin, bp.tile_elems, unroll, [&](int64_t e, int bytes) {
                for (int i = 0; i < bytes / 4; ++i) {
                    if (e + i >= jb.len) fail("batched element outside its job");
                    else seen[lo][e + i] += 1;
                }
                for (int k = 0; k < nreads; ++k) {
                    const uintptr_t ad = (uintptr_t)bp.ptrs[(size_t)lo * ptrs_per_job + k] + (uintptr_t)(e * 4);
                    if (!inside(ad, bytes)) fail("batched read outside its buffer");
                    if (ad % 4) fail("batched read off the element grid");
                }
            });
            for (int r = 0; r < R; ++r) {
                const uintptr_t base = (uintptr_t)bp.ptrs[(size_t)lo * ptrs_per_job + nreads + r];
                WriteCount& wc = bwrites[lo][r];
                tile_elements(jb.len, jb.phase, t - jb.tile_begin, bp.tile_elems, unroll,
                              [&](int64_t e, int bytes) { count_write(wc, base, e, bytes, jb.len, "batched"); });
            }
        }
        for (size_t j = 0; j < bp.jobs.size(); ++j) {
            for (int64_t e = 0; e < bp.jobs[j].len; ++e)
                if (seen[j][e] != 1) {
                    fail("batched job element not produced exactly once");
                    break;
                }
            for (int r = 0; r < R; ++r) expect_once(bwrites[j][r], "batched job output");
        }
        ++batches;
    }
    // copy batches: all_to_all_single and the list form of all_gather; every
    // destination element written exactly once, every access in bounds
    int copies = 0;
    int full_copy_batches = 0;     // copy batches on the whole-tile kernel
    int shifted_copy_batches = 0;  // and on its shifted form
    for (int it = 0; it < iters / 2; ++it) {
        g_bufs.clear();
        const int R = 1 + (int)(rng() % 16);
        bool a2a = rng() % 2;
        int64_t m = (int64_t)(rng() % 3 == 0 ? rng() % 40000 : rng() % 300);
        if (rng() % 4 == 0) m = 2048 * (1 + (int64_t)(rng() % 3));  // whole tiles for every tile size tried
        if (rng() % 4 == 0) m = 512 * (1 + (int64_t)(rng() % 80));  // whole tiles, several groups per XCD
        // 3: the list all_gather in whole tiles with the destinations of odd
        // ranks off their 64-byte bursts (the shifted copy kernel; sources and
        // even ranks' destinations aligned keep the aligned class the heaviest)
        const int mis_mode = (int)(rng() % 4);
        if (mis_mode == 3) {
            m = 512 * (1 + (int64_t)(rng() % 80));
            a2a = false;
        }
        auto mis = [&](int r) { return mis_mode == 0 ? 0 : (mis_mode == 1 ? 1 : (r * 3 + it) % 4); };
        auto dst_mis = [&](int i) {  // destination i = r * R + k of the list
            if (mis_mode != 3) return mis(i + 2);
            const int r = i / R;
            return r % 2 == 0 ? 0 : 1 + (r * 5 + it) % 15;
        };
        std::vector<rc_buf> bufs(R);
        std::vector<void*> recv_list;
        // destination buffers, with per-element write counts
        struct Dst {
            uintptr_t lo;
            int64_t n;
            std::vector<uint8_t> hits;
        };
        std::vector<Dst> dsts;
        const int64_t n = a2a ? m * R : m;
        for (int r = 0; r < R; ++r) {
            void* s = (void*)alloc(std::max<int64_t>(n, 1) * 4, mis_mode == 3 ? 0 : mis(r));
            void* o = nullptr;
            if (a2a) {
                o = (void*)alloc(std::max<int64_t>(n, 1) * 4, mis(r + 1));
                dsts.push_back({(uintptr_t)o, n, std::vector<uint8_t>((size_t)n, 0)});
            }
            bufs[r] = make(s, o, n);
        }
        if (!a2a)
            for (int i = 0; i < R * R; ++i) {
                void* o = (void*)alloc(std::max<int64_t>(m, 1) * 4, dst_mis(i));
                recv_list.push_back(o);
                dsts.push_back({(uintptr_t)o, m, std::vector<uint8_t>((size_t)m, 0)});
            }
        Checked ck;
        Error e = validate(a2a ? Coll::AllToAll : Coll::AllGatherList, R, bufs.data(), &ck,
                           a2a ? nullptr : recv_list.data());
        if (e.code) {
            fail("copy validation rejected a valid call: " + e.msg);
            continue;
        }
        Config cfg;
        cfg.waves_per_cu = (int)(rng() % 9);
        cfg.max_workgroups = rng() % 3 == 0 && mis_mode != 3 ? (int)(1 + rng() % 50) : 0;
        const int64_t tes[] = {0, 0, 2048, 8192};
        cfg.tile_elems = mis_mode == 3 ? 0 : tes[rng() % 4];
        const BatchPlan bp = plan_copies(ck, cfg, dev);
        const int per_job = 1 + bp.nout;
        if (ck.count > 0 && (!bp.copy || bp.ptrs.size() != bp.jobs.size() * (size_t)per_job))
            fail("copy plan has the wrong shape");
        for (size_t j = 0; j < bp.jobs.size(); ++j) {
            const auto* tp = &bp.ptrs[j * per_job];
            std::vector<uintptr_t> ins{(uintptr_t)tp[0]}, outs;
            for (int k = 1; k < per_job; ++k) outs.push_back((uintptr_t)tp[k]);
            if (!phase_fits_heaviest(ins, outs, (uint8_t)bp.jobs[j].phase))
                fail("copy job not tiled on its heaviest alignment class");
        }
        // the (job, tile) pairs the launch visits: one-shot 2-D grid (y = job,
        // tiles past the job's own count exit) or the 1-D group lookup
        std::vector<std::pair<int, int64_t>> visits;
        if (bp.grid_2d) {
            if (bp.grid_y != (int)bp.jobs.size()) fail("copy 2-D grid height is not the job count");
            for (int j = 0; j < bp.grid_y; ++j) {
                const BatchJob& jb = bp.jobs[j];
                const int64_t own = tiles_of(jb.len, (uint8_t)jb.phase, bp.tile_elems);
                if (own > bp.grid) fail("copy 2-D grid narrower than a job");
                if (bp.full_tiles && (!bp.by_value || jb.phase != 0 || bp.tile_elems != kBlock * kVec * kCopyUnroll ||
                                      jb.len != bp.grid * (int64_t)bp.tile_elems))
                    fail("whole-tile copy batch on a job that is not whole tiles");
                for (int64_t bx = 0; bx < bp.grid; ++bx) {
                    const int64_t lt = bp.shift_out ? xcd_group_tile(bx, bp.grid) : bx;
                    if (bp.full_tiles || lt < own) visits.push_back({j, lt});
                }
            }
            if (bp.full_tiles) ++full_copy_batches;
            if (bp.shift_out) {
                ++shifted_copy_batches;
                if (!bp.full_tiles) fail("shifted copy batch off whole tiles");
                const size_t per = (size_t)per_job;
                for (size_t j = 0; j < bp.jobs.size(); ++j)
                    for (size_t k = 1; k < per; ++k) {
                        const uintptr_t d = (uintptr_t)bp.ptrs[j * per + k];
                        for (size_t i = 0; i < bp.jobs.size(); ++i) {
                            const uintptr_t sp = (uintptr_t)bp.ptrs[i * per];
                            if (d < sp + (uintptr_t)(bp.jobs[i].len * 4) && sp < d + (uintptr_t)(bp.jobs[j].len * 4))
                                fail("shifted copy batch with a destination over a source");
                        }
                    }
            }
        } else {
            const int64_t ngroups = (int64_t)bp.group_job.size();
            for (int64_t t = 0; t < bp.total_tiles; ++t) {
                const int lo = find_job(bp.jobs.data(), bp.group_job.data(), ngroups, (int)bp.jobs.size(), t);
                const int64_t next = lo + 1 < (int)bp.jobs.size() ? bp.jobs[lo + 1].tile_begin : bp.total_tiles;
                if (!(bp.jobs[lo].tile_begin <= t && t < next)) fail("copy group lookup found the wrong job");
                visits.push_back({lo, t - bp.jobs[lo].tile_begin});
            }
        }
        for (const auto& v : visits) {
            const int lo = v.first;
            const BatchJob& jb = bp.jobs[lo];
            auto visit_copy_tile = [&](auto&& visit) {
                if (bp.full_tiles) {  // copy_args_full_kernel: one whole round from lt*tile_elems
                    for (int64_t el = v.second * bp.tile_elems; el < (v.second + 1) * bp.tile_elems; el += kVec)
                        visit(el, 16);
                } else {
                    tile_elements(jb.len, jb.phase, v.second, bp.tile_elems, kCopyUnroll, visit);
                }
            };
            visit_copy_tile([&](int64_t el, int bytes) {
                const uintptr_t ad = (uintptr_t)bp.ptrs[(size_t)lo * per_job] + (uintptr_t)(el * 4);
                if (!inside(ad, bytes)) fail("copy read outside its buffer");
                if (ad % 4) fail("copy read off the element grid");
            });
            if (bp.shift_out) {  // the source read ahead of the tile
                int mmax = 0;
                for (int k = 1; k < per_job; ++k)
                    mmax = std::max(mmax, burst_offset((uintptr_t)bp.ptrs[(size_t)lo * per_job + k]));
                const int npre = pre_vectors(mmax, v.second == 0);
                for (int lane = 0; lane < npre; ++lane) {
                    const int64_t el = v.second * bp.tile_elems - (int64_t)(npre - lane) * kVec;
                    const uintptr_t ad = (uintptr_t)bp.ptrs[(size_t)lo * per_job] + (uintptr_t)(el * 4);
                    if (el < 0 || !inside(ad, 16)) fail("copy read ahead of a tile outside its job or buffer");
                }
            }
            for (int k = 1; k < per_job; ++k) {
                const uintptr_t base = (uintptr_t)bp.ptrs[(size_t)lo * per_job + k];
                auto write = [&](int64_t el, int bytes) {
                    const uintptr_t ad = base + (uintptr_t)(el * 4);
                    if (!inside(ad, bytes)) fail("copy write outside its buffer");
                    if (ad % 4) fail("copy write off the element grid");
                    if (el < 0 || el + bytes / 4 > jb.len) fail("copy write outside its job");
                    for (Dst& d : dsts)
                        if (ad >= d.lo && ad < d.lo + (uintptr_t)d.n * 4)
                            for (int i = 0; i < bytes / 4; ++i) d.hits[(ad - d.lo) / 4 + i] += 1;
                };
                const int msh = bp.shift_out ? burst_offset(base) : 0;
                if (msh) {
                    shifted_tile_writes(v.second, bp.grid, bp.tile_elems, msh, write);
                    shifted_tile_writes(v.second, bp.grid, bp.tile_elems, msh, [&](int64_t el, int bytes) {
                        if (bytes == 16 && (base + (uintptr_t)(el * 4)) % 16) fail("shifted copy write off grid");
                    });
                } else if (bp.full_tiles) {
                    for (int64_t el = v.second * bp.tile_elems; el < (v.second + 1) * bp.tile_elems; el += kVec)
                        write(el, 16);
                } else {
                    tile_elements(jb.len, jb.phase, v.second, bp.tile_elems, kCopyUnroll, write);
                }
            }
        }
        for (const Dst& d : dsts)
            for (int64_t i = 0; i < d.n; ++i)
                if (d.hits[i] != 1) {
                    fail(std::string(a2a ? "all_to_all" : "all_gather_list") + ": destination element written " +
                         std::to_string(d.hits[i]) + " times");
                    i = d.n;
                }
        ++copies;
    }
    if (iters >= 100 && full_plans == 0) fail("no plan took the whole-tile path");
    if (iters >= 100 && shifted_plans == 0) fail("no plan took the shifted whole-tile kernel");
    if (iters >= 100 && split_plans == 0) fail("no fold was split");
    if (iters >= 100 && g_acc_table_plans == 0) fail("no fold with accumulators took the table kernel");
    if (iters >= 100 && shifted_copy_batches == 0) fail("no copy batch took the shifted whole-tile kernel");
    if (iters >= 100 && full_copy_batches == 0) fail("no copy batch took the whole-tile path");
    // occupancy tuner: candidates are the rule's W and the two below (never
    // under 2), each timed kTuneSamples times in turn, and the lowest median
    // wins (ties keep the rule's value); nothing is timed once a value is chosen
    for (int rule : {2, 3, 7, 10, 32}) {
        for (int fastest = 0; fastest < kTuneCands; ++fastest) {
            TuneEntry t;
            std::vector<std::pair<int, int>> issued;  // (W, cand)
            for (int call = 0; call < 3 * kTuneCands * kTuneSamples; ++call) {
                int cand = -1;
                const int w = tune_pick(t, rule, &cand);
                if (w < 2 || w > rule) fail("tuner picked a wave count outside [2, rule]");
                if (cand >= 0) {
                    if (t.cand[cand] != w) fail("tuner candidate and wave count disagree");
                    issued.push_back({w, cand});
                } else if (!t.chosen && w != rule) {
                    fail("untimed launch before the choice does not use the rule's value");
                }
                // read the oldest timed launch two calls late
                if (issued.size() > 2 || (cand < 0 && !issued.empty())) {
                    const auto s0 = issued.front();
                    issued.erase(issued.begin());
                    const int pos = rule - s0.first;  // 0 = rule
                    tune_record(t, s0.second, pos == fastest ? 100.0f : 120.0f + (float)pos);
                }
            }
            const int expect_n = std::min(kTuneCands, rule - 1);
            if (t.ncand != expect_n) fail("tuner candidate count");
            const int want = fastest < t.ncand ? rule - fastest : rule;
            if (t.chosen != want)
                fail("tuner chose " + std::to_string(t.chosen) + " for rule " + std::to_string(rule) + ", want " +
                     std::to_string(want));
            int c2 = 0;
            if (tune_pick(t, rule, &c2) != want || c2 != -1) fail("tuner still timing after its choice");
        }
    }
    {
        // medians, not best samples: one lucky sample does not win, and a
        // candidate must beat the rule's W by kTuneMargin
        auto run = [](const std::vector<std::vector<float>>& samples) {  // [cand][sample], cand 0 = rule
            TuneEntry t;
            int c = 0;
            std::vector<int> next(kTuneCands, 0);
            for (int i = 0; i < kTuneCands * kTuneSamples; ++i) {
                tune_pick(t, 7, &c);
                tune_record(t, c, samples[c][next[c]++]);
            }
            return t.chosen;
        };
        static_assert(kTuneSamples == 5, "the cases below list five samples per candidate");
        if (run({{110, 110, 110, 110, 110}, {115, 115, 115, 115, 115}, {90, 80, 130, 130, 130}}) != 7)
            fail("tuner followed two lucky samples");
        if (run({{110, 110, 110, 110, 110}, {107.5f, 107.5f, 107.5f, 107.5f, 107.5f}, {120, 120, 120, 120, 120}}) != 7)
            fail("tuner switched for a gain inside the margin");
        if (run({{110, 110, 110, 110, 110}, {104, 200, 104, 90, 104}, {120, 120, 120, 120, 120}}) != 6)
            fail("tuner missed a clear gain");
    }
    {
        TuneEntry t;  // equal times: the rule's value stays
        int c = 0;
        for (int i = 0; i < kTuneCands * kTuneSamples; ++i) {
            tune_pick(t, 7, &c);
            tune_record(t, c, 50.0f);
        }
        if (t.chosen != 7) fail("tuner left the rule's value on a tie");
    }
    std::printf("checked %d plans (%d whole-tile, %d shifted, %d split; %d tables, %d with accumulators), "
                "%d batches and %d copy batches (%d whole-tile, %d shifted): %d failures\n",
                plans, full_plans, shifted_plans, split_plans, g_table_plans, g_acc_table_plans, batches, copies,
                full_copy_batches, shifted_copy_batches, g_fail);
    return g_fail ? 1 : 0;
}
