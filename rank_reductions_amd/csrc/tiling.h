// Index arithmetic of a job (one ring segment of one tensor) shared by the
// planner on the host, the kernels on the GPU and the CPU replay of the
// kernels' accesses: how a job's elements split into a scalar head, 16-byte
// vectors and a scalar tail, which vectors each tile covers, how many tiles a
// job has, and which job a tile of a launch belongs to.  One definition, so
// that what the planner sizes is what the kernels run.
//
// The ring segments themselves follow the ruCCL README (ja), "CUDA tensor
// example" (a ring AllReduce over logical ranks on one GPU): segment c of N
// elements over R ranks is [c*S, min((c+1)*S, N)) with S = ceil(N/R).
#pragma once

#include <cstdint>

// Functions compiled for both sides: device code under hipcc, plain inline
// functions under the host compiler that builds the planner.
#if defined(__HIPCC__)
#define RC_HD __host__ __device__ __forceinline__
#define RC_UNROLL _Pragma("unroll")
#else
#define RC_HD inline
#define RC_UNROLL
#endif

namespace rc {

constexpr int kMaxRanks = 16;        // equals RC_MAX_RANKS of rc.h
constexpr int kBlock = 64;           // threads per workgroup: one wave64
constexpr int kVec = 4;              // 32-bit elements per 16-byte vector
constexpr int kTileAlignBytes = 256; // full tiles start on this boundary of the reference stream

// A job's phase packs where its reference stream (the address its tiles are
// aligned to, chosen by the planner) reaches alignment: bits 0-1 hold the
// scalar elements before the reference reaches a 16-byte boundary, bits 2-5
// the 16-byte vectors after that before it reaches a kTileAlignBytes
// boundary.  Those vectors form a short first tile, so that every full tile
// starts on the boundary.  The job's other streams are accessed at the same
// element offsets; where they are not aligned like the reference their
// 16-byte accesses are only 4-byte aligned.
RC_HD constexpr uint8_t phase_code(int head, int lead) { return (uint8_t)(head | (lead << 2)); }
RC_HD constexpr int phase_head(uint8_t phase) { return phase & 3; }
RC_HD constexpr int phase_lead(uint8_t phase) { return (phase >> 2) & 15; }

RC_HD int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
RC_HD int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

// Length of job c of a launch whose jobs are consecutive runs of `seg`
// elements of an index space of n (the last ones possibly short or empty).
RC_HD int64_t job_len(int64_t n, int64_t seg, int c) { return max64(0, min64(seg, n - (int64_t)c * seg)); }

// How a job of `len` elements splits: `head` scalar elements, then `nvec`
// 16-byte vectors, then scalars from `tail0` to len.  With `lead` > 0, tile 0
// holds the first `lead` vectors alone and tile t >= 1 starts at vector
// lead + (t-1)*tv; otherwise tile t starts at vector t*tv.
struct JobSplit {
    int64_t head;
    int64_t nvec;
    int64_t tail0;
    int64_t lead;
    int64_t tv;     // vectors per full tile
};

RC_HD JobSplit job_split(int64_t len, uint8_t phase, int64_t tile_elems) {
    JobSplit s;
    s.head = min64(phase_head(phase), len);
    s.nvec = (len - s.head) / kVec;
    s.tail0 = s.head + s.nvec * kVec;
    s.lead = min64(phase_lead(phase), s.nvec);
    s.tv = tile_elems / kVec;
    return s;
}

// Tiles of a job (0 for an empty job; at least 1 otherwise, the scalars of a
// job with no whole vector riding on tile 0).
RC_HD int64_t tiles_of(int64_t len, uint8_t phase, int64_t tile_elems) {
    if (len <= 0) return 0;
    const JobSplit s = job_split(len, phase, tile_elems);
    return max64(1, (s.lead > 0 ? 1 : 0) + (s.nvec - s.lead + s.tv - 1) / s.tv);
}

// Vectors [*v0, *v1) of tile lt.
RC_HD void tile_vectors(const JobSplit& s, int64_t lt, int64_t* v0, int64_t* v1) {
    const int64_t shift = s.lead > 0 ? s.lead - s.tv : 0;
    *v0 = max64(0, lt * s.tv + shift);
    *v1 = min64((lt + 1) * s.tv + shift, s.nvec);
}

// Scalars of a job (head and tail together, at most 6), done by the first
// lanes of tile 0: lane `lane` < scalars_of(s, len) takes element
// scalar_elem(s, lane).
RC_HD int64_t scalars_of(const JobSplit& s, int64_t len) { return s.head + (len - s.tail0); }
RC_HD int64_t scalar_elem(const JobSplit& s, int64_t lane) {
    return lane < s.head ? lane : s.tail0 + (lane - s.head);
}

// Job of tile t in a launch of up to kMaxRanks jobs: the number of job
// boundaries at or below t, where prefix[j] is the first tile of job j and
// entries past the last job equal the tile total, which t never reaches.
RC_HD int job_of(const int32_t* prefix, int t) {
    int c = 0;
    RC_UNROLL
    for (int j = 1; j < kMaxRanks; ++j) c += t >= prefix[j] ? 1 : 0;
    return c;
}

// The job's tile that workgroup x of a 2-D grid takes when the job's tiles
// [from, from + count) belong to another launch (the interior of a split
// fold, done on the whole-tile kernels).
RC_HD int skipped_tile(int x, int from, int count) { return x < from ? x : x + count; }

// A fold job's aligned interior, for a split launch: the job's tiles from 1
// on that are whole (tile 0, which also does the job's scalars, stays with
// the general kernel).  Tile t >= 1 starts at vector job_interior_vec +
// (t - 1) * tv, on a kTileAlignBytes boundary of the reference stream;
// job_interior_tiles of them are whole, from element job_interior_start.
RC_HD int64_t job_interior_vec(const JobSplit& s) { return s.lead > 0 ? s.lead : s.tv; }
RC_HD int64_t job_interior_start(const JobSplit& s) { return s.head + job_interior_vec(s) * kVec; }
RC_HD int64_t job_interior_tiles(const JobSplit& s) {
    const int64_t v = job_interior_vec(s);
    return s.tv > 0 && s.nvec > v ? (s.nvec - v) / s.tv : 0;
}

// Which ranks' outputs a job writes (each at out[r] + c*out_stride).
enum OutMode : int32_t {
    kOutMask = 0,          // the ranks in out_mask
    kOutOwner = 1,         // only rank c, the segment's owner
    kOutMaskButOwner = 2,  // the ranks in out_mask except rank c
};

RC_HD uint32_t out_mask_of(int32_t out_mode, uint32_t out_mask, int c) {
    if (out_mode == kOutOwner) return 1u << c;
    if (out_mode == kOutMaskButOwner) return out_mask & ~(1u << c);
    return out_mask;
}

// Fold operand k of job c is rank (c + 1 + k) mod R: the ring order that
// leaves segment c at its owner c.
RC_HD int fold_rank(int c, int k, int nranks) {
    const int r = c + 1 + k;
    return r >= nranks ? r - nranks : r;
}

// Whole-tile folds with outputs off a 64-byte write burst.  HBM is written
// in 64-byte bursts: a store that covers part of one costs the memory a
// read-modify-write.  A job's tiles are whole multiples of 64 bytes, so an
// output that starts the job m elements past a burst boundary starts every
// tile m elements past one (burst_offset), and with straight tiles the burst
// at each tile boundary would be written half by each of two waves.  The
// shifted whole-tile kernel writes such an output over burst-aligned ranges
// instead: tile x of T elements writes its elements [x*T - m, (x+1)*T - m),
// taking the values before its tile from pre_vectors extra vectors that it
// folds ahead of the tile; the job's first tile skips the elements before
// the job (lanes whose vector starts fewer than m elements into the shifted
// range write from element shifted_first on), and its last tile also writes
// the job's last m elements, lane l < m taking element T - m + l.  Outputs on
// a boundary are written straight, as by the unshifted kernel.
constexpr int kBurstBytes = 64;
constexpr int kBurstElems = kBurstBytes / 4;

RC_HD int burst_offset(uintptr_t addr) { return (int)((addr % kBurstBytes) / 4); }

// Vectors before the tile that a tile folds for outputs up to mmax elements
// past a burst boundary (none on the job's first tile).
RC_HD int pre_vectors(int mmax, bool first) { return first ? 0 : (mmax + kVec - 1) / kVec; }

// The first element, of the 4 in the vector w elements into the shifted
// range [x*T - m, ...), that the tile writes (4: none of them).
RC_HD int shifted_first(bool first, int64_t w, int m) { return first ? (int)min64(max64(m - w, 0), kVec) : 0; }

// Whether `lane` writes one of the job's last m elements.
RC_HD bool shifted_tail(bool last, int m, int lane) { return last && lane < m; }

// The shifted kernel's tile for workgroup bx of a job's nx: groups of
// kXcdGroup consecutive tiles per XCD.  Workgroups go to the 8 XCDs in turn,
// so without the grouping a tile's neighbour runs on another XCD and the
// 128-byte line of each operand that the tile reads ahead of itself comes
// from HBM a second time; grouped, the neighbour that read it a moment
// before shares the XCD's L2.  Tiles past the last whole group of
// 8*kXcdGroup keep their place.  A permutation of [0, nx).
constexpr int kXcdCount = 8;
constexpr int kXcdGroup = 4;
RC_HD int64_t xcd_group_tile(int64_t bx, int64_t nx) {
    constexpr int64_t span = (int64_t)kXcdCount * kXcdGroup;
    if (bx >= nx / span * span) return bx;
    return bx / span * span + (bx % kXcdCount) * kXcdGroup + (bx / kXcdCount) % kXcdGroup;
}

// LDS the shifted kernel stages a round in: the round and the kBurstElems
// elements before it.
RC_HD constexpr int shift_lds_bytes(int unroll) { return (kBurstElems + kBlock * kVec * unroll) * 4; }

// One job of a launch over a job table in device memory (the batched
// all-reduce, and copy batches too large for kernel arguments).
struct BatchJob {
    int64_t tile_begin;  // first tile of this job in the launch's tile space
    int64_t len;         // elements in the job (> 0)
    int32_t phase;       // phase_code of the job's reference stream
    int32_t pad;
};

// Batched launches index their tiles in groups of 2^kGroupShift: a tile's job
// lies between the jobs holding the first tiles of its group and of the next
// (group_job[g] is the job holding tile g << kGroupShift); a binary search
// over that range, usually empty, finds it.
constexpr int kGroupShift = 8;

RC_HD int find_job(const BatchJob* jobs, const int32_t* group_job, int64_t ngroups, int njobs, int64_t t) {
    const int64_t g = t >> kGroupShift;
    int lo = group_job[g];
    int hi = g + 1 < ngroups ? group_job[g + 1] : njobs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (jobs[mid].tile_begin <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

}  // namespace rc
