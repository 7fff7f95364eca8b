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
